"""Seeded synthetic workloads for the MoE feed-forward layer.

This module only draws inputs; it holds none of the layer's arithmetic.  Both the HIP path and the CPU
oracle consume the tensors it returns.  Shapes follow the DeepSeek-V3 layer described on
"DeepSeek-V3.2-Exp / Mixture of experts / Shared expert" ("Exact per-instance accounting": 7168 x 2048
projections) and "DeepSeek-V3 Architecture: MoE Design, Specifications, and API Fit" (spec table: 256
routed experts + 1 shared, 8 activated per token).

Recipe (per tensor tag a torch.Generator seeded with seed * 1000 + tag id, on the requested device):
  x ~ N(0, 1);  Wg, W1, W3, S1, S3 ~ N(0, 1/d);  W2 ~ N(0, 1/inter);  S2 ~ N(0, 1/inter_shared).
  bf16 tensors are the fp32 draws rounded to nearest-even by torch.
  fp8 tensors: per 128x128 block, s = U * amax / 448 with U ~ U[0.5, 2] (tag "U"), and the code is torch's
  float8_e4m3fn rounding of clamp(W / s, -448, 448).  (codes, scales) define the weight.
  Skewed routing: bias[e] = -1.2 * ln(rank_e) over a seeded permutation pi (expert pi[r-1] has rank r),
  i.e. the logit bias log(p_e) + const for p_e proportional to rank_e^-1.2.
Draws depend on the device (torch's CPU and GPU generators differ); every comparison draws once and
hands the same tensors to both sides.
"""
from dataclasses import dataclass, replace
import math

import torch

F32, BF16, FP8_E4M3 = 0, 1, 2
DTYPE_NAMES = {F32: "f32", BF16: "bf16", FP8_E4M3: "fp8_e4m3"}

_TAGS = {"x": 1, "Wg": 2, "W1": 3, "W3": 4, "W2": 5, "S1": 6, "S3": 7, "S2": 8, "perm": 9, "U": 10}


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    d: int
    E: int
    k: int
    inter: int
    inter_shared: int
    act_dtype: int
    w_dtype: int
    skew: bool = False

    def shape(self) -> dict:
        return dict(T=self.T, d=self.d, E=self.E, k=self.k, inter=self.inter, inter_shared=self.inter_shared,
                    act_dtype=self.act_dtype, w_dtype=self.w_dtype)

    def with_T(self, T: int) -> "Workload":
        return replace(self, T=T, name=f"{self.name}@T{T}")


# The five measured configurations.
TINY_F32 = Workload("tiny-fp32-T128-d512-E32-k4", 128, 512, 32, 4, 256, 256, F32, F32)
DECODE_BF16 = Workload("decode-bf16-T64-d7168-E256-k8", 64, 7168, 256, 8, 2048, 2048, BF16, BF16)
PREFILL_BF16 = Workload("prefill-bf16-T4096-d7168-E256-k8", 4096, 7168, 256, 8, 2048, 2048, BF16, BF16)
SKEW_BF16 = Workload("skewed-bf16-T16384-d7168-E256-k8", 16384, 7168, 256, 8, 2048, 2048, BF16, BF16, skew=True)
FP8_T32768 = Workload("fp8-T32768-d7168-E256-k8", 32768, 7168, 256, 8, 2048, 2048, BF16, FP8_E4M3)

CONFIGS = [TINY_F32, DECODE_BF16, PREFILL_BF16, SKEW_BF16, FP8_T32768]
BY_NAME = {w.name: w for w in CONFIGS}


def _gen(seed: int, tag: str, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed * 1000 + _TAGS[tag])
    return g


def _normal(shape, std, gen, device):
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32) * std


def _fp8_blocks(wf: torch.Tensor, u: torch.Tensor):
    """fp32 [R, C] -> (E4M3 codes as uint8 [R, C], fp32 scales [R/128, C/128])."""
    R, C = wf.shape
    blk = wf.view(R // 128, 128, C // 128, 128)
    amax = blk.abs().amax(dim=(1, 3))
    s = (u * amax / 448.0).to(torch.float32)
    s = torch.where(s > 0, s, torch.ones_like(s))
    q = (blk / s[:, None, :, None]).clamp(-448.0, 448.0).view(R, C).to(torch.float8_e4m3fn)
    return q.view(torch.uint8), s


def _weight_stack(n, rows, cols, std, seed, tag, device, w_dtype, stack: bool):
    """n matrices [rows, cols] drawn one by one (bounded temporaries).  Returns (W, scales or None)."""
    g = _gen(seed, tag, device)
    gu = _gen(seed, "U", device) if w_dtype == FP8_E4M3 else None
    if gu is not None:  # separate U stream per tag: skip ahead by the tag id so tags differ
        gu.manual_seed(seed * 1000 + _TAGS["U"] * 100 + _TAGS[tag])
    wdt = {F32: torch.float32, BF16: torch.bfloat16, FP8_E4M3: torch.uint8}[w_dtype]
    shape = (n, rows, cols) if stack else (rows, cols)
    W = torch.empty(shape, dtype=wdt, device=device)
    S = None
    if w_dtype == FP8_E4M3:
        S = torch.empty(((n,) if stack else ()) + (rows // 128, cols // 128), dtype=torch.float32, device=device)
    for e in range(n if stack else 1):
        wf = _normal((rows, cols), std, g, device)
        dst = W[e] if stack else W
        if w_dtype == FP8_E4M3:
            u = torch.rand((rows // 128, cols // 128), generator=gu, device=device) * 1.5 + 0.5
            q, s = _fp8_blocks(wf, u)
            dst.copy_(q)
            (S[e] if stack else S).copy_(s)
        else:
            dst.copy_(wf.to(wdt))
    return W, S


def skew_bias(E: int, seed: int, device="cpu") -> torch.Tensor:
    g = _gen(seed, "perm", "cpu")
    perm = torch.randperm(E, generator=g)
    bias = torch.empty(E, dtype=torch.float64)
    bias[perm] = -1.2 * torch.log(torch.arange(1, E + 1, dtype=torch.float64))
    return bias.to(torch.float32).to(device)


def generate(wl: Workload, seed: int = 0, device="cpu", weights=True) -> dict:
    """All inputs of one layer invocation as torch tensors on `device`.

    Keys: x [T,d]; Wg [E,d] fp32 (the gate's nn.Linear weight); bias [E] fp32 or None; W1, W3 [E,inter,d]; W2 [E,d,inter];
    S1, S3 [inter_s,d]; S2 [d,inter_s]; fp8 only: W1s, W3s [E,inter/128,d/128], W2s [E,d/128,inter/128],
    S1s, S3s [inter_s/128,d/128], S2s [d/128,inter_s/128].
    """
    act = torch.float32 if wl.act_dtype == F32 else torch.bfloat16
    out = {}
    out["x"] = _normal((wl.T, wl.d), 1.0, _gen(seed, "x", device), device).to(act)
    out["Wg"] = _normal((wl.E, wl.d), 1.0 / math.sqrt(wl.d), _gen(seed, "Wg", device), device)
    out["bias"] = skew_bias(wl.E, seed, device) if wl.skew else None
    if not weights:
        return out
    sd, si, ss = 1.0 / math.sqrt(wl.d), 1.0 / math.sqrt(wl.inter), 1.0 / math.sqrt(wl.inter_shared)
    out["W1"], out["W1s"] = _weight_stack(wl.E, wl.inter, wl.d, sd, seed, "W1", device, wl.w_dtype, True)
    out["W3"], out["W3s"] = _weight_stack(wl.E, wl.inter, wl.d, sd, seed, "W3", device, wl.w_dtype, True)
    out["W2"], out["W2s"] = _weight_stack(wl.E, wl.d, wl.inter, si, seed, "W2", device, wl.w_dtype, True)
    out["S1"], out["S1s"] = _weight_stack(1, wl.inter_shared, wl.d, sd, seed, "S1", device, wl.w_dtype, False)
    out["S3"], out["S3s"] = _weight_stack(1, wl.inter_shared, wl.d, sd, seed, "S3", device, wl.w_dtype, False)
    out["S2"], out["S2s"] = _weight_stack(1, wl.d, wl.inter_shared, ss, seed, "S2", device, wl.w_dtype, False)
    return out


def to_numpy(t):
    """Host numpy view for the oracle: bf16 -> uint16 bits, fp8 codes stay uint8."""
    if t is None:
        return None
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.uint16).numpy() if hasattr(torch, "uint16") else t.view(torch.int16).numpy().view("uint16")
    return t.numpy()


def weight_shapes(wl: Workload) -> dict:
    """Shapes of the weight tensors `generate` returns (no allocation)."""
    return dict(Wg=(wl.E, wl.d), W1=(wl.E, wl.inter, wl.d), W3=(wl.E, wl.inter, wl.d), W2=(wl.E, wl.d, wl.inter),
                S1=(wl.inter_shared, wl.d), S3=(wl.inter_shared, wl.d), S2=(wl.d, wl.inter_shared))
