"""Benchmark of the MoE feed-forward layer forward pass on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

A step is one moe_forward call (router, top-k, permutation, grouped up GEMM with the shared expert,
grouped down GEMM, combine) over one batch of synthetic tokens already resident in HBM.  Prints one JSON
line: tokens/s, the dominant kernel's roofline figures (its average duration from HIP events recorded
around it on the launch stream, over the timed steps) and the CPU oracle timed on a bounded sample.
"""
import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from sparse_mixture_experts_08_amd import binding as B  # noqa: E402
from sparse_mixture_experts_08_amd import workloads as W  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_PEAK_TFLOPS = {W.BF16: 2500.0, W.FP8_E4M3: 5000.0, W.F32: 157.3}


class HipEvents:
    """A set of hipEvent_t handles created through the HIP runtime (timing enabled)."""

    def __init__(self, n):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.arr = (ctypes.c_void_p * n)()
        for i in range(n):
            slot = ctypes.cast(ctypes.addressof(self.arr) + i * ctypes.sizeof(ctypes.c_void_p),
                               ctypes.POINTER(ctypes.c_void_p))
            if self.hip.hipEventCreate(slot):
                raise RuntimeError("hipEventCreate failed")

    def elapsed_ms(self, i, j):
        self.hip.hipEventSynchronize(self.arr[j])
        ms = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), self.arr[i], self.arr[j]):
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def close(self):
        for i in range(len(self.arr)):
            self.hip.hipEventDestroy(self.arr[i])


def algorithmic(wl, counts):
    """Algorithmic bytes and flops of the up GEMM, the down GEMM and the whole layer for this routing."""
    wb = {W.F32: 4, W.BF16: 2, W.FP8_E4M3: 1}[wl.w_dtype]
    ab = 4 if wl.act_dtype == W.F32 else 2
    touched = int((counts > 0).sum())
    rows = wl.T * wl.k + wl.T
    sblk = 4.0 / (128 * 128) if wl.w_dtype == W.FP8_E4M3 else 0.0      # fp32 block scale per 128x128
    up_w = (touched * wl.inter + wl.inter_shared) * 2 * wl.d * (wb + sblk)
    dn_w = (touched * wl.inter + wl.inter_shared) * wl.d * (wb + sblk)
    up_bytes = up_w + wl.T * wl.d * ab + rows * (wl.inter if wl.inter >= wl.inter_shared else wl.inter_shared) * ab
    dn_bytes = dn_w + rows * wl.d * ab
    up_flops = 2.0 * 2 * wl.d * (wl.T * wl.k * wl.inter + wl.T * wl.inter_shared)
    dn_flops = 2.0 * wl.d * (wl.T * wl.k * wl.inter + wl.T * wl.inter_shared)
    layer_bytes = up_w + dn_w + wl.d * wl.E * 4 + 2 * wl.T * wl.d * ab
    return dict(touched=touched, up_bytes=up_bytes, dn_bytes=dn_bytes, up_flops=up_flops, dn_flops=dn_flops,
                layer_bytes=layer_bytes, layer_flops=up_flops + dn_flops + 2.0 * wl.T * wl.d * wl.E)


def measured_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE summary, if it
    was taken on the current GEMM source (else None)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        rec = json.load(open(path))[workload]
    except (OSError, KeyError, ValueError):
        return None
    src = os.path.join(ROOT, "sparse_mixture_experts_08_amd", "csrc", "gemm.hip")
    if hashlib.sha256(open(src, "rb").read()).hexdigest()[:16] != rec.get("gemm_source_sha256_16"):
        return None
    k = rec.get(kernel)
    return None if not k else k["bytes"]


def cpu_baseline(wl, inp, max_tokens):
    """The CPU oracle on a bounded sample of the same workload: routing of every token plus experts and
    combine for up to max_tokens tokens; tokens/s from the per-token cost of both parts."""
    from oracle import oracle as O
    h = {n: W.to_numpy(t) for n, t in inp.items()}
    t0 = time.perf_counter()
    r = O.route(h["x"], h["Wg"], h.get("bias"), wl.k, wl.act_dtype)
    t_route = time.perf_counter() - t0
    n = min(max_tokens, wl.T)
    toks = np.arange(n, dtype=np.int32)
    sc = {k: h.get(k) for k in ("W1s", "W3s", "W2s", "S1s", "S3s", "S2s")}
    t0 = time.perf_counter()
    O.forward(wl.shape(), h["x"], h["W1"], h["W3"], h["W2"], h["S1"], h["S3"], h["S2"], r["idx"], r["w"],
              tokens=toks, **sc)
    t_fwd = time.perf_counter() - t0
    per_token = t_route / wl.T + t_fwd / n
    return {"value": 1.0 / per_token, "unit": "tokens/s", "cores": O.num_threads(), "kind": "oracle",
            "sample": f"routing of all {wl.T} tokens ({t_route:.2f} s) + experts and combine of {n} tokens "
                      f"({t_fwd:.2f} s); tokens/s = 1 / (route s/token + expert s/token)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=W.DECODE_BF16.name, choices=[w.name for w in W.CONFIGS])
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=64)
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after the timed steps, one plain device copy of this many MiB (a known-size reference "
                         "for hardware byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this layer runs unsharded on a single MI355X (asked for --gpus "
              f"{args.gpus}); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)

    wl = W.BY_NAME[args.workload]
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    inp = W.generate(wl, seed=args.seed, device=dev)
    shape = B.make_shape(wl.T, wl.d, wl.E, wl.k, wl.inter, wl.inter_shared, wl.act_dtype, wl.w_dtype)
    ws = torch.empty(B.moe_workspace_size(shape), dtype=torch.uint8, device=dev)
    y = torch.empty_like(inp["x"])
    _, r = B.forward_inputs(inp, wl.k, y=y, workspace=ws, routing=True)
    torch.cuda.synchronize()
    alg = algorithmic(wl, r["counts"].cpu().numpy())

    # headline: plain moe_forward steps
    for _ in range(args.warmup):
        B.forward_inputs(inp, wl.k, y=y, workspace=ws)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        B.forward_inputs(inp, wl.k, y=y, workspace=ws)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    ms_per_step = dt * 1e3 / args.steps

    # per-stage device time: HIP events recorded between stages on the launch stream
    ns = B.NUM_STAGES
    ev = HipEvents((ns + 1) * args.steps)
    for s in range(args.steps):
        sub = (ctypes.c_void_p * (ns + 1)).from_buffer(ev.arr, s * (ns + 1) * ctypes.sizeof(ctypes.c_void_p))
        B.forward_inputs(inp, wl.k, y=y, workspace=ws, events=sub)
    torch.cuda.synchronize()
    stage_ms = np.zeros(ns)
    for s in range(args.steps):
        for i in range(ns):
            stage_ms[i] += ev.elapsed_ms(s * (ns + 1) + i, s * (ns + 1) + i + 1)
    stage_ms /= args.steps
    ev.close()

    up_ms, dn_ms = stage_ms[4], stage_ms[5]
    # the binding roofline of the up GEMM: the larger of its HBM time and its MFMA time at peak
    hbm_bound = alg["up_bytes"] / (HBM_PEAK_GBS * 1e9) >= alg["up_flops"] / (MFMA_PEAK_TFLOPS[wl.w_dtype] * 1e12)
    if hbm_bound:
        roof = {"bound": "hbm", "achieved": alg["up_bytes"] / (up_ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS,
                "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": alg["up_flops"] / (up_ms * 1e-3) / 1e12,
                "peak": MFMA_PEAK_TFLOPS[wl.w_dtype], "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = measured_traffic(wl.name, "up_gemm")
    roof["kernel"] = "grouped up GEMM (W1, W3, SiLU*mul; routed + shared)"
    roof["kernel_ms"] = up_ms

    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    out = {
        "metric": "MoE-layer tokens/s at d=7168, 256 experts top-8; % of HBM or MFMA roofline",
        "value": wl.T / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {W.F32: "f32", W.BF16: "bf16", W.FP8_E4M3: "fp8_e4m3"}[wl.w_dtype],
        "data": "synthetic",
        "config": {"workload": wl.name, "T": wl.T, "d": wl.d, "E": wl.E, "k": wl.k, "inter": wl.inter,
                   "inter_shared": wl.inter_shared, "parallelism": "none (one GPU)"},
        "roofline": roof,
        "layer": {"algorithmic_GB": alg["layer_bytes"] / 1e9, "touched_experts": alg["touched"],
                  "GB_per_s": alg["layer_bytes"] / (ms_per_step * 1e-3) / 1e9,
                  "hbm_frac": alg["layer_bytes"] / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
                  "TFLOP_per_s": alg["layer_flops"] / (ms_per_step * 1e-3) / 1e12,
                  "stage_ms": {n: float(v) for n, v in zip(B.STAGE_NAMES, stage_ms)},
                  "down_gemm_GB_per_s": alg["dn_bytes"] / (dn_ms * 1e-3) / 1e9 if dn_ms > 0 else None},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, inp, args.cpu_tokens)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
