"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI and the CPU oracle on the
same seeded inputs, and compare.  Routing artefacts must match bit for bit; weights within 1e-6; the
layer output within a relative Frobenius error bound."""
import sys
import time

import numpy as np
import torch

from oracle import oracle as O
from sparse_mixture_experts_08_amd import binding as B
from sparse_mixture_experts_08_amd import workloads as W

# Relative Frobenius bounds on y: bf16 1e-2 and fp8 3e-2 (the stated bars); fp32: the GPU's fp32
# accumulation against the oracle's fp64 sums at these depths stays orders of magnitude below 1e-5.
TOL = {(W.F32, W.F32): 1e-5, (W.BF16, W.BF16): 1e-2, (W.BF16, W.FP8_E4M3): 3e-2}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def host(inp):
    return {n: W.to_numpy(t) for n, t in inp.items()}


def y_to_f64(y, act_dtype):
    if act_dtype == W.F32:
        return np.asarray(y, np.float64)
    return (np.asarray(y).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def oracle_route(wl, h):
    return O.route(h["x"], h["Wg"], h.get("bias"), wl.k, wl.act_dtype)


def oracle_forward(wl, h, r, tokens=None):
    sc = {n: h.get(n) for n in ("W1s", "W3s", "W2s", "S1s", "S3s", "S2s")}
    return O.forward(wl.shape(), h["x"], h["W1"], h["W3"], h["W2"], h["S1"], h["S3"], h["S2"], r["idx"], r["w"],
                     tokens=tokens, **sc)


def check_routing(wl, gpu_r, orc):
    """gpu_r: device tensors from moe_route; orc: oracle dict."""
    g = {k: v.cpu().numpy() for k, v in gpu_r.items()}
    assert np.array_equal(g["idx"], orc["idx"]), "idx differs"
    assert np.array_equal(g["counts"], orc["counts"]), "counts differ"
    assert np.array_equal(g["offsets"], orc["offsets"]), "offsets differ"
    assert np.array_equal(g["sorted_slots"], orc["sorted_slots"]), "sorted_slots differ"
    assert np.array_equal(g["pos"], orc["pos"]), "pos differs"
    dw = np.abs(g["w"].astype(np.float64) - orc["w"].astype(np.float64)).max()
    assert dw <= 1e-6, f"w differs by {dw}"


def rel_fro(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    n = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (n if n > 0 else 1.0))


def run_parity(wl, inp, tokens=None, check_route=True):
    """Full comparison of one workload whose inputs `inp` are on the GPU.  Returns the error."""
    say(f"[parity] {wl.name} shape={wl.shape()} sample={'all' if tokens is None else len(tokens)}")
    t0 = time.time()
    y, rt = B.forward_inputs(inp, wl.k, routing=True)
    rr = B.moe_route(inp["x"], inp["Wg"], inp.get("bias"), wl.k) if check_route else None
    torch.cuda.synchronize()
    say(f"  gpu done {time.time() - t0:.1f}s")
    h = host(inp)
    orc = oracle_route(wl, h)
    say(f"  oracle routing done {time.time() - t0:.1f}s")
    if check_route:
        check_routing(wl, rr, orc)
    assert np.array_equal(rt["idx"].cpu().numpy(), orc["idx"]) and np.array_equal(rt["counts"].cpu().numpy(), orc["counts"])
    out, yref = oracle_forward(wl, h, orc, tokens)
    say(f"  oracle forward done {time.time() - t0:.1f}s")
    yg = y.cpu()
    if tokens is not None:
        yg = yg[torch.as_tensor(tokens, dtype=torch.long)]
    err = rel_fro(y_to_f64(W.to_numpy(yg), wl.act_dtype), y_to_f64(yref, wl.act_dtype))
    say(f"  rel_fro={err:.3e} (bound {TOL[(wl.act_dtype, wl.w_dtype)]})")
    assert err <= TOL[(wl.act_dtype, wl.w_dtype)], err
    return err
