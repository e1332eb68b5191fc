"""Benchmark of the MoE feed-forward layer forward pass on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--variant V] [--no-cpu-baseline]

A step is one moe_forward call (router, top-k, permutation, grouped up GEMM with the shared expert,
grouped down GEMM, combine) over one batch of synthetic tokens already resident in HBM.  Prints one JSON
line: tokens/s, the dominant kernel's roofline figures (its average duration from HIP events recorded
around it on the launch stream, over the timed steps) and the CPU oracle timed on a bounded sample.

--variant selects another entry point on the same workload (one JSON line each):
  shard-ep8      moe_forward_shard of one of 8 expert-parallel ranks (E/8 experts, 1/8 of the shared
                 expert's features; the all-reduce over ranks is not part of it)
  route-limited  moe_route_limited with the experts of one of 8 devices allowed
  route-grouped  moe_route_grouped: two experts from each of the k / 2 best of 8 expert groups
  utilization    moe_expert_utilization over the workload's expert counts
"""
import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from sparse_mixture_experts_08_amd import binding as B  # noqa: E402
from sparse_mixture_experts_08_amd.build import code_fingerprint  # noqa: E402
from sparse_mixture_experts_08_amd import workloads as W  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_PEAK_TFLOPS = {W.BF16: 2500.0, W.FP8_E4M3: 5000.0, W.F32: 157.3}
# fp32 vector peak without packed FMA (the kernels are compiled with packed fp32 ops off): 256 CUs x 4 SIMDs x 16 lanes x 2 flops x 2.4 GHz
FP32_VALU_PEAK_TFLOPS = 78.6
# the router's logit kernel: fp32 FMA chains on the vector ALU up to this many tokens, fp32 MFMA above
ROUTER_FEW_MAX_T = 512
PROBE_LIB = os.path.join(ROOT, "sparse_mixture_experts_08_amd", "libmoe_probe.so")


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


def measured_peaks(dev, read_gib=16, reps=3):
    """What this GPU sustains, as the measured denominators of the roofline fractions: a streaming read of
    read_gib GiB (far beyond the 256 MB last-level cache) with libmoe_probe.so's read kernel; back-to-back
    bf16 and fp8 MFMAs (eight independent chains per wavefront, two wavefronts per SIMD) with its MFMA
    kernel; and a large dense bf16 GEMM through torch.matmul (the vendor library).  Best of `reps` runs."""
    L = ctypes.CDLL(PROBE_LIB)
    L.moe_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_uint, ctypes.c_void_p,
                                        ctypes.c_void_p]
    L.moe_probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_uint, ctypes.c_void_p,
                                 ctypes.POINTER(ctypes.c_double), ctypes.c_void_p]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    out = {}
    nbytes = read_gib << 30
    buf = torch.ones(nbytes, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1 << 16, dtype=torch.int32, device=dev)
    grid = 8192

    def read():
        if L.moe_probe_stream_read(ctypes.c_void_p(buf.data_ptr()), nbytes, grid, ctypes.c_void_p(sink.data_ptr()),
                                   stream):
            raise RuntimeError("moe_probe_stream_read failed")
    read()
    out["hbm_read_GBs"] = max(nbytes / (event_ms(read, 1) * 1e-3) / 1e9 for _ in range(reps))
    del buf
    torch.cuda.empty_cache()
    flops = ctypes.c_double()
    for name, dt in (("mfma_bf16_TFLOPs", 1), ("mfma_fp8_TFLOPs", 2)):
        def mfma():
            if L.moe_probe_mfma(dt, 20000, 512, ctypes.c_void_p(sink.data_ptr()), ctypes.byref(flops), stream):
                raise RuntimeError("moe_probe_mfma failed")
        mfma()
        out[name] = max(flops.value / (event_ms(mfma, 1) * 1e-3) / 1e12 for _ in range(reps))
    a = torch.randn(8192, 8192, device=dev).to(torch.bfloat16)
    b = torch.randn(8192, 8192, device=dev).to(torch.bfloat16)
    c = torch.empty(8192, 8192, device=dev, dtype=torch.bfloat16)
    torch.matmul(a, b, out=c)
    out["gemm_bf16_TFLOPs"] = max(2.0 * 8192 ** 3 / (event_ms(lambda: torch.matmul(a, b, out=c), 5) * 1e-3) / 1e12
                                  for _ in range(reps))
    del a, b, c
    torch.cuda.empty_cache()
    out["how"] = (f"streaming read of {read_gib} GiB ({grid} blocks of 256 threads, each reading 256 KB chunks with "
                  "16-byte non-temporal loads); 2048 wavefronts "
                  "x 8 chains of back-to-back v_mfma_f32_32x32x16_bf16 / v_mfma_scale_f32_16x16x128_f8f6f4; "
                  "torch.matmul bf16 8192^3; best of 3")
    return out


def with_measured(roof, peaks, w_dtype):
    """Adds the fraction against the measured ceiling of the roofline's bound to a roofline dict."""
    if peaks is None:
        return roof
    key = {"hbm": "hbm_read_GBs", "mfma": {W.BF16: "mfma_bf16_TFLOPs", W.FP8_E4M3: "mfma_fp8_TFLOPs"}.get(w_dtype)}
    k = key.get(roof["bound"])
    if k:
        roof["peak_measured"] = peaks[k]
        roof["frac_measured"] = roof["achieved"] / peaks[k]
    return roof


def algorithmic(wl, counts, e0=0, e1=None, n_shared=None):
    """Algorithmic bytes and flops of the up GEMM, the down GEMM and the whole call for this routing, over
    the routed experts [e0, e1) and n_shared shared features (default: the whole layer)."""
    e1 = wl.E if e1 is None else e1
    n_shared = wl.inter_shared if n_shared is None else n_shared
    wb = {W.F32: 4, W.BF16: 2, W.FP8_E4M3: 1}[wl.w_dtype]
    ab = 4 if wl.act_dtype == W.F32 else 2
    c = counts[e0:e1]
    touched = int((c > 0).sum())
    routed_rows = int(c.sum())
    shared_rows = wl.T if n_shared else 0
    rows = routed_rows + shared_rows
    sblk = 4.0 / (128 * 128) if wl.w_dtype == W.FP8_E4M3 else 0.0      # fp32 block scale per 128x128
    up_w = (touched * wl.inter + n_shared) * 2 * wl.d * (wb + sblk)
    dn_w = (touched * wl.inter + n_shared) * wl.d * (wb + sblk)
    # h is written by the up GEMM and read by the down GEMM; fp8 weights store it as E4M3 codes
    hb = 1 + 4.0 / 128 if wl.w_dtype == W.FP8_E4M3 else ab
    h_bytes = (routed_rows * wl.inter + shared_rows * n_shared) * hb
    up_bytes = up_w + wl.T * wl.d * ab + h_bytes
    dn_bytes = dn_w + h_bytes + rows * wl.d * ab
    up_flops = 2.0 * 2 * wl.d * (routed_rows * wl.inter + shared_rows * n_shared)
    dn_flops = 2.0 * wl.d * (routed_rows * wl.inter + shared_rows * n_shared)
    full = e0 == 0 and e1 == wl.E and n_shared == wl.inter_shared
    out_b = wl.T * wl.d * (ab if full else 4)
    layer_bytes = up_w + dn_w + wl.d * wl.E * 4 + wl.T * wl.d * ab + out_b
    return dict(touched=touched, up_bytes=up_bytes, dn_bytes=dn_bytes, up_flops=up_flops, dn_flops=dn_flops,
                layer_bytes=layer_bytes, layer_flops=up_flops + dn_flops + 2.0 * wl.T * wl.d * wl.E)


def measured_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE summary, if it
    was taken on the current GEMM code (its comment-free fingerprint; else None)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        rec = json.load(open(path))[workload]
    except (OSError, KeyError, ValueError):
        return None
    src = os.path.join(ROOT, "sparse_mixture_experts_08_amd", "csrc", "gemm.hip")
    if code_fingerprint(src) != rec.get("gemm_code_sha256_16"):
        return None
    k = rec.get(kernel)
    return None if not k else k["bytes"]


def cpu_baseline(wl, inp, max_tokens, shard=None, min_seconds=10.0):
    """The CPU oracle on a bounded sample of the same workload: routing of every token plus experts and
    combine for up to max_tokens tokens, the latter repeated until about min_seconds of CPU work (at most
    8 passes); tokens/s from the per-token cost of both parts.  With shard = (e0, e1, s0, s1): the
    oracle's expert-parallel partial of that rank instead of the whole layer."""
    from oracle import oracle as O
    h = {n: W.to_numpy(t) for n, t in inp.items()}
    t0 = time.perf_counter()
    r = O.route(h["x"], h["Wg"], h.get("bias"), wl.k, wl.act_dtype)
    t_route = time.perf_counter() - t0
    n = min(max_tokens, wl.T)
    toks = np.arange(n, dtype=np.int32)
    sc = {k: h.get(k) for k in ("W1s", "W3s", "W2s", "S1s", "S3s", "S2s")}
    t_fwd, passes = 0.0, 0
    while passes < 8 and (passes == 0 or t_fwd < min_seconds):
        t0 = time.perf_counter()
        if shard is None:
            O.forward(wl.shape(), h["x"], h["W1"], h["W3"], h["W2"], h["S1"], h["S3"], h["S2"], r["idx"], r["w"],
                      tokens=toks, **sc)
        else:
            O.forward_shard(wl.shape(), h["x"], h["W1"], h["W3"], h["W2"], h["S1"], h["S3"], h["S2"], r["idx"],
                            r["w"], *shard, tokens=toks, **sc)
        t_fwd += time.perf_counter() - t0
        passes += 1
    per_token = t_route / wl.T + t_fwd / (n * passes)
    return {"value": 1.0 / per_token, "unit": "tokens/s", "cores": len(os.sched_getaffinity(0)),
            "omp_threads": O.num_threads(), "kind": "oracle",
            "sample": f"routing of all {wl.T} tokens ({t_route:.2f} s) + experts and combine of {n} tokens, "
                      f"{passes} passes ({t_fwd:.2f} s); tokens/s = 1 / (route s/token + expert s/token)"}


def roofline_of(bytes_, flops, ms, peak_tflops, kernel):
    """Roofline figures of one kernel: bound by whichever of HBM bytes and MFMA flops takes longer at peak."""
    if bytes_ / (HBM_PEAK_GBS * 1e9) >= flops / (peak_tflops * 1e12):
        roof = {"bound": "hbm", "achieved": bytes_ / (ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": flops / (ms * 1e-3) / 1e12, "peak": peak_tflops, "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["kernel"] = kernel
    roof["kernel_ms"] = ms
    return roof


def wall_ms(fn, steps, warmup):
    """Wall-clock ms per call of fn over `steps` calls after `warmup`, synchronised on both sides."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


def staged_ms(fn, steps):
    """Mean device ms of each stage: fn(events) records NUM_STAGES + 1 HIP events on the launch stream."""
    ns = B.NUM_STAGES
    ev = HipEvents((ns + 1) * steps)
    for s in range(steps):
        fn((ctypes.c_void_p * (ns + 1)).from_buffer(ev.arr, s * (ns + 1) * ctypes.sizeof(ctypes.c_void_p)))
    torch.cuda.synchronize()
    stage = np.zeros(ns)
    for s in range(steps):
        for i in range(ns):
            stage[i] += ev.elapsed_ms(s * (ns + 1) + i, s * (ns + 1) + i + 1)
    ev.close()
    return stage / steps


def event_ms(fn, steps):
    """Mean device ms of one fn() call from HIP events recorded around each call on torch's stream."""
    ev = HipEvents(2 * steps)
    hip = ev.hip
    hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for s in range(steps):
        hip.hipEventRecord(ev.arr[2 * s], stream)
        fn()
        hip.hipEventRecord(ev.arr[2 * s + 1], stream)
    torch.cuda.synchronize()
    ms = sum(ev.elapsed_ms(2 * s, 2 * s + 1) for s in range(steps)) / steps
    ev.close()
    return ms


def ep8_ranges(wl, rank):
    """Experts and shared features of expert-parallel rank `rank` of 8."""
    if wl.E % 8 or wl.inter_shared % (8 * 128):
        raise SystemExit(f"{wl.name}: E and inter_shared / 128 must split 8 ways for shard-ep8")
    ne, ns = wl.E // 8, wl.inter_shared // 8
    return rank * ne, (rank + 1) * ne, rank * ns, (rank + 1) * ns


def base_record(wl, args, metric, value, unit, ms, higher=True):
    return {
        "metric": metric, "value": value, "unit": unit, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": higher, "scaling": "weak", "vs_baseline": None,
        "dtype": {W.F32: "f32", W.BF16: "bf16", W.FP8_E4M3: "fp8_e4m3"}[wl.w_dtype], "data": "synthetic",
        "config": {"workload": wl.name, "T": wl.T, "d": wl.d, "E": wl.E, "k": wl.k, "inter": wl.inter,
                   "inter_shared": wl.inter_shared, "parallelism": "none (one GPU)"},
    }


def run_layer(wl, inp, args, dev):
    shape = B.make_shape(wl.T, wl.d, wl.E, wl.k, wl.inter, wl.inter_shared, wl.act_dtype, wl.w_dtype)
    ws = torch.empty(B.moe_workspace_size(shape), dtype=torch.uint8, device=dev)
    shard = None
    if args.variant == "shard-ep8":
        shard = ep8_ranges(wl, args.rank)
        lw = B.shard_weights(inp, *shard)
        e0, e1, s0, s1 = shard
        yp = torch.empty((wl.T, wl.d), dtype=torch.float32, device=dev)
        sc = {n: lw[n] for n in ("W1s", "W3s", "W2s", "S1s", "S3s", "S2s") if n in lw} or None

        def call(events=None, routing=False):
            return B.moe_forward_shard(inp["x"], inp["Wg"], inp.get("bias"), wl.k, e0, e1, lw["W1"], lw["W3"],
                                       lw["W2"], lw["S1"], lw["S3"], lw["S2"], wl.inter, wl.inter_shared,
                                       scales=sc, y_partial=yp, workspace=ws, routing=routing, events=events)
    else:
        y = torch.empty_like(inp["x"])

        def call(events=None, routing=False):
            return B.forward_inputs(inp, wl.k, y=y, workspace=ws, routing=routing, events=events)
    _, r = call(routing=True)
    torch.cuda.synchronize()
    counts = r["counts"].cpu().numpy()
    alg = algorithmic(wl, counts) if shard is None else algorithmic(wl, counts, shard[0], shard[1],
                                                                    shard[3] - shard[2])
    ms_per_step = wall_ms(call, args.steps, args.warmup)
    stage_ms = staged_ms(lambda ev: call(events=ev), args.steps)
    up_ms, dn_ms = stage_ms[4], stage_ms[5]
    roof = roofline_of(alg["up_bytes"], alg["up_flops"], up_ms, MFMA_PEAK_TFLOPS[wl.w_dtype],
                       "grouped up GEMM (W1, W3, SiLU*mul; routed + shared)")
    roof["traffic"] = measured_traffic(wl.name if shard is None else f"{wl.name}/shard-ep8", "up_gemm")
    # keep the documented key order: bound, achieved, peak, unit, frac, traffic
    roof = {k: roof[k] for k in ("bound", "achieved", "peak", "unit", "frac", "traffic", "kernel", "kernel_ms")}
    peaks = None if args.no_peaks else measured_peaks(dev)
    roof = with_measured(roof, peaks, wl.w_dtype)

    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    if shard is None:
        metric = "MoE-layer tokens/s at d=7168, 256 experts top-8; % of HBM or MFMA roofline"
    else:
        metric = (f"expert-parallel rank {args.rank}/8 tokens/s (experts [{shard[0]},{shard[1]}), shared features "
                  f"[{shard[2]},{shard[3]}); fp32 partial, all-reduce excluded)")
    out = base_record(wl, args, metric, wl.T / (ms_per_step * 1e-3), "tokens/s", ms_per_step)
    if shard is not None:
        out["config"]["parallelism"] = f"ep8 rank {args.rank} (one GPU's share)"
    out["roofline"] = roof
    out["peaks_measured"] = peaks
    out["layer"] = {"algorithmic_GB": alg["layer_bytes"] / 1e9, "touched_experts": alg["touched"],
                    "GB_per_s": alg["layer_bytes"] / (ms_per_step * 1e-3) / 1e9,
                    "hbm_frac": alg["layer_bytes"] / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
                    "TFLOP_per_s": alg["layer_flops"] / (ms_per_step * 1e-3) / 1e12,
                    "stage_ms": {n: float(v) for n, v in zip(B.STAGE_NAMES, stage_ms)},
                    "down_gemm_GB_per_s": alg["dn_bytes"] / (dn_ms * 1e-3) / 1e9 if dn_ms > 0 else None}
    # the gate's logits on their own roofline: fp32 FMA chains on the vector ALU up to ROUTER_FEW_MAX_T
    # tokens, fp32 MFMA (K = 1 steps) above
    router_ms = stage_ms[0]
    if router_ms > 0:
        on_mfma = wl.T > ROUTER_FEW_MAX_T
        rpeak = MFMA_PEAK_TFLOPS[W.F32] if on_mfma else FP32_VALU_PEAK_TFLOPS
        rt = 2.0 * wl.T * wl.d * wl.E / (router_ms * 1e-3) / 1e12
        out["layer"]["router"] = {"unit": "mfma fp32" if on_mfma else "valu fp32", "TFLOP_per_s": rt,
                                  "peak_TFLOPs": rpeak, "frac": rt / rpeak}
    out["cpu_baseline"] = None
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, inp, args.cpu_tokens, shard, args.cpu_seconds)
    return out


def run_route(wl, inp, args, dev, grouped):
    """Routing alone: device-limited (the experts of device `rank` of 8, contiguous blocks of E/8, as a
    device_expert_map would list them) or group-limited (8 groups, two experts from each of k / 2)."""
    ne = max(wl.E // 8, wl.k)
    allowed = torch.zeros(wl.E, dtype=torch.uint8)
    allowed[args.rank * ne:(args.rank + 1) * ne] = 1
    a_dev = allowed.to(dev)
    n_group = 8
    shape = B.make_shape(wl.T, wl.d, wl.E, wl.k, 128, 128, wl.act_dtype, wl.act_dtype)
    ws = torch.empty(B.moe_workspace_size(shape), dtype=torch.uint8, device=dev)
    if grouped:
        call = lambda: B.moe_route_grouped(inp["x"], inp["Wg"], inp.get("bias"), wl.k, n_group, workspace=ws)  # noqa
    else:
        call = lambda: B.moe_route_limited(inp["x"], inp["Wg"], inp.get("bias"), a_dev, wl.k, workspace=ws)  # noqa
    ms_per_step = wall_ms(call, args.steps, args.warmup)
    dev_ms = event_ms(call, args.steps)
    ab = 4 if wl.act_dtype == W.F32 else 2
    bytes_ = wl.T * wl.d * ab + wl.d * wl.E * 4 + wl.E + wl.T * wl.k * (4 + 4 + 4 + 4) + (2 * wl.E + 1) * 4
    flops = 2.0 * wl.T * wl.d * wl.E
    # the logits' fp32 FMA chains (bit-exact): vector ALU for few tokens, fp32 MFMA (K = 1 steps) above
    on_mfma = wl.T > ROUTER_FEW_MAX_T
    peak = MFMA_PEAK_TFLOPS[W.F32] if on_mfma else FP32_VALU_PEAK_TFLOPS
    if bytes_ / (HBM_PEAK_GBS * 1e9) >= flops / (peak * 1e12):
        roof = {"bound": "hbm", "achieved": bytes_ / (dev_ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    else:
        roof = {"bound": "mfma" if on_mfma else "alu", "achieved": flops / (dev_ms * 1e-3) / 1e12, "peak": peak,
                "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = None
    name = "moe_route_grouped" if grouped else "moe_route_limited"
    roof["kernel"] = f"whole {name} call (router logits + {'grouped' if grouped else 'masked'} top-k + permutation)"
    roof["kernel_ms"] = dev_ms
    metric = (f"group-limited routing tokens/s ({n_group} groups, {wl.k // 2} kept)" if grouped else
              f"device-limited routing tokens/s ({int(allowed.sum())} of {wl.E} experts allowed)")
    out = base_record(wl, args, metric, wl.T / (ms_per_step * 1e-3), "tokens/s", ms_per_step)
    out["roofline"] = roof
    out["cpu_baseline"] = None
    if not args.no_cpu_baseline:
        from oracle import oracle as O
        h = {n: W.to_numpy(inp[n]) for n in ("x", "Wg")}
        b = W.to_numpy(inp.get("bias"))
        t0 = time.perf_counter()
        if grouped:
            O.route_grouped(h["x"], h["Wg"], b, wl.k, n_group, wl.act_dtype)
        else:
            O.route_limited(h["x"], h["Wg"], b, allowed.numpy(), wl.k, wl.act_dtype)
        dt = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": wl.T / dt, "unit": "tokens/s", "cores": len(os.sched_getaffinity(0)),
                               "omp_threads": O.num_threads(), "kind": "oracle",
                               "sample": f"{'route_grouped' if grouped else 'route_limited'} of all {wl.T} tokens "
                                         f"({dt:.2f} s)"}
    return out


def run_utilization(wl, inp, args, dev):
    r = B.moe_route(inp["x"], inp["Wg"], inp.get("bias"), wl.k)
    counts = r["counts"]
    util = torch.empty(wl.E, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    call = lambda: B.moe_expert_utilization(counts)  # noqa: E731
    steps = max(args.steps, 200)
    ms_per_step = wall_ms(call, steps, args.warmup)
    dev_ms = event_ms(call, steps)
    bytes_ = wl.E * (4 + 4 + 4) + 8
    roof = {"bound": "hbm", "achieved": bytes_ / (dev_ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = None
    roof["kernel"] = "expert_utilization_kernel (one block; launch-latency bound at this size)"
    roof["kernel_ms"] = dev_ms
    out = base_record(wl, args, "expert-utilisation monitor latency per call (us)", ms_per_step * 1e3, "us",
                      ms_per_step, higher=False)
    out["steps"] = steps
    out["roofline"] = roof
    out["cpu_baseline"] = None
    del util
    if not args.no_cpu_baseline:
        from oracle import oracle as O
        c = counts.cpu().numpy()
        n = 2000
        t0 = time.perf_counter()
        for _ in range(n):
            O.expert_utilization(c)
        dt = (time.perf_counter() - t0) / n
        out["cpu_baseline"] = {"value": dt * 1e6, "unit": "us", "cores": 1, "kind": "oracle",
                               "sample": f"{n} calls of expert_utilization on the same {wl.E} counts"}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=W.DECODE_BF16.name, choices=[w.name for w in W.CONFIGS])
    ap.add_argument("--variant", default="layer",
                    choices=["layer", "shard-ep8", "route-limited", "route-grouped", "utilization"])
    ap.add_argument("--rank", type=int, default=0, choices=range(8), help="expert-parallel rank / device (of 8)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-peaks", action="store_true", help="skip measuring the GPU's sustained HBM / MFMA ceilings")
    ap.add_argument("--cpu-tokens", type=int, default=64)
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="CPU work of the oracle baseline (about)")
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
    inp = W.generate(wl, seed=args.seed, device=dev, weights=args.variant in ("layer", "shard-ep8"))
    if args.variant in ("layer", "shard-ep8"):
        out = run_layer(wl, inp, args, dev)
    elif args.variant in ("route-limited", "route-grouped"):
        out = run_route(wl, inp, args, dev, grouped=args.variant == "route-grouped")
    else:
        out = run_utilization(wl, inp, args, dev)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
