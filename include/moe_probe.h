/*
 * moe_probe.h -- measurement kernels of libmoe_probe.so, used by the benchmark to state each roofline
 * fraction against what this GPU sustains as well as against its published peaks, and one self-check of an
 * arithmetic shortcut the layer takes (used by the tests).  They are not part of the layer (moe.h); they
 * compute nothing of it.  The HBM ceiling they measure is the one the pages say
 * decides serving ("DeepSeek-V3's mixture-of-experts architecture explained", "Inference reality check":
 * loading the experts' weights dominates), the MFMA one the ceiling of the expert GEMMs at large batch.
 * Conventions as in moe.h: device pointers, work enqueued on `stream`, no host synchronisation; return 0
 * on success, 1 for a bad argument, 2 for an unsupported dtype, 4 for a launch failure.
 */
#ifndef MOE_PROBE_H
#define MOE_PROBE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Streaming read: `grid` blocks of 256 threads read all `bytes` of `buf` (16-byte aligned) once, block b
 * the 256 KB chunks b, b + grid, ..., with 16-byte non-temporal loads, eight in flight per thread.  sink: [grid]
 * uint32 device array (practically never written).
 * Bytes / elapsed time is the read rate; with a buffer far beyond the 256 MB last-level cache it is the
 * HBM read ceiling.
 */
int moe_probe_stream_read(const void* buf, size_t bytes, unsigned grid, uint32_t* sink, hipStream_t stream);

/*
 * Back-to-back MFMAs: `grid` blocks of four wavefronts; each wavefront advances eight independent
 * accumulators `iters` times with v_mfma_f32_32x32x16_bf16 (dtype 1) or v_mfma_scale_f32_16x16x128_f8f6f4
 * with E4M3 operands and unit scales (dtype 2).  *flops (host) receives the floating-point operations the
 * launch performs; flops / elapsed time is the sustained dense MFMA rate.  sink: [grid] fp32 device array
 * (practically never written).
 */
int moe_probe_mfma(int dtype, int iters, unsigned grid, float* sink, double* flops, hipStream_t stream);

/*
 * Self-check of the fp8 quantisation's division (the rule of moe_quantize_e4m3 in moe.h: codes = E4M3 of
 * v / s in fp32, s = amax / 448), which the library computes from a correctly rounded reciprocal and one
 * fused residual correction instead of the IEEE division.  counts: 2 device uint64; counts[0] receives
 * the number of s in [2^-90, 2^126) (every mantissa) whose reciprocal differs from IEEE 1 / s, counts[1]
 * the number of (amax, v) pairs, over amax[0 .. n_amax) (positive finite fp32, device memory) and every
 * float v with |v| <= amax, whose E4M3 code differs from that of the IEEE quotient.  Both are 0 when the
 * shortcut is exact.  About 5 ms of GPU time per amax value at amax near 2^127, less below.
 */
int moe_probe_check_quant_division(const float* amax, int n_amax, unsigned long long* counts, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_PROBE_H */
