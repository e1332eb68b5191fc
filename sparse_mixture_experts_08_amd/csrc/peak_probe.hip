// peak_probe.hip -- measurement kernels for the denominators of the roofline fractions: the HBM read rate
// a plain streaming kernel reaches, and the MFMA rate back-to-back matrix instructions reach, on the GPU
// at hand (the published 8 TB/s and 2.5 / 5.0 PFLOP/s are peaks at the nominal clock; these are what the
// chip sustains).  Also a self-check of one arithmetic shortcut of the layer's fp8 quantisation step.  Not
// part of the layer: libmoe_probe.so, used by the benchmark and the tests only.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe_probe.h"
#include "moe_common.h"

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

// Block b reads the 256 KB chunks b, b + grid, b + 2 grid, ... of the buffer, each thread eight 16-byte
// vectors in flight per step, and folds them into an xor; the fold is stored only when it equals a value no
// finite buffer of ones produces, so the loads cannot be removed and nothing is written in practice.
// The loads carry the non-temporal hint, which streams faster on MI355X (4 GiB, 8192 blocks: 7.1 against
// 6.4 TB/s without it); contiguous chunks per block stream faster than a grid-stride walk over the whole
// buffer (6.0 / 5.6-5.7 TB/s for grids of 8192 / 2048 blocks, without the hint), and 64 KB - 4 MB chunks,
// 16 vectors in flight or 512- and 1024-thread blocks reach no more.
__global__ __launch_bounds__(256) void stream_read_kernel(const i32x4* __restrict__ p, uint64_t n16, uint32_t* sink)
{
    constexpr uint64_t CH16 = (256u << 10) / 16;       // 16-byte vectors per chunk
    constexpr int U = 8;
    uint32_t acc = 0;
    for (uint64_t c = blockIdx.x; c * CH16 < n16; c += gridDim.x) {
        const uint64_t end = min((c + 1) * CH16, n16);
        for (uint64_t i = c * CH16 + threadIdx.x; i < end; i += U * 256) {
            i32x4 v[U];
#pragma unroll
            for (int u = 0; u < U; u++)
                v[u] = i + u * 256 < end ? __builtin_nontemporal_load(p + i + u * 256) : (i32x4){0, 0, 0, 0};
#pragma unroll
            for (int u = 0; u < U; u++) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
        }
    }
    if (acc == 0x9E3779B9u) sink[blockIdx.x] = acc;
}

// CHAINS independent accumulators per wavefront, each advanced by one MFMA per iteration: the matrix pipe
// never waits on a result.  Operands are lane values that cannot be folded at compile time.
template <int CHAINS>
__global__ __launch_bounds__(256) void mfma_bf16_kernel(int iters, float* sink)
{
    const float s = (float)(threadIdx.x & 7) * 0.125f;
    bf16x8 a, b;
    for (int e = 0; e < 8; e++) {
        a[e] = (__bf16)(s + e);
        b[e] = (__bf16)(s - e);
    }
    f32x16 acc[CHAINS];
    for (int c = 0; c < CHAINS; c++) acc[c] = (f32x16){};
    for (int it = 0; it < iters; it++) {
#pragma unroll
        for (int c = 0; c < CHAINS; c++) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
#pragma unroll
        for (int c = 0; c < CHAINS; c++) asm volatile("" : "+a"(acc[c]));   // keeps every chain in its registers
    }
    float t = 0.f;
    for (int c = 0; c < CHAINS; c++)
        for (int e = 0; e < 16; e++) t += acc[c][e];
    if (t == 1.2345f) sink[blockIdx.x] = t;
}

template <int CHAINS>
__global__ __launch_bounds__(256) void mfma_fp8_kernel(int iters, float* sink)
{
    const int s = (int)(threadIdx.x & 7);
    i32x8 a, b;
    for (int e = 0; e < 8; e++) {
        a[e] = 0x38383838 + s + e;
        b[e] = 0x30303030 + s - e;
    }
    f32x4 acc[CHAINS];
    for (int c = 0; c < CHAINS; c++) acc[c] = (f32x4){};
    for (int it = 0; it < iters; it++) {
#pragma unroll
        for (int c = 0; c < CHAINS; c++)
            acc[c] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc[c], 0, 0, 0, 127, 0, 127);
#pragma unroll
        for (int c = 0; c < CHAINS; c++) asm volatile("" : "+a"(acc[c]));   // keeps every chain in its registers
    }
    float t = 0.f;
    for (int c = 0; c < CHAINS; c++)
        for (int e = 0; e < 4; e++) t += acc[c][e];
    if (t == 1.2345f) sink[blockIdx.x] = t;
}

}  // namespace

// The quantisation's division shortcut (moe_common.h: quant_div_fast, recip_rn, quant_div) against IEEE
// fp32 division.  recip_check: every s = 2^e (1 + m 2^-23) with 2^-90 <= s < 2^126 against 1.0f / s.
// code_check: per amax (blockIdx.y strides over them), every float v with |v| <= amax (bit patterns 0 ..
// bits(amax), both signs) with s = amax / 448: the E4M3 code of the library's quotient against that of
// v / s.  Mismatches are counted with one atomic per thread.
__global__ __launch_bounds__(256) void recip_check_kernel(unsigned long long* count)
{
    constexpr uint32_t E0 = 127 - 90, E1 = 127 + 125;  // biased exponents of the checked s
    const uint64_t n = (uint64_t)(E1 - E0 + 1) << 23;
    unsigned long long bad = 0;
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (uint64_t)gridDim.x * blockDim.x) {
        const float s = __uint_as_float(((E0 + (uint32_t)(i >> 23)) << 23) | (uint32_t)(i & 0x7FFFFF));
        bad += __float_as_uint(moe::recip_rn(s)) != __float_as_uint(1.0f / s);
    }
    if (bad) atomicAdd(count, bad);
}

__global__ __launch_bounds__(256) void code_check_kernel(const float* amaxes, int n_amax, unsigned long long* count)
{
    unsigned long long bad = 0;
    for (int a = blockIdx.y; a < n_amax; a += gridDim.y) {
        const float amax = amaxes[a];
        const float s = amax / 448.0f;
        const bool fast = moe::quant_div_fast(s);
        const float r = moe::recip_rn(s);
        const uint64_t top = (uint64_t)(__float_as_uint(amax) & 0x7FFFFFFFu) + 1;
        for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < 2 * top; i += (uint64_t)gridDim.x * blockDim.x) {
            const float v = __uint_as_float((uint32_t)(i >> 1) | ((uint32_t)(i & 1) << 31));
            const float q = fast ? moe::quant_div(v, s, r) : v / s;
            bad += (moe::f32x2_to_e4m3(q, 0.f) & 0xFFu) != (moe::f32x2_to_e4m3(v / s, 0.f) & 0xFFu);
        }
    }
    if (bad) atomicAdd(count, bad);
}

__global__ void zero2_kernel(unsigned long long* c) { c[0] = c[1] = 0; }

extern "C" int moe_probe_check_quant_division(const float* amax, int n_amax, unsigned long long* counts,
                                              hipStream_t stream)
{
    if (!amax || !counts || n_amax <= 0) return 1;
    zero2_kernel<<<1, 1, 0, stream>>>(counts);
    recip_check_kernel<<<8192, 256, 0, stream>>>(counts);
    code_check_kernel<<<dim3(4096, 64), 256, 0, stream>>>(amax, n_amax, counts + 1);
    return hipGetLastError() == hipSuccess ? 0 : 4;
}

extern "C" int moe_probe_stream_read(const void* buf, size_t bytes, unsigned grid, uint32_t* sink, hipStream_t stream)
{
    if (!buf || !sink || bytes < 16 || ((uintptr_t)buf & 15) || grid == 0) return 1;
    stream_read_kernel<<<grid, 256, 0, stream>>>((const i32x4*)buf, bytes / 16, sink);
    return hipGetLastError() == hipSuccess ? 0 : 4;
}

extern "C" int moe_probe_mfma(int dtype, int iters, unsigned grid, float* sink, double* flops, hipStream_t stream)
{
    if (!sink || !flops || iters <= 0 || grid == 0) return 1;
    constexpr int CHAINS = 8;
    const double waves = (double)grid * 4;
    if (dtype == 1) {
        mfma_bf16_kernel<CHAINS><<<grid, 256, 0, stream>>>(iters, sink);
        *flops = waves * iters * CHAINS * (2.0 * 32 * 32 * 16);
    } else if (dtype == 2) {
        mfma_fp8_kernel<CHAINS><<<grid, 256, 0, stream>>>(iters, sink);
        *flops = waves * iters * CHAINS * (2.0 * 16 * 16 * 128);
    } else {
        return 2;
    }
    return hipGetLastError() == hipSuccess ? 0 : 4;
}
