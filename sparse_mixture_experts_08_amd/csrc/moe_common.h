// moe_common.h -- device helpers, workspace layout and kernel launchers shared by the HIP sources of
// the MoE layer library (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

// ------------------------------------------------------------------------------------------------
// Scalar conversions (finite inputs).
// ------------------------------------------------------------------------------------------------

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Two floats rounded to the nearest bf16 (ties to even) by the hardware conversion (v_cvt_pk_bf16_f32:
// one instruction for both, against three integer operations each for the same rounding done on the bit
// pattern), packed as a | b << 16.  For every finite float, subnormals included, it gives the bit pattern
// of u + 0x7FFF + (u >> 16 & 1), shifted right by 16; NaNs stay NaNs.
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float a, float b)
{
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
}

// Round to the nearest bf16 (ties to even) and return its bit pattern.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return (uint16_t)f32x2_to_bf16x2(f, 0.f); }

// Round to the nearest bf16 (ties to even), returned as the (exact) float value.
__device__ __forceinline__ float round_bf16(float f) { return bf16_to_f32(f32_to_bf16(f)); }

// a and b rounded to the nearest bf16 in place, by one conversion.
__device__ __forceinline__ void round_bf16x2(float& a, float& b)
{
    const uint32_t p = f32x2_to_bf16x2(a, b);
    a = __uint_as_float(p << 16);
    b = __uint_as_float(p & 0xFFFF0000u);
}

// Value rounded to the activation dtype (fp32: identity).
template <bool ACT_BF16>
__device__ __forceinline__ float round_act(float f) { return ACT_BF16 ? round_bf16(f) : f; }

// The quotient v / s of the E4M3 quantisation (s = amax / 448 of the group, |v| <= amax), with the
// E4M3 code of the IEEE fp32 division in four instructions instead of about ten.  recip_rn(s) is the
// correctly rounded 1/s (hardware reciprocal, one Newton step) for every s in [2^-90, 2^126); from it
// the product v * (1/s) and one fused residual correction give the correctly rounded quotient
// (Markstein's division), except where the residual underflows, which needs |v / s| < 2^-12, where both
// quotients are below 2^-10 and round to a zero code; the sign copy keeps the sign of v there (-0 -> -0).
// For the other s the callers divide.  Checked on the GPU: the reciprocal for every mantissa of that
// range, the codes for every v in [-amax, amax] at 4096 values of amax from 2^-81 to 2^127 (libmoe_probe's
// moe_probe_check_quant_division runs the same helpers).
__device__ __forceinline__ bool quant_div_fast(float s) { return s >= 0x1p-90f && s < 0x1p126f; }
__device__ __forceinline__ float recip_rn(float s)
{
    const float r0 = __builtin_amdgcn_rcpf(s);
    return __builtin_fmaf(__builtin_fmaf(-s, r0, 1.0f), r0, r0);
}
__device__ __forceinline__ float quant_div(float v, float s, float r)
{
    const float q0 = v * r;
    return __builtin_copysignf(__builtin_fmaf(__builtin_fmaf(-s, q0, v), r, q0), v);
}

// Maximum of a non-negative, non-NaN x over each aligned group of 16 lanes (a DPP row), returned to every
// lane of the group: four DPP moves (the neighbour in a pair, the other pair of a quad, the mirrored quad
// of a half-row, the mirrored half-row) instead of four LDS permutes.  Such floats order as their bit
// patterns do, so the maxima are integer maxima (no NaN canonicalisation).  Every lane of a group must be
// active.
template <int CTRL> __device__ __forceinline__ uint32_t dpp_u32(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ float row16_max(float x)
{
    uint32_t u = __float_as_uint(x);
    u = max(u, dpp_u32<0xB1>(u));                      // quad_perm [1, 0, 3, 2]
    u = max(u, dpp_u32<0x4E>(u));                      // quad_perm [2, 3, 0, 1]
    u = max(u, dpp_u32<0x141>(u));                     // row_half_mirror
    u = max(u, dpp_u32<0x140>(u));                     // row_mirror
    return __uint_as_float(u);
}

// Two floats -> two OCP E4M3 codes (round to nearest even; |v| <= 448 here), packed in the low 16 bits.
__device__ __forceinline__ uint32_t f32x2_to_e4m3(float a, float b)
{
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
}

// Exclusive prefix sum of one int per thread over a block of NT threads (NT a multiple of 64, <= 1024).
// `lds` holds NT/64 + 1 ints.  Returns the thread's exclusive prefix; *total gets the block sum.
template <int NT>
__device__ __forceinline__ int block_exclusive_scan(int v, int* total, int* lds)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    if (lane == 63) lds[wave] = x;
    __syncthreads();
    if (threadIdx.x == 0) {
        int run = 0;
        for (int w = 0; w < NT / 64; w++) {
            const int t = lds[w];
            lds[w] = run;
            run += t;
        }
        lds[NT / 64] = run;
    }
    __syncthreads();
    const int excl = x - v + lds[wave];
    *total = lds[NT / 64];
    __syncthreads();
    return excl;
}

// ------------------------------------------------------------------------------------------------
// Vector types for 16-byte loads and MFMA operands.
// ------------------------------------------------------------------------------------------------
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

// ------------------------------------------------------------------------------------------------
// Workspace layout.  Every region is 256-byte aligned; offsets are computed from the shape only.
// ------------------------------------------------------------------------------------------------
struct Workspace {
    float* logits;          // [T, E] router logits
    int32_t* idx;           // [T, k]
    float* w;               // [T, k]
    int32_t* counts;        // [E]
    int32_t* offsets;       // [E + 1]
    int32_t* chunk_counts;  // [nchunks, E]  tokens of a 64-token chunk routed to each expert
    int32_t* chunk_prefix;  // [nchunks, E]  exclusive prefix of chunk_counts over chunks, per expert
    uint64_t* chunk_bits;   // [nchunks, E]  which of the chunk's 64 tokens chose each expert
    int32_t* sorted_slots;  // [T * k]
    int32_t* pos;           // [T * k]
    int32_t* row_token;     // [T * k + T]  token of each expert-sorted row; shared rows last
    int4* tiles;            // [max_tiles]  (group, first row, rows, 0); group E is the shared expert
    int32_t* sync;          // [4]  sync[0]: number of tiles (written with the tile list)
    uint8_t* xq;            // [T, d] E4M3 codes of x (fp8 weights only)
    float* xs;              // [T, d / 128] their scales
    void* h;                // [T * k + T, inter_max] act dtype, or E4M3 codes (fp8 weights)
    float* hs;              // [T * k + T, inter_max / 128] (fp8 weights only)
    void* y_rows;           // [T * k + T, d] act dtype: each row's expert output
    size_t total;
    int64_t max_tiles, nchunks, inter_max;
};

// Groups that get GEMM tiles: routed experts [g0, g1), and the shared expert when `shared` is set.
struct TileRange {
    int g0, g1, shared;
};

// Rows per grouped-GEMM tile for this shape.
int tile_rows(const moe_shape_t& s);

// Compute the layout (pointers relative to `base`; base may be null to size it).
Workspace carve_workspace(const moe_shape_t& s, void* base);

// ------------------------------------------------------------------------------------------------
// Kernel launchers (all enqueue on `stream`, return hipGetLastError()).
// ------------------------------------------------------------------------------------------------
hipError_t launch_router_logits(const moe_shape_t& s, const void* x, const float* Wg, const float* bias,
                                float* logits, hipStream_t stream);
hipError_t launch_topk(const moe_shape_t& s, const float* logits, const uint8_t* allowed, int32_t* idx, float* w,
                       const Workspace& ws, hipStream_t stream, int n_group = 0);
bool routing_is_fused(const moe_shape_t& s);
hipError_t launch_routing_fused(const moe_shape_t& s, const float* logits, const uint8_t* allowed, int32_t* idx, float* w,
                                int32_t* counts, int32_t* offsets, int32_t* sorted_slots, int32_t* pos,
                                const Workspace& ws, int bm, TileRange tr, hipStream_t stream);
hipError_t launch_permute(const moe_shape_t& s, const int32_t* idx, int32_t* counts, int32_t* offsets,
                          int32_t* sorted_slots, int32_t* pos, const Workspace& ws, int bm, TileRange tr,
                          hipStream_t stream);
hipError_t launch_act_quant(const moe_shape_t& s, const void* x, const Workspace& ws, hipStream_t stream);
hipError_t launch_quantize_e4m3(int64_t rows, int cols, const void* x, uint8_t* q, float* scales, hipStream_t stream);
// e_base: the expert stored first in W1/W3/W2 (0 for the whole layer); n_shared: the shared hidden
// features held in S1/S3 ([n_shared, d]) and S2 ([d, n_shared]).
hipError_t launch_up_gemm(const moe_shape_t& s, const void* x, const void* W1, const void* W3, const float* W1s,
                          const float* W3s, const void* S1, const void* S3, const float* S1s, const float* S3s,
                          const Workspace& ws, hipStream_t stream, int e_base, int n_shared);
hipError_t launch_down_gemm(const moe_shape_t& s, const void* W2, const float* W2s, const void* S2, const float* S2s,
                            const Workspace& ws, hipStream_t stream, int e_base, int n_shared);
hipError_t launch_combine_partial(const moe_shape_t& s, const int32_t* idx, const int32_t* pos, const float* w,
                                  const Workspace& ws, int e0, int e1, int with_shared, float* y_partial,
                                  hipStream_t stream);
hipError_t launch_expert_utilization(int E, const int32_t* counts, float* util, int32_t* flags, int32_t* summary,
                                     hipStream_t stream);
hipError_t launch_combine(const moe_shape_t& s, const int32_t* pos, const float* w, const Workspace& ws, void* y,
                          hipStream_t stream);

}  // namespace moe
