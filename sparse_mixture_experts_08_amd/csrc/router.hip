// router.hip -- router logits, top-k selection and softmax over the selected logits.
//
// Gate as "DeepSeek-V3's mixture-of-experts architecture explained" states it (block pseudocode of
// "The architecture in one diagram"): router_logits = gate(x); the top-8 values and indices of the
// logits; a softmax over those selected values only.
//
// Logits.  Each logit is one fp32 fused-multiply-add chain over i ascending, starting from +0.0f, then
// one fp32 add of the optional bias.  Both kernels below are fp32 GEMMs whose K loop runs in order with
// no split, so every (token, expert) output keeps exactly that chain and the routing decision is a
// deterministic function of x, Wg and bias.
//
// Top-k.  One wavefront per token; each lane holds E/64 logits as 64-bit keys (order-preserving bits of
// the logit, then the complemented expert index), so a wave-wide max picks the largest logit and, among
// equal logits, the lower expert index.  k rounds give the experts in descending-logit order.
#include "moe_common.h"
#include "topk.h"

namespace moe {

// x tile element as float.
template <typename XT> __device__ __forceinline__ float ldx(const XT* p);
template <> __device__ __forceinline__ float ldx<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float ldx<uint16_t>(const uint16_t* p) { return bf16_to_f32(*p); }

// Eight consecutive x elements (16-byte aligned for bf16, 32-byte for fp32) as floats.
__device__ __forceinline__ void ldx8(const uint16_t* p, float* v)
{
    const uint4 r = *(const uint4*)p;
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int j = 0; j < 4; j++) {
        v[2 * j] = __uint_as_float(w[j] << 16);
        v[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
    }
}
__device__ __forceinline__ void ldx8(const float* p, float* v)
{
    const float4 a = *(const float4*)p, b = *(const float4*)(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// Many tokens: L[t][e] = fma chain over i of x[t][i] * Wg[i][e] (+ bias[e]).  Block tile 64 tokens x
// 64 experts, thread tile 4 x 4, K staged through double-buffered LDS 32 at a time (the next stage's
// global loads are in flight during the current stage's FMAs).  x is stored transposed ([i][t]) with
// consecutive lanes on consecutive tokens, so the transposing stores and the 16-byte reads are free of
// bank conflicts.  Per output the K loop runs in order: the chain is exactly the contract's.
template <typename XT>
__global__ __launch_bounds__(256) void router_logits_many_kernel(const XT* __restrict__ x, const float* __restrict__ Wg,
                                                                 const float* __restrict__ bias, float* __restrict__ L,
                                                                 int T, int d, int E, int vec)
{
    constexpr int BT = 64, BE = 64, BK = 32;
    __shared__ __attribute__((aligned(16))) float xs[2][BK][BT];
    __shared__ __attribute__((aligned(16))) float wsm[2][BK][BE];
    const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
    const int e0 = blockIdx.x * BE, t0 = blockIdx.y * BT;
    // loader roles: x -> token (tid & 63), 8 consecutive i at (tid >> 6) * 8; Wg -> rows tid / 16 and
    // tid / 16 + 16, 4 experts at (tid & 15) * 4
    const int lx_t = tid & 63, lx_k = (tid >> 6) * 8;
    const int lw_k = tid >> 4, lw_c = (tid & 15) * 4;
    float xr[8];
    float4 wr[2];
    auto load = [&](int k0) {
        if (t0 + lx_t < T) {
            ldx8(x + (size_t)(t0 + lx_t) * d + k0 + lx_k, xr);
        } else {
#pragma unroll
            for (int j = 0; j < 8; j++) xr[j] = 0.f;
        }
#pragma unroll
        for (int h = 0; h < 2; h++) {
            const float* row = Wg + (size_t)(k0 + lw_k + 16 * h) * E + e0 + lw_c;
            if (vec && e0 + lw_c + 4 <= E) {
                wr[h] = *(const float4*)row;
            } else {
                wr[h].x = e0 + lw_c + 0 < E ? row[0] : 0.f;
                wr[h].y = e0 + lw_c + 1 < E ? row[1] : 0.f;
                wr[h].z = e0 + lw_c + 2 < E ? row[2] : 0.f;
                wr[h].w = e0 + lw_c + 3 < E ? row[3] : 0.f;
            }
        }
    };
    auto store = [&](int b) {
#pragma unroll
        for (int j = 0; j < 8; j++) xs[b][lx_k + j][lx_t] = xr[j];
#pragma unroll
        for (int h = 0; h < 2; h++) *(float4*)&wsm[b][lw_k + 16 * h][lw_c] = wr[h];
    };

    float acc[4][4];
#pragma unroll
    for (int r = 0; r < 4; r++)
#pragma unroll
        for (int c = 0; c < 4; c++) acc[r][c] = 0.0f;

    const int ns = d / BK;
    load(0);
    store(0);
    __syncthreads();
    for (int s = 0; s < ns; s++) {
        const int b = s & 1;
        if (s + 1 < ns) load((s + 1) * BK);
#pragma unroll 8
        for (int kk = 0; kk < BK; kk++) {
            const float4 a = *(const float4*)&xs[b][kk][ty * 4];
            const float4 w = *(const float4*)&wsm[b][kk][tx * 4];
            const float av[4] = {a.x, a.y, a.z, a.w}, wv[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int r = 0; r < 4; r++)
#pragma unroll
                for (int c = 0; c < 4; c++) acc[r][c] = __builtin_fmaf(av[r], wv[c], acc[r][c]);
        }
        if (s + 1 < ns) store(b ^ 1);
        __syncthreads();
    }
#pragma unroll
    for (int r = 0; r < 4; r++) {
        const int t = t0 + ty * 4 + r;
        if (t >= T) continue;
#pragma unroll
        for (int c = 0; c < 4; c++) {
            const int e = e0 + tx * 4 + c;
            if (e >= E) continue;
            float v = acc[r][c];
            if (bias) v = v + bias[e];
            L[(size_t)t * E + e] = v;
        }
    }
}

// Few tokens: one chain per lane.  Block = 16 tokens x 16 experts, 4 wavefronts (wave w: tokens
// 4w..4w+3; lane (tt, el) = (lane / 16, lane % 16)).  Per 128-wide K stage the block loads the Wg tile
// [128 i][16 e] (64-byte row segments) and the x tile [16 t][128 i] and stores them in LDS transposed
// ([e][i], [t][i]) so each lane reads four consecutive i of its expert and of its token with one 16-byte
// LDS read.  Global loads run two stages ahead of the FMAs (two register sets, loop unrolled by two).
template <typename XT>
__global__ __launch_bounds__(256) void router_logits_few_kernel(const XT* __restrict__ x, const float* __restrict__ Wg,
                                                                const float* __restrict__ bias, float* __restrict__ L,
                                                                int T, int d, int E, int vec)
{
    constexpr int BK = 128, PAD = 4;
    __shared__ __attribute__((aligned(16))) float wT[2][16][BK + PAD];
    __shared__ __attribute__((aligned(16))) float xT[2][16][BK + PAD];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, tt = wave * 4 + (lane >> 4), el = lane & 15;
    const int e0 = blockIdx.x * 16, t0 = blockIdx.y * 16;
    const int wr_row = tid >> 1, wr_col = (tid & 1) * 8;       // Wg tile element loaded by this thread
    const int xr_tok = tid >> 4, xr_i = (tid & 15) * 8;        // x tile element loaded by this thread

    struct Regs {
        float4 w0, w1;
        float x[8];
    };
    auto load = [&](Regs& r, int k0) {
        const float* row = Wg + (size_t)(k0 + wr_row) * E + e0 + wr_col;
        if (vec) {
            r.w0 = *(const float4*)row;
            r.w1 = *(const float4*)(row + 4);
        } else {
            float v[8];
#pragma unroll
            for (int j = 0; j < 8; j++) v[j] = e0 + wr_col + j < E ? row[j] : 0.f;
            r.w0 = make_float4(v[0], v[1], v[2], v[3]);
            r.w1 = make_float4(v[4], v[5], v[6], v[7]);
        }
        if (t0 + xr_tok < T) {
            ldx8(x + (size_t)(t0 + xr_tok) * d + k0 + xr_i, r.x);
        } else {
#pragma unroll
            for (int j = 0; j < 8; j++) r.x[j] = 0.f;
        }
    };
    auto store = [&](const Regs& r, int b) {
        wT[b][wr_col + 0][wr_row] = r.w0.x;
        wT[b][wr_col + 1][wr_row] = r.w0.y;
        wT[b][wr_col + 2][wr_row] = r.w0.z;
        wT[b][wr_col + 3][wr_row] = r.w0.w;
        wT[b][wr_col + 4][wr_row] = r.w1.x;
        wT[b][wr_col + 5][wr_row] = r.w1.y;
        wT[b][wr_col + 6][wr_row] = r.w1.z;
        wT[b][wr_col + 7][wr_row] = r.w1.w;
        *(float4*)&xT[b][xr_tok][xr_i] = make_float4(r.x[0], r.x[1], r.x[2], r.x[3]);
        *(float4*)&xT[b][xr_tok][xr_i + 4] = make_float4(r.x[4], r.x[5], r.x[6], r.x[7]);
    };
    float acc = 0.0f;
    auto compute = [&](int b) {
#pragma unroll 8
        for (int i = 0; i < BK; i += 4) {
            const float4 a = *(const float4*)&xT[b][tt][i];
            const float4 w = *(const float4*)&wT[b][el][i];
            acc = __builtin_fmaf(a.x, w.x, acc);
            acc = __builtin_fmaf(a.y, w.y, acc);
            acc = __builtin_fmaf(a.z, w.z, acc);
            acc = __builtin_fmaf(a.w, w.w, acc);
        }
    };

    const int ns = d / BK;
    Regs ra, rb;
    load(ra, 0);
    if (ns > 1) load(rb, BK);
    store(ra, 0);
    __syncthreads();
    for (int s = 0; s < ns; s += 2) {
        // stage s is in LDS buffer 0; rb holds stage s + 1 (in flight)
        if (s + 2 < ns) load(ra, (s + 2) * BK);
        compute(0);
        if (s + 1 >= ns) break;
        store(rb, 1);
        __syncthreads();
        // stage s + 1 is in LDS buffer 1; ra holds stage s + 2 (in flight)
        if (s + 3 < ns) load(rb, (s + 3) * BK);
        compute(1);
        if (s + 2 < ns) store(ra, 0);
        __syncthreads();
    }
    const int t = t0 + tt, e = e0 + el;
    if (t < T && e < E) {
        if (bias) acc = acc + bias[e];
        L[(size_t)t * E + e] = acc;
    }
}

hipError_t launch_router_logits(const moe_shape_t& s, const void* x, const float* Wg, const float* bias,
                                float* logits, hipStream_t stream)
{
    const int T = (int)s.T, d = (int)s.d, E = (int)s.E;
    const bool bf = s.act_dtype == MOE_BF16;
    if (T <= 512) {
        const int vec = (E % 16 == 0) && (((uintptr_t)Wg & 15) == 0);
        dim3 grid((E + 15) / 16, (T + 15) / 16);
        if (bf)
            router_logits_few_kernel<uint16_t><<<grid, 256, 0, stream>>>((const uint16_t*)x, Wg, bias, logits, T, d, E, vec);
        else
            router_logits_few_kernel<float><<<grid, 256, 0, stream>>>((const float*)x, Wg, bias, logits, T, d, E, vec);
    } else {
        const int vec = (E % 4 == 0) && (((uintptr_t)Wg & 15) == 0);
        dim3 grid((E + 63) / 64, (T + 63) / 64);
        if (bf)
            router_logits_many_kernel<uint16_t><<<grid, 256, 0, stream>>>((const uint16_t*)x, Wg, bias, logits, T, d, E, vec);
        else
            router_logits_many_kernel<float><<<grid, 256, 0, stream>>>((const float*)x, Wg, bias, logits, T, d, E, vec);
    }
    return hipGetLastError();
}

// ------------------------------------------------------------------------------------------------
// Top-k + softmax for many tokens: one wavefront per token, 64 tokens (one chunk) per block of 16
// wavefronts.  Also records, per chunk, which tokens chose each expert (a 64-bit mask) and how many.
// ------------------------------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void topk_softmax_kernel(const float* __restrict__ L, const uint8_t* __restrict__ allowed,
                                                            int T, int E, int k,
                                                            int32_t* __restrict__ idx, float* __restrict__ w,
                                                            uint64_t* __restrict__ chunk_bits,
                                                            int32_t* __restrict__ chunk_counts,
                                                            int32_t* __restrict__ sync)
{
    __shared__ uint32_t bits_lo[1024], bits_hi[1024];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, c = blockIdx.x;
    if (c == 0 && threadIdx.x < 4) sync[threadIdx.x] = 0;   // reset the permutation's counters
    for (int e = threadIdx.x; e < E; e += 1024) bits_lo[e] = bits_hi[e] = 0;
    __syncthreads();
    for (int tl = wave; tl < 64; tl += 16) {
        const int t = c * 64 + tl;
        if (t >= T) break;
        int my_e;
        float my_w;
        topk_group<64, 16>(L + (size_t)t * E, allowed, E, k, lane, my_e, my_w);
        if (lane < k) {
            idx[(size_t)t * k + lane] = my_e;
            w[(size_t)t * k + lane] = my_w;
            if (tl < 32) atomicOr(&bits_lo[my_e], 1u << tl);
            else atomicOr(&bits_hi[my_e], 1u << (tl - 32));
        }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += 1024) {
        const uint64_t b = ((uint64_t)bits_hi[e] << 32) | bits_lo[e];
        chunk_bits[(size_t)c * E + e] = b;
        chunk_counts[(size_t)c * E + e] = __popcll(b);
    }
}

hipError_t launch_topk(const moe_shape_t& s, const float* logits, const uint8_t* allowed, int32_t* idx, float* w,
                       const Workspace& ws, hipStream_t stream)
{
    topk_softmax_kernel<<<(unsigned)ws.nchunks, 1024, 0, stream>>>(logits, allowed, (int)s.T, (int)s.E, (int)s.k, idx, w,
                                                                     ws.chunk_bits, ws.chunk_counts, ws.sync);
    return hipGetLastError();
}

}  // namespace moe
