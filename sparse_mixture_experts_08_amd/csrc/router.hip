// router.hip -- router logits, top-k selection and softmax over the selected logits.
//
// Gate as "DeepSeek-V3's mixture-of-experts architecture explained" states it (block pseudocode of
// "The architecture in one diagram"): router_logits = gate(x); the top-8 values and indices of the
// logits; a softmax over those selected values only.
//
// Logits.  Each logit is one fp32 fused-multiply-add chain over i ascending, starting from +0.0f, then
// one fp32 add of the optional bias.  The kernel is a register-tiled fp32 GEMM whose K loop runs in
// order with no split, so every (token, expert) output keeps exactly that chain and the routing decision
// is a deterministic function of x, Wg and bias.
//
// Top-k.  One wavefront per token; each lane holds E/64 logits as 64-bit keys (order-preserving bits of
// the logit, then the complemented expert index), so a wave-wide max picks the largest logit and, among
// equal logits, the lower expert index.  k rounds give the experts in descending-logit order.
#include "moe_common.h"

namespace moe {

// x tile element as float.
template <typename XT> __device__ __forceinline__ float ldx(const XT* p);
template <> __device__ __forceinline__ float ldx<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float ldx<uint16_t>(const uint16_t* p) { return bf16_to_f32(*p); }

// L[t][e] = fma chain over i of x[t][i] * Wg[i][e] (+ bias[e]).
// Block tile BT tokens x BE experts, thread tile RT x RE, K staged through LDS in BK steps.
template <typename XT, int BT, int BE, int RT, int RE, int BK>
__global__ __launch_bounds__(256) void router_logits_kernel(const XT* __restrict__ x, const float* __restrict__ Wg,
                                                            const float* __restrict__ bias, float* __restrict__ L,
                                                            int T, int d, int E)
{
    constexpr int TX = BE / RE, TY = BT / RT;
    static_assert(TX * TY == 256, "256 threads");
    __shared__ float xs[BK][BT];
    __shared__ float wsm[BK][BE];
    const int tid = threadIdx.x, tx = tid % TX, ty = tid / TX;
    const int e0 = blockIdx.x * BE, t0 = blockIdx.y * BT;

    float acc[RT][RE];
#pragma unroll
    for (int r = 0; r < RT; r++)
#pragma unroll
        for (int c = 0; c < RE; c++) acc[r][c] = 0.0f;

    for (int k0 = 0; k0 < d; k0 += BK) {
        for (int f = tid; f < BT * BK; f += 256) {           // x tile, stored transposed
            const int t = f / BK, kk = f % BK;
            xs[kk][t] = (t0 + t < T) ? ldx<XT>(x + (size_t)(t0 + t) * d + k0 + kk) : 0.0f;
        }
        for (int f = tid; f < BK * BE; f += 256) {           // Wg tile, rows of BE experts
            const int kk = f / BE, c = f % BE;
            wsm[kk][c] = (e0 + c < E) ? Wg[(size_t)(k0 + kk) * E + e0 + c] : 0.0f;
        }
        __syncthreads();
#pragma unroll 8
        for (int kk = 0; kk < BK; kk++) {
            float a[RT], b[RE];
#pragma unroll
            for (int r = 0; r < RT; r++) a[r] = xs[kk][ty * RT + r];
#pragma unroll
            for (int c = 0; c < RE; c++) b[c] = wsm[kk][tx * RE + c];
#pragma unroll
            for (int r = 0; r < RT; r++)
#pragma unroll
                for (int c = 0; c < RE; c++) acc[r][c] = __builtin_fmaf(a[r], b[c], acc[r][c]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int r = 0; r < RT; r++) {
        const int t = t0 + ty * RT + r;
        if (t >= T) continue;
#pragma unroll
        for (int c = 0; c < RE; c++) {
            const int e = e0 + tx * RE + c;
            if (e >= E) continue;
            float v = acc[r][c];
            if (bias) v = v + bias[e];
            L[(size_t)t * E + e] = v;
        }
    }
}

hipError_t launch_router_logits(const moe_shape_t& s, const void* x, const float* Wg, const float* bias,
                                float* logits, hipStream_t stream)
{
    const int T = (int)s.T, d = (int)s.d, E = (int)s.E;
    const bool bf = s.act_dtype == MOE_BF16;
    if (T <= 512) {
        dim3 grid((E + 63) / 64, (T + 3) / 4);
        if (bf)
            router_logits_kernel<uint16_t, 4, 64, 1, 1, 64><<<grid, 256, 0, stream>>>((const uint16_t*)x, Wg, bias, logits, T, d, E);
        else
            router_logits_kernel<float, 4, 64, 1, 1, 64><<<grid, 256, 0, stream>>>((const float*)x, Wg, bias, logits, T, d, E);
    } else {
        dim3 grid((E + 63) / 64, (T + 63) / 64);
        if (bf)
            router_logits_kernel<uint16_t, 64, 64, 4, 4, 32><<<grid, 256, 0, stream>>>((const uint16_t*)x, Wg, bias, logits, T, d, E);
        else
            router_logits_kernel<float, 64, 64, 4, 4, 32><<<grid, 256, 0, stream>>>((const float*)x, Wg, bias, logits, T, d, E);
    }
    return hipGetLastError();
}

// ------------------------------------------------------------------------------------------------
// Top-k + softmax, one wavefront per token, 64 tokens (one chunk) per block of 4 wavefronts.
// Also records, per chunk, which tokens chose each expert (a 64-bit mask) and how many did.
// ------------------------------------------------------------------------------------------------

// Order-preserving map of a finite float to uint32 (+0 and -0 map to the same key).
__device__ __forceinline__ uint32_t ordered_bits(float f)
{
    uint32_t u = __float_as_uint(f == 0.0f ? 0.0f : f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const uint32_t lo = __shfl_xor((uint32_t)v, off, 64), hi = __shfl_xor((uint32_t)(v >> 32), off, 64);
        const uint64_t o = ((uint64_t)hi << 32) | lo;
        v = o > v ? o : v;
    }
    return v;
}

__global__ __launch_bounds__(256) void topk_softmax_kernel(const float* __restrict__ L, int T, int E, int k,
                                                           int32_t* __restrict__ idx, float* __restrict__ w,
                                                           uint64_t* __restrict__ chunk_bits,
                                                           int32_t* __restrict__ chunk_counts,
                                                           int32_t* __restrict__ sync)
{
    __shared__ uint32_t bits_lo[1024], bits_hi[1024];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, c = blockIdx.x;
    if (c == 0 && threadIdx.x < 4) sync[threadIdx.x] = 0;   // reset the permutation's counters
    for (int e = threadIdx.x; e < E; e += 256) bits_lo[e] = bits_hi[e] = 0;
    __syncthreads();

    const int nq = (E + 63) / 64;   // logits per lane (<= 16)
    for (int tl = wave; tl < 64; tl += 4) {
        const int t = c * 64 + tl;
        if (t >= T) break;
        uint64_t key[16];
#pragma unroll
        for (int q = 0; q < 16; q++) {
            const int e = lane + 64 * q;
            key[q] = 0;
            if (q < nq && e < E)
                key[q] = ((uint64_t)ordered_bits(L[(size_t)t * E + e]) << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)e);
        }
        int my_e = 0;
        float my_l = 0.0f;
        for (int j = 0; j < k; j++) {
            uint64_t best = 0;
#pragma unroll
            for (int q = 0; q < 16; q++) best = key[q] > best ? key[q] : best;
            best = wave_max_u64(best);
            const int e = (int)(0xFFFFFFFFu - (uint32_t)best);
            if ((e & 63) == lane) {
#pragma unroll
                for (int q = 0; q < 16; q++)
                    if (q == (e >> 6)) key[q] = 0;
            }
            if (lane == j) {
                my_e = e;
                my_l = L[(size_t)t * E + e];
            }
        }
        // softmax over the k selected logits; the first one is the largest
        const float m = __shfl(my_l, 0, 64);
        float z = lane < k ? expf(my_l - m) : 0.0f;
        float sum = z;
#pragma unroll
        for (int off = 8; off >= 1; off >>= 1) sum += __shfl_xor(sum, off, 64);   // lanes 0..15, fixed tree
        sum = __shfl(sum, 0, 64);
        if (lane < k) {
            idx[(size_t)t * k + lane] = my_e;
            w[(size_t)t * k + lane] = z / sum;
            if (tl < 32) atomicOr(&bits_lo[my_e], 1u << tl);
            else atomicOr(&bits_hi[my_e], 1u << (tl - 32));
        }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += 256) {
        const uint64_t b = ((uint64_t)bits_hi[e] << 32) | bits_lo[e];
        chunk_bits[(size_t)c * E + e] = b;
        chunk_counts[(size_t)c * E + e] = __popcll(b);
    }
}

hipError_t launch_topk(const moe_shape_t& s, const float* logits, int32_t* idx, float* w, const Workspace& ws,
                       hipStream_t stream)
{
    topk_softmax_kernel<<<(unsigned)ws.nchunks, 256, 0, stream>>>(logits, (int)s.T, (int)s.E, (int)s.k, idx, w,
                                                                    ws.chunk_bits, ws.chunk_counts, ws.sync);
    return hipGetLastError();
}

}  // namespace moe
