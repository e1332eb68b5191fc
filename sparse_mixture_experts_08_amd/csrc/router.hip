// router.hip -- router logits, top-k selection and softmax over the selected logits.
//
// Gate as "DeepSeek-V3's mixture-of-experts architecture explained" states it (block pseudocode of
// "The architecture in one diagram"): router_logits = gate(x); the top-8 values and indices of the
// logits; a softmax over those selected values only.
//
// Logits.  Each logit is one fp32 fused-multiply-add chain over i ascending, starting from +0.0f, then
// one fp32 add of the optional bias.  Wg is the gate's nn.Linear weight, [E, d]: one contiguous row per
// expert.  Both logit kernels below run the K loop in order with no split, the few-token one on the
// vector ALU and the many-token one on the matrix cores (whose fp32 K = 1 MFMA is that same fused
// multiply-add), so every (token, expert) output keeps exactly that chain and the routing decision is a
// deterministic function of x, Wg and bias.
//
// Top-k.  A group of lanes per token (16 lanes when E <= 256, four tokens per wavefront; a whole wavefront
// when E <= 1024); each lane holds its share of the logits as 64-bit keys (order-preserving bits of the
// logit, then the complemented expert index), so a group-wide max picks the largest logit and, among
// equal logits, the lower expert index.  k rounds give the experts in descending-logit order.
#include "moe_common.h"
#include "topk.h"

namespace moe {

// Global loads of x and Wg are kept raw (storage format, no conversion) from the load to the LDS store,
// at clamped in-bounds addresses, and out-of-range elements are zeroed at the store with a select.
// Converting inside a branch around the load would make the compiler wait for each load where it is
// issued, which serialises them and defeats the prefetch.

// Eight consecutive x elements (16-byte aligned for bf16, 32-byte for fp32).
template <typename XT> struct X8;
template <> struct X8<uint16_t> {
    uint4 r;
    __device__ __forceinline__ void load(const uint16_t* p) { r = *(const uint4*)p; }
    __device__ __forceinline__ void get(float* v, bool valid) const
    {
        const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
        for (int j = 0; j < 4; j++) {
            v[2 * j] = valid ? __uint_as_float(w[j] << 16) : 0.f;
            v[2 * j + 1] = valid ? __uint_as_float(w[j] & 0xFFFF0000u) : 0.f;
        }
    }
};
template <> struct X8<float> {
    float4 a, b;
    __device__ __forceinline__ void load(const float* p)
    {
        a = *(const float4*)p;
        b = *(const float4*)(p + 4);
    }
    __device__ __forceinline__ void get(float* v, bool valid) const
    {
        v[0] = valid ? a.x : 0.f; v[1] = valid ? a.y : 0.f; v[2] = valid ? a.z : 0.f; v[3] = valid ? a.w : 0.f;
        v[4] = valid ? b.x : 0.f; v[5] = valid ? b.y : 0.f; v[6] = valid ? b.z : 0.f; v[7] = valid ? b.w : 0.f;
    }
};

// Four consecutive elements of one gate row (Wg is [E, d], the gate's nn.Linear weight; rows 16-byte
// aligned).  Rows past E are clamped to the last row and zeroed at get().
struct W4 {
    float4 r;
    __device__ __forceinline__ void load(const float* Wg, int e, int i, int E, int d)
    {
        r = *(const float4*)(Wg + (size_t)min(e, E - 1) * d + i);
    }
    __device__ __forceinline__ float4 get(bool valid) const
    {
        return make_float4(valid ? r.x : 0.f, valid ? r.y : 0.f, valid ? r.z : 0.f, valid ? r.w : 0.f);
    }
};

// Many tokens, on the matrix cores: v_mfma_f32_16x16x1_4b_f32 computes, per element of four 16 x 16 blocks,
// d = a * b + c with one rounding -- an fp32 fused multiply-add, bit for bit (including subnormals), so
// every logit is still the contract's chain of fmaf steps over i ascending from +0.0f, at twice the rate
// of one FMA per lane on the vector ALU.  Operand layout of the instruction: A row i of block b comes from
// lane 16 b + i, B column j from lane 16 b + j, and result register r of lane l is block r / 4, row
// 4 (l / 16) + r % 4, column l % 16.  Each lane supplies x of token l % 16 (the same 16 tokens for the four
// blocks) and the gate row of expert l, so one instruction advances 16 tokens x 64 experts by one step of
// i; a wavefront keeps NS such chains over consecutive 64-expert groups (NS independent instructions per
// step of i).  Block = 4 wavefronts x 16 tokens = 64 tokens, x 64 NS experts; K staged through
// double-buffered LDS 32 at a time ([t][i] and [e][i] rows padded to 144 bytes, so 16 lanes reading
// 16 B each hit distinct banks), global loads two stages ahead as in the kernels above.
// FLAT: the stage loop walks whole pairs of stages with an odd last stage after it, which keeps the
// accumulators in one register range (the form with a break inside the pair copies them between two
// ranges every pair: 32 extra moves per 64 MFMAs).  With four or more wavefronts per SIMD (above 8192
// tokens) that is faster (16384 / 32768 tokens: 0.683 -> 0.662 / 1.219 -> 1.178 ms, logits bitwise
// equal); with one (4096 tokens) the compiler's schedule of the other form hides the LDS reads better
// (0.225 against 0.261 ms).
template <typename XT, int NS, bool FLAT>
__global__ __launch_bounds__(256) void router_logits_mfma_kernel(const XT* __restrict__ x, const float* __restrict__ Wg,
                                                                const float* __restrict__ bias, float* __restrict__ L,
                                                                int T, int d, int E)
{
    constexpr int BT = 64, BE = 64 * NS, BK = 32, PAD = 4, WH = BE * BK / 4 / 256;
    typedef float f32x16 __attribute__((ext_vector_type(16)));
    __shared__ __attribute__((aligned(16))) float xs[2][BT][BK + PAD];
    __shared__ __attribute__((aligned(16))) float ws[2][BE][BK + PAD];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int e0 = blockIdx.x * BE, t0 = blockIdx.y * BT;
    // loaders: x -> token tid / 4, 8 consecutive i at (tid % 4) * 8; Wg -> experts tid / 8 + 32 h, 4
    // consecutive i at (tid % 8) * 4
    const int lx_t = tid >> 2, lx_k = (tid & 3) * 8;
    const int lw_e = tid >> 3, lw_k = (tid & 7) * 4;
    const bool x_ok = t0 + lx_t < T;
    const XT* xrow = x + (size_t)min(t0 + lx_t, T - 1) * d + lx_k;
    struct Regs {
        X8<XT> x;
        W4 w[WH];
    };
    auto load = [&](Regs& r, int k0) {
        r.x.load(xrow + k0);
#pragma unroll
        for (int h = 0; h < WH; h++) r.w[h].load(Wg, e0 + lw_e + 32 * h, k0 + lw_k, E, d);
    };
    auto store = [&](const Regs& r, int b) {
        float v[8];
        r.x.get(v, x_ok);
        *(float4*)&xs[b][lx_t][lx_k] = make_float4(v[0], v[1], v[2], v[3]);
        *(float4*)&xs[b][lx_t][lx_k + 4] = make_float4(v[4], v[5], v[6], v[7]);
#pragma unroll
        for (int h = 0; h < WH; h++) *(float4*)&ws[b][lw_e + 32 * h][lw_k] = r.w[h].get(e0 + lw_e + 32 * h < E);
    };

    const int my_t = wave * 16 + (lane & 15);          // the token this lane supplies
    f32x16 acc[NS];
#pragma unroll
    for (int s = 0; s < NS; s++) acc[s] = (f32x16){};
    auto compute = [&](int b) {
#pragma unroll
        for (int kq = 0; kq < BK; kq += 4) {
            const float4 a = *(const float4*)&xs[b][my_t][kq];
            float4 w[NS];
#pragma unroll
            for (int s = 0; s < NS; s++) w[s] = *(const float4*)&ws[b][64 * s + lane][kq];
            const float av[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
            for (int kk = 0; kk < 4; kk++)
#pragma unroll
                for (int s = 0; s < NS; s++) {
                    const float wv = kk == 0 ? w[s].x : kk == 1 ? w[s].y : kk == 2 ? w[s].z : w[s].w;
                    acc[s] = __builtin_amdgcn_mfma_f32_16x16x1f32(av[kk], wv, acc[s], 0, 0, 0);
                }
        }
    };
    const int ns = d / BK;
    Regs ra, rb;
    load(ra, 0);
    if (ns > 1) load(rb, BK);
    store(ra, 0);
    __syncthreads();
    if constexpr (FLAT) {
        int s = 0;
        for (; s + 1 < ns; s += 2) {
            // stage s is in LDS buffer 0; rb holds stage s + 1 (in flight)
            if (s + 2 < ns) load(ra, (s + 2) * BK);
            compute(0);
            store(rb, 1);
            __syncthreads();
            // stage s + 1 is in LDS buffer 1; ra holds stage s + 2 (in flight)
            if (s + 3 < ns) load(rb, (s + 3) * BK);
            compute(1);
            if (s + 2 < ns) store(ra, 0);
            __syncthreads();
        }
        if (s < ns) compute(0);                        // an odd stage count: the last stage, in buffer 0
    } else {
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
    }
#pragma unroll
    for (int s = 0; s < NS; s++)
#pragma unroll
        for (int r = 0; r < 16; r++) {
            const int t = t0 + wave * 16 + 4 * (lane >> 4) + (r & 3);
            const int e = e0 + 64 * s + 16 * (r >> 2) + (lane & 15);
            if (t >= T || e >= E) continue;
            float v = acc[s][r];
            if (bias) v = v + bias[e];
            L[(size_t)t * E + e] = v;
        }
}


// Few tokens: one chain per lane.  Block = TPB tokens x 16 experts, TPB / 4 wavefronts (lane (tt, el)
// = (thread / 16, thread % 16)).  Per BK-wide K stage the block copies the Wg tile (16 gate rows) and the
// x tile (TPB token rows) into LDS as [e][i] and [t][i], so each lane reads four consecutive i of its
// expert and of its token with one 16-byte read.  Global loads run two stages ahead of the FMAs (two
// register sets, loop unrolled by two) and are issued without a branch around them (past the end the
// last stage is loaded again): behind a branch the compiler waits for every load in flight before
// issuing the next set.  With one chain per lane a stage is short next to the load latency, so the
// stages are wide (BK = 256 where d allows; decode router, T = 64: 50 us with 128-wide stages and no LDS
// prefetch, 40 us here).
template <typename XT, int TPB, int BK>
__global__ __launch_bounds__(TPB * 16) void router_logits_few_kernel(const XT* __restrict__ x, const float* __restrict__ Wg,
                                                                     const float* __restrict__ bias, float* __restrict__ L,
                                                                     int T, int d, int E)
{
    constexpr int PAD = 4, NT = TPB * 16, Q = BK / 128;
    constexpr int WPT = 16 * 16 / NT;                          // 8-float Wg chunks per thread per 128 i
    static_assert(TPB % 4 == 0 && TPB <= 16, "whole wavefronts, at most 16 tokens");
    static_assert(BK % 128 == 0, "whole 128-wide loader steps");
    __shared__ __attribute__((aligned(16))) float wT[2][16][BK + PAD];
    __shared__ __attribute__((aligned(16))) float xT[2][TPB][BK + PAD];
    const int tid = threadIdx.x, tt = tid >> 4, el = tid & 15;
    const int e0 = blockIdx.x * 16, t0 = blockIdx.y * TPB;
    const int li = (tid & 15) * 8;                             // first i of this thread's chunks, per 128
    const bool x_ok = t0 + tt < T;
    const XT* xrow = x + (size_t)min(t0 + tt, T - 1) * d + li;

    struct Regs {
        W4 w[Q][WPT][2];
        X8<XT> x[Q];
    };
    auto load = [&](Regs& r, int k0) {
#pragma unroll
        for (int q = 0; q < Q; q++) {
#pragma unroll
            for (int p = 0; p < WPT; p++) {
                const int e = (tid >> 4) + p * TPB;
                r.w[q][p][0].load(Wg, e0 + e, k0 + 128 * q + li, E, d);
                r.w[q][p][1].load(Wg, e0 + e, k0 + 128 * q + li + 4, E, d);
            }
            r.x[q].load(xrow + k0 + 128 * q);
        }
    };
    auto store = [&](const Regs& r, int b) {
#pragma unroll
        for (int q = 0; q < Q; q++) {
#pragma unroll
            for (int p = 0; p < WPT; p++) {
                const int e = (tid >> 4) + p * TPB;
                *(float4*)&wT[b][e][128 * q + li] = r.w[q][p][0].get(e0 + e < E);
                *(float4*)&wT[b][e][128 * q + li + 4] = r.w[q][p][1].get(e0 + e < E);
            }
            float v[8];
            r.x[q].get(v, x_ok);
            *(float4*)&xT[b][tt][128 * q + li] = make_float4(v[0], v[1], v[2], v[3]);
            *(float4*)&xT[b][tt][128 * q + li + 4] = make_float4(v[4], v[5], v[6], v[7]);
        }
    };
    float acc = 0.0f;
    // The stage's LDS reads run D steps of four i ahead of the single FMA chain (pinned there by the
    // scheduling barriers): with one wavefront per SIMD nothing else hides their latency.
    auto compute = [&](int b) {
        constexpr int N = BK / 4, D = 16;
        float4 fa[N], fw[N];
#pragma unroll
        for (int j = 0; j < D; j++) {
            fa[j] = *(const float4*)&xT[b][tt][4 * j];
            fw[j] = *(const float4*)&wT[b][el][4 * j];
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < N; i++) {
            if (i + D < N) {
                fa[i + D] = *(const float4*)&xT[b][tt][4 * (i + D)];
                fw[i + D] = *(const float4*)&wT[b][el][4 * (i + D)];
            }
            acc = __builtin_fmaf(fa[i].x, fw[i].x, acc);
            acc = __builtin_fmaf(fa[i].y, fw[i].y, acc);
            acc = __builtin_fmaf(fa[i].z, fw[i].z, acc);
            acc = __builtin_fmaf(fa[i].w, fw[i].w, acc);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    const int ns = d / BK;
    Regs ra, rb;
    load(ra, 0);
    load(rb, min(1, ns - 1) * BK);
    store(ra, 0);
    __syncthreads();
    for (int s = 0; s < ns; s += 2) {
        // stage s is in LDS buffer 0; rb holds stage s + 1 (in flight)
        load(ra, min(s + 2, ns - 1) * BK);
        compute(0);
        if (s + 1 >= ns) break;
        store(rb, 1);
        __syncthreads();
        // stage s + 1 is in LDS buffer 1; ra holds stage s + 2 (in flight)
        load(rb, min(s + 3, ns - 1) * BK);
        compute(1);
        store(ra, 0);
        __syncthreads();
    }
    const int t = t0 + tt, e = e0 + el;
    if (t < T && e < E) {
        if (bias) acc = acc + bias[e];
        L[(size_t)t * E + e] = acc;
    }
}


// The few-token kernel with 256-wide K stages where d allows (512-wide ones measured slower), else 128.
template <typename XT, int TPB>
static void launch_few(dim3 grid, const XT* x, const float* Wg, const float* bias, float* logits, int T, int d, int E,
                       hipStream_t stream)
{
    if (d % 256 == 0)
        router_logits_few_kernel<XT, TPB, 256><<<grid, TPB * 16, 0, stream>>>(x, Wg, bias, logits, T, d, E);
    else
        router_logits_few_kernel<XT, TPB, 128><<<grid, TPB * 16, 0, stream>>>(x, Wg, bias, logits, T, d, E);
}

// Router kernel by token count: the few-token kernel (vector ALU) up to 512 tokens, the MFMA kernel above
// (one 64-expert chain group per wavefront, which measured faster than two or four: T = 4096 / 16384 /
// 32768 in 0.224 / 0.670 / 1.167 ms, against 0.332 / 0.912 / 1.502 ms with the vector-ALU register-tile
// and DPP row-rotation kernels it replaces, routing bitwise equal).
static constexpr int ROUTER_FEW_MAX_T = 512;
static constexpr int ROUTER_MFMA_NS = 1;
// Above this many tokens the MFMA logit kernel takes its FLAT stage loop (four or more wavefronts per SIMD).
static constexpr int64_t ROUTER_FLAT_MIN_T = 8192;

hipError_t launch_router_logits(const moe_shape_t& s, const void* x, const float* Wg, const float* bias,
                                float* logits, hipStream_t stream)
{
    const int T = (int)s.T, d = (int)s.d, E = (int)s.E;
    const bool bf = s.act_dtype == MOE_BF16;
    if (T <= 256) {
        // 8 tokens per block: twice the blocks of the 16-token form, more loads in flight per token
        dim3 grid((E + 15) / 16, (T + 7) / 8);
        if (bf) launch_few<uint16_t, 8>(grid, (const uint16_t*)x, Wg, bias, logits, T, d, E, stream);
        else launch_few<float, 8>(grid, (const float*)x, Wg, bias, logits, T, d, E, stream);
    } else if (T <= ROUTER_FEW_MAX_T) {
        dim3 grid((E + 15) / 16, (T + 15) / 16);
        if (bf) launch_few<uint16_t, 16>(grid, (const uint16_t*)x, Wg, bias, logits, T, d, E, stream);
        else launch_few<float, 16>(grid, (const float*)x, Wg, bias, logits, T, d, E, stream);
    } else {
        dim3 grid((E + 64 * ROUTER_MFMA_NS - 1) / (64 * ROUTER_MFMA_NS), (T + 63) / 64);
        const bool flat = T > ROUTER_FLAT_MIN_T;
        if (bf)
            flat ? router_logits_mfma_kernel<uint16_t, ROUTER_MFMA_NS, true>
                       <<<grid, 256, 0, stream>>>((const uint16_t*)x, Wg, bias, logits, T, d, E)
                 : router_logits_mfma_kernel<uint16_t, ROUTER_MFMA_NS, false>
                       <<<grid, 256, 0, stream>>>((const uint16_t*)x, Wg, bias, logits, T, d, E);
        else
            flat ? router_logits_mfma_kernel<float, ROUTER_MFMA_NS, true>
                       <<<grid, 256, 0, stream>>>((const float*)x, Wg, bias, logits, T, d, E)
                 : router_logits_mfma_kernel<float, ROUTER_MFMA_NS, false>
                       <<<grid, 256, 0, stream>>>((const float*)x, Wg, bias, logits, T, d, E);
    }
    return hipGetLastError();
}

// ------------------------------------------------------------------------------------------------
// Top-k + softmax for many tokens: W lanes per token (16 when E <= 256: four tokens per wavefront at
// once; a wavefront when E <= 1024), 64 tokens (one chunk) per block of 16 wavefronts.  Also records,
// per chunk, which tokens chose each expert (a 64-bit mask) and how many.
// ------------------------------------------------------------------------------------------------
// NQ: logits per lane (E <= W * NQ).  GROUPED: group-limited selection over n_group groups (topk_grouped)
// instead of the plain (optionally masked) top-k.
template <int W, int NQ, bool GROUPED>
__global__ __launch_bounds__(1024) void topk_softmax_kernel(const float* __restrict__ L, const uint8_t* __restrict__ allowed,
                                                            int T, int E, int k, int n_group,
                                                            int32_t* __restrict__ idx, float* __restrict__ w,
                                                            uint64_t* __restrict__ chunk_bits,
                                                            int32_t* __restrict__ chunk_counts)
{
    constexpr int TPW = 64 / W;                        // tokens per wavefront pass
    __shared__ uint32_t bits_lo[1024], bits_hi[1024];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, c = blockIdx.x;
    const int sub = lane % W, grp = lane / W;
    for (int e = threadIdx.x; e < E; e += 1024) bits_lo[e] = bits_hi[e] = 0;
    __syncthreads();
    for (int tl0 = wave * TPW; tl0 < 64; tl0 += 16 * TPW) {
        const int tl = tl0 + grp, t = c * 64 + tl;
        if (c * 64 + tl0 >= T) break;                  // wavefront-uniform
        const bool valid = t < T;                      // the W-lane group of a token past T reads token 0
        int my_e;
        float my_w;
        if constexpr (GROUPED) topk_grouped<W, NQ>(L + (size_t)(valid ? t : 0) * E, E, k, n_group, sub, my_e, my_w);
        else topk_group<W, NQ>(L + (size_t)(valid ? t : 0) * E, allowed, E, k, sub, my_e, my_w);
        if (valid && sub < k) {
            idx[(size_t)t * k + sub] = my_e;
            w[(size_t)t * k + sub] = my_w;
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
                       const Workspace& ws, hipStream_t stream, int n_group)
{
    const unsigned grid = (unsigned)ws.nchunks;
    const int T = (int)s.T, E = (int)s.E, k = (int)s.k;
    if (n_group > 0) {
        if (E <= 256)
            topk_softmax_kernel<16, 16, true><<<grid, 1024, 0, stream>>>(logits, nullptr, T, E, k, n_group, idx, w,
                                                                          ws.chunk_bits, ws.chunk_counts);
        else
            topk_softmax_kernel<64, 16, true><<<grid, 1024, 0, stream>>>(logits, nullptr, T, E, k, n_group, idx, w,
                                                                          ws.chunk_bits, ws.chunk_counts);
    } else if (E <= 256) {
        topk_softmax_kernel<16, 16, false><<<grid, 1024, 0, stream>>>(logits, allowed, T, E, k, 0, idx, w, ws.chunk_bits,
                                                                       ws.chunk_counts);
    } else {
        topk_softmax_kernel<64, 16, false><<<grid, 1024, 0, stream>>>(logits, allowed, T, E, k, 0, idx, w, ws.chunk_bits,
                                                                       ws.chunk_counts);
    }
    return hipGetLastError();
}

}  // namespace moe
