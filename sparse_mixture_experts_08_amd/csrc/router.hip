// router.hip -- router logits, top-k selection and softmax over the selected logits.
//
// Gate as "DeepSeek-V3's mixture-of-experts architecture explained" states it (block pseudocode of
// "The architecture in one diagram"): router_logits = gate(x); the top-8 values and indices of the
// logits; a softmax over those selected values only.
//
// Logits.  Each logit is one fp32 fused-multiply-add chain over i ascending, starting from +0.0f, then
// one fp32 add of the optional bias.  Wg is the gate's nn.Linear weight, [E, d]: one contiguous row per
// expert.  Both kernels below are fp32 GEMMs whose K loop runs in order with no split, so every
// (token, expert) output keeps exactly that chain and the routing decision is a deterministic function
// of x, Wg and bias.
//
// Top-k.  One wavefront per token; each lane holds E/64 logits as 64-bit keys (order-preserving bits of
// the logit, then the complemented expert index), so a wave-wide max picks the largest logit and, among
// equal logits, the lower expert index.  k rounds give the experts in descending-logit order.
#include <type_traits>

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

// Four consecutive x elements (8-byte aligned for bf16, 16-byte for fp32).
template <typename XT> struct X4;
template <> struct X4<uint16_t> {
    uint2 r;
    __device__ __forceinline__ void load(const uint16_t* p) { r = *(const uint2*)p; }
    __device__ __forceinline__ void get(float* v, bool valid) const
    {
        v[0] = valid ? __uint_as_float(r.x << 16) : 0.f;
        v[1] = valid ? __uint_as_float(r.x & 0xFFFF0000u) : 0.f;
        v[2] = valid ? __uint_as_float(r.y << 16) : 0.f;
        v[3] = valid ? __uint_as_float(r.y & 0xFFFF0000u) : 0.f;
    }
};
template <> struct X4<float> {
    float4 a;
    __device__ __forceinline__ void load(const float* p) { a = *(const float4*)p; }
    __device__ __forceinline__ void get(float* v, bool valid) const
    {
        v[0] = valid ? a.x : 0.f; v[1] = valid ? a.y : 0.f; v[2] = valid ? a.z : 0.f; v[3] = valid ? a.w : 0.f;
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

// Many tokens: L[t][e] = fma chain over i of x[t][i] * Wg[e][i] (+ bias[e]).  Block tile BT (64 or 32)
// tokens x 64 experts, thread tile TT (4 or 2) tokens x 4 experts, K staged through double-buffered LDS
// 32 at a time; global loads run two stages ahead of the FMAs (two register sets), so a CU with a single
// block still covers their latency.  Both tiles are stored K-major ([i][t], [i][e]) so a thread reads its
// tokens and four experts of one i with two LDS reads; the x transposing stores put consecutive lanes on
// consecutive tokens (conflict-free) and the Wg rows are padded so its transposing stores spread over the
// banks.  Calls above the rotated-operand kernel's range use 64 x 4: with wavefronts plenty, four
// tokens per thread keep the most FMAs per LDS read.  Per output the K loop runs in order: the chain is
// exactly the contract's.
template <typename XT, int BT, int TT>
__global__ __launch_bounds__(BT / TT * 16) void router_logits_many_kernel(const XT* __restrict__ x, const float* __restrict__ Wg,
                                                                          const float* __restrict__ bias, float* __restrict__ L,
                                                                          int T, int d, int E)
{
    constexpr int BE = 64, BK = 32, WPAD = 4, NT = BT / TT * 16;
    constexpr int WH = BE * BK / 4 / NT;               // float4 Wg loads per thread
    constexpr int XPT = BT * BK / NT;                  // x elements per thread per stage (8 or 4)
    static_assert((BT == 64 || BT == 32) && (TT == 4 || TT == 2), "64- or 32-token tiles, 4 or 2 tokens per thread");
    __shared__ __attribute__((aligned(16))) float xs[2][BK][BT];
    __shared__ __attribute__((aligned(16))) float wsm[2][BK][BE + WPAD];
    const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
    const int e0 = blockIdx.x * BE, t0 = blockIdx.y * BT;
    // loader roles: x -> token tid % BT, XPT consecutive i at (tid / BT) * XPT; Wg -> experts tid / 8 +
    // (NT / 8) * h, 4 consecutive i at (tid % 8) * 4
    const int lx_t = tid % BT, lx_k = (tid / BT) * XPT;
    const int lw_e = tid >> 3, lw_k = (tid & 7) * 4;
    const bool x_ok = t0 + lx_t < T;
    const XT* xrow = x + (size_t)min(t0 + lx_t, T - 1) * d + lx_k;
    using XL = typename std::conditional<XPT == 8, X8<XT>, X4<XT>>::type;
    struct Regs {
        XL x;
        W4 w[WH];
    };
    auto load = [&](Regs& r, int k0) {
        r.x.load(xrow + k0);
#pragma unroll
        for (int h = 0; h < WH; h++) r.w[h].load(Wg, e0 + lw_e + (NT / 8) * h, k0 + lw_k, E, d);
    };
    auto store = [&](const Regs& r, int b) {
        float v[XPT];
        r.x.get(v, x_ok);
#pragma unroll
        for (int j = 0; j < XPT; j++) xs[b][lx_k + j][lx_t] = v[j];
#pragma unroll
        for (int h = 0; h < WH; h++) {
            const int e = lw_e + (NT / 8) * h;
            const float4 w = r.w[h].get(e0 + e < E);
            wsm[b][lw_k + 0][e] = w.x;
            wsm[b][lw_k + 1][e] = w.y;
            wsm[b][lw_k + 2][e] = w.z;
            wsm[b][lw_k + 3][e] = w.w;
        }
    };

    float acc[TT][4];
#pragma unroll
    for (int r = 0; r < TT; r++)
#pragma unroll
        for (int c = 0; c < 4; c++) acc[r][c] = 0.0f;

    auto compute = [&](int b) {
#pragma unroll 8
        for (int kk = 0; kk < BK; kk++) {
            float av[TT];
            if constexpr (TT == 4) {
                const float4 a = *(const float4*)&xs[b][kk][ty * 4];
                av[0] = a.x; av[1] = a.y; av[2] = a.z; av[3] = a.w;
            } else {
                const float2 a = *(const float2*)&xs[b][kk][ty * 2];
                av[0] = a.x; av[1] = a.y;
            }
            const float4 w = *(const float4*)&wsm[b][kk][tx * 4];
            const float wv[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int r = 0; r < TT; r++)
#pragma unroll
                for (int c = 0; c < 4; c++) acc[r][c] = __builtin_fmaf(av[r], wv[c], acc[r][c]);
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
#pragma unroll
    for (int r = 0; r < TT; r++) {
        const int t = t0 + ty * TT + r;
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

// Seven more chains per lane for the price of one operand read: acc[j] (j = 1..7) += w' * x, where w'
// is the first source taken from lane (l - j) mod 16 of the same 16-lane row (DPP row rotation inside
// v_fmac_f32, which the compiler does not fold from a separate DPP move), for the four K steps of w and
// x in order.  The leading s_nop gives the two wait states a DPP read needs after a VALU write of its
// source.
#define MOE_DPP_FMA(D, J, W, X) "v_fmac_f32_dpp %" #D ", %" #W ", %" #X " row_ror:" #J " row_mask:0xf bank_mask:0xf\n"
#define MOE_DPP_FMA7(W, X)                                                                                      \
    MOE_DPP_FMA(0, 1, W, X) MOE_DPP_FMA(1, 2, W, X) MOE_DPP_FMA(2, 3, W, X) MOE_DPP_FMA(3, 4, W, X)             \
    MOE_DPP_FMA(4, 5, W, X) MOE_DPP_FMA(5, 6, W, X) MOE_DPP_FMA(6, 7, W, X)
__device__ __forceinline__ void fma_rotated8(float (&a)[8], float4 w, float4 x)
{
    a[0] = __builtin_fmaf(x.x, w.x, a[0]);
    a[0] = __builtin_fmaf(x.y, w.y, a[0]);
    a[0] = __builtin_fmaf(x.z, w.z, a[0]);
    a[0] = __builtin_fmaf(x.w, w.w, a[0]);
    asm("s_nop 1\n" MOE_DPP_FMA7(7, 11) MOE_DPP_FMA7(8, 12) MOE_DPP_FMA7(9, 13) MOE_DPP_FMA7(10, 14)
        : "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(a[4]), "+v"(a[5]), "+v"(a[6]), "+v"(a[7])
        : "v"(w.x), "v"(w.y), "v"(w.z), "v"(w.w), "v"(x.x), "v"(x.y), "v"(x.z), "v"(x.w));
}
#undef MOE_DPP_FMA7
#undef MOE_DPP_FMA

#ifndef MOE_DPP_BK
#define MOE_DPP_BK 64
#endif

// Mid-sized T: per 16-lane row an outer product of 16 tokens x 8 experts with one LDS read per operand
// per lane and K step.  Lane l reads x of token l and the gate row of expert l % 8 and, through
// fma_rotated8, keeps eight chains: token l with the experts of lanes (l - j) mod 16, j = 0..7, which are
// the eight experts of the row.  (The register tiles of router_logits_many_kernel read six floats per
// eight FMAs, more than the LDS delivers at two wavefronts per SIMD.)  Block = 4 wavefronts = 64 tokens
// x 32 experts: wavefront w takes tokens 16 w .. 16 w + 15, its four rows the four 8-expert groups.  K is
// staged 64 at a time through double-buffered LDS as [t][i] and [e][i] rows, so a lane reads four
// consecutive i of each operand with one 16-byte read; global loads run two stages ahead.  Every chain
// runs over i in order.  (Prefill router, T = 4096: 0.345 ms with the register tiles, 0.31 ms here.  The
// DPP forms issue somewhat slower than plain FMAs, so where there are enough wavefronts for the 4 x 4
// register tiles -- T above 8192 -- those stay faster.)
template <typename XT>
__global__ __launch_bounds__(256) void router_logits_dpp_kernel(const XT* __restrict__ x, const float* __restrict__ Wg,
                                                               const float* __restrict__ bias, float* __restrict__ L,
                                                               int T, int d, int E)
{
    constexpr int BT = 64, BE = 32, BK = MOE_DPP_BK, PAD = 4, NQ = BK / 32;
    static_assert(BK % 32 == 0, "whole 32-wide loader steps");
    __shared__ __attribute__((aligned(16))) float xs[2][BT][BK + PAD];
    __shared__ __attribute__((aligned(16))) float ws[2][BE][BK + PAD];
    const int tid = threadIdx.x, lane = tid & 63, l = lane & 15, row = lane >> 4, wave = tid >> 6;
    const int e0 = blockIdx.x * BE, t0 = blockIdx.y * BT;
    // loaders, per 32 i of the stage: x -> token tid / 4, 8 consecutive i at (tid % 4) * 8; Wg -> expert
    // tid / 8, 4 consecutive i at (tid % 8) * 4
    const int lx_t = tid >> 2, lx_k = (tid & 3) * 8;
    const int lw_e = tid >> 3, lw_k = (tid & 7) * 4;
    const bool x_ok = t0 + lx_t < T;
    const XT* xrow = x + (size_t)min(t0 + lx_t, T - 1) * d + lx_k;
    struct Regs {
        X8<XT> x[NQ];
        W4 w[NQ];
    };
    auto load = [&](Regs& r, int k0) {
#pragma unroll
        for (int q = 0; q < NQ; q++) {
            r.x[q].load(xrow + k0 + 32 * q);
            r.w[q].load(Wg, e0 + lw_e, k0 + 32 * q + lw_k, E, d);
        }
    };
    auto store = [&](const Regs& r, int b) {
#pragma unroll
        for (int q = 0; q < NQ; q++) {
            float v[8];
            r.x[q].get(v, x_ok);
            *(float4*)&xs[b][lx_t][32 * q + lx_k] = make_float4(v[0], v[1], v[2], v[3]);
            *(float4*)&xs[b][lx_t][32 * q + lx_k + 4] = make_float4(v[4], v[5], v[6], v[7]);
            *(float4*)&ws[b][lw_e][32 * q + lw_k] = r.w[q].get(e0 + lw_e < E);
        }
    };

    const int my_t = wave * 16 + l, my_e = row * 8 + (l & 7);
    float acc[8];
#pragma unroll
    for (int j = 0; j < 8; j++) acc[j] = 0.0f;
    auto compute = [&](int b) {
#pragma unroll
        for (int kq = 0; kq < BK; kq += 4)
            fma_rotated8(acc, *(const float4*)&ws[b][my_e][kq], *(const float4*)&xs[b][my_t][kq]);
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
    const int t = t0 + my_t;
    if (t >= T) return;
#pragma unroll
    for (int j = 0; j < 8; j++) {
        const int e = e0 + row * 8 + ((l - j) & 7);        // row_ror:j read lane (l - j) mod 16
        if (e >= E) continue;
        float v = acc[j];
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

#ifndef MOE_ROUTER_FEW_MAX_T
#define MOE_ROUTER_FEW_MAX_T 512
#endif
#ifndef MOE_ROUTER_DPP_MAX_T
#define MOE_ROUTER_DPP_MAX_T 8192
#endif

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
    } else if (T <= MOE_ROUTER_FEW_MAX_T) {
        dim3 grid((E + 15) / 16, (T + 15) / 16);
        if (bf) launch_few<uint16_t, 16>(grid, (const uint16_t*)x, Wg, bias, logits, T, d, E, stream);
        else launch_few<float, 16>(grid, (const float*)x, Wg, bias, logits, T, d, E, stream);
    } else if (T <= MOE_ROUTER_DPP_MAX_T) {
        dim3 grid((E + 31) / 32, (T + 63) / 64);
        if (bf)
            router_logits_dpp_kernel<uint16_t><<<grid, 256, 0, stream>>>((const uint16_t*)x, Wg, bias, logits, T, d, E);
        else
            router_logits_dpp_kernel<float><<<grid, 256, 0, stream>>>((const float*)x, Wg, bias, logits, T, d, E);
    } else {
        dim3 grid((E + 63) / 64, (T + 63) / 64);
        if (bf)
            router_logits_many_kernel<uint16_t, 64, 4><<<grid, 256, 0, stream>>>((const uint16_t*)x, Wg, bias, logits, T, d, E);
        else
            router_logits_many_kernel<float, 64, 4><<<grid, 256, 0, stream>>>((const float*)x, Wg, bias, logits, T, d, E);
    }
    return hipGetLastError();
}

// ------------------------------------------------------------------------------------------------
// Top-k + softmax for many tokens: W lanes per token (16 when E <= 256: four tokens per wavefront at
// once; a wavefront when E <= 1024), 64 tokens (one chunk) per block of 16 wavefronts.  Also records,
// per chunk, which tokens chose each expert (a 64-bit mask) and how many.
// ------------------------------------------------------------------------------------------------
// NQ: logits per lane (E <= W * NQ).
template <int W, int NQ>
__global__ __launch_bounds__(1024) void topk_softmax_kernel(const float* __restrict__ L, const uint8_t* __restrict__ allowed,
                                                            int T, int E, int k,
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
        topk_group<W, NQ>(L + (size_t)(valid ? t : 0) * E, allowed, E, k, sub, my_e, my_w);
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

#ifndef MOE_TOPK_W16
#define MOE_TOPK_W16 1
#endif

hipError_t launch_topk(const moe_shape_t& s, const float* logits, const uint8_t* allowed, int32_t* idx, float* w,
                       const Workspace& ws, hipStream_t stream)
{
    if (s.E <= 256 && MOE_TOPK_W16)
        topk_softmax_kernel<16, 16><<<(unsigned)ws.nchunks, 1024, 0, stream>>>(logits, allowed, (int)s.T, (int)s.E, (int)s.k,
                                                                                idx, w, ws.chunk_bits, ws.chunk_counts);
    else if (s.E <= 256)
        topk_softmax_kernel<64, 4><<<(unsigned)ws.nchunks, 1024, 0, stream>>>(logits, allowed, (int)s.T, (int)s.E, (int)s.k,
                                                                               idx, w, ws.chunk_bits, ws.chunk_counts);
    else
        topk_softmax_kernel<64, 16><<<(unsigned)ws.nchunks, 1024, 0, stream>>>(logits, allowed, (int)s.T, (int)s.E, (int)s.k,
                                                                                idx, w, ws.chunk_bits, ws.chunk_counts);
    return hipGetLastError();
}

}  // namespace moe
