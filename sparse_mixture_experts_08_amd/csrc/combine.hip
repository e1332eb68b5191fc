// combine.hip -- weighted sum of each token's expert outputs plus the shared expert's output.
//
// The MoE forward excerpt on "DeepSeek-V3.2-Exp / Mixture of experts" accumulates
// expert(x) * weight into an fp32 zero tensor expert by expert (ascending expert index), then adds
// shared_experts(x).  Here each token gathers its k expert-output rows (the expert-sorted rows written
// by the down GEMM; pos[t*k+j] is the row of slot j) in ascending row order, which is ascending expert
// order, adds the shared row (row T*k + t) last, and rounds once to the activation dtype.  The order is
// fixed, so the result is bitwise deterministic; no float atomics are involved.
#include "moe_common.h"

namespace moe {

// K > 0: k fixed at compile time, so the slot sort is a register-only network and the k + 1 row loads of a
// vector are all in flight together; K = 0: any k <= 16, one row load at a time.
template <bool ACT_BF16, int K>
__global__ __launch_bounds__(512) void combine_kernel(const int32_t* __restrict__ pos, const float* __restrict__ w,
                                                      const uint8_t* __restrict__ y_rows, int T, int d, int k_rt,
                                                      uint8_t* __restrict__ y)
{
    constexpr int EB = ACT_BF16 ? 2 : 4;           // bytes per element
    constexpr int VE = 16 / EB;                    // elements per 16-byte vector
    constexpr int KM = K > 0 ? K : 16;
    const int k = K > 0 ? K : k_rt;
    const int t = blockIdx.x;
    int rr[KM];
    float ww[KM];
    for (int j = 0; j < k; j++) {
        rr[j] = pos[(size_t)t * k + j];
        ww[j] = w[(size_t)t * k + j];
    }
    // ascending row order (the same on every thread)
    if constexpr (K > 0) {
        // odd-even transposition: K rounds of compare-exchange on fixed pairs sort K entries
#pragma unroll
        for (int p = 0; p < K; p++)
#pragma unroll
            for (int b = p & 1; b + 1 < K; b += 2) {
                const bool sw = rr[b] > rr[b + 1];
                const int r0 = rr[b], r1 = rr[b + 1];
                const float w0 = ww[b], w1 = ww[b + 1];
                rr[b] = sw ? r1 : r0;
                rr[b + 1] = sw ? r0 : r1;
                ww[b] = sw ? w1 : w0;
                ww[b + 1] = sw ? w0 : w1;
            }
    } else {
        for (int a = 1; a < k; a++) {              // insertion sort of <= 16 entries
            const int r = rr[a];
            const float v = ww[a];
            int b = a - 1;
            while (b >= 0 && rr[b] > r) {
                rr[b + 1] = rr[b];
                ww[b + 1] = ww[b];
                b--;
            }
            rr[b + 1] = r;
            ww[b + 1] = v;
        }
    }
    const int64_t shared_row = (int64_t)T * k + t;
    auto add_row = [&](float (&acc)[VE], const uint4 raw, float wj) {
        const uint32_t wv[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int e = 0; e < VE; e++) {
            float v;
            if constexpr (ACT_BF16) v = __uint_as_float(e & 1 ? (wv[e / 2] & 0xFFFF0000u) : (wv[e / 2] << 16));
            else v = __uint_as_float(wv[e]);
            acc[e] = acc[e] + v * wj;
        }
    };
    auto finish = [&](const float (&acc)[VE], const uint4 raw, int c) {
        const uint32_t wv[4] = {raw.x, raw.y, raw.z, raw.w};
        uint32_t o[4];
        if constexpr (ACT_BF16) {
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const float a0 = acc[2 * e] + __uint_as_float(wv[e] << 16);
                const float a1 = acc[2 * e + 1] + __uint_as_float(wv[e] & 0xFFFF0000u);
                o[e] = f32x2_to_bf16x2(a0, a1);
            }
        } else {
#pragma unroll
            for (int e = 0; e < 4; e++) o[e] = __float_as_uint(acc[e] + __uint_as_float(wv[e]));
        }
        *(uint4*)(y + ((int64_t)t * d + c) * EB) = make_uint4(o[0], o[1], o[2], o[3]);
    };
    const int step = gridDim.y * blockDim.x * VE;
    int c = (blockIdx.y * blockDim.x + threadIdx.x) * VE;
    if constexpr (K > 0) {
        // The k + 1 rows of the next vector are loaded while this one is summed (past the row end the
        // current vector again, with no branch around the loads).
        auto load = [&](uint4 (&rows)[K + 1], int cc) {
#pragma unroll
            for (int j = 0; j < K; j++) rows[j] = *(const uint4*)(y_rows + ((int64_t)rr[j] * d + cc) * EB);
            rows[K] = *(const uint4*)(y_rows + (shared_row * d + cc) * EB);
        };
        if (c >= d) return;
        uint4 cur[K + 1];
        load(cur, c);
        for (; c < d; c += step) {
            uint4 nxt[K + 1];
            load(nxt, c + step < d ? c + step : c);
            float acc[VE];
#pragma unroll
            for (int e = 0; e < VE; e++) acc[e] = 0.0f;
#pragma unroll
            for (int j = 0; j < K; j++) add_row(acc, cur[j], ww[j]);
            finish(acc, cur[K], c);
#pragma unroll
            for (int j = 0; j <= K; j++) cur[j] = nxt[j];
        }
    } else {
        for (; c < d; c += step) {
            float acc[VE];
#pragma unroll
            for (int e = 0; e < VE; e++) acc[e] = 0.0f;
            for (int j = 0; j < k; j++) add_row(acc, *(const uint4*)(y_rows + ((int64_t)rr[j] * d + c) * EB), ww[j]);
            finish(acc, *(const uint4*)(y_rows + (shared_row * d + c) * EB), c);
        }
    }
}

// Threads per block.  Grid: with few tokens one block per (token, column chunk) of 256-thread blocks, so
// decode-sized T still spreads over the CUs; with many tokens one block per token, which amortises the slot
// sort over the row, of 448 threads, which step a 7168-wide bf16 row in exactly two 16-byte vectors each
// (32768-token fp8 layer 0.908 -> 0.879 ms against 256 threads' three and a half, 16384-token skewed 0.446
// -> 0.431 ms; 512 threads 0.881 / 0.433, 224 0.909 / 0.444; 128 and 64 threads slower still, 0.917 /
// 0.451 and 0.953 / 0.477 against 256 threads at 0.939 / 0.469 in an earlier run).
static int combine_threads(const moe_shape_t& s) { return s.T >= 1024 ? 448 : 256; }
static dim3 combine_grid(const moe_shape_t& s, int threads)
{
    const int ve = s.act_dtype == MOE_BF16 ? 8 : 4;
    const int chunk = threads * ve;
    return dim3((unsigned)s.T, s.T >= 1024 ? 1u : (unsigned)((s.d + chunk - 1) / chunk));
}

template <bool ACT_BF16>
static void launch_combine_t(const moe_shape_t& s, const int32_t* pos, const float* w, const Workspace& ws, void* y,
                             hipStream_t stream)
{
    const int nt = combine_threads(s);
    const dim3 grid = combine_grid(s, nt);
    const int T = (int)s.T, d = (int)s.d, k = (int)s.k;
    const uint8_t* rows = (const uint8_t*)ws.y_rows;
    uint8_t* out = (uint8_t*)y;
    switch (k) {
    case 4: combine_kernel<ACT_BF16, 4><<<grid, nt, 0, stream>>>(pos, w, rows, T, d, k, out); break;
    case 6: combine_kernel<ACT_BF16, 6><<<grid, nt, 0, stream>>>(pos, w, rows, T, d, k, out); break;
    case 8: combine_kernel<ACT_BF16, 8><<<grid, nt, 0, stream>>>(pos, w, rows, T, d, k, out); break;
    default: combine_kernel<ACT_BF16, 0><<<grid, nt, 0, stream>>>(pos, w, rows, T, d, k, out); break;
    }
}

hipError_t launch_combine(const moe_shape_t& s, const int32_t* pos, const float* w, const Workspace& ws, void* y,
                          hipStream_t stream)
{
    if (s.act_dtype == MOE_BF16) launch_combine_t<true>(s, pos, w, ws, y, stream);
    else launch_combine_t<false>(s, pos, w, ws, y, stream);
    return hipGetLastError();
}

// One expert-parallel rank's partial output ("DeepSeek-V3.2-Exp / Mixture of experts", MoE forward: the
// rank adds its local experts' weighted outputs and its shared-expert slice into an fp32 y that
// dist.all_reduce(y) then sums over ranks).  Same fixed order as combine_kernel, restricted to the slots
// whose expert lies in [e0, e1), plus the shared row when with_shared; stored in fp32 without rounding.
template <bool ACT_BF16>
__global__ __launch_bounds__(256) void combine_partial_kernel(const int32_t* __restrict__ idx, const int32_t* __restrict__ pos,
                                                              const float* __restrict__ w, const uint8_t* __restrict__ y_rows,
                                                              int T, int d, int k, int e0, int e1, int with_shared,
                                                              float* __restrict__ out)
{
    constexpr int EB = ACT_BF16 ? 2 : 4;
    constexpr int VE = 16 / EB;
    const int t = blockIdx.x;
    int rr[16];
    float ww[16];
    int n = 0;
    for (int j = 0; j < k; j++) {
        const int e = idx[(size_t)t * k + j];
        if (e < e0 || e >= e1) continue;
        rr[n] = pos[(size_t)t * k + j];
        ww[n] = w[(size_t)t * k + j];
        n++;
    }
    for (int a = 1; a < n; a++) {                 // ascending row order = ascending expert
        const int r = rr[a];
        const float v = ww[a];
        int b = a - 1;
        while (b >= 0 && rr[b] > r) {
            rr[b + 1] = rr[b];
            ww[b + 1] = ww[b];
            b--;
        }
        rr[b + 1] = r;
        ww[b + 1] = v;
    }
    const int64_t shared_row = (int64_t)T * k + t;
    // block (t, column chunk): 256 threads x one 16-byte vector each
    for (int c = (blockIdx.y * 256 + threadIdx.x) * VE; c < d; c += gridDim.y * 256 * VE) {
        float acc[VE];
#pragma unroll
        for (int e = 0; e < VE; e++) acc[e] = 0.0f;
        for (int j = 0; j < n; j++) {
            const uint4 raw = *(const uint4*)(y_rows + ((int64_t)rr[j] * d + c) * EB);
            const uint32_t wv[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
            for (int e = 0; e < VE; e++) {
                float v;
                if constexpr (ACT_BF16) v = __uint_as_float(e & 1 ? (wv[e / 2] & 0xFFFF0000u) : (wv[e / 2] << 16));
                else v = __uint_as_float(wv[e]);
                acc[e] = acc[e] + v * ww[j];
            }
        }
        if (with_shared) {
            const uint4 raw = *(const uint4*)(y_rows + (shared_row * d + c) * EB);
            const uint32_t wv[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
            for (int e = 0; e < VE; e++) {
                float v;
                if constexpr (ACT_BF16) v = __uint_as_float(e & 1 ? (wv[e / 2] & 0xFFFF0000u) : (wv[e / 2] << 16));
                else v = __uint_as_float(wv[e]);
                acc[e] = acc[e] + v;
            }
        }
#pragma unroll
        for (int e = 0; e < VE; e += 4)
            *(float4*)(out + (int64_t)t * d + c + e) = make_float4(acc[e], acc[e + 1], acc[e + 2], acc[e + 3]);
    }
}

hipError_t launch_combine_partial(const moe_shape_t& s, const int32_t* idx, const int32_t* pos, const float* w,
                                  const Workspace& ws, int e0, int e1, int with_shared, float* y_partial,
                                  hipStream_t stream)
{
    if (s.act_dtype == MOE_BF16)
        combine_partial_kernel<true><<<combine_grid(s, 256), 256, 0, stream>>>(idx, pos, w, (const uint8_t*)ws.y_rows, (int)s.T,
                                                                        (int)s.d, (int)s.k, e0, e1, with_shared, y_partial);
    else
        combine_partial_kernel<false><<<combine_grid(s, 256), 256, 0, stream>>>(idx, pos, w, (const uint8_t*)ws.y_rows, (int)s.T,
                                                                         (int)s.d, (int)s.k, e0, e1, with_shared, y_partial);
    return hipGetLastError();
}

// Expert utilisation ("DeepSeek-V3's mixture-of-experts architecture explained", "Where the
// architecture struggles", log_expert_utilization): utilisation = counts / sum(counts) in fp32, and an
// alert flag per expert above 2x or below 0.1x the mean utilisation 1/E, decided on the exact integers
// (counts[e] * E > 2 * total, 10 * counts[e] * E < total).  One block; summary = (#over, #under).
__global__ __launch_bounds__(1024) void expert_utilization_kernel(int E, const int32_t* __restrict__ counts,
                                                                  float* __restrict__ util, int32_t* __restrict__ flags,
                                                                  int32_t* __restrict__ summary)
{
    __shared__ long long tot_lds[16];
    __shared__ int n_over, n_under;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    long long part = 0;
    for (int e = tid; e < E; e += 1024) part += counts[e];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) part += __shfl_xor(part, off, 64);
    if (lane == 0) tot_lds[wave] = part;
    if (tid == 0) n_over = n_under = 0;
    __syncthreads();
    long long total = 0;
    for (int i = 0; i < 16; i++) total += tot_lds[i];
    for (int e = tid; e < E; e += 1024) {
        const long long c = counts[e];
        util[e] = total > 0 ? (float)c / (float)total : 0.0f;
        const int over = total > 0 && c * E > 2 * total, under = total > 0 && 10 * c * E < total;
        flags[e] = over ? 1 : under ? -1 : 0;
        if (over) atomicAdd(&n_over, 1);
        if (under) atomicAdd(&n_under, 1);
    }
    __syncthreads();
    if (tid == 0) {
        summary[0] = n_over;
        summary[1] = n_under;
    }
}

hipError_t launch_expert_utilization(int E, const int32_t* counts, float* util, int32_t* flags, int32_t* summary,
                                     hipStream_t stream)
{
    expert_utilization_kernel<<<1, 1024, 0, stream>>>(E, counts, util, flags, summary);
    return hipGetLastError();
}

}  // namespace moe
