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

template <bool ACT_BF16>
__global__ __launch_bounds__(256) void combine_kernel(const int32_t* __restrict__ pos, const float* __restrict__ w,
                                                      const uint8_t* __restrict__ y_rows, int T, int d, int k,
                                                      uint8_t* __restrict__ y)
{
    constexpr int EB = ACT_BF16 ? 2 : 4;           // bytes per element
    constexpr int VE = 16 / EB;                    // elements per 16-byte vector
    const int t = blockIdx.x;
    int rr[16];
    float ww[16];
    for (int j = 0; j < k; j++) {
        rr[j] = pos[(size_t)t * k + j];
        ww[j] = w[(size_t)t * k + j];
    }
    // ascending row order (insertion sort of <= 16 entries; same on every thread)
    for (int a = 1; a < k; a++) {
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
    for (int c = threadIdx.x * VE; c < d; c += 256 * VE) {
        float acc[VE];
#pragma unroll
        for (int e = 0; e < VE; e++) acc[e] = 0.0f;
        for (int j = 0; j < k; j++) {
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
        const uint4 raw = *(const uint4*)(y_rows + (shared_row * d + c) * EB);
        const uint32_t wv[4] = {raw.x, raw.y, raw.z, raw.w};
        uint32_t o[4];
        if constexpr (ACT_BF16) {
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const float a0 = acc[2 * e] + __uint_as_float(wv[e] << 16);
                const float a1 = acc[2 * e + 1] + __uint_as_float(wv[e] & 0xFFFF0000u);
                o[e] = (uint32_t)f32_to_bf16(a0) | ((uint32_t)f32_to_bf16(a1) << 16);
            }
        } else {
#pragma unroll
            for (int e = 0; e < 4; e++) o[e] = __float_as_uint(acc[e] + __uint_as_float(wv[e]));
        }
        *(uint4*)(y + ((int64_t)t * d + c) * EB) = make_uint4(o[0], o[1], o[2], o[3]);
    }
}

hipError_t launch_combine(const moe_shape_t& s, const int32_t* pos, const float* w, const Workspace& ws, void* y,
                          hipStream_t stream)
{
    if (s.act_dtype == MOE_BF16)
        combine_kernel<true><<<(unsigned)s.T, 256, 0, stream>>>(pos, w, (const uint8_t*)ws.y_rows, (int)s.T, (int)s.d,
                                                                (int)s.k, (uint8_t*)y);
    else
        combine_kernel<false><<<(unsigned)s.T, 256, 0, stream>>>(pos, w, (const uint8_t*)ws.y_rows, (int)s.T, (int)s.d,
                                                                 (int)s.k, (uint8_t*)y);
    return hipGetLastError();
}

}  // namespace moe
