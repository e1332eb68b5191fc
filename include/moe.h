/*
 * moe.h -- C ABI of the MI355X (gfx950) forward pass of one DeepSeek-V3-style mixture-of-experts
 * feed-forward layer.
 *
 * The layer (per token t, x[t] a row of d activations):
 *   logits[e] = sum_i x[t][i] * Wg[e][i]  (+ bias[e])                       router, fp32
 *   (idx, v)  = the k largest logits, descending, equal logits -> lower e
 *   w         = softmax(v) over the k selected logits only
 *   y[t]      = sum_j w[j] * SwiGLU_{idx[j]}(x[t]) + SwiGLU_shared(x[t])
 *   SwiGLU(x) = W2 (silu(W1 x) * (W3 x))
 * as stated on "DeepSeek-V3's mixture-of-experts architecture explained" (block pseudocode of
 * "The architecture in one diagram": gate, topk, softmax over the selected values) and on
 * "DeepSeek-V3.2-Exp / Mixture of experts / Shared expert" ("All 5 steps"; the MoE forward excerpt:
 * fp32 accumulation of expert(x) * weight per expert, then + shared_experts(x); the MLP forward
 * excerpt: silu * mul formed in fp32, cast back to the activation dtype before w2).
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers, row-major, densely packed, owned by the caller.  The
 *    library allocates and frees nothing and keeps no state between calls, except moe_forward_noalloc's
 *    static device scratch (see there).
 *  - All work is enqueued on `stream` (a hipStream_t; NULL = the default stream) without any host
 *    synchronisation; results are valid once the caller synchronises the stream.
 *  - Argument errors are detected on the host before any launch; nothing is written then.
 *    Launch failures return MOE_ERR_HIP.  Device faults surface at the caller's next synchronisation.
 *  - Calls are reentrant.  Concurrent calls must use different workspaces and outputs.
 *  - fp8 weights are quantised in 128 x 128 blocks and fp8 activations in 1 x 128 groups: the block
 *    edge is fixed at 128 (the configurations' quantisation block), so d, inter and inter_shared are
 *    multiples of 128 for every dtype.
 *  - Inputs are assumed finite; NaN/Inf inputs are outside the contract.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = 1,   /* null required pointer, negative size, k > E, y aliasing x, bad alignment */
    MOE_ERR_UNSUPPORTED = 2,   /* dtype combination, d / inter not multiples of 128, k > 16, E > 1024 */
    MOE_ERR_WORKSPACE = 3,     /* workspace smaller than moe_workspace_size() */
    MOE_ERR_HIP = 4,           /* a kernel launch failed */
    MOE_ERR_SCRATCH = 5        /* moe_forward_noalloc: the shape needs more than MOE_NOALLOC_SCRATCH_BYTES */
} moe_status_t;

typedef enum {
    MOE_F32 = 0,               /* IEEE binary32 */
    MOE_BF16 = 1,              /* bfloat16 */
    MOE_FP8_E4M3 = 2           /* OCP 8-bit E4M3 ("FN": max 448, no infinities), weights only */
} moe_dtype_t;

/*
 * Sizes and dtypes of one layer invocation.
 *   T             tokens (rows of x and y), T >= 0
 *   d             model width (7168 for DeepSeek-V3), multiple of 128
 *   E             routed experts (256), 1 <= E <= 1024
 *   k             experts per token (8), 1 <= k <= min(E, 16)
 *   inter         routed expert width (2048), multiple of 128
 *   inter_shared  shared expert width (n_shared * inter = 2048), multiple of 128
 *   act_dtype     dtype of x, y and every activation between linears: MOE_F32 or MOE_BF16
 *   w_dtype       dtype of W1, W3, W2 and S1, S3, S2.  Supported pairs (act, w):
 *                 (F32, F32), (BF16, BF16), (BF16, FP8_E4M3).
 * The router is fp32 in every case (Wg, bias and logits).
 */
typedef struct {
    int64_t T, d, E, k, inter, inter_shared;
    int32_t act_dtype, w_dtype;
} moe_shape_t;

/*
 * Bytes of device workspace moe_route / moe_forward need for `shape` (a pure host function; 0 on an
 * invalid shape).  The workspace must be 256-byte aligned.  Its contents need no initialisation and
 * are undefined afterwards.
 */
size_t moe_workspace_size(const moe_shape_t* shape);

/*
 * Routing only: router logits, top-k, softmax and the expert-sorted permutation.
 * Gate: "DeepSeek-V3's mixture-of-experts architecture explained", "The architecture in one diagram",
 * block pseudocode (router_logits = self.gate(x); weights, indices = topk(router_logits, k=8); weights =
 * softmax(weights)); counts and the expert-sorted rows: "DeepSeek-V3.2-Exp / Mixture of experts", MoE
 * forward excerpt (bincount of the indices; torch.where(indices == i) per expert, row-major).
 *   x            [T, d] act_dtype
 *   Wg           [E, d] fp32 router weight, the gate's nn.Linear(d, E) weight (logits = x Wg^T);
 *                16-byte aligned.  This is the transpose of the math-orientation [d, E] ("Wg 7168 x 256"
 *                in the configurations): the nn.Linear [out, in] layout the pages' gate wraps, which
 *                gives every expert's FMA chain one contiguous row.  A [d, E] array is passed as its
 *                transpose.
 *   bias         [E] fp32 logit bias added before selection, or NULL
 *   idx    out   [T, k] int32 selected experts, descending logit, ties -> lower expert index
 *   w      out   [T, k] fp32 softmax over the k selected logits
 *   counts out   [E] int32 tokens routed to each expert (torch.bincount of idx)
 *   offsets out  [E + 1] int32 exclusive prefix sum of counts
 *   sorted_slots out [T * k] int32 slot ids t*k+j, expert by expert, tokens ascending within an expert
 *   pos    out   [T * k] int32 inverse of sorted_slots, or NULL
 * Logits are one fp32 fused-multiply-add chain per (token, expert) over i ascending, then one fp32 add
 * of bias[e], so routing is a deterministic function of the inputs.
 */
moe_status_t moe_route(const moe_shape_t* shape, const void* x, const float* Wg, const float* bias,
                       int32_t* idx, float* w, int32_t* counts, int32_t* offsets, int32_t* sorted_slots,
                       int32_t* pos, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * The whole layer: routing, routed SwiGLU experts, shared SwiGLU expert and the weighted combine.
 * "DeepSeek-V3.2-Exp / Mixture of experts / Shared expert": MoE forward excerpt (y = zeros in fp32;
 * y[idx] += expert(x[idx]) * weights[idx, top] per expert; y += shared_experts(x)), "All 5 steps" and the
 * MLP forward excerpt (w2(silu(w1(x)) * w3(x)), silu * mul in fp32, cast back before w2); routing as in
 * moe_route.
 *   x        [T, d] act_dtype (not modified; must not alias y)
 *   Wg, bias as in moe_route
 *   W1, W3   [E, inter, d] w_dtype (nn.Linear [out, in] layout: g = x W1^T per expert)
 *   W2       [E, d, inter] w_dtype
 *   S1, S3   [inter_shared, d] w_dtype;  S2 [d, inter_shared] w_dtype
 *   W1s, W3s [E, inter/128, d/128] fp32, W2s [E, d/128, inter/128] fp32, S1s, S3s
 *            [inter_shared/128, d/128] fp32, S2s [d/128, inter_shared/128] fp32: one scale per 128x128
 *            weight block, value = code * scale.  Required iff w_dtype == MOE_FP8_E4M3, else ignored.
 *   y    out [T, d] act_dtype
 *   idx_out, w_out [T, k], counts_out [E]: optional copies of the routing (NULL to skip)
 * Rounding: each linear's output is rounded to act_dtype; silu(g)*u is formed in fp32 and rounded to
 * act_dtype; with fp8 weights, x and h are quantised per 1x128 group (s = amax/448, codes = E4M3
 * round-to-nearest-even of v/s); the combine accumulates w * expert output and the shared output in
 * fp32 in a fixed order and rounds once to act_dtype.  The result is bitwise deterministic.
 */
moe_status_t moe_forward(const moe_shape_t* shape, const void* x, const float* Wg, const float* bias,
                         const void* W1, const void* W3, const void* W2,
                         const float* W1s, const float* W3s, const float* W2s,
                         const void* S1, const void* S3, const void* S2,
                         const float* S1s, const float* S3s, const float* S2s,
                         void* y, int32_t* idx_out, float* w_out, int32_t* counts_out,
                         void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * moe_forward with stage timing: identical work and results, and events[i] (hipEvent_t, created by the
 * caller) is recorded on `stream` before stage i and events[MOE_NUM_STAGES] after the last stage, so
 * hipEventElapsedTime(events[i], events[i+1]) is the device time of stage i.  Stages, in order:
 *   0 router logits, 1 top-k + softmax (with T <= 256 also the permutation and tile list, one launch),
 *   2 permutation and tile list (empty when done in stage 1), 3 x quantisation (fp8 weights only;
 *   empty otherwise), 4 grouped up GEMM (W1, W3, SiLU*mul; routed and shared), 5 grouped down GEMM
 *   (W2), 6 combine.
 * events may be NULL (then it is moe_forward).
 */
#define MOE_NUM_STAGES 7
moe_status_t moe_forward_staged(const moe_shape_t* shape, const void* x, const float* Wg, const float* bias,
                                const void* W1, const void* W3, const void* W2,
                                const float* W1s, const float* W3s, const float* W2s,
                                const void* S1, const void* S3, const void* S2,
                                const float* S1s, const float* S3s, const float* S2s,
                                void* y, int32_t* idx_out, float* w_out, int32_t* counts_out,
                                void* workspace, size_t workspace_bytes, hipStream_t stream,
                                hipEvent_t* events);

/*
 * Device-limited routing ("DeepSeek-V3's mixture-of-experts architecture explained", "Why 256 experts
 * with top-8 routing?", device_limited_routing: logits outside the experts of the current device get a
 * -inf mask before the top-k).  moe_route with one extra input:
 *   allowed  [E] uint8 device array, nonzero = the expert may be selected; the same mask for every
 *            token.  Required (NULL -> MOE_ERR_INVALID_ARG).
 * Selection is the top-k of (logit + mask) with the mask -inf outside `allowed` and 0 inside, equal
 * values -> lower expert index; the softmax is over those k masked values.  When fewer than k experts
 * are allowed, the surplus slots select the lowest-index experts outside `allowed` and get weight 0.
 * At least one entry of `allowed` must be nonzero (it lives in device memory, so this is not
 * checked); with none, every weight is NaN.  All other arguments, outputs and guarantees as moe_route.
 */
moe_status_t moe_route_limited(const moe_shape_t* shape, const void* x, const float* Wg, const float* bias,
                               const uint8_t* allowed, int32_t* idx, float* w, int32_t* counts, int32_t* offsets,
                               int32_t* sorted_slots, int32_t* pos, void* workspace, size_t workspace_bytes,
                               hipStream_t stream);

/*
 * fp8 activation quantisation, the layer's step for activations entering an fp8 linear (the fp8
 * configuration's 1 x 128 activation groups; "DeepSeek-V3.2-Exp / Mixture of experts / Shared expert",
 * the FP8 block-scale note under the parameter table: the checkpoint's weights carry block scales), on its
 * own: for every row and every group of 128 consecutive columns, s = amax / 448 in fp32 (s = 1 when the
 * group is all zeros) and q = E4M3(v / s), v / s an IEEE fp32 division, rounded to nearest even and
 * saturated to +-448 (OCP E4M3 "FN": no infinities).  moe_forward applies the same rule to x and to h.
 *   x       [rows, cols] bf16 (uint16 bit patterns), 16-byte aligned
 *   q       [rows, cols] E4M3 codes (uint8), 16-byte aligned (written)
 *   scales  [rows, cols / 128] fp32 (written)
 * cols a positive multiple of 128 (else MOE_ERR_UNSUPPORTED), rows >= 0 (rows = 0: a no-op).  Null or
 * misaligned pointers return MOE_ERR_INVALID_ARG before any launch.
 */
moe_status_t moe_quantize_e4m3(int64_t rows, int64_t cols, const void* x, uint8_t* q, float* scales,
                               hipStream_t stream);

/*
 * Group-limited routing ("Technical Architecture and Core Innovations", "Architectural Breakthroughs",
 * item 1, "Hierarchical Dynamic Routing": a two-layer gate first distributes tokens over expert groups by
 * a softmax, then selects two experts per group).  Taken as: the E experts form n_group groups of
 * E / n_group consecutive experts (expert e in group e / (E / n_group)); a group's candidates are its two
 * largest logits (equal logits -> lower index) and its score is the fp32 sum of those two logits; the
 * k / 2 groups with the largest scores are kept (equal scores -> lower group index), and the token's k
 * experts are their candidates, in descending-logit order as moe_route's slots.  w is the softmax over
 * those k logits, as in moe_route.  With 8 groups and k = 8 this is two experts from each of four groups.
 *   n_group  groups: divides E, E / n_group >= 2, k even, k / 2 <= n_group, and n_group <= 16 for
 *            E <= 256 (<= 64 above); otherwise MOE_ERR_UNSUPPORTED (n_group < 1: MOE_ERR_INVALID_ARG).
 * All other arguments, outputs and guarantees as moe_route (the bias is added before selection).
 */
moe_status_t moe_route_grouped(const moe_shape_t* shape, int64_t n_group, const void* x, const float* Wg,
                               const float* bias, int32_t* idx, float* w, int32_t* counts, int32_t* offsets,
                               int32_t* sorted_slots, int32_t* pos, void* workspace, size_t workspace_bytes,
                               hipStream_t stream);

/*
 * One expert-parallel rank's share of the layer ("DeepSeek-V3.2-Exp / Mixture of experts", MoE
 * __init__ and forward excerpts: a rank owns the routed experts [experts_start_idx, experts_end_idx)
 * and a slice of the shared expert, adds their outputs into an fp32 y, and dist.all_reduce(y) sums the
 * ranks' y).  Every token is routed over all E experts (or the `allowed` ones), as each rank runs the
 * full gate; only the rank's experts and shared slice are computed.
 *   allowed   [E] uint8 routing mask as in moe_route_limited, or NULL for plain routing
 *   e0, e1    routed experts of this rank, 0 <= e0 <= e1 <= E (e0 == e1: none)
 *   n_shared  shared-expert hidden features of this rank, 0 <= n_shared <= inter_shared, multiple of 128
 *   W1, W3    [e1 - e0, inter, d] w_dtype, W2 [e1 - e0, d, inter]: the rank's experts only (expert e
 *             at index e - e0); scales W1s, W3s, W2s likewise.  May be NULL when e0 == e1.
 *   S1, S3    [n_shared, d] w_dtype, S2 [d, n_shared]: the rank's slice of the shared expert (rows of
 *             S1/S3 and the matching columns of S2, stored densely); scales S1s, S3s
 *             [n_shared/128, d/128], S2s [d/128, n_shared/128].  May be NULL when n_shared == 0.
 *   y_partial out [T, d] fp32:  sum over the token's selected experts e in [e0, e1), ascending e, of
 *             w * expert_e(x) (each expert output rounded to act_dtype, the products summed in fp32),
 *             then + the shared slice's output (its W2 product rounded to act_dtype).  Not rounded.
 *   idx_out, w_out, counts_out  optional copies of the full routing, as in moe_forward.
 * With e0 = 0, e1 = E, n_shared = inter_shared, rounding y_partial to act_dtype gives moe_forward's y
 * bitwise.  The sum of y_partial over ranks that partition the experts and the shared features is the
 * layer output up to fp32 reassociation and the rounding of each shared slice.
 * shape->inter_shared is the full shared width (it sizes the workspace; moe_workspace_size applies).
 * events: NULL, or MOE_NUM_STAGES + 1 caller-created events recorded between the stages as in
 * moe_forward_staged (stage 6 is the partial combine).
 */
moe_status_t moe_forward_shard(const moe_shape_t* shape, const void* x, const float* Wg, const float* bias,
                               const uint8_t* allowed, int64_t e0, int64_t e1, int64_t n_shared,
                               const void* W1, const void* W3, const void* W2,
                               const float* W1s, const float* W3s, const float* W2s,
                               const void* S1, const void* S3, const void* S2,
                               const float* S1s, const float* S3s, const float* S2s,
                               float* y_partial, int32_t* idx_out, float* w_out, int32_t* counts_out,
                               void* workspace, size_t workspace_bytes, hipStream_t stream, hipEvent_t* events);

/*
 * Expert-utilisation monitor ("DeepSeek-V3's mixture-of-experts architecture explained", "Where the
 * architecture struggles", log_expert_utilization: utilisation = bincount / its sum, with an alert for
 * experts above 2x or below 0.1x the mean).  One single-block launch.
 *   counts      [E] int32 device: tokens per expert (the counts output of moe_route / moe_forward)
 *   util   out  [E] fp32: float(counts[e]) / float(sum of counts), correctly rounded; 0 if the sum is 0
 *   flags  out  [E] int32: +1 if util > 2/E, -1 if util < 0.1/E, else 0, decided exactly on the
 *               integers (counts[e] * E > 2 * sum, 10 * counts[e] * E < sum); all 0 if the sum is 0
 *   summary out [2] int32: number of +1 flags, number of -1 flags
 * E >= 1 (else MOE_ERR_INVALID_ARG); counts must be >= 0.
 */
moe_status_t moe_expert_utilization(int64_t E, const int32_t* counts, float* util, int32_t* flags,
                                    int32_t* summary, hipStream_t stream);

/*
 * moe_forward for callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): the same arguments, results and guarantees as
 * moe_forward, without the workspace arguments.  Its workspace is a static device array of
 * MOE_NOALLOC_SCRATCH_BYTES inside the library: each GPU the library runs on holds one copy from the
 * moment the library's kernels are loaded on it until the process ends (64 MiB; enough for moe_forward's
 * workspace at decode sizes, e.g. T <= 256 tokens at d = 7168, E = 256, k = 8, inter = 2048).
 *  - A shape whose moe_workspace_size() exceeds MOE_NOALLOC_SCRATCH_BYTES returns MOE_ERR_SCRATCH
 *    before any device work.  Argument errors as moe_forward.
 *  - The call allocates and frees nothing.  Its first call on a device looks up the array's device
 *    address there (hipGetSymbolAddress); failure returns MOE_ERR_HIP.
 *  - The array used is the current device's (hipGetDevice): `stream` must belong to that device (the
 *    null stream does), as every pointer argument must point to its memory.
 *  - Every call on one GPU uses that GPU's one array, which keeps the last call's contents (no call reads
 *    what an earlier one left: nothing in it needs clearing).  Calls that overlap on one GPU -- on
 *    different streams, or from different host threads without ordering -- race on it: serialise them,
 *    or use moe_forward with a workspace per concurrent call.
 */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
moe_status_t moe_forward_noalloc(const moe_shape_t* shape, const void* x, const float* Wg, const float* bias,
                                 const void* W1, const void* W3, const void* W2,
                                 const float* W1s, const float* W3s, const float* W2s,
                                 const void* S1, const void* S3, const void* S2,
                                 const float* S1s, const float* S3s, const float* S2s,
                                 void* y, int32_t* idx_out, float* w_out, int32_t* counts_out,
                                 hipStream_t stream);

/* Static description of a status code. */
const char* moe_status_string(moe_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
