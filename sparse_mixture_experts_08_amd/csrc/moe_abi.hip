// moe_abi.hip -- the C entry points of moe.h: argument validation, workspace layout and the launch
// sequence of the layer (router -> top-k -> permutation -> [x quantisation] -> grouped up GEMM ->
// grouped down GEMM -> combine), all enqueued on the caller's stream with no host synchronisation.
#include <string.h>

#include <mutex>

#include "moe_common.h"

namespace moe {

static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

int tile_rows(const moe_shape_t& s)
{
    // By the average rows per routed expert: decode-sized groups (<= 24 rows) -> 16-row tiles (weight
    // streaming).  Otherwise bf16 takes 256-row tiles: an expert of up to 256 rows reads its weights once,
    // and a 256 x 256 output block needs fewer staged bytes per MFMA than 128 x 512; row blocks past a
    // tile's end are skipped.  fp8 takes 256-row tiles above 192 rows per expert (fewer staged bytes and
    // LDS fragment reads per MFMA), else 128; fp32 keeps 128.
    const int64_t per_expert = s.T * s.k / (s.E > 0 ? s.E : 1);
    if (per_expert <= 24) return 16;
    if (s.w_dtype == MOE_FP8_E4M3) return per_expert > 192 ? 256 : 128;
    if (s.act_dtype == MOE_F32) return 128;
    return 256;
}

Workspace carve_workspace(const moe_shape_t& s, void* base)
{
    Workspace w;
    memset(&w, 0, sizeof(w));
    const int64_t T = s.T, E = s.E, k = s.k, d = s.d;
    const int64_t rows = T * k + T;
    const int bm = tile_rows(s);
    w.nchunks = (T + 63) / 64;
    w.max_tiles = rows / bm + E + 2;
    w.inter_max = s.inter > s.inter_shared ? s.inter : s.inter_shared;
    const bool fp8 = s.w_dtype == MOE_FP8_E4M3;
    const size_t act = s.act_dtype == MOE_F32 ? 4 : 2;
    size_t off = 0;
    char* b = (char*)base;
    auto take = [&](size_t bytes) -> void* {
        void* p = b ? (void*)(b + off) : nullptr;
        off += align256(bytes);
        return p;
    };
    w.logits = (float*)take(sizeof(float) * T * E);
    w.idx = (int32_t*)take(sizeof(int32_t) * T * k);
    w.w = (float*)take(sizeof(float) * T * k);
    w.counts = (int32_t*)take(sizeof(int32_t) * E);
    w.offsets = (int32_t*)take(sizeof(int32_t) * (E + 1));
    w.chunk_counts = (int32_t*)take(sizeof(int32_t) * w.nchunks * E);
    w.chunk_prefix = (int32_t*)take(sizeof(int32_t) * w.nchunks * E);
    w.chunk_bits = (uint64_t*)take(sizeof(uint64_t) * w.nchunks * E);
    w.sorted_slots = (int32_t*)take(sizeof(int32_t) * T * k);
    w.pos = (int32_t*)take(sizeof(int32_t) * T * k);
    w.row_token = (int32_t*)take(sizeof(int32_t) * rows);
    w.tiles = (int4*)take(sizeof(int4) * w.max_tiles);
    w.sync = (int32_t*)take(sizeof(int32_t) * 4);
    if (fp8) {
        w.xq = (uint8_t*)take((size_t)T * d);
        w.xs = (float*)take(sizeof(float) * T * (d / 128));
        w.h = take((size_t)rows * w.inter_max);
        w.hs = (float*)take(sizeof(float) * rows * (w.inter_max / 128));
    } else {
        w.h = take(act * rows * w.inter_max);
    }
    w.y_rows = take(act * rows * d);
    w.total = off;
    return w;
}

// Host-side validation shared by both entry points.
static moe_status_t check_shape(const moe_shape_t* s)
{
    if (!s) return MOE_ERR_INVALID_ARG;
    if (s->T < 0 || s->d <= 0 || s->E <= 0 || s->k <= 0 || s->inter <= 0 || s->inter_shared <= 0)
        return MOE_ERR_INVALID_ARG;
    if (s->k > s->E) return MOE_ERR_INVALID_ARG;
    if (s->k > 16 || s->E > 1024) return MOE_ERR_UNSUPPORTED;
    if (s->d % 128 || s->inter % 128 || s->inter_shared % 128) return MOE_ERR_UNSUPPORTED;
    const bool ok = (s->act_dtype == MOE_F32 && s->w_dtype == MOE_F32) ||
                    (s->act_dtype == MOE_BF16 && s->w_dtype == MOE_BF16) ||
                    (s->act_dtype == MOE_BF16 && s->w_dtype == MOE_FP8_E4M3);
    if (!ok) return MOE_ERR_UNSUPPORTED;
    // int32 indexing of rows and elements inside the kernels
    if (s->T > (1 << 24) || (s->T * (s->k + 1)) * s->d > ((int64_t)1 << 40)) return MOE_ERR_UNSUPPORTED;
    // 32-bit byte offsets inside the GEMM operands: x, h, and one expert's weights each under 4 GB
    const int64_t ab = s->act_dtype == MOE_F32 ? 4 : 2, wb = s->w_dtype == MOE_FP8_E4M3 ? 1 : ab;
    const int64_t inter_max = s->inter > s->inter_shared ? s->inter : s->inter_shared;
    const int64_t lim = (int64_t)1 << 32;
    if (s->T * s->d * ab >= lim || s->T * (s->k + 1) * inter_max * ab >= lim ||
        inter_max * s->d * wb >= lim)
        return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

static bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

}  // namespace moe

using namespace moe;

extern "C" size_t moe_workspace_size(const moe_shape_t* shape)
{
    if (check_shape(shape) != MOE_OK) return 0;
    return carve_workspace(*shape, nullptr).total;
}

extern "C" const char* moe_status_string(moe_status_t st)
{
    switch (st) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape or dtype combination";
    case MOE_ERR_WORKSPACE: return "workspace too small or misaligned";
    case MOE_ERR_HIP: return "HIP launch failure";
    case MOE_ERR_SCRATCH: return "shape needs more workspace than the static scratch of moe_forward_noalloc holds";
    }
    return "unknown status";
}

#define MOE_TRY(expr)                                    \
    do {                                                 \
        if ((expr) != hipSuccess) return MOE_ERR_HIP;    \
    } while (0)

// Routing with an optional per-expert mask (allowed == NULL: every expert), or group-limited over
// n_group groups (n_group > 0; no mask).
static moe_status_t route_impl(const moe_shape_t* shape, const void* x, const float* Wg, const float* bias,
                               const uint8_t* allowed, int n_group, int32_t* idx, float* w, int32_t* counts,
                               int32_t* offsets, int32_t* sorted_slots, int32_t* pos, void* workspace,
                               size_t workspace_bytes, hipStream_t stream)
{
    moe_status_t st = check_shape(shape);
    if (st != MOE_OK) return st;
    const moe_shape_t& s = *shape;
    if (n_group > 0 && (s.E % n_group || s.E / n_group < 2 || s.k % 2 || s.k / 2 > n_group ||
                        n_group > (s.E <= 256 ? 16 : 64)))
        return MOE_ERR_UNSUPPORTED;
    if (s.T == 0) return MOE_OK;
    if (!x || !Wg || !idx || !w || !counts || !offsets || !sorted_slots || !workspace) return MOE_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(Wg)) return MOE_ERR_INVALID_ARG;
    Workspace ws = carve_workspace(s, workspace);
    if (workspace_bytes < ws.total || ((uintptr_t)workspace & 255)) return MOE_ERR_WORKSPACE;
    const TileRange all = {0, (int)s.E, 1};
    MOE_TRY(launch_router_logits(s, x, Wg, bias, ws.logits, stream));
    if (n_group == 0 && routing_is_fused(s)) {
        MOE_TRY(launch_routing_fused(s, ws.logits, allowed, idx, w, counts, offsets, sorted_slots, pos ? pos : ws.pos,
                                     ws, tile_rows(s), all, stream));
    } else {
        MOE_TRY(launch_topk(s, ws.logits, allowed, idx, w, ws, stream, n_group));
        MOE_TRY(launch_permute(s, idx, counts, offsets, sorted_slots, pos ? pos : ws.pos, ws, tile_rows(s), all,
                               stream));
    }
    return MOE_OK;
}

extern "C" moe_status_t moe_route(const moe_shape_t* shape, const void* x, const float* Wg, const float* bias,
                                  int32_t* idx, float* w, int32_t* counts, int32_t* offsets,
                                  int32_t* sorted_slots, int32_t* pos, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream)
{
    return route_impl(shape, x, Wg, bias, nullptr, 0, idx, w, counts, offsets, sorted_slots, pos, workspace,
                      workspace_bytes, stream);
}

extern "C" moe_status_t moe_route_grouped(const moe_shape_t* shape, int64_t n_group, const void* x, const float* Wg,
                                          const float* bias, int32_t* idx, float* w, int32_t* counts,
                                          int32_t* offsets, int32_t* sorted_slots, int32_t* pos, void* workspace,
                                          size_t workspace_bytes, hipStream_t stream)
{
    if (n_group < 1 || n_group > 1024) return MOE_ERR_INVALID_ARG;
    return route_impl(shape, x, Wg, bias, nullptr, (int)n_group, idx, w, counts, offsets, sorted_slots, pos,
                      workspace, workspace_bytes, stream);
}

extern "C" moe_status_t moe_route_limited(const moe_shape_t* shape, const void* x, const float* Wg,
                                          const float* bias, const uint8_t* allowed, int32_t* idx, float* w,
                                          int32_t* counts, int32_t* offsets, int32_t* sorted_slots, int32_t* pos,
                                          void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    if (!allowed) return MOE_ERR_INVALID_ARG;
    return route_impl(shape, x, Wg, bias, allowed, 0, idx, w, counts, offsets, sorted_slots, pos, workspace,
                      workspace_bytes, stream);
}

// Host-side checks of a layer call (everything but the workspace), shared by the entry points.
static moe_status_t check_layer_args(const moe_shape_t* shape, const void* x, const float* Wg, int64_t e0, int64_t e1,
                                     int64_t n_shared, const void* W1, const void* W3, const void* W2,
                                     const float* W1s, const float* W3s, const float* W2s, const void* S1,
                                     const void* S3, const void* S2, const float* S1s, const float* S3s,
                                     const float* S2s, const void* out)
{
    moe_status_t st = check_shape(shape);
    if (st != MOE_OK) return st;
    const moe_shape_t& s = *shape;
    if (e0 < 0 || e1 > s.E || e0 > e1 || n_shared < 0 || n_shared > s.inter_shared) return MOE_ERR_INVALID_ARG;
    if (n_shared % 128) return MOE_ERR_UNSUPPORTED;
    if (s.T == 0) return MOE_OK;
    const bool routed = e1 > e0, with_shared = n_shared > 0;
    const bool fp8 = s.w_dtype == MOE_FP8_E4M3;
    if (!x || !Wg || !out) return MOE_ERR_INVALID_ARG;
    if (routed && (!W1 || !W3 || !W2 || (fp8 && (!W1s || !W3s || !W2s)))) return MOE_ERR_INVALID_ARG;
    if (with_shared && (!S1 || !S3 || !S2 || (fp8 && (!S1s || !S3s || !S2s)))) return MOE_ERR_INVALID_ARG;
    if (x == out) return MOE_ERR_INVALID_ARG;
    const void* ptrs[] = {x, Wg, out, routed ? W1 : x, routed ? W3 : x, routed ? W2 : x, with_shared ? S1 : x,
                          with_shared ? S3 : x, with_shared ? S2 : x};
    for (const void* p : ptrs)
        if (!aligned16(p)) return MOE_ERR_INVALID_ARG;
    return MOE_OK;
}

// The layer or one expert-parallel rank's share of it.  Routed experts [e0, e1) (weights of expert e at
// index e - e0 of W1/W3/W2), n_shared shared hidden features; y (act dtype, rounded) or y_partial (fp32).
static moe_status_t layer_impl(const moe_shape_t* shape, const void* x, const float* Wg, const float* bias,
                               const uint8_t* allowed, int64_t e0, int64_t e1, int64_t n_shared, const void* W1,
                               const void* W3, const void* W2, const float* W1s, const float* W3s,
                               const float* W2s, const void* S1, const void* S3, const void* S2, const float* S1s,
                               const float* S3s, const float* S2s, void* y, float* y_partial, int32_t* idx_out,
                               float* w_out, int32_t* counts_out, void* workspace, size_t workspace_bytes,
                               hipStream_t stream, hipEvent_t* events)
{
    void* out = y ? y : (void*)y_partial;
    moe_status_t st = check_layer_args(shape, x, Wg, e0, e1, n_shared, W1, W3, W2, W1s, W3s, W2s, S1, S3, S2, S1s,
                                       S3s, S2s, out);
    if (st != MOE_OK) return st;
    const moe_shape_t& s = *shape;
    if (s.T == 0) return MOE_OK;
    const bool with_shared = n_shared > 0;
    const bool fp8 = s.w_dtype == MOE_FP8_E4M3;
    if (!workspace) return MOE_ERR_INVALID_ARG;
    Workspace ws = carve_workspace(s, workspace);
    if (workspace_bytes < ws.total || ((uintptr_t)workspace & 255)) return MOE_ERR_WORKSPACE;

    int32_t* idx = idx_out ? idx_out : ws.idx;
    float* w = w_out ? w_out : ws.w;
    int32_t* counts = counts_out ? counts_out : ws.counts;
    const TileRange tr = {(int)e0, (int)e1, with_shared ? 1 : 0};
    const int bm = tile_rows(s);
    auto mark = [&](int i) -> hipError_t { return events ? hipEventRecord(events[i], stream) : hipSuccess; };
    MOE_TRY(mark(0));
    MOE_TRY(launch_router_logits(s, x, Wg, bias, ws.logits, stream));
    MOE_TRY(mark(1));
    if (routing_is_fused(s)) {
        MOE_TRY(launch_routing_fused(s, ws.logits, allowed, idx, w, counts, ws.offsets, ws.sorted_slots, ws.pos, ws, bm,
                                     tr, stream));
        MOE_TRY(mark(2));
    } else {
        MOE_TRY(launch_topk(s, ws.logits, allowed, idx, w, ws, stream));
        MOE_TRY(mark(2));
        MOE_TRY(launch_permute(s, idx, counts, ws.offsets, ws.sorted_slots, ws.pos, ws, bm, tr, stream));
    }
    MOE_TRY(mark(3));
    if (fp8) MOE_TRY(launch_act_quant(s, x, ws, stream));
    MOE_TRY(mark(4));
    MOE_TRY(launch_up_gemm(s, x, W1, W3, W1s, W3s, S1, S3, S1s, S3s, ws, stream, (int)e0, (int)n_shared));
    MOE_TRY(mark(5));
    MOE_TRY(launch_down_gemm(s, W2, W2s, S2, S2s, ws, stream, (int)e0, (int)n_shared));
    MOE_TRY(mark(6));
    if (y) MOE_TRY(launch_combine(s, ws.pos, w, ws, y, stream));
    else MOE_TRY(launch_combine_partial(s, idx, ws.pos, w, ws, (int)e0, (int)e1, with_shared, y_partial, stream));
    MOE_TRY(mark(7));
    return MOE_OK;
}

extern "C" moe_status_t moe_forward_staged(const moe_shape_t* shape, const void* x, const float* Wg,
                                           const float* bias, const void* W1, const void* W3, const void* W2,
                                           const float* W1s, const float* W3s, const float* W2s, const void* S1,
                                           const void* S3, const void* S2, const float* S1s, const float* S3s,
                                           const float* S2s, void* y, int32_t* idx_out, float* w_out,
                                           int32_t* counts_out, void* workspace, size_t workspace_bytes,
                                           hipStream_t stream, hipEvent_t* events)
{
    if (!shape) return MOE_ERR_INVALID_ARG;
    return layer_impl(shape, x, Wg, bias, nullptr, 0, shape->E, shape->inter_shared, W1, W3, W2, W1s, W3s, W2s, S1,
                      S3, S2, S1s, S3s, S2s, y, nullptr, idx_out, w_out, counts_out, workspace, workspace_bytes,
                      stream, events);
}

extern "C" moe_status_t moe_forward(const moe_shape_t* shape, const void* x, const float* Wg, const float* bias,
                                    const void* W1, const void* W3, const void* W2, const float* W1s,
                                    const float* W3s, const float* W2s, const void* S1, const void* S3,
                                    const void* S2, const float* S1s, const float* S3s, const float* S2s, void* y,
                                    int32_t* idx_out, float* w_out, int32_t* counts_out, void* workspace,
                                    size_t workspace_bytes, hipStream_t stream)
{
    return moe_forward_staged(shape, x, Wg, bias, W1, W3, W2, W1s, W3s, W2s, S1, S3, S2, S1s, S3s, S2s, y, idx_out,
                              w_out, counts_out, workspace, workspace_bytes, stream, nullptr);
}

extern "C" moe_status_t moe_forward_shard(const moe_shape_t* shape, const void* x, const float* Wg,
                                          const float* bias, const uint8_t* allowed, int64_t e0, int64_t e1,
                                          int64_t n_shared, const void* W1, const void* W3, const void* W2,
                                          const float* W1s, const float* W3s, const float* W2s, const void* S1,
                                          const void* S3, const void* S2, const float* S1s, const float* S3s,
                                          const float* S2s, float* y_partial, int32_t* idx_out, float* w_out,
                                          int32_t* counts_out, void* workspace, size_t workspace_bytes,
                                          hipStream_t stream, hipEvent_t* events)
{
    return layer_impl(shape, x, Wg, bias, allowed, e0, e1, n_shared, W1, W3, W2, W1s, W3s, W2s, S1, S3, S2, S1s, S3s,
                      S2s, nullptr, y_partial, idx_out, w_out, counts_out, workspace, workspace_bytes, stream,
                      events);
}

extern "C" moe_status_t moe_quantize_e4m3(int64_t rows, int64_t cols, const void* x, uint8_t* q, float* scales,
                                          hipStream_t stream)
{
    if (rows < 0 || cols <= 0) return MOE_ERR_INVALID_ARG;
    if (cols % 128 || cols > (1 << 30) || rows > ((int64_t)1 << 40) / cols) return MOE_ERR_UNSUPPORTED;
    if (rows == 0) return MOE_OK;
    if (!x || !q || !scales || !aligned16(x) || !aligned16(q) || ((uintptr_t)scales & 3)) return MOE_ERR_INVALID_ARG;
    MOE_TRY(launch_quantize_e4m3(rows, (int)cols, x, q, scales, stream));
    return MOE_OK;
}

extern "C" moe_status_t moe_expert_utilization(int64_t E, const int32_t* counts, float* util, int32_t* flags,
                                               int32_t* summary, hipStream_t stream)
{
    if (E <= 0 || E > (1 << 30) || !counts || !util || !flags || !summary) return MOE_ERR_INVALID_ARG;
    MOE_TRY(launch_expert_utilization((int)E, counts, util, flags, summary, stream));
    return MOE_OK;
}

// ---------------------------------------------------------------------------------------------------
// moe_forward without a workspace argument, for callers that cannot allocate device memory.  The
// workspace is this file-scope device array: every GPU the library runs on holds its own copy, from the
// loading of the library's code object on that GPU until the process ends.  In host code `scratch` names
// a host-side stand-in, not device memory, so its device address is looked up once per device (with that
// device current) and only that address is handed to the kernels.
// ---------------------------------------------------------------------------------------------------
static __device__ __attribute__((aligned(256))) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

static constexpr int NOALLOC_MAX_DEVICES = 64;

// Device address of `scratch` on the current device (looked up on the first call per device), or null
// with *err set.
static void* scratch_on_current_device(hipError_t* err)
{
    static std::mutex mu;
    static void* addr[NOALLOC_MAX_DEVICES] = {};
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        *err = e;
        return nullptr;
    }
    if (dev < 0 || dev >= NOALLOC_MAX_DEVICES) {
        *err = hipErrorInvalidDevice;
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            *err = e != hipSuccess ? e : hipErrorInvalidSymbol;
            return nullptr;
        }
        addr[dev] = p;
    }
    return addr[dev];
}

extern "C" moe_status_t moe_forward_noalloc(const moe_shape_t* shape, const void* x, const float* Wg,
                                            const float* bias, const void* W1, const void* W3, const void* W2,
                                            const float* W1s, const float* W3s, const float* W2s, const void* S1,
                                            const void* S3, const void* S2, const float* S1s, const float* S3s,
                                            const float* S2s, void* y, int32_t* idx_out, float* w_out,
                                            int32_t* counts_out, hipStream_t stream)
{
    if (!shape) return MOE_ERR_INVALID_ARG;
    moe_status_t st = check_layer_args(shape, x, Wg, 0, shape->E, shape->inter_shared, W1, W3, W2, W1s, W3s, W2s,
                                       S1, S3, S2, S1s, S3s, S2s, y);
    if (st != MOE_OK) return st;
    if (shape->T == 0) return MOE_OK;
    if (carve_workspace(*shape, nullptr).total > MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_SCRATCH;
    hipError_t err = hipSuccess;
    void* ws = scratch_on_current_device(&err);
    if (!ws) return MOE_ERR_HIP;
    return layer_impl(shape, x, Wg, bias, nullptr, 0, shape->E, shape->inter_shared, W1, W3, W2, W1s, W3s, W2s, S1,
                      S3, S2, S1s, S3s, S2s, y, nullptr, idx_out, w_out, counts_out, ws, MOE_NOALLOC_SCRATCH_BYTES,
                      stream, nullptr);
}
