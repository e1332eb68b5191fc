// permute.hip -- per-expert counts, offsets, the expert-sorted slot order and the grouped-GEMM tile list.
//
// What it computes is what the MoE forward excerpt on "DeepSeek-V3.2-Exp / Mixture of experts" does on
// the host: a bincount of the selected indices, then per expert the (token, slot) pairs that chose it,
// tokens ascending (torch.where scans row-major).  Here it runs on 64-token chunks with no host
// synchronisation and no order-dependent atomics:
//   - a 64-bit mask per (chunk, expert) of the chunk's tokens that chose it (built with the top-k);
//   - counts = popcounts summed over chunks; offsets = exclusive scan of counts over experts;
//   - a slot's position is offsets[e] + (tokens of earlier chunks in e) + (earlier tokens of its own
//     chunk in e's mask), so positions are unique and ascending in token order within each expert.
// Sorted rows [0, T*k) hold the routed slots; rows [T*k, T*k + T) are the shared expert's, token order.
//
// Two paths: up to 256 tokens, one block does top-k, masks, scans, scatter and tiles in one launch;
// beyond that, a top-k kernel per chunk (router.hip), a per-expert scan over the chunks, and a scatter
// kernel whose every block scans the expert counts itself (block 0 also stores offsets and the tiles).
// Group-limited routing takes the second path at every token count.
#include "moe_common.h"
#include "topk.h"

namespace moe {

constexpr int kFusedMaxTokens = 256;

// Tile list for groups with counts cnt[0..E) and offsets off[0..E]: shared expert (group E, rows
// [T*k, T*k + T)) first when `shared` is set, then the experts of [g0, g1) ascending, each cut into
// ceil(rows / bm) tiles of at most bm rows.  One thread per expert; called by all NT threads of the block.
template <int NT>
__device__ void write_tiles(const int* cnt, const int* off, int E, int T, int k, int bm, TileRange tr, int4* tiles,
                            int32_t* ntiles, int* scan_lds)
{
    const int nshared = tr.shared ? (T + bm - 1) / bm : 0;
    for (int i = threadIdx.x; i < nshared; i += NT) tiles[i] = make_int4(E, T * k + i * bm, min(bm, T - i * bm), 0);
    int carry = nshared;
    for (int e0 = 0; e0 < E; e0 += NT) {
        const int e = e0 + threadIdx.x;
        const int c = (e < E && e >= tr.g0 && e < tr.g1) ? cnt[e] : 0;
        const int nt = (c + bm - 1) / bm;
        int total;
        const int base = carry + block_exclusive_scan<NT>(nt, &total, scan_lds);
        // The expert's ceil(c / 16) blocks of 16 rows dealt evenly over its nt = ceil(c / bm) tiles (tile i
        // takes blocks [i nb / nt, (i + 1) nb / nt), 1 to bm rows, only the last one ragged), so an expert
        // just over a multiple of bm rows gets no nearly empty last tile.
        const int nb = (c + 15) / 16;
        for (int i = 0; i < nt; i++) {
            const int r0 = 16 * (int)((int64_t)i * nb / nt), r1 = min(16 * (int)((int64_t)(i + 1) * nb / nt), c);
            tiles[base + i] = make_int4(e, off[e] + r0, r1 - r0, 0);
        }
        carry += total;
    }
    if (threadIdx.x == 0) ntiles[0] = carry;
}

// ---------------------------------------------------------------------------------------------------
// Fused path (T <= 256): one block of 1024 threads.
// ---------------------------------------------------------------------------------------------------
// SMALL_E: E <= 256 (16 lanes per token); otherwise a wavefront per token (E <= 1024).
template <bool SMALL_E>
__global__ __launch_bounds__(1024) void route_fused_kernel(const float* __restrict__ L, const uint8_t* __restrict__ allowed,
                                                           int T, int E, int k, int bm, TileRange tr,
                                                           int32_t* __restrict__ idx, float* __restrict__ w,
                                                           int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ sorted_slots, int32_t* __restrict__ pos,
                                                           int32_t* __restrict__ row_token, int4* __restrict__ tiles,
                                                           int32_t* __restrict__ sync)
{
    __shared__ uint32_t bits_lo[4][1024], bits_hi[4][1024];   // [chunk][expert]
    __shared__ int cnt[1024], off[1025], cpre[4][1024];
    __shared__ int idx_s[kFusedMaxTokens * 16];
    __shared__ int scan_lds[17];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nch = (T + 63) / 64;
    for (int i = tid; i < 4 * 1024; i += 1024) (&bits_lo[0][0])[i] = (&bits_hi[0][0])[i] = 0;
    __syncthreads();

    // top-k: 16 lanes per token when E <= 256, else a whole wavefront per token
    if constexpr (SMALL_E) {
        const int g = lane >> 4, sub = lane & 15;
        for (int t0 = wave * 4; t0 < T; t0 += 64) {
            const int t = t0 + g;
            const bool valid = t < T;
            int my_e;
            float my_w;
            topk_group<16, 16>(L + (size_t)(valid ? t : 0) * E, allowed, E, k, sub, my_e, my_w);
            if (valid && sub < k) {
                idx[(size_t)t * k + sub] = my_e;
                w[(size_t)t * k + sub] = my_w;
                idx_s[t * k + sub] = my_e;
                const int c = t >> 6, tl = t & 63;
                if (tl < 32) atomicOr(&bits_lo[c][my_e], 1u << tl);
                else atomicOr(&bits_hi[c][my_e], 1u << (tl - 32));
            }
        }
    } else {
        for (int t = wave; t < T; t += 16) {
            int my_e;
            float my_w;
            topk_group<64, 16>(L + (size_t)t * E, allowed, E, k, lane, my_e, my_w);
            if (lane < k) {
                idx[(size_t)t * k + lane] = my_e;
                w[(size_t)t * k + lane] = my_w;
                idx_s[t * k + lane] = my_e;
                const int c = t >> 6, tl = t & 63;
                if (tl < 32) atomicOr(&bits_lo[c][my_e], 1u << tl);
                else atomicOr(&bits_hi[c][my_e], 1u << (tl - 32));
            }
        }
    }
    __syncthreads();

    // counts and per-chunk prefixes (one thread per expert)
    int my_cnt = 0;
    if (tid < E) {
        for (int c = 0; c < nch; c++) {
            cpre[c][tid] = my_cnt;
            my_cnt += __popcll(((uint64_t)bits_hi[c][tid] << 32) | bits_lo[c][tid]);
        }
        cnt[tid] = my_cnt;
    }
    int total;
    const int excl = block_exclusive_scan<1024>(tid < E ? my_cnt : 0, &total, scan_lds);
    if (tid < E) {
        off[tid] = excl;
        counts[tid] = my_cnt;
        offsets[tid] = excl;
    }
    if (tid == 0) {
        off[E] = total;
        offsets[E] = total;
    }
    __syncthreads();

    // scatter
    for (int s = tid; s < T * k; s += 1024) {
        const int t = s / k, e = idx_s[s], c = t >> 6, tl = t & 63;
        const uint64_t mask = ((uint64_t)bits_hi[c][e] << 32) | bits_lo[c][e];
        const uint64_t below = tl ? (~0ull >> (64 - tl)) : 0ull;
        const int p = off[e] + cpre[c][e] + __popcll(mask & below);
        pos[s] = p;
        sorted_slots[p] = s;
        row_token[p] = t;
    }
    for (int t = tid; t < T; t += 1024) row_token[T * k + t] = t;
    write_tiles<1024>(cnt, off, E, T, k, bm, tr, tiles, sync, scan_lds);
}

// ---------------------------------------------------------------------------------------------------
// Multi-block path.
// ---------------------------------------------------------------------------------------------------
// One block per expert: the exclusive scan of its per-chunk counts over the chunks, and its total.
__global__ __launch_bounds__(256) void chunk_scan_kernel(const int32_t* __restrict__ chunk_counts, int nchunks, int E,
                                                         int32_t* __restrict__ chunk_prefix, int32_t* __restrict__ counts)
{
    __shared__ int scan_lds[5];
    const int e = blockIdx.x, tid = threadIdx.x;
    const int per = (nchunks + 255) / 256;
    const int c0 = tid * per, c1 = min(c0 + per, nchunks);
    int sum = 0;
    for (int c = c0; c < c1; c++) sum += chunk_counts[(size_t)c * E + e];
    int total;
    int run = block_exclusive_scan<256>(sum, &total, scan_lds);
    for (int c = c0; c < c1; c++) {
        const int v = chunk_counts[(size_t)c * E + e];
        chunk_prefix[(size_t)c * E + e] = run;
        run += v;
    }
    if (tid == 0) counts[e] = total;
}

// One thread per (token, slot) s: its sorted row is the expert's offset, plus the chunk prefix of earlier
// chunks, plus the tokens of its own chunk below it in the expert's mask.  Every block first scans the E
// counts into offsets in LDS (E <= 1024 values: cheaper than a grid-wide hand-off); block 0 also stores
// the offsets and the tile list.  Threads s < T write the shared expert's row table.
__global__ __launch_bounds__(256) void scatter_kernel(const int32_t* __restrict__ idx, const uint64_t* __restrict__ chunk_bits,
                                                      const int32_t* __restrict__ chunk_prefix,
                                                      const int32_t* __restrict__ counts, int T, int E, int k, int bm,
                                                      TileRange tr, int32_t* __restrict__ offsets,
                                                      int32_t* __restrict__ sorted_slots, int32_t* __restrict__ pos,
                                                      int32_t* __restrict__ row_token, int4* __restrict__ tiles,
                                                      int32_t* __restrict__ ntiles)
{
    __shared__ int cnt[1024], off[1025];
    __shared__ int scan_lds[5];
    const int tid = threadIdx.x;
    int carry = 0;
    for (int g0 = 0; g0 < E; g0 += 256) {
        const int g = g0 + tid;
        const int c = g < E ? counts[g] : 0;
        int tot;
        const int ex = carry + block_exclusive_scan<256>(c, &tot, scan_lds);
        if (g < E) {
            cnt[g] = c;
            off[g] = ex;
        }
        carry += tot;
    }
    if (tid == 0) off[E] = carry;
    __syncthreads();
    if (blockIdx.x == 0) {                              // block-uniform
        for (int g = tid; g <= E; g += 256) offsets[g] = off[g];
        write_tiles<256>(cnt, off, E, T, k, bm, tr, tiles, ntiles, scan_lds);
    }

    const int s = blockIdx.x * 256 + tid;
    if (s < T) row_token[T * k + s] = s;
    if (s >= T * k) return;
    const int t = s / k, c = t >> 6, tl = t & 63;
    const int e = idx[s];
    const size_t ce = (size_t)c * E + e;
    const uint64_t below = tl ? (~0ull >> (64 - tl)) : 0ull;
    const int p = off[e] + chunk_prefix[ce] + __popcll(chunk_bits[ce] & below);
    pos[s] = p;
    sorted_slots[p] = s;
    row_token[p] = t;
}

bool routing_is_fused(const moe_shape_t& s) { return s.T <= kFusedMaxTokens; }

hipError_t launch_routing_fused(const moe_shape_t& s, const float* logits, const uint8_t* allowed, int32_t* idx, float* w,
                                int32_t* counts, int32_t* offsets, int32_t* sorted_slots, int32_t* pos,
                                const Workspace& ws, int bm, TileRange tr, hipStream_t stream)
{
    if (s.E <= 256)
        route_fused_kernel<true><<<1, 1024, 0, stream>>>(logits, allowed, (int)s.T, (int)s.E, (int)s.k, bm, tr, idx, w, counts,
                                                         offsets, sorted_slots, pos, ws.row_token, ws.tiles, ws.sync);
    else
        route_fused_kernel<false><<<1, 1024, 0, stream>>>(logits, allowed, (int)s.T, (int)s.E, (int)s.k, bm, tr, idx, w, counts,
                                                          offsets, sorted_slots, pos, ws.row_token, ws.tiles, ws.sync);
    return hipGetLastError();
}

hipError_t launch_permute(const moe_shape_t& s, const int32_t* idx, int32_t* counts, int32_t* offsets,
                          int32_t* sorted_slots, int32_t* pos, const Workspace& ws, int bm, TileRange tr,
                          hipStream_t stream)
{
    const int T = (int)s.T, E = (int)s.E, k = (int)s.k, nch = (int)ws.nchunks;
    chunk_scan_kernel<<<E, 256, 0, stream>>>(ws.chunk_counts, nch, E, ws.chunk_prefix, counts);
    scatter_kernel<<<(T * k + 255) / 256, 256, 0, stream>>>(idx, ws.chunk_bits, ws.chunk_prefix, counts, T, E, k, bm, tr,
                                                            offsets, sorted_slots, pos, ws.row_token, ws.tiles, ws.sync);
    return hipGetLastError();
}

}  // namespace moe
