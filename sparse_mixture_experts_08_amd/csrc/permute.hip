// permute.hip -- per-expert counts, offsets, the expert-sorted slot order and the grouped-GEMM tile list.
//
// What it computes is what the MoE forward excerpt on "DeepSeek-V3.2-Exp / Mixture of experts" does on
// the host: a bincount of the selected indices, then per expert the (token, slot) pairs that chose it,
// tokens ascending (torch.where scans row-major).  Here it is three passes over 64-token chunks with no
// host synchronisation and no order-dependent atomics:
//   1. (in the top-k kernel) a 64-bit mask per (chunk, expert) of the chunk's tokens that chose it;
//   2. one block per expert: exclusive prefix of the chunk counts; the last block to finish (a ticket
//      counter) scans the expert counts into offsets and writes the tile list;
//   3. one wavefront per chunk: a slot's position is offsets[e] + its chunk's prefix for e + the number
//      of earlier tokens of the chunk in e's mask.
// Sorted rows [0, T*k) hold the routed slots; rows [T*k, T*k + T) are the shared expert's, token order.
#include "moe_common.h"

namespace moe {

__global__ __launch_bounds__(256) void chunk_scan_kernel(const int32_t* __restrict__ chunk_counts, int nchunks, int E,
                                                         int T, int k, int bm, int32_t* __restrict__ chunk_prefix,
                                                         int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                         int4* __restrict__ tiles, int32_t* __restrict__ sync)
{
    __shared__ int32_t part[256];
    __shared__ int32_t scan[1025];
    __shared__ int is_last;
    const int e = blockIdx.x, tid = threadIdx.x;
    const int per = (nchunks + 255) / 256;
    const int c0 = tid * per, c1 = min(c0 + per, nchunks);
    int sum = 0;
    for (int c = c0; c < c1; c++) sum += chunk_counts[(size_t)c * E + e];
    part[tid] = sum;
    __syncthreads();
    if (tid == 0) {          // 256 partial sums, scanned in order
        int run = 0;
        for (int i = 0; i < 256; i++) {
            const int v = part[i];
            part[i] = run;
            run += v;
        }
        counts[e] = run;
    }
    __syncthreads();
    int run = part[tid];
    for (int c = c0; c < c1; c++) {
        const int v = chunk_counts[(size_t)c * E + e];
        chunk_prefix[(size_t)c * E + e] = run;
        run += v;
    }

    // The last block to arrive sees every count: offsets and tile list.
    __threadfence();
    __syncthreads();
    if (tid == 0) is_last = atomicAdd(&sync[1], 1) == E - 1;
    __syncthreads();
    if (!is_last) return;
    __threadfence();
    for (int g = tid; g < E; g += 256) scan[g] = __hip_atomic_load(&counts[g], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (tid == 0) {          // exclusive scan of the counts, in expert order
        int acc = 0;
        for (int g = 0; g < E; g++) {
            const int c = scan[g];
            scan[g] = acc;
            acc += c;
        }
        scan[E] = acc;       // == T * k
    }
    __syncthreads();
    for (int g = tid; g <= E; g += 256) offsets[g] = scan[g];
    // Tiles: shared expert (group E, rows [T*k, T*k+T)) first, then experts ascending.
    __shared__ int tbase[1024];
    const int nshared = (T + bm - 1) / bm;
    if (tid == 0) {
        int nt = nshared;
        for (int g = 0; g < E; g++) {
            tbase[g] = nt;
            nt += (scan[g + 1] - scan[g] + bm - 1) / bm;
        }
        sync[0] = nt;
        sync[1] = 0;
    }
    __syncthreads();
    for (int i = tid; i < nshared; i += 256) tiles[i] = make_int4(E, T * k + i * bm, min(bm, T - i * bm), 0);
    for (int g = tid; g < E; g += 256) {
        const int c = scan[g + 1] - scan[g];
        for (int r = 0; r < c; r += bm) tiles[tbase[g] + r / bm] = make_int4(g, scan[g] + r, min(bm, c - r), 0);
    }
}

__global__ __launch_bounds__(64) void scatter_kernel(const int32_t* __restrict__ idx, const uint64_t* __restrict__ chunk_bits,
                                                     const int32_t* __restrict__ chunk_prefix,
                                                     const int32_t* __restrict__ offsets, int T, int E, int k,
                                                     int32_t* __restrict__ sorted_slots, int32_t* __restrict__ pos,
                                                     int32_t* __restrict__ row_token)
{
    const int c = blockIdx.x, lane = threadIdx.x, t = c * 64 + lane;
    if (t >= T) return;
    const uint64_t below = lane ? (~0ull >> (64 - lane)) : 0ull;
    for (int j = 0; j < k; j++) {
        const int s = t * k + j;
        const int e = idx[s];
        const size_t ce = (size_t)c * E + e;
        const int p = offsets[e] + chunk_prefix[ce] + __popcll(chunk_bits[ce] & below);
        pos[s] = p;
        sorted_slots[p] = s;
        row_token[p] = t;
    }
    row_token[T * k + t] = t;
}

hipError_t launch_permute(const moe_shape_t& s, const int32_t* idx, int32_t* counts, int32_t* offsets,
                          int32_t* sorted_slots, int32_t* pos, const Workspace& ws, int bm, hipStream_t stream)
{
    const int T = (int)s.T, E = (int)s.E, k = (int)s.k, nch = (int)ws.nchunks;
    chunk_scan_kernel<<<E, 256, 0, stream>>>(ws.chunk_counts, nch, E, T, k, bm, ws.chunk_prefix, counts, offsets,
                                             ws.tiles, ws.sync);
    scatter_kernel<<<nch, 64, 0, stream>>>(idx, ws.chunk_bits, ws.chunk_prefix, offsets, T, E, k, sorted_slots, pos,
                                           ws.row_token);
    return hipGetLastError();
}

}  // namespace moe
