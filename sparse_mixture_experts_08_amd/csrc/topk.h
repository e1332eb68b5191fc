// topk.h -- top-k selection with a softmax over the selected logits, for one token held by a group of
// lanes of a wavefront (gate of "DeepSeek-V3's mixture-of-experts architecture explained", block
// pseudocode: topk of the router logits, then softmax over those k values).
//
// Each logit becomes a 64-bit key: its order-preserving bit pattern (+0 and -0 equal) in the high word
// and the complemented expert index in the low word, so the maximum key is the largest logit and,
// among equal logits, the lowest expert index.  k rounds of a group-wide maximum give the experts in
// descending-logit order.  The softmax subtracts the first (largest) selected logit, exponentiates in
// fp32 and divides by a fixed-order sum.
#pragma once

#include "moe_common.h"

namespace moe {

// Order-preserving map of a float (finite or -inf) to uint32; +0 and -0 map to the same key, and every
// key is nonzero.
__device__ __forceinline__ uint32_t ordered_bits(float f)
{
    uint32_t u = __float_as_uint(f == 0.0f ? 0.0f : f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t logit_key(float l, int e)
{
    return ((uint64_t)ordered_bits(l) << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)e);
}

__device__ __forceinline__ int key_expert(uint64_t key) { return (int)(0xFFFFFFFFu - (uint32_t)key); }

// Maximum of a 64-bit value over groups of W consecutive lanes.
template <int W>
__device__ __forceinline__ uint64_t group_max_u64(uint64_t v)
{
#pragma unroll
    for (int off = W / 2; off >= 1; off >>= 1) {
        const uint32_t lo = __shfl_xor((uint32_t)v, off, W), hi = __shfl_xor((uint32_t)(v >> 32), off, W);
        const uint64_t o = ((uint64_t)hi << 32) | lo;
        v = o > v ? o : v;
    }
    return v;
}

// Inverse of ordered_bits (-0 comes back as +0, which compares and subtracts the same).
__device__ __forceinline__ float key_logit(uint64_t key)
{
    const uint32_t u = (uint32_t)(key >> 32);
    return __uint_as_float((u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u);
}

// Softmax over the k slot logits held by lanes 0 .. k - 1 of a group of W lanes (slot 0 the largest):
// exponentials in fp32 relative to slot 0, a fixed-order sum, one IEEE division per slot.
template <int W>
__device__ __forceinline__ float softmax_slots(float my_l, int k, int sub)
{
    const float m = __shfl(my_l, 0, W);
    const float z = sub < k ? expf(my_l - m) : 0.0f;
    float sum = z;
#pragma unroll
    for (int off = (W < 16 ? W : 16) / 2; off >= 1; off >>= 1) sum += __shfl_xor(sum, off, W);
    sum = __shfl(sum, 0, W);
    return z / sum;
}

// Top-k of row L[0..E) held by a group of W lanes (sub = lane index in the group), each lane holding the
// logits e = sub + W * q for q < NQ (NQ * W >= E).  On return, lane sub < k of the group holds slot
// sub's expert and weight.  k <= min(W, 16).  allowed (nullable): the routing mask.
template <int W, int NQ>
__device__ __forceinline__ void topk_group(const float* __restrict__ Lrow, const uint8_t* __restrict__ allowed, int E,
                                           int k, int sub, int& my_e, float& my_w)
{
    // All loads first, at clamped in-bounds indices, so they are in flight together; then the keys.
    // The device-limited routing mask (allowed[e] == 0) makes the logit -inf: the page's `logits + mask`
    // with mask -inf outside the allowed experts and 0 inside.
    float lv[NQ];
    uint8_t av[NQ];
#pragma unroll
    for (int q = 0; q < NQ; q++) lv[q] = Lrow[min(sub + W * q, E - 1)];
    if (allowed) {
#pragma unroll
        for (int q = 0; q < NQ; q++) av[q] = allowed[min(sub + W * q, E - 1)];
    }
    uint64_t key[NQ];
#pragma unroll
    for (int q = 0; q < NQ; q++) {
        const int e = sub + W * q;
        const float l = (allowed && !av[q]) ? -INFINITY : lv[q];
        key[q] = e < E ? logit_key(l, e) : 0ull;
    }
    my_e = 0;
    float my_l = 0.0f;
    for (int j = 0; j < k; j++) {
        uint64_t best = 0;
#pragma unroll
        for (int q = 0; q < NQ; q++) best = key[q] > best ? key[q] : best;
        best = group_max_u64<W>(best);
        const int e = key_expert(best);
        if (e % W == sub) {
#pragma unroll
            for (int q = 0; q < NQ; q++)
                if (q == e / W) key[q] = 0ull;
        }
        if (sub == j) {
            my_e = e;
            my_l = key_logit(best);
        }
    }
    my_w = softmax_slots<W>(my_l, k, sub);
}

// Group-limited top-k ("Technical Architecture and Core Innovations", "Architectural Breakthroughs", item 1:
// tokens are first distributed over expert groups by a softmax, then two experts per group are selected).
// The E experts form G groups of E / G consecutive experts; a group's two best keys are its candidates
// and the fp32 sum of their logits its score; the k / 2 groups with the largest scores are kept (equal
// scores: the lower group), and their candidates, in key order, fill the k slots.  Layout as topk_group;
// group g's candidates and score live on lane g, so G <= W.  k even, k / 2 <= G, E / G >= 2.
template <int W, int NQ>
__device__ __forceinline__ void topk_grouped(const float* __restrict__ Lrow, int E, int k, int G, int sub, int& my_e,
                                             float& my_w)
{
    float lv[NQ];
#pragma unroll
    for (int q = 0; q < NQ; q++) lv[q] = Lrow[min(sub + W * q, E - 1)];
    const int gs = E / G;
    uint64_t key[NQ];
    int grp[NQ];
#pragma unroll
    for (int q = 0; q < NQ; q++) {
        const int e = sub + W * q;
        key[q] = e < E ? logit_key(lv[q], e) : 0ull;
        grp[q] = e / gs;                               // past E: a group >= G, never asked for
    }
    // each group's best two keys, by two group-wide maxima over that group's keys
    uint64_t c1 = 0ull, c2 = 0ull;
    for (int g = 0; g < G; g++) {
        uint64_t b = 0ull;
#pragma unroll
        for (int q = 0; q < NQ; q++) b = (grp[q] == g && key[q] > b) ? key[q] : b;
        const uint64_t k1 = group_max_u64<W>(b);
        b = 0ull;
#pragma unroll
        for (int q = 0; q < NQ; q++) b = (grp[q] == g && key[q] != k1 && key[q] > b) ? key[q] : b;
        const uint64_t k2 = group_max_u64<W>(b);
        if (sub == g) {
            c1 = k1;
            c2 = k2;
        }
    }
    // group keys: the score's order-preserving bits, then the complemented group index
    uint64_t gkey = 0ull;
    if (sub < G) {
        const float score = key_logit(c1) + key_logit(c2);
        gkey = ((uint64_t)ordered_bits(score) << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)sub);
    }
    bool kept = false;
    for (int r = 0; r < k / 2; r++) {
        const uint64_t best = group_max_u64<W>(gkey);
        if (sub == (int)(0xFFFFFFFFu - (uint32_t)best)) {
            kept = true;
            gkey = 0ull;
        }
    }
    uint64_t cand0 = kept ? c1 : 0ull, cand1 = kept ? c2 : 0ull;
    my_e = 0;
    float my_l = 0.0f;
    for (int j = 0; j < k; j++) {
        const uint64_t best = group_max_u64<W>(cand0 > cand1 ? cand0 : cand1);
        if (cand0 == best) cand0 = 0ull;
        else if (cand1 == best) cand1 = 0ull;
        if (sub == j) {
            my_e = key_expert(best);
            my_l = key_logit(best);
        }
    }
    my_w = softmax_slots<W>(my_l, k, sub);
}

}  // namespace moe
