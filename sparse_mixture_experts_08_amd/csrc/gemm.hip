// gemm.hip -- grouped expert GEMMs on CDNA4 MFMA.
//
// Expert math from "DeepSeek-V3.2-Exp / Mixture of experts / Shared expert" ("All 5 steps"):
// g = x W1, u = x W3, a = g sigma(g), h = a (.) u, y = h W2; the MLP forward excerpt forms
// silu(g) * u in fp32 from the linears' outputs and casts it back to the activation dtype before W2.
// Each linear's output is rounded to the activation dtype, as a bf16 linear returns bf16.
//
// Work list.  Rows are the expert-sorted (token, slot) pairs of every routed expert followed by one
// row per token for the shared expert (group E); the tile list cuts each group into BM-row tiles.
// A block computes one (tile, n-block): rows of that group against BN output features.
//   up   : A = x rows gathered through row_token, B = [W1 rows n0..n0+BN) ; W3 rows n0..n0+BN)],
//          epilogue h = round(silu(round(g)) * round(u)) -> h rows (fp8 weights: E4M3 codes of h per
//          1x128 group plus one scale per group);
//   down : A = h rows (already in sorted order), B = W2 rows, epilogue y_rows = round(acc).
// Empty experts create no tiles and read no weights.
//
// Data path.  A and B tiles are staged through LDS in 128-byte-per-row K stages (16-byte chunks
// XOR-swizzled by row) and read back as MFMA fragments with 16-byte LDS reads.  Three kernels:
//   grouped_gemm_kernel    : global loads into registers one stage ahead, then LDS stores (16-row decode
//                            tiles of every dtype; fp32 128-row tiles);
//   grouped_gemm_w_kernel  : bf16 256-row tiles, eight wavefronts of 128 x 64 outputs in 32x32 MFMAs,
//                            stages copied global -> LDS by direct-to-LDS loads;
//   grouped_gemm_f8_kernel : fp8 128- or 256-row tiles, direct-to-LDS staging of the operands and their
//                            scales.
// MFMA per element type:
//   fp32 : v_mfma_f32_16x16x4_f32   (4 per 16-byte fragment; lane group q holds k = 4q + e)
//   bf16 : v_mfma_f32_16x16x32_bf16 (one per 16-byte fragment), v_mfma_f32_32x32x16_bf16 (wide kernel)
//   fp8  : v_mfma_scale_f32_16x16x128_f8f6f4 with unit exponent scales, one per 128-byte stage, whose
//          fp32 result is multiplied by (activation scale of the row) * (weight block scale) and
//          added to the accumulator: a 128-wide K stage is exactly one 128x128 weight block.
// Since A and B fragments use the same lane -> k assignment, any consistent K permutation inside a
// stage gives the same dot product.
#include "moe_common.h"

namespace moe {

enum { ET_F32 = 0, ET_BF16 = 1, ET_FP8 = 2 };

struct GemmArgs {
    const int4* tiles;        // tile list
    const int32_t* ntiles;    // number of valid tiles
    const int32_t* row_token; // up: sorted row -> token (A row)
    const uint8_t* A;         // up: x or its E4M3 codes; down: h
    const float* As;          // fp8: scales of A rows per 128-K block ([rows, K/128])
    int64_t lda;              // bytes between A rows
    int64_t ldas;             // floats between rows of As
    const uint8_t* B1;        // routed weights (up: W1, down: W2) [experts e_base.., N, K]
    const uint8_t* B3;        // up: W3
    const float* B1s;         // fp8 block scales [E, N/128, K/128]
    const float* B3s;
    const uint8_t* S1;        // shared-expert weights [N_s rows of ld_s elements, K_s used]
    const uint8_t* S3;
    const float* S1s;
    const float* S3s;
    uint8_t* out;             // up: h; down: y_rows
    float* outs;              // up with fp8: scales of h [rows, inter_max/128]
    int64_t ldo;              // elements between output rows
    int64_t ldos;             // floats between rows of outs
    int E;                    // group E is the shared expert
    int e_base;               // expert held at index 0 of B1/B3 (and their scales)
    int N_r, N_s;             // output features: routed / shared
    int K_r, K_s;             // reduction length: routed / shared
    int n_blocks;             // n-blocks per tile (over the larger N)
    int64_t ld_s;             // elements between shared weight rows (a slice of a wider expert)
    int nkb_s;                // fp8: scale blocks between shared scale rows
    int max_tiles;
    int krot;                 // K-stage rotation per n-block (0: every block walks K from stage 0)
    int group_m;              // 0: block b -> (tile b / n_blocks, n-block b % n_blocks); else the XCD-aware
                              // grouped order below, with group_m tiles per group
};

template <int ET> struct Elem;
template <> struct Elem<ET_F32> { static constexpr int bytes = 4; };
template <> struct Elem<ET_BF16> { static constexpr int bytes = 2; };
template <> struct Elem<ET_FP8> { static constexpr int bytes = 1; };

__device__ __forceinline__ int swz(int row, int chunk) { return row * 128 + ((chunk ^ (row & 7)) << 4); }

__device__ __forceinline__ float silu_mul(float g, float u)
{
    const float sig = 1.0f / (1.0f + expf(-g));
    return (g * sig) * u;
}

// silu(g) * u for an h that is rounded to bf16 (the bf16 and fp8 layers): the sigmoid from the hardware
// base-2 exponential and reciprocal (v_exp_f32, v_rcp_f32, each within about an ulp), five instructions
// where expf and the IEEE division take about 25.  Its error, under 1e-6 relative, is far below a bf16
// ulp (2^-8): over normally distributed g an emulation moves 1 to 2 in 10^5 of the rounded h values by
// one bf16 ulp against the IEEE form.  The fp32 layer keeps silu_mul.  In the large-tile GEMMs the
// epilogue runs with the matrix pipe idle, so its cost adds to the kernel's time.
__device__ __forceinline__ float silu_mul_fast(float g, float u)
{
    const float e = __builtin_amdgcn_exp2f(g * -1.44269504088896341f);   // exp(-g)
    const float sig = __builtin_amdgcn_rcpf(1.0f + e);
    return (g * sig) * u;
}

// One K stage of MFMAs for a wave's WM x WN blocks (and the W3 half for the up GEMM).
template <int ET, bool UP, int WM, int WN, int BN>
__device__ __forceinline__ void mma_stage(const uint8_t* As_lds, const uint8_t* Bs_lds, const float* sA_lds,
                                          float sb1, float sb3, int wm0, int wn0, int lane,
                                          f32x4 (&acc1)[WM][WN], f32x4 (&acc3)[WM][WN])
{
    const int r16 = lane & 15, q = lane >> 4;
    if constexpr (ET == ET_FP8) {
        // B fragments of the whole stage stay in registers; A fragments are read one row block at a time.
        i32x8 b1[WN], b3[WN];
#pragma unroll
        for (int j = 0; j < WN; j++) {
            const int row = wn0 + j * 16 + r16;
            i32x4 lo = *(const i32x4*)(Bs_lds + swz(row, 2 * q));
            i32x4 hi = *(const i32x4*)(Bs_lds + swz(row, 2 * q + 1));
            b1[j] = (i32x8){lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
            if constexpr (UP) {
                lo = *(const i32x4*)(Bs_lds + swz(BN + row, 2 * q));
                hi = *(const i32x4*)(Bs_lds + swz(BN + row, 2 * q + 1));
                b3[j] = (i32x8){lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
            }
        }
#pragma unroll
        for (int i = 0; i < WM; i++) {
            const int row = wm0 + i * 16 + r16;
            const i32x4 lo = *(const i32x4*)(As_lds + swz(row, 2 * q));
            const i32x4 hi = *(const i32x4*)(As_lds + swz(row, 2 * q + 1));
            const i32x8 a = (i32x8){lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
            float s1[4], s3[4];
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const float sa = sA_lds[wm0 + i * 16 + 4 * q + r];
                s1[r] = sa * sb1;
                s3[r] = sa * sb3;
            }
#pragma unroll
            for (int j = 0; j < WN; j++) {
                const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
                const f32x4 p1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b1[j], zero, 0, 0, 0, 127, 0, 127);
#pragma unroll
                for (int r = 0; r < 4; r++) acc1[i][j][r] += p1[r] * s1[r];
                if constexpr (UP) {
                    const f32x4 p3 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b3[j], zero, 0, 0, 0, 127, 0, 127);
#pragma unroll
                    for (int r = 0; r < 4; r++) acc3[i][j][r] += p3[r] * s3[r];
                }
            }
        }
    } else {
#pragma unroll
        for (int ks = 0; ks < 2; ks++) {          // two 64-byte K slices per stage
            const int chunk = ks * 4 + q;
            i32x4 a[WM], b1[WN], b3[WN];
#pragma unroll
            for (int i = 0; i < WM; i++) a[i] = *(const i32x4*)(As_lds + swz(wm0 + i * 16 + r16, chunk));
#pragma unroll
            for (int j = 0; j < WN; j++) {
                b1[j] = *(const i32x4*)(Bs_lds + swz(wn0 + j * 16 + r16, chunk));
                if constexpr (UP) b3[j] = *(const i32x4*)(Bs_lds + swz(BN + wn0 + j * 16 + r16, chunk));
            }
#pragma unroll
            for (int i = 0; i < WM; i++)
#pragma unroll
                for (int j = 0; j < WN; j++) {
                    if constexpr (ET == ET_BF16) {
                        acc1[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[i]),
                                                                             __builtin_bit_cast(bf16x8, b1[j]), acc1[i][j], 0, 0, 0);
                        if constexpr (UP)
                            acc3[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[i]),
                                                                                 __builtin_bit_cast(bf16x8, b3[j]), acc3[i][j], 0, 0, 0);
                    } else {
                        const f32x4 af = __builtin_bit_cast(f32x4, a[i]), bf1 = __builtin_bit_cast(f32x4, b1[j]);
#pragma unroll
                        for (int e = 0; e < 4; e++) acc1[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[e], bf1[e], acc1[i][j], 0, 0, 0);
                        if constexpr (UP) {
                            const f32x4 bf3 = __builtin_bit_cast(f32x4, b3[j]);
#pragma unroll
                            for (int e = 0; e < 4; e++) acc3[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[e], bf3[e], acc3[i][j], 0, 0, 0);
                        }
                    }
                }
        }
    }
}

// Epilogue of the 16x16-MFMA kernels.  Accumulator layout: lane holds rows 4*(lane/16) + r, column
// lane % 16.  UP: h = round(silu(round g) * round u), with fp8 weights quantised per 1x128 group through
// `smem` (BM x BN floats; the caller has finished with the staging buffers); down: y rows = round(acc).
template <int ET, bool UP, bool ACT_BF16, int BM, int BN, int WM, int WN, int NT>
__device__ __forceinline__ void gemm_epilogue(const GemmArgs& g, uint8_t* smem, const f32x4 (&acc1)[WM][WN],
                                              const f32x4 (&acc3)[WM][WN], int rows, int row0, int n0, int wm0,
                                              int wn0, int tid)
{
    constexpr bool FP8 = ET == ET_FP8;
    const int lane = tid & 63;
    const int r16 = lane & 15, q = lane >> 4;
    if constexpr (UP && FP8) {
        float* hs = (float*)smem;                      // [BM][BN] h values, then quantised per 128 group
#pragma unroll
        for (int i = 0; i < WM; i++)
#pragma unroll
            for (int j = 0; j < WN; j++)
#pragma unroll
                for (int r = 0; r < 4; r++) {
                    float gg = acc1[i][j][r], uu = acc3[i][j][r];
                    round_bf16x2(gg, uu);
                    hs[(wm0 + i * 16 + 4 * q + r) * BN + wn0 + j * 16 + r16] = round_bf16(silu_mul_fast(gg, uu));
                }
        __syncthreads();
        // 16 threads per (row, 128-column group), 8 columns each
        constexpr int GROUPS = BM * (BN / 128);
        for (int gi = tid >> 4; gi < GROUPS; gi += NT / 16) {
            const int row = gi / (BN / 128), grp128 = gi % (BN / 128);
            const int sub = tid & 15;
            const float* v = hs + row * BN + grp128 * 128 + sub * 8;
            float amax = 0.f;
#pragma unroll
            for (int e = 0; e < 8; e++) amax = fmaxf(amax, fabsf(v[e]));
            amax = row16_max(amax);
            const float sc = amax > 0.f ? amax / 448.0f : 1.0f;
            if (row < rows) {
                float q[8];
                if (quant_div_fast(sc)) {
                    const float r = recip_rn(sc);
#pragma unroll
                    for (int e = 0; e < 8; e++) q[e] = quant_div(v[e], sc, r);
                } else {
#pragma unroll
                    for (int e = 0; e < 8; e++) q[e] = v[e] / sc;
                }
                uint32_t lo = f32x2_to_e4m3(q[0], q[1]) | (f32x2_to_e4m3(q[2], q[3]) << 16);
                uint32_t hi = f32x2_to_e4m3(q[4], q[5]) | (f32x2_to_e4m3(q[6], q[7]) << 16);
                const int64_t orow = row0 + row;
                *(uint2*)(g.out + orow * g.ldo + n0 + grp128 * 128 + sub * 8) = make_uint2(lo, hi);
                if (sub == 0) g.outs[orow * g.ldos + (n0 + grp128 * 128) / 128] = sc;
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < WM; i++)
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const int row = wm0 + i * 16 + 4 * q + r;
                if (row >= rows) continue;
                const int64_t orow = row0 + row;
#pragma unroll
                for (int j = 0; j < WN; j++) {
                    const int col = n0 + wn0 + j * 16 + r16;
                    float v;
                    if constexpr (UP) {
                        const float gg = round_act<ACT_BF16>(acc1[i][j][r]), uu = round_act<ACT_BF16>(acc3[i][j][r]);
                        v = ACT_BF16 ? silu_mul_fast(gg, uu) : silu_mul(gg, uu);
                    } else {
                        v = acc1[i][j][r];
                    }
                    if constexpr (ACT_BF16) ((uint16_t*)g.out)[orow * g.ldo + col] = f32_to_bf16(v);
                    else ((float*)g.out)[orow * g.ldo + col] = v;
                }
            }
    }
}

// block -> (tile, n-block); false when the block has no work.  group_m == 0 (decode-sized tiles):
// consecutive blocks walk one tile's n-blocks.  Otherwise the work list is cut into groups of group_m
// consecutive tiles x all n-blocks, walked n-block by n-block with the group's tiles fastest, and the
// groups are dealt round-robin to the 8 XCDs (block b runs on XCD b % 8; XCD x takes groups x, x + 8,
// x + 16, ..., one after the other).  Blocks that run together on one XCD share A rows (same tile) and
// weight panels (same expert, n-block) in that XCD's L2, and every XCD gets a like share of hot, cold and
// shared-expert tiles: cut into 8 contiguous ranges instead, the list gave one XCD all 16 shared tiles of
// the 4096-token layer (about a quarter more work than the others) and the skewed layer's XCDs 5-6 % more
// or less than their mean.  launch_blocks() is the grid this needs.
__device__ __forceinline__ bool block_work(const GemmArgs& g, int& tile, int& nb)
{
    const int bid = blockIdx.x;
    const int nt = *g.ntiles;
    if (g.group_m == 0) {
        tile = bid / g.n_blocks;
        nb = bid % g.n_blocks;
        return tile < nt;
    }
    const int items = g.group_m * g.n_blocks;          // work items of a full group
    const int j = bid >> 3;                            // the block's place in its XCD's list
    const int c = (bid & 7) + 8 * (j / items), r = j % items;
    if (c * g.group_m >= nt) return false;
    const int gm = min(g.group_m, nt - c * g.group_m); // the last group may be short
    if (r >= gm * g.n_blocks) return false;
    nb = r / gm;
    tile = c * g.group_m + r % gm;
    return true;
}

// Grid of a grouped-GEMM launch: enough blocks for max_tiles tiles under block_work's mapping.
static int64_t launch_blocks(const GemmArgs& a)
{
    if (a.group_m == 0) return ((int64_t)a.n_blocks * a.max_tiles + 7) / 8 * 8;
    const int64_t groups = (a.max_tiles + a.group_m - 1) / a.group_m;
    return 8 * ((groups + 7) / 8) * a.group_m * a.n_blocks;
}

// NBUF: LDS stages (2 = double buffered, one barrier per K stage; 1 = single buffer, two barriers per
// stage but half the LDS, so two blocks share a CU and cover each other's barriers).  MINW: minimum
// wavefronts per SIMD the register allocation must allow.
template <int ET, bool UP, bool ACT_BF16, int BM, int BN, int WAVES_M, int WAVES_N, int NBUF, int MINW>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N, MINW) void grouped_gemm_kernel(GemmArgs g)
{
    constexpr int NB = UP ? 2 * BN : BN;               // B rows per stage
    constexpr int ROWS = BM + NB;                      // LDS rows per stage (128 bytes each)
    constexpr int NT = 64 * WAVES_M * WAVES_N;         // threads per block
    constexpr int WM = BM / 16 / WAVES_M, WN = BN / 16 / WAVES_N;
    constexpr int KE = 128 / Elem<ET>::bytes;          // K elements per stage
    constexpr bool FP8 = ET == ET_FP8;
    static_assert((WAVES_M * WAVES_N == 4 || WAVES_M * WAVES_N == 8) && WM >= 1 && WN >= 1, "4 or 8 waves");
    static_assert(NBUF == 1 || NBUF == 2, "single- or double-buffered stages (the loop below knows no other)");
    static_assert(BM <= NT, "one thread per tile row for the row tables");
    static_assert(!FP8 || (WN * 16 <= 128 && 128 % (WN * 16) == 0), "a wavefront's columns share one fp8 block scale");
    static_assert(!(FP8 && UP) || BN % 128 == 0, "fp8 h quantisation needs whole 128-column groups");

    static_assert(!(FP8 && UP) || BM * BN * 4 <= NBUF * ROWS * 128, "h tile must fit the staging LDS");
    __shared__ __attribute__((aligned(16))) uint8_t smem[NBUF * ROWS * 128];
    __shared__ float sA[NBUF][BM];
    __shared__ int s_tok[BM];

    int tile, nb;
    if (!block_work(g, tile, nb)) return;
    const int4 td = g.tiles[tile];
    const int grp = td.x, row0 = td.y, rows = td.z;
    const bool shared = grp == g.E;
    const int N = shared ? g.N_s : g.N_r, K = shared ? g.K_s : g.K_r;
    const int n0 = nb * BN;
    if (n0 >= N) return;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm0 = (wave / WAVES_N) * WM * 16, wn0 = (wave % WAVES_N) * WN * 16;
    const int64_t ldb = (shared ? g.ld_s : (int64_t)K) * Elem<ET>::bytes;  // bytes per weight row
    const int64_t lgrp = grp - g.e_base;               // index of the expert in the weight arrays
    const uint8_t* W1 = shared ? g.S1 : g.B1 + lgrp * N * ldb;
    const uint8_t* W3 = UP ? (shared ? g.S3 : g.B3 + lgrp * N * ldb) : nullptr;
    const int nkb = shared ? g.nkb_s : K / 128;        // fp8 scale blocks per weight-scale row
    // fp8: the block scales of this wavefront's output columns (its column span lies in one 128-block)
    const float* W1s = FP8 ? (shared ? g.S1s : g.B1s + lgrp * (N / 128) * nkb) + ((n0 + wn0) / 128) * nkb : nullptr;
    const float* W3s = (FP8 && UP) ? (shared ? g.S3s : g.B3s + lgrp * (N / 128) * nkb) + ((n0 + wn0) / 128) * nkb : nullptr;

    // A row of every tile row.  Rows past the tile's end: with fp8 operands they repeat the tile's first
    // row (valid memory, finite values: computed, never stored); otherwise they are not loaded (-1).
    if (tid < BM) {
        if constexpr (FP8) {
            const int r = tid < rows ? tid : 0;
            s_tok[tid] = UP ? g.row_token[row0 + r] : row0 + r;
        } else {
            s_tok[tid] = tid < rows ? (UP ? g.row_token[row0 + tid] : row0 + tid) : -1;
        }
    }
    __syncthreads();

    // K-stage order: rotated by the n-block, so blocks streaming weight rows at the same time read
    // different column offsets of them and spread over the HBM channels.  (The fp32 sum over K stages
    // then runs in a rotated but fixed order per output column: still deterministic.)
    const int nstages = K / KE;
    const int kshift = (nb * g.krot) % nstages;
    auto kst = [&](int s) { return s + kshift >= nstages ? s + kshift - nstages : s + kshift; };

    // Staging, bf16 and fp32: a 64-bit source pointer per 16-byte chunk (null for rows past the tile's
    // end, which stay zero), advanced by 128 bytes per K stage; x rows in src, weight rows in wsrc.
    // Weight rows are read with the non-temporal hint: here each weight byte is read by one block and not
    // again, and the hint lets the stream run closer to the HBM peak (4096 x 7168 x 2 bytes per touched
    // expert at 64 tokens: up GEMM 2.12 -> 1.88 ms, down 1.07 -> 0.97 ms).  x rows, which every
    // n-block and expert of a token reads again, keep the default policy.  (Two pointer arrays, so the
    // two loads are not merged into one that drops the hint.)
    constexpr int CHUNKS = ROWS * 8;                   // 16-byte chunks per stage
    constexpr int PER = FP8 ? 1 : (CHUNKS + NT - 1) / NT;
    const uint8_t* src[PER];
    const uint8_t* wsrc[PER];
    int dst[PER];
    i32x4 reg[PER];
    if constexpr (!FP8) {
#pragma unroll
        for (int p = 0; p < PER; p++) {
            const int c = tid + p * NT;
            src[p] = wsrc[p] = nullptr;
            dst[p] = -1;
            if (c < CHUNKS) {
                const int row = c >> 3, ch = c & 7;
                dst[p] = swz(row, ch);
                if (row < BM) {
                    const int r = s_tok[row];
                    if (r >= 0) src[p] = g.A + (int64_t)r * g.lda + ch * 16;
                } else if (!UP || row < BM + BN) {
                    wsrc[p] = W1 + (int64_t)(n0 + row - BM) * ldb + ch * 16;
                } else {
                    wsrc[p] = W3 + (int64_t)(n0 + row - BM - BN) * ldb + ch * 16;
                }
            }
        }
    }
    // Staging, fp8 (weight rows with the non-temporal hint, as above): each region (A rows, W1 rows, W3
    // rows) is a block-uniform base plus a 32-bit per-lane offset fixed across K, and the K stage moves the
    // base, so the loads take the scalar-base form with no per-load address arithmetic or branch: the fp8
    // kernels are bound by vector-ALU issue (the per-block rescaling of every MFMA result), and this frees
    // it.  (The host keeps A and each expert's weights under 4 GB.)
    constexpr int A_CH = BM * 8, B_CH = BN * 8;        // 16-byte chunks per stage: A tile, one B tile
    constexpr int A_PER = FP8 ? (A_CH + NT - 1) / NT : 1, B_PER = FP8 ? (B_CH + NT - 1) / NT : 1;
    constexpr bool A_EXACT = A_CH % NT == 0, B_EXACT = B_CH % NT == 0;
    uint32_t offA[A_PER], offB[B_PER];
    int dstA[A_PER], dstB[B_PER];
    i32x4 ra[A_PER], rb1[B_PER], rb3[B_PER];
    if constexpr (FP8) {
#pragma unroll
        for (int p = 0; p < A_PER; p++) {
            const int c = A_EXACT ? tid + p * NT : min(tid + p * NT, A_CH - 1);
            const int row = c >> 3, ch = c & 7;
            offA[p] = (uint32_t)s_tok[row] * (uint32_t)g.lda + ch * 16;
            dstA[p] = (A_EXACT || tid + p * NT < A_CH) ? swz(row, ch) : -1;
        }
#pragma unroll
        for (int p = 0; p < B_PER; p++) {
            const int c = B_EXACT ? tid + p * NT : min(tid + p * NT, B_CH - 1);
            const int row = c >> 3, ch = c & 7;
            offB[p] = (uint32_t)(n0 + row) * (uint32_t)ldb + ch * 16;
            dstB[p] = (B_EXACT || tid + p * NT < B_CH) ? swz(BM + row, ch) : -1;
        }
    }

    auto load_stage = [&](int s0) {
        if constexpr (FP8) {
            const int64_t koff = (int64_t)kst(s0) * 128;
            const uint8_t* a = g.A + koff;
            const uint8_t* b1 = W1 + koff;
#pragma unroll
            for (int p = 0; p < A_PER; p++) ra[p] = *(const i32x4*)(a + offA[p]);
#pragma unroll
            for (int p = 0; p < B_PER; p++) rb1[p] = __builtin_nontemporal_load((const i32x4*)(b1 + offB[p]));
            if constexpr (UP) {
                const uint8_t* b3 = W3 + koff;
#pragma unroll
                for (int p = 0; p < B_PER; p++) rb3[p] = __builtin_nontemporal_load((const i32x4*)(b3 + offB[p]));
            }
        } else {
            const int s = kst(s0);
#pragma unroll
            for (int p = 0; p < PER; p++) {
                reg[p] = (i32x4){0, 0, 0, 0};
                if (src[p]) reg[p] = *(const i32x4*)(src[p] + (int64_t)s * 128);
                if (wsrc[p]) reg[p] = __builtin_nontemporal_load((const i32x4*)(wsrc[p] + (int64_t)s * 128));
            }
        }
    };
    auto store_stage = [&](int buf) {
        uint8_t* base = smem + buf * ROWS * 128;
        if constexpr (FP8) {
#pragma unroll
            for (int p = 0; p < A_PER; p++)
                if (A_EXACT || dstA[p] >= 0) *(i32x4*)(base + dstA[p]) = ra[p];
#pragma unroll
            for (int p = 0; p < B_PER; p++) {
                if (B_EXACT || dstB[p] >= 0) {
                    *(i32x4*)(base + dstB[p]) = rb1[p];
                    if constexpr (UP) *(i32x4*)(base + dstB[p] + BN * 128) = rb3[p];
                }
            }
        } else {
#pragma unroll
            for (int p = 0; p < PER; p++)
                if (dst[p] >= 0) *(i32x4*)(base + dst[p]) = reg[p];
        }
    };
    auto load_scales = [&](int s, int buf) {
        if constexpr (FP8) {
            if (tid < BM) sA[buf][tid] = g.As[(int64_t)s_tok[tid] * g.ldas + s];
        }
    };

    f32x4 acc1[WM][WN], acc3[WM][WN];
#pragma unroll
    for (int i = 0; i < WM; i++)
#pragma unroll
        for (int j = 0; j < WN; j++) acc1[i][j] = acc3[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};

    load_stage(0);
    store_stage(0);
    load_scales(kst(0), 0);
    __syncthreads();
    for (int s = 0; s < nstages; s++) {
        const int buf = NBUF == 2 ? (s & 1) : 0;
        if (s + 1 < nstages) load_stage(s + 1);
        float sb1 = 0.f, sb3 = 0.f;
        if constexpr (FP8) {
            sb1 = W1s[kst(s)];
            if constexpr (UP) sb3 = W3s[kst(s)];
        }
        mma_stage<ET, UP, WM, WN, BN>(smem + buf * ROWS * 128, smem + buf * ROWS * 128 + BM * 128, sA[buf], sb1, sb3,
                                      wm0, wn0, lane, acc1, acc3);
        if constexpr (NBUF == 1) __syncthreads();
        if (s + 1 < nstages) {
            store_stage(NBUF == 2 ? buf ^ 1 : 0);
            load_scales(kst(s + 1), NBUF == 2 ? buf ^ 1 : 0);
        }
        __syncthreads();
    }

    gemm_epilogue<ET, UP, ACT_BF16, BM, BN, WM, WN, NT>(g, smem, acc1, acc3, rows, row0, n0, wm0, wn0, tid);
}

// ---------------------------------------------------------------------------------------------------
// Machinery of the direct-to-LDS forms below.  K stages are copied global -> LDS by the direct-to-LDS
// load (global_load_lds_dwordx4: a wavefront's 64 lanes write 1 KB at M0 + 16 * lane), so staging uses
// no registers, no LDS store instructions and no per-load vector-ALU work: each lane's source is a
// block-uniform base in SGPRs (moved by the K stage) plus a 32-bit offset fixed for the whole K walk.
// The loads are issued from asm, so the compiler knows of no load into LDS and schedules fragment reads
// freely; an explicit vmcnt wait and barrier per stage order the reads after the loads of their stage.
//
// LDS row layout: 16-byte chunk c of row r stored at chunk c ^ f(r), f(r) = (r ^ (r >> 3 & 1)) & 7 for
// 128-byte rows, ((r >> 1) ^ (r >> 3)) & 3 for 64-byte rows: a fragment read (lanes 0..31: 32
// consecutive rows, one chunk) hits distinct banks for any 8 or 16 consecutive lanes, and f is unchanged
// by adding 16 (resp. 32) rows.  The loads apply the swizzle on the source side (lane l writes stored
// chunk l % (RB / 16) of row l / (RB / 16), so it reads the logical chunk that belongs there).
// Rows past the tile's end load the tile's first row (valid memory); their results are never stored.
// ---------------------------------------------------------------------------------------------------
typedef float f32x16 __attribute__((ext_vector_type(16)));
template <int N> struct IntC {
    static constexpr int value = N;
};

// f(IntC<n>{}) for a runtime n in [0, N] (n outside: f(IntC<0>{})).
template <int N, typename F> __device__ __forceinline__ void with_count(int n, F&& f)
{
    if constexpr (N == 0) {
        f(IntC<0>{});
    } else {
        if (n == N) f(IntC<N>{});
        else with_count<N - 1>(n, f);
    }
}

template <int N> __device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// Barrier without the vmcnt(0) that __syncthreads implies: loads into the other ring buffers stay in flight.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <int RB> __device__ __forceinline__ int swzr(int row, int chunk)
{
    if constexpr (RB == 128) return row * 128 + ((chunk ^ ((row ^ (row >> 3 & 1)) & 7)) << 4);
    else return row * 64 + ((chunk ^ (((row >> 1) ^ (row >> 3)) & 3)) << 4);
}

__device__ __forceinline__ uint32_t lds_addr(const void* p)
{
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// One direct-to-LDS load: lane l copies 16 bytes from sbase + voff to LDS address lds + 16 l.  M0 carries
// the LDS address and is written here (one wait state before the load uses it); nothing else in the
// kernels that use this keeps a value in M0.  No memory clobber: the load writes a ring buffer that no
// LDS access nearby touches, and as a volatile asm it keeps its place relative to the barrier asm.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const uint8_t* sbase, uint32_t voff, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(lds)
                 : "m0");
}
// The 4-byte form: lane l copies 4 bytes from sbase + voff to LDS address lds + 4 l.
__device__ __forceinline__ void dma4(const uint8_t* sbase, uint32_t voff, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(sbase), "s"(lds)
                 : "m0");
}
#pragma clang diagnostic pop

// Coalesced store of a block's bf16 output tile: the wavefronts have written it row-major into LDS (row
// stride OSTR bytes, padded so the two row groups of one LDS write fall on different banks); every
// thread then copies 16-byte chunks of rows < rows to out (row0 + row, col0 ..), ldo elements apart.
// Against per-lane 2-byte global stores straight from the accumulators this writes whole lines (and
// against 8-byte stores straight from the fp8 kernel's accumulators, 32 contiguous bytes a row: fp8 down
// GEMM 4.83 -> 5.35 ms).  NTS: stores with the non-temporal hint, for the down GEMMs' expert-output rows,
// which only the combine reads, after the whole GEMM (prefill down GEMM 1.795 -> 1.695 ms, fp8 down GEMM
// 4.77 -> 4.68 ms, skewed down GEMM 0.3 % slower).
template <int BM, int OC, int OSTR, int NT, bool NTS = false>
__device__ __forceinline__ void store_tile_bf16(const uint8_t* tile, uint8_t* out, int64_t ldo, int row0, int rows,
                                                int col0)
{
    typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
    constexpr int CH = OC * 2 / 16;                    // 16-byte chunks per row
    for (int idx = threadIdx.x; idx < BM * CH; idx += NT) {
        const int row = idx / CH, ch = idx % CH;
        if (row < rows) {
            u32x4_t* dst = (u32x4_t*)(out + (((int64_t)row0 + row) * ldo + col0 + ch * 8) * 2);
            const u32x4_t v = *(const u32x4_t*)(tile + row * OSTR + ch * 16);
            if constexpr (NTS) __builtin_nontemporal_store(v, dst);
            else *dst = v;
        }
    }
}

// ---------------------------------------------------------------------------------------------------
// Wide form for bf16 tiles of BM = 128 or 256 rows, v_mfma_f32_32x32x16_bf16.  NW = 4: one wavefront
// per SIMD owning a 128 x 128 output block (UP: 64 columns of W1 and the same 64 of W3) in 16 accumulators
// of 32 x 32 (BM = 128 -> 1 x 4 wavefronts, BM = 256 -> 2 x 2).  NW = 8 (used: BM = 256): the same
// 256 x 256 block tile as 2 x 4 wavefronts of 128 x 64, two per SIMD, so one wavefront issues MFMAs
// while the other waits on a fragment read or the stage barrier (skewed workload 16.2 -> 15.1 ms).
// K stages of RB / 2 elements in a ring of NSTG, copied by direct-to-LDS loads; at the end of each stage
// the barrier publishing the next stage, the refill of the freed buffer and the first fragment reads of
// the next stage sit under the MFMAs of the stage's last K step.  With whole-line (128-byte) rows the
// time of this kernel on MI355X is set mostly by the global -> LDS copies (the same loop without MFMAs
// takes 77-94 % of it, without the copies about 60 %).  The copy path itself is not the cap: the same
// direct-to-LDS loads alone stream 58-61 B/clock per CU from L2 and the same panel pattern 6.1 TB/s from
// HBM; deeper rings, copies issued ahead of the barrier, other XCD groupings and K rotations did not
// shorten it.  Fewer staged bytes per MFMA did, which is why the block tile is as large as the register
// file allows.
// ---------------------------------------------------------------------------------------------------
template <bool UP, int BM, int RB, int NA, int NBS, int NW>
__global__ __launch_bounds__(64 * NW, 1) void grouped_gemm_w_kernel(GemmArgs g)
{
    constexpr int WAVES_M = BM / 128, WAVES_N = NW / WAVES_M;
    constexpr int NJ = (UP ? 2 : 4) * 4 / NW;          // 32-column MFMA blocks per half (UP) or per wavefront
    constexpr int WCOL = 32 * NJ;                      // wavefront columns (per half for UP)
    constexpr int BN = WAVES_N * WCOL;                  // block columns (per half for UP)
    constexpr int NB = UP ? 2 * BN : BN;               // B rows per stage
    constexpr int ROWS = BM + NB;
    constexpr int ASTAGE = BM * RB, BSTAGE = NB * RB;  // one stage of A rows / of weight rows
    constexpr int CPR = RB / 16, RPL = 64 / CPR;       // 16-byte chunks per row, rows per 1-KB load
    constexpr int PERW = ROWS / RPL / NW;              // 1-KB loads per wavefront per stage
    constexpr int PA = BM / RPL / NW, PB1 = BN / RPL / NW; // ... of which A rows, W1 (or W2) rows
    constexpr int PBW = PERW - PA;                     // ... of which weight rows
    constexpr int KS = RB / 32;                        // 16-element K steps per stage
    static_assert(BM == 128 || BM == 256, "128- or 256-row tiles");
    static_assert(RB == 64 || RB == 128, "64- or 128-byte rows");
    static_assert(NA >= 2 && NBS >= NA, "the weight ring is at least as deep as the A ring");
    static_assert(ROWS % (NW * RPL) == 0 && BM % (NW * RPL) == 0 && BN % (NW * RPL) == 0 &&
                  (NA - 1) * PA + (NBS - 1) * PBW < 64, "whole loads per wavefront, vmcnt range");
    static_assert(NJ >= 1, "at least one 32-column block per wavefront");
    static_assert(BM * 4 <= ASTAGE, "row table fits the first stage buffer");

    constexpr int OSTR = BN * 2 + 16;                  // epilogue: padded LDS row of the block's output tile
    constexpr int RINGS = NA * ASTAGE + NBS * BSTAGE;
    constexpr int RING = RINGS > BM * OSTR ? RINGS : BM * OSTR;
    __shared__ __attribute__((aligned(1024))) uint8_t ring[RING];
    uint8_t* const ringB = ring + NA * ASTAGE;         // the weight rows' ring follows the A rows' ring
    int* s_tok = (int*)ring;                           // row table, dead before the first load into the ring

    int tile, nb;
    if (!block_work(g, tile, nb)) return;
    const int4 td = g.tiles[tile];
    const int grp = td.x, row0 = td.y, rows = td.z;
    const bool shared = grp == g.E;
    const int N = shared ? g.N_s : g.N_r, K = shared ? g.K_s : g.K_r;
    const int n0 = nb * BN;
    if (n0 >= N) return;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm0 = (wave / WAVES_N) * 128, wn0 = (wave % WAVES_N) * WCOL;
    const int64_t ldb = (shared ? g.ld_s : (int64_t)K) * 2;
    const int64_t lgrp = grp - g.e_base;
    const uint8_t* W1 = shared ? g.S1 : g.B1 + lgrp * N * ldb;
    const uint8_t* W3 = UP ? (shared ? g.S3 : g.B3 + lgrp * N * ldb) : W1;

    if (tid < BM) s_tok[tid] = UP ? g.row_token[row0 + (tid < rows ? tid : 0)] : row0 + (tid < rows ? tid : 0);
    __syncthreads();
    uint32_t off[PERW];
#pragma unroll
    for (int p = 0; p < PERW; p++) {
        const int row = (NW * p + wave) * RPL + lane / CPR;
        const int lc = (swzr<RB>(row, lane % CPR) - row * RB) >> 4;  // logical chunk stored at chunk lane % CPR
        if (p < PA) off[p] = (uint32_t)s_tok[row] * (uint32_t)g.lda + lc * 16;
        else if (p < PA + PB1) off[p] = (uint32_t)(n0 + row - BM) * (uint32_t)ldb + lc * 16;
        else off[p] = (uint32_t)(n0 + row - BM - BN) * (uint32_t)ldb + lc * 16;
    }
    __syncthreads();                                   // the row table is dead from here

    // 32-row MFMA blocks holding tile rows (per wavefront, wave-uniform).  Blocks past the tile's end get
    // no MFMAs and no fragment reads; their A rows are still copied (the row table repeats the tile's first
    // row there, so the copies hit in cache): every wavefront issues the same loads each stage with no
    // branch between them, which was no slower than the copies it saved (prefill up GEMM 3.47 -> 3.44 ms,
    // within the kernel's run-to-run spread) and keeps one vmcnt value for every wavefront.
    const int nrb = max(0, min(4, (rows - wm0 + 31) / 32));

    // K stages walked from a start rotated by the n-block (as in grouped_gemm_kernel), in a fixed order.
    const int nstages = K / (RB / 2);
    const int kshift = (nb * g.krot) % nstages;
    const uint32_t ringA0 = lds_addr(ring), ringB0 = lds_addr(ringB);
    auto kstage = [&](int s) { return (int64_t)(s + kshift >= nstages ? s + kshift - nstages : s + kshift) * RB; };
    // The A rows of stage s into A buffer buf: this wavefront's loads 0 .. PA - 1.
    auto issue_a = [&](int buf, int s) {
        const uint8_t* a = g.A + kstage(s);
        const uint32_t dst = ringA0 + buf * ASTAGE + wave * 1024;
#pragma unroll
        for (int p = 0; p < PA; p++) dma16(a, off[p], dst + p * NW * 1024);
    };
    // The weight rows of stage s into weight buffer buf: this wavefront's loads PA .. PERW - 1.
    auto issue_b = [&](int buf, int s) {
        const int64_t koff = kstage(s);
        const uint8_t* b1 = W1 + koff;
        const uint8_t* b3 = W3 + koff;
        const uint32_t dst = ringB0 + buf * BSTAGE + wave * 1024;
#pragma unroll
        for (int p = PA; p < PERW; p++) dma16(p < PA + PB1 ? b1 : b3, off[p], dst + (p - PA) * NW * 1024);
    };

    f32x16 acc1[4][NJ], acc3[4][UP ? NJ : 1];
#pragma unroll
    for (int i = 0; i < 4; i++) {
#pragma unroll
        for (int j = 0; j < NJ; j++) acc1[i][j] = (f32x16){};
#pragma unroll
        for (int j = 0; j < (UP ? NJ : 1); j++) acc3[i][j] = (f32x16){};
    }

    const int r32 = lane & 31, kh = lane >> 5;
    struct Frags {
        bf16x8 a[4], b1[NJ], b3[UP ? NJ : 1];
    };

    // The K loop for NRB computed row blocks (a compile-time count, so the MFMA / fragment-read
    // interleave below stays one straight-line schedule).
    auto k_loop = [&](auto nrb_tag) {
        constexpr int NRB = decltype(nrb_tag)::value;
        constexpr int NF = NRB == 0 ? 0 : NRB + (UP ? 2 * NJ : NJ);   // fragment reads per K step
        constexpr int NM = NRB * (UP ? 2 * NJ : NJ);                   // MFMAs per K step
        // (The row swizzle repeats every 16 rows, so a weight row keeps it without the BM offset it has in
        // the load offsets above.)
        auto read = [&](int abuf, int bbuf, int kk, Frags& f) {
            if constexpr (NRB > 0) {
                const uint8_t* sa = ring + abuf * ASTAGE;
                const uint8_t* sb = ringB + bbuf * BSTAGE;
                const int ch = 2 * kk + kh;
#pragma unroll
                for (int i = 0; i < NRB; i++) f.a[i] = *(const bf16x8*)(sa + swzr<RB>(wm0 + 32 * i + r32, ch));
#pragma unroll
                for (int j = 0; j < NJ; j++) {
                    f.b1[j] = *(const bf16x8*)(sb + swzr<RB>(wn0 + 32 * j + r32, ch));
                    if constexpr (UP) f.b3[j] = *(const bf16x8*)(sb + swzr<RB>(BN + wn0 + 32 * j + r32, ch));
                }
            }
        };
        auto mma = [&](const Frags& f) {
#pragma unroll
            for (int i = 0; i < NRB; i++)
#pragma unroll
                for (int j = 0; j < NJ; j++) {
                    acc1[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b1[j], acc1[i][j], 0, 0, 0);
                    if constexpr (UP)
                        acc3[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b3[j], acc3[i][j], 0, 0, 0);
                }
        };
        // One K step: the fragments of the next step are read (one read after each of the first NF MFMAs).
        auto kstep = [&](const Frags& cur, int abuf_next, int bbuf_next, int kk_next, Frags& nxt) {
            read(abuf_next, bbuf_next, kk_next, nxt);
            mma(cur);
#pragma unroll
            for (int m = 0; m < NM; m++) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (m < NF) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
        };

        // Rings: stage t's A rows live in A buffer t % NA and its weight rows in weight buffer t % NBS.  The
        // prologue loads the A rows of stages 0 .. NA - 1 and the weight rows of stages 0 .. NBS - 1; at the
        // end of stage s (all its fragments read) stage s + 1 is awaited and published, and stage s's
        // buffers are refilled with the A rows of stage s + NA and the weight rows of stage s + NBS (past the
        // end: the last stage again, into buffers nobody reads).  Weight rows, which stream from HBM or the
        // last-level cache, thus have NBS - 1 stages of lead, A rows (L2 hits mostly) NA - 1.  Loads are issued
        // in the order A(s + NA), weights(s + NBS), so every wait for stage s + 1 is the same vmcnt: only the
        // weight loads issued after it (PBW per wavefront) may remain in flight.
        // The refill sits around the K step that follows the barrier: the A rows before it, the weight rows
        // after it for the up GEMM (before it for the down GEMM).
        auto refill = [&](int ab, int bb, int s, auto&& step) {
            issue_a(ab, min(s + NA, nstages - 1));
            if constexpr (!UP) issue_b(bb, min(s + NBS, nstages - 1));
            step();
            if constexpr (UP) issue_b(bb, min(s + NBS, nstages - 1));
        };
#pragma unroll
        for (int t = 0; t < NBS; t++) {
            if (t < NA) issue_a(t, min(t, nstages - 1));
            issue_b(t, min(t, nstages - 1));
        }
        wait_vmcnt<(NA - 1) * PA + (NBS - 1) * PBW>(); // stage 0 only, its successors stay in flight
        lds_barrier();
        Frags f0, f1;
        read(0, 0, 0, f0);
        int ab = 0, bb = 0;
        for (int s = 0; s + 1 < nstages; s++) {
            const int nab = ab + 1 == NA ? 0 : ab + 1, nbb = bb + 1 == NBS ? 0 : bb + 1;
            if constexpr (KS == 4) {
                kstep(f0, ab, bb, 1, f1);
                kstep(f1, ab, bb, 2, f0);
                kstep(f0, ab, bb, 3, f1);
            } else {
                kstep(f0, ab, bb, 1, f1);
            }
            wait_vmcnt<PBW>();
            lds_barrier();
            refill(ab, bb, s, [&] { kstep(f1, nab, nbb, 0, f0); });
            ab = nab;
            bb = nbb;
        }
        if constexpr (KS == 4) {
            kstep(f0, ab, bb, 1, f1);
            kstep(f1, ab, bb, 2, f0);
            kstep(f0, ab, bb, 3, f1);
            mma(f1);
        } else {
            kstep(f0, ab, bb, 1, f1);
            mma(f1);
        }
    };
    switch (nrb) {
    case 4: k_loop(IntC<4>{}); break;
    case 3: k_loop(IntC<3>{}); break;
    case 2: k_loop(IntC<2>{}); break;
    case 1: k_loop(IntC<1>{}); break;
    default: k_loop(IntC<0>{}); break;
    }
    wait_vmcnt<0>();                                   // no load may still target this block's LDS
    __syncthreads();                                   // every wavefront is done with the ring

    // Epilogue (32x32 accumulator layout: lane holds column lane % 32, rows 8 (r / 4) + 4 (lane / 32) + r % 4):
    // the block's bf16 tile (UP: h = silu(g) * u, BN columns) into LDS, then coalesced to global memory.
    // Rows come in pairs (r, r + 1 share a 4-row group), so one conversion rounds both outputs (and for UP
    // one rounds g and u of each).
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
            const int row = wm0 + 32 * i + 8 * (r >> 2) + 4 * kh + (r & 3);
#pragma unroll
            for (int j = 0; j < NJ; j++) {
                float v0 = acc1[i][j][r], v1 = acc1[i][j][r + 1];
                if constexpr (UP) {
                    float u0 = acc3[i][j][r], u1 = acc3[i][j][r + 1];
                    round_bf16x2(v0, u0);
                    round_bf16x2(v1, u1);
                    v0 = silu_mul_fast(v0, u0);
                    v1 = silu_mul_fast(v1, u1);
                }
                const uint32_t p = f32x2_to_bf16x2(v0, v1);
                uint8_t* o = ring + row * OSTR + (wn0 + 32 * j + r32) * 2;
                *(uint16_t*)o = (uint16_t)p;
                *(uint16_t*)(o + OSTR) = (uint16_t)(p >> 16);
            }
        }
    __syncthreads();
    store_tile_bf16<BM, BN, OSTR, 64 * NW, !UP>(ring, g.out, g.ldo, row0, rows, n0);
}

// One 128-wide K stage of fp8 MFMAs for the direct-to-LDS fp8 kernel: the wavefront's WM x WN blocks of
// 16 x 16 (and the W3 half for the up GEMM), each the product of one 16-row weight fragment (first MFMA
// operand) and one 16-row activation fragment (second), so a result holds [feature][token]: lane l has
// features 4 (l / 16) + r, r = 0..3, of token l % 16.  All four values of a lane then share one row
// scale, and the per-K-block rescale acc += p * (row scale * weight block scale) needs one scale product
// per lane and row block (against four rows per lane in [token][feature] order: 2 instead of 8 multiplies
// per four MFMAs).  B fragments and the lane's row scales of the stage stay in registers; A fragments are
// read one row block ahead (two in the pipelined form).  With more than 64 accumulator VGPRs a row
// block's MFMAs also wait for the rescaling of the previous block's results, so only one block's MFMA
// results are live and a 128 x 64 wavefront tile (128 accumulator VGPRs) fits two wavefronts per SIMD.
// mid() runs once in the stage, at row block MID_AT (at the end when the wavefront computes fewer row
// blocks): the kernel issues the second half of a ring refill there.  Only the first NB of the WM row blocks hold tile rows; the
// others get no MFMAs, no rescale and no fragment reads (their accumulators stay zero, never stored).
// In the pipelined form (TIGHT below) a stage's last row block is not rescaled before the stage barrier:
// its MFMA results and scale products are carried into the next stage and rescaled after that stage's
// first row block's MFMAs, like any other block's one block later.  Each accumulator still receives its K
// blocks' terms in K order.  The carry starts as zeros (adding 0 * 0 leaves +0 accumulators as they are)
// and f8_flush applies the last stage's after the walk.
template <int NP> struct F8Carry {
    f32x4 p[NP];
    float s1, s3;
};

template <bool UP, int WM, int WN> constexpr bool f8_tight() { return WM * WN * (UP ? 2 : 1) > 16; }

template <bool UP, int WM, int WN, int NB, int NP>
__device__ __forceinline__ void f8_flush(const F8Carry<NP>& car, f32x4 (&acc1)[WM][WN], f32x4 (&acc3)[WM][WN])
{
    if constexpr (f8_tight<UP, WM, WN>() && NB > 0) {
#pragma unroll
        for (int j = 0; j < WN; j++)
#pragma unroll
            for (int r = 0; r < 4; r++) {
                acc1[NB - 1][j][r] += car.p[j][r] * car.s1;
                if constexpr (UP) acc3[NB - 1][j][r] += car.p[WN + j][r] * car.s3;
            }
    }
}

template <bool UP, int WM, int WN, int BN, int NB, int MID_AT, typename MID>
__device__ __forceinline__ void mma_f8(const uint8_t* As_lds, const uint8_t* Bs_lds, const float* sA_lds, float sb1,
                                       float sb3, int wm0, int wn0, int lane, f32x4 (&acc1)[WM][WN],
                                       f32x4 (&acc3)[WM][WN], F8Carry<UP ? 2 * WN : WN>& car, MID&& mid)
{
    static_assert(NB >= 0 && NB <= WM, "row blocks");
    static_assert(WM > MID_AT, "mid() runs inside the row-block loop");
    const int r16 = lane & 15, q = lane >> 4;
    constexpr bool TIGHT = f8_tight<UP, WM, WN>();     // more than 64 accumulator VGPRs
    auto frag = [&](const uint8_t* base, int row) {
        const i32x4 lo = *(const i32x4*)(base + swzr<128>(row, 2 * q));
        const i32x4 hi = *(const i32x4*)(base + swzr<128>(row, 2 * q + 1));
        return (i32x8){lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    };
    i32x8 b1[WN], b3[UP ? WN : 1];
#pragma unroll
    for (int j = 0; j < WN; j++) {
        b1[j] = frag(Bs_lds, wn0 + j * 16 + r16);
        if constexpr (UP) b3[j] = frag(Bs_lds, BN + wn0 + j * 16 + r16);
    }
    // The lane's WM row scales (rows wm0 + 16 i + r16) sit in the stage's scale copy in groups of four
    // (rows of blocks 4v .. 4v + 3 at wm0 + 64 v + 4 r16), so WM / 4 16-byte reads at the start of the
    // stage fetch them all, the 16 lanes of a read covering 256 consecutive bytes (no bank conflicts).  A
    // 4-byte read per row block, issued with the next A fragment, made each scale product wait for that
    // fragment too (LDS reads complete in order).
    static_assert(WM % 4 == 0, "row scales as 16-byte vectors");
    f32x4 sv[WM / 4];
#pragma unroll
    for (int v = 0; v < WM / 4; v++) sv[v] = *(const f32x4*)(sA_lds + wm0 + 64 * v + 4 * r16);
    auto scale = [&](int i) { return sv[i >> 2][i & 3]; };   // row scale of the lane's token in row block i
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    if constexpr (NB == 0) {
        mid();
        return;
    }
    i32x8 a = frag(As_lds, wm0 + r16);
    float sa = scale(0);
    if constexpr (TIGHT) {
        // Software pipeline over row blocks: block i's MFMAs are issued before the previous block's results
        // are rescaled (block i - 1, or for i = 0 the previous stage's last block, from the carry), so the
        // matrix pipe runs while the vector ALU rescales.  A fragments are read two blocks ahead; block
        // i + 2's passes through an empty asm that also takes the rescaled accumulators, so its read has
        // landed by the end of block i and at most two blocks' MFMA results are live.
        constexpr int NP = UP ? 2 * WN : WN;          // MFMA results per row block
        f32x4 pc[NP], pp[NP];
        float s1 = car.s1, s3 = car.s3;                // scale products of the previous block
#pragma unroll
        for (int n = 0; n < NP; n++) pp[n] = car.p[n];
        i32x8 a2 = a;                                  // block i + 1's A fragment, read one block early
        if (NB > 1) a2 = frag(As_lds, wm0 + 16 + r16);
#pragma unroll
        for (int i = 0; i < NB; i++) {
            const int ip = i > 0 ? i - 1 : NB - 1;     // the block rescaled here
            const i32x8 a_next = a2;
#pragma unroll
            for (int j = 0; j < WN; j++) {
                pc[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b1[j], a, zero, 0, 0, 0, 127, 0, 127);
                if constexpr (UP)
                    pc[WN + j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b3[j], a, zero, 0, 0, 0, 127, 0, 127);
            }
            if (UP && i == MID_AT) mid();
            if (i + 2 < NB) a2 = frag(As_lds, wm0 + (i + 2) * 16 + r16);
#pragma unroll
            for (int j = 0; j < WN; j++) {
#pragma unroll
                for (int r = 0; r < 4; r++) acc1[ip][j][r] += pp[j][r] * s1;
                if constexpr (UP) {
#pragma unroll
                    for (int r = 0; r < 4; r++) acc3[ip][j][r] += pp[WN + j][r] * s3;
                }
            }
            // After each MFMA of block i, four of the previous block's rescale FMAs (and block i + 2's
            // fragment reads after the first), so the vector ALU works while the matrix pipe runs.  The
            // scheduling barrier at the end of the block keeps the compiler from hoisting block i's own
            // rescale (next block's work) up to just behind its MFMAs, where it would wait for their results.
#pragma unroll
            for (int m = 0; m < NP; m++) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (m == 0) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
            }
#pragma unroll
            for (int j = 0; j < WN; j++) {
                if constexpr (UP) asm volatile("" : "+v"(a2) : "v"(acc1[ip][j]), "v"(acc3[ip][j]));
                else asm volatile("" : "+v"(a2) : "v"(acc1[ip][j]));
            }
            if (!UP && i == MID_AT) mid();
            s1 = scale(i) * sb1;
            s3 = scale(i) * sb3;
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int n = 0; n < NP; n++) pp[n] = pc[n];
            a = a_next;
        }
#pragma unroll
        for (int n = 0; n < NP; n++) car.p[n] = pp[n];
        car.s1 = s1;
        car.s3 = s3;
        if constexpr (NB <= MID_AT) mid();
        return;
    }
#pragma unroll
    for (int i = 0; i < NB; i++) {
        i32x8 a_next = a;
        float sa_next = sa;
        if (i + 1 < NB) {
            a_next = frag(As_lds, wm0 + (i + 1) * 16 + r16);
            sa_next = scale(i + 1);
        }
        const float s1 = sa * sb1, s3 = sa * sb3;
#pragma unroll
        for (int j = 0; j < WN; j++) {
            const f32x4 p1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b1[j], a, zero, 0, 0, 0, 127, 0, 127);
#pragma unroll
            for (int r = 0; r < 4; r++) acc1[i][j][r] += p1[r] * s1;
            if constexpr (UP) {
                const f32x4 p3 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b3[j], a, zero, 0, 0, 0, 127, 0, 127);
#pragma unroll
                for (int r = 0; r < 4; r++) acc3[i][j][r] += p3[r] * s3;
            }
        }
        if (i == MID_AT) mid();
        a = a_next;
        sa = sa_next;
    }
    if constexpr (NB <= MID_AT) mid();
}

// Epilogue of the direct-to-LDS fp8 kernel, for the [feature][token] accumulator layout of mma_f8 (lane
// l holds features 4 (l / 16) + r of token l % 16).  UP: h = round(silu(round g) * round u) through LDS
// (BM x BN floats, each row's 16-byte chunks XOR-swizzled by token so a wavefront's 16 tokens write
// distinct banks), then quantised per 1 x 128 group to E4M3 codes plus one scale per group.  Down: the
// bf16 output tile through LDS (padded rows), then whole-line copies to the output rows.
template <bool UP, int BM, int BN, int WM, int WN, int NT>
__device__ __forceinline__ void f8_epilogue(const GemmArgs& g, uint8_t* smem, const f32x4 (&acc1)[WM][WN],
                                            const f32x4 (&acc3)[WM][WN], int rows, int row0, int n0, int wm0,
                                            int wn0, int tid)
{
    const int lane = tid & 63;
    const int r16 = lane & 15, q = lane >> 4;
    if constexpr (UP) {
        static_assert(BN / 4 >= 16, "the chunk swizzle flips the low four bits of a row's chunk index");
        float* hs = (float*)smem;                      // [BM][BN]; logical chunk c of row t at chunk c ^ (t % 16)
#pragma unroll
        for (int i = 0; i < WM; i++) {
            const int t = wm0 + i * 16 + r16;
#pragma unroll
            for (int j = 0; j < WN; j++) {
                float gv[4], uv[4];
#pragma unroll
                for (int r = 0; r < 4; r++) {
                    gv[r] = acc1[i][j][r];
                    uv[r] = acc3[i][j][r];
                    round_bf16x2(gv[r], uv[r]);
                    gv[r] = silu_mul_fast(gv[r], uv[r]);
                }
                round_bf16x2(gv[0], gv[1]);
                round_bf16x2(gv[2], gv[3]);
                const f32x4 v = {gv[0], gv[1], gv[2], gv[3]};
                const int c = ((wn0 + j * 16) >> 2) + q;
                *(f32x4*)(hs + t * BN + ((c ^ (t & 15)) << 2)) = v;
            }
        }
        __syncthreads();
        // 16 threads per (row, 128-column group), 8 columns (two chunks) each
        constexpr int GROUPS = BM * (BN / 128);
        for (int gi = tid >> 4; gi < GROUPS; gi += NT / 16) {
            const int row = gi / (BN / 128), grp128 = gi % (BN / 128);
            const int sub = tid & 15;
            const int c0 = grp128 * 32 + 2 * sub;
            const f32x4 va = *(const f32x4*)(hs + row * BN + ((c0 ^ (row & 15)) << 2));
            const f32x4 vb = *(const f32x4*)(hs + row * BN + (((c0 + 1) ^ (row & 15)) << 2));
            const float v[8] = {va[0], va[1], va[2], va[3], vb[0], vb[1], vb[2], vb[3]};
            float amax = 0.f;
#pragma unroll
            for (int e = 0; e < 8; e++) amax = fmaxf(amax, fabsf(v[e]));
            amax = row16_max(amax);
            const float sc = amax > 0.f ? amax / 448.0f : 1.0f;
            if (row < rows) {
                float q[8];
                if (quant_div_fast(sc)) {
                    const float r = recip_rn(sc);
#pragma unroll
                    for (int e = 0; e < 8; e++) q[e] = quant_div(v[e], sc, r);
                } else {
#pragma unroll
                    for (int e = 0; e < 8; e++) q[e] = v[e] / sc;
                }
                uint32_t lo = f32x2_to_e4m3(q[0], q[1]) | (f32x2_to_e4m3(q[2], q[3]) << 16);
                uint32_t hi = f32x2_to_e4m3(q[4], q[5]) | (f32x2_to_e4m3(q[6], q[7]) << 16);
                const int64_t orow = row0 + row;
                *(uint2*)(g.out + orow * g.ldo + n0 + grp128 * 128 + sub * 8) = make_uint2(lo, hi);
                if (sub == 0) g.outs[orow * g.ldos + (n0 + grp128 * 128) / 128] = sc;
            }
        }
    } else {
        constexpr int OSTR = BN * 2 + 16;              // padded LDS row of the bf16 output tile
#pragma unroll
        for (int i = 0; i < WM; i++)
#pragma unroll
            for (int j = 0; j < WN; j++) {
                const uint32_t lo = f32x2_to_bf16x2(acc1[i][j][0], acc1[i][j][1]);
                const uint32_t hi = f32x2_to_bf16x2(acc1[i][j][2], acc1[i][j][3]);
                *(uint2*)(smem + (wm0 + i * 16 + r16) * OSTR + (wn0 + j * 16 + 4 * q) * 2) = make_uint2(lo, hi);
            }
        __syncthreads();
        store_tile_bf16<BM, BN, OSTR, NT, true>(smem, g.out, g.ldo, row0, rows, n0);
    }
}

// ---------------------------------------------------------------------------------------------------
// fp8 form with direct-to-LDS staging (128- or 256-row tiles, eight wavefronts as 2 x 4, the 16x16x128
// fp8 MFMA and per-K-block rescaling of mma_f8).  A K stage is 128 fp8 elements: one 128-byte line of every A
// row, W1 row and W3 row, its 16-byte chunks XOR-swizzled over a 16-row period (swzr<128>), so the 16-row
// fragment reads of mma_f8 hit distinct banks.  The stages sit in a ring of NSTG buffers filled by global_load_lds (no
// staging registers, no LDS stores), NSTG - 1 of them in flight while one is computed.  The scales of a
// stage ride in the same ring: wavefronts 0-1 copy the A row scales of the stage (one 4-byte load per
// row), wavefront 2 the W1 block scales, wavefront 3 the W3 block scales, the others a dummy copy, so
// every wavefront issues the same number of loads per stage and one vmcnt value waits for a stage.
// ---------------------------------------------------------------------------------------------------
template <bool UP, int BM, int BN, int NSTG>
__global__ __launch_bounds__(512, 2) void grouped_gemm_f8_kernel(GemmArgs g)
{
    constexpr int WAVES_M = 2, WAVES_N = 4, NW = 8, NT = 512;
    constexpr int WM = BM / 16 / WAVES_M, WN = BN / 16 / WAVES_N;
    constexpr int NB = UP ? 2 * BN : BN;               // B rows per stage
    constexpr int ROWS = BM + NB;                      // 128-byte LDS rows per stage
    constexpr int STAGE = ROWS * 128;
    constexpr int LOADS = ROWS / 8;                    // 1-KB loads per stage
    constexpr int PERW = LOADS / NW;                   // ... per wavefront
    constexpr int PA = BM / 8 / NW;                    // ... of which A rows
    constexpr int PB1 = BN / 8 / NW;                   // ... W1 (or W2) rows
    constexpr int NL = PERW + 1;                       // loads per wavefront per stage (with the scale copy)
    static_assert(LOADS % NW == 0 && BN % 128 == 0 && BN / 128 <= 64, "whole loads per wavefront");
    static_assert(WN * 16 <= 128 && 128 % (WN * 16) == 0, "a wavefront's columns share one fp8 block scale");
    static_assert((NSTG - 1) * NL < 64, "vmcnt range");
    static_assert(!UP || BM * BN * 4 <= NSTG * STAGE, "h tile must fit the ring");
    static_assert(BM == 128 || BM == 256, "128- or 256-row tiles");
    constexpr int SW = BM / 64;                        // wavefronts copying A row scales; W1, W3 next

    constexpr int OSTR = BN * 2 + 16;                  // down epilogue: padded LDS row of the bf16 output tile
    constexpr int RING = (UP || NSTG * STAGE > BM * OSTR) ? NSTG * STAGE : BM * OSTR;
    __shared__ __attribute__((aligned(1024))) uint8_t ring[RING];
    __shared__ __attribute__((aligned(256))) float scl[NSTG][NW * 64];   // per stage: A row scales, W1, W3 block scales
    __shared__ int s_tok[BM];

    int tile, nb;
    if (!block_work(g, tile, nb)) return;
    const int4 td = g.tiles[tile];
    const int grp = td.x, row0 = td.y, rows = td.z;
    const bool shared = grp == g.E;
    const int N = shared ? g.N_s : g.N_r, K = shared ? g.K_s : g.K_r;
    const int n0 = nb * BN;
    if (n0 >= N) return;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm0 = (wave / WAVES_N) * WM * 16, wn0 = (wave % WAVES_N) * WN * 16;
    const int64_t ldb = shared ? g.ld_s : (int64_t)K;  // bytes per weight row
    const int64_t lgrp = grp - g.e_base;
    const uint8_t* W1 = shared ? g.S1 : g.B1 + lgrp * N * ldb;
    const uint8_t* W3 = UP ? (shared ? g.S3 : g.B3 + lgrp * N * ldb) : W1;
    const int nkb = shared ? g.nkb_s : K / 128;        // scale blocks per weight-scale row
    const float* W1s = (shared ? g.S1s : g.B1s + lgrp * (N / 128) * nkb) + (n0 / 128) * nkb;
    const float* W3s = UP ? (shared ? g.S3s : g.B3s + lgrp * (N / 128) * nkb) + (n0 / 128) * nkb : W1s;

    // rows past the tile's end repeat its first row (valid memory, finite values; never stored)
    if (tid < BM) s_tok[tid] = UP ? g.row_token[row0 + (tid < rows ? tid : 0)] : row0 + (tid < rows ? tid : 0);
    __syncthreads();

    // Per-lane source offsets, fixed over the K walk.  Load p of wavefront w fills LDS rows
    // (p * NW + w) * 8 .. + 8; lane l writes stored chunk l % 8 of row l / 8, which holds the logical chunk
    // stored there by swzr<128> (the row's swizzle repeats every 16 rows, so A and B rows share it).
    uint32_t off[PERW];
#pragma unroll
    for (int p = 0; p < PERW; p++) {
        const int row = (p * NW + wave) * 8 + (lane >> 3);
        const int lc = (swzr<128>(row, lane & 7) - row * 128) >> 4;
        if (p < PA) off[p] = (uint32_t)s_tok[row] * (uint32_t)g.lda + lc * 16;
        else if (p < PA + PB1) off[p] = (uint32_t)(n0 + row - BM) * (uint32_t)ldb + lc * 16;
        else off[p] = (uint32_t)(n0 + row - BM - BN) * (uint32_t)ldb + lc * 16;
    }
    // scale copy of this wavefront: byte offset from its base, the base moved by the K stage below
    uint32_t soff = 0;
    if (wave < SW) {
        // A row scales in the order mma_f8 reads them: position wm0 + 64 v + 4 r16 + e holds row
        // wm0 + 16 (4 v + e) + r16
        const int p = wave * 64 + lane, rem = p % (WM * 16);
        soff = (uint32_t)s_tok[p - rem + 16 * (4 * (rem / 64) + rem % 4) + (rem % 64) / 4] * (uint32_t)g.ldas * 4u;
    }
    else if (wave == SW || (UP && wave == SW + 1)) soff = (uint32_t)(lane < BN / 128 ? lane : 0) * (uint32_t)nkb * 4u;

    const int nstages = K / 128;
    const int kshift = (nb * g.krot) % nstages;
    const uint32_t ring0 = lds_addr(ring), scl0 = lds_addr(&scl[0][0]);
    // Stage s into ring buffer buf: this wavefront's operand loads p0 .. p1 - 1, and its scale load if asked.
    auto issue = [&](int buf, int s, int p0, int p1, bool with_scales) {
        const int ks = s + kshift >= nstages ? s + kshift - nstages : s + kshift;
        const int64_t koff = (int64_t)ks * 128;
        const uint32_t dst = ring0 + buf * STAGE + wave * 1024;
#pragma unroll
        for (int p = p0; p < p1; p++) dma16((p < PA ? g.A : p < PA + PB1 ? W1 : W3) + koff, off[p], dst + p * NW * 1024);
        const uint8_t* sb = wave < SW ? (const uint8_t*)(g.As + ks)
                          : wave == SW ? (const uint8_t*)(W1s + ks)
                          : (UP && wave == SW + 1) ? (const uint8_t*)(W3s + ks) : (const uint8_t*)W1s;
        if (with_scales) dma4(sb, soff, scl0 + (buf * NW * 64 + wave * 64) * 4);
    };

    f32x4 acc1[WM][WN], acc3[WM][WN];
#pragma unroll
    for (int i = 0; i < WM; i++)
#pragma unroll
        for (int j = 0; j < WN; j++) acc1[i][j] = acc3[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};

    const int cb = wn0 / 128;                          // the wavefront's weight block within the n-block
    // 16-row blocks of this wavefront that hold tile rows (wave-uniform)
    const int nrb = __builtin_amdgcn_readfirstlane(max(0, min(WM, (rows - wm0 + 15) / 16)));
#pragma unroll
    for (int t = 0; t < NSTG; t++) issue(t, min(t, nstages - 1), 0, PERW, true);
    wait_vmcnt<(NSTG - 1) * NL>();
    lds_barrier();
    // A freed buffer is refilled in two halves: the first right after the barrier, the rest (with the
    // scales) from inside the next stage's MFMAs, so no wavefront stalls on a burst of loads before its
    // MFMAs (fp8 up GEMM 11.48 -> 11.19 ms with the second half after the second row block).  Every load
    // of the refill still precedes the next wait.
    // The K walk for NB computed row blocks (a compile-time count, so the MFMA / rescale pipeline of mma_f8
    // stays one straight-line schedule; the walk is instantiated per count, like the bf16 kernel's).
    auto k_walk = [&](auto nb_tag) {
        constexpr int NB = decltype(nb_tag)::value;
        F8Carry<UP ? 2 * WN : WN> car;
#pragma unroll
        for (int n = 0; n < (UP ? 2 * WN : WN); n++) car.p[n] = (f32x4){0.f, 0.f, 0.f, 0.f};
        car.s1 = car.s3 = 0.f;
        int buf = 0, pbuf = -1, pst = 0;
        for (int s = 0; s < nstages; s++) {
            const float* sc = scl[buf];
            const uint8_t* st = ring + buf * STAGE;
            mma_f8<UP, WM, WN, BN, NB, UP ? 3 : 0>(st, st + BM * 128, sc, sc[BM + cb], UP ? sc[BM + 64 + cb] : 0.f,
                                                   wm0, wn0, lane, acc1, acc3, car,
                                                   [&] { if (pbuf >= 0) issue(pbuf, pst, PERW / 2, PERW, true); });
            pbuf = -1;
            if (s + 1 < nstages) {
                wait_vmcnt<(NSTG - 2) * NL>();         // stage s + 1 has landed
                lds_barrier();                         // ... for every wavefront; stage s is read
                pst = min(s + NSTG, nstages - 1);      // past the end: the last stage again (never read)
                issue(buf, pst, 0, PERW / 2, false);
                pbuf = buf;
                buf = buf + 1 == NSTG ? 0 : buf + 1;
            }
        }
        f8_flush<UP, WM, WN, NB>(car, acc1, acc3);
    };
    with_count<WM>(nrb, k_walk);
    wait_vmcnt<0>();                                   // no load may still target this block's LDS
    lds_barrier();
    f8_epilogue<UP, BM, BN, WM, WN, NT>(g, ring, acc1, acc3, rows, row0, n0, wm0, wn0, tid);
}

// fp8 activation quantisation of x: per row, per 128-column group, s = amax / 448 (1 if amax = 0),
// codes = E4M3(round to nearest even)(x / s).  16 threads per group, 8 elements each.
__global__ __launch_bounds__(256) void act_quant_kernel(const uint16_t* __restrict__ x, int64_t ngroups, int d,
                                                        uint8_t* __restrict__ xq, float* __restrict__ xs)
{
    const int64_t gi = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
    const int sub = threadIdx.x & 15;
    if (gi >= ngroups) return;                         // whole 16-lane groups exit together
    const int64_t row = gi / (d / 128), col = (gi % (d / 128)) * 128 + sub * 8;
    const uint4 raw = *(const uint4*)(x + row * d + col);
    const uint32_t wv[4] = {raw.x, raw.y, raw.z, raw.w};
    float v[8];
#pragma unroll
    for (int e = 0; e < 4; e++) {
        v[2 * e] = __uint_as_float(wv[e] << 16);
        v[2 * e + 1] = __uint_as_float(wv[e] & 0xFFFF0000u);
    }
    float amax = 0.f;
#pragma unroll
    for (int e = 0; e < 8; e++) amax = fmaxf(amax, fabsf(v[e]));
    amax = row16_max(amax);
    const float sc = amax > 0.f ? amax / 448.0f : 1.0f;
    float q[8];
    if (quant_div_fast(sc)) {
        const float r = recip_rn(sc);
#pragma unroll
        for (int e = 0; e < 8; e++) q[e] = quant_div(v[e], sc, r);
    } else {
#pragma unroll
        for (int e = 0; e < 8; e++) q[e] = v[e] / sc;
    }
    const uint32_t lo = f32x2_to_e4m3(q[0], q[1]) | (f32x2_to_e4m3(q[2], q[3]) << 16);
    const uint32_t hi = f32x2_to_e4m3(q[4], q[5]) | (f32x2_to_e4m3(q[6], q[7]) << 16);
    *(uint2*)(xq + row * d + col) = make_uint2(lo, hi);
    if (sub == 0) xs[gi] = sc;
}

hipError_t launch_quantize_e4m3(int64_t rows, int cols, const void* x, uint8_t* q, float* scales, hipStream_t stream)
{
    const int64_t ngroups = rows * (cols / 128);
    act_quant_kernel<<<(unsigned)((ngroups + 15) / 16), 256, 0, stream>>>((const uint16_t*)x, ngroups, cols, q, scales);
    return hipGetLastError();
}

hipError_t launch_act_quant(const moe_shape_t& s, const void* x, const Workspace& ws, hipStream_t stream)
{
    return launch_quantize_e4m3(s.T, (int)s.d, x, ws.xq, ws.xs, stream);
}

template <int ET, bool UP, bool ACT_BF16, int BM, int BN, int WAVES_M, int WAVES_N, int NBUF = 2, int MINW = 1>
static void launch_one(GemmArgs a, hipStream_t stream)
{
    const int64_t nblk = launch_blocks(a);
    grouped_gemm_kernel<ET, UP, ACT_BF16, BM, BN, WAVES_M, WAVES_N, NBUF, MINW>
        <<<(unsigned)nblk, 64 * WAVES_M * WAVES_N, 0, stream>>>(a);
}

// K-stage rotation per n-block: the down GEMM (rows of inter elements) and the large-tile up GEMMs gain
// from it; the up GEMM with 16-row tiles already streams at the HBM ceiling without it.
static constexpr int KROT_UP16 = 0;
static constexpr int KROT_UP = 3;
static constexpr int KROT_WDN = 3;   // wide-kernel down GEMM (rotations 0 / 1 / 5 / 7 / 13 measured slower)
static constexpr int KROT_DN = 1;
// Tiles per group of the large-tile block order (block_work: groups dealt round-robin to the XCDs).
// Four for the GEMMs in general (skewed layer, groups of 2 / 3 / 4 / 6 / 8 tiles: 13.66 / 13.64 / 13.56 /
// 13.79 / 13.82 ms; fp8 layer 4 / 8 / 16: 16.15 / 16.14 / 16.29 ms; all bitwise equal); the fp8 down GEMM,
// whose h rows are short (inter bytes) and whose 256-wide n-blocks are many (d / 256), does best with
// groups of two (fp8 layer, down GEMM with 1 / 2 / 4: 4.70 / 4.67 / 4.76 ms).
static constexpr int GROUP_M = 4;
static constexpr int GROUP_M_F8_DN = 2;

// bf16 256-row tiles: 128-byte K stages in a ring of two (64-byte stages in deeper rings request twice
// the lines and measured slower), eight wavefronts (four, one per SIMD with 128 x 128 each, measured
// 7 % slower on the skewed workload).  Both GEMMs walk K with the up GEMM's rotation here (other rotations
// measured no different).
template <bool UP>
static void launch_w(GemmArgs a, hipStream_t stream)
{
    const int64_t nblk = launch_blocks(a);
    grouped_gemm_w_kernel<UP, 256, 128, 2, 3, 8><<<(unsigned)nblk, 512, 0, stream>>>(a);
}

// fp8 tiles of 128 or 256 rows: a ring of three stages for 128-row tiles, two for 256 (LDS).
template <bool UP, int BM, int BN>
static void launch_f8(GemmArgs a, hipStream_t stream)
{
    const int64_t nblk = launch_blocks(a);
    grouped_gemm_f8_kernel<UP, BM, BN, BM == 128 ? 3 : 2><<<(unsigned)nblk, 512, 0, stream>>>(a);
}

// 16-row tiles (bf16): output features per block, wavefronts, minimum wavefronts per SIMD.  inter and
// inter_shared must be multiples of SMALL_UP_BN (the host requires multiples of 128).  The up GEMM's
// 128-wide blocks of eight wavefronts stream W1 and W3 a little faster than 64-wide blocks of four
// (64-token bf16 layer: 1.881 -> 1.852 ms, bitwise equal; 128 on four wavefronts 1.854, 256 on eight
// 1.969); the down GEMM gains nothing from 128-wide blocks (0.962 -> 0.959 / 0.960 ms on four / eight).
static constexpr int SMALL_UP_BN = 128, SMALL_UP_WAVES = 8, SMALL_UP_MINW = 1;
static constexpr int SMALL_DN_BN = 64, SMALL_DN_WAVES = 4, SMALL_DN_MINW = 1;

// Common fields of both GEMMs' arguments.
static GemmArgs base_args(const moe_shape_t& s, const Workspace& ws, int e_base)
{
    GemmArgs a = {};
    a.e_base = e_base;
    a.tiles = ws.tiles;
    a.ntiles = ws.sync;
    a.max_tiles = (int)ws.max_tiles;
    a.E = (int)s.E;
    a.group_m = tile_rows(s) == 16 ? 0 : GROUP_M;
    return a;
}

// Kernel per (dtype, tile rows):
//   16-row tiles          grouped_gemm_kernel (register-staged), every dtype
//   fp32, 128-row tiles   grouped_gemm_kernel
//   bf16, 256-row tiles   grouped_gemm_w_kernel; the down GEMM with d an odd multiple of 128 takes
//                         grouped_gemm_kernel with 128-wide n-blocks
//   fp8, 128/256-row      grouped_gemm_f8_kernel
hipError_t launch_up_gemm(const moe_shape_t& s, const void* x, const void* W1, const void* W3, const float* W1s,
                          const float* W3s, const void* S1, const void* S3, const float* S1s, const float* S3s,
                          const Workspace& ws, hipStream_t stream, int e_base, int n_shared)
{
    const bool fp8 = s.w_dtype == MOE_FP8_E4M3, f32 = s.act_dtype == MOE_F32;
    const int64_t act = f32 ? 4 : 2;
    GemmArgs up = base_args(s, ws, e_base);
    up.row_token = ws.row_token;
    up.A = fp8 ? ws.xq : (const uint8_t*)x;
    up.As = ws.xs;
    up.lda = s.d * (fp8 ? 1 : act);
    up.ldas = s.d / 128;
    up.B1 = (const uint8_t*)W1;
    up.B3 = (const uint8_t*)W3;
    up.B1s = W1s;
    up.B3s = W3s;
    // shared expert: n_shared hidden features, rows of d elements
    up.S1 = (const uint8_t*)S1;
    up.S3 = (const uint8_t*)S3;
    up.S1s = S1s;
    up.S3s = S3s;
    up.ld_s = s.d;
    up.nkb_s = (int)(s.d / 128);
    up.out = (uint8_t*)ws.h;
    up.outs = ws.hs;
    up.ldo = ws.inter_max;
    up.ldos = ws.inter_max / 128;
    up.N_r = (int)s.inter;
    up.N_s = n_shared;
    up.K_r = up.K_s = (int)s.d;
    const int bm = tile_rows(s);
    up.krot = bm == 16 ? KROT_UP16 : KROT_UP;
    // bf16 large tiles with at most one tile per expert on average (prefill): weight panels are not shared
    // between tiles, so each tile's n-blocks run together and walk K in step, sharing the tile's gathered x
    // rows in L2 (4096-token bf16 layer: up GEMM 3.05 -> 3.01-3.02 ms; groups of 2 or 4 tiles the same, 8 no
    // gain, and with the K rotation kept it is slower, 3.09 ms).
    if (!fp8 && !f32 && bm > 16 && s.T * s.k <= (int64_t)s.E * bm) {
        up.group_m = 1;
        up.krot = 0;
    }
    if (fp8) {
        up.n_blocks = (int)(ws.inter_max / 128);
        if (bm == 16) launch_one<ET_FP8, true, true, 16, 128, 1, 4>(up, stream);
        else if (bm == 128) launch_f8<true, 128, 128>(up, stream);
        else launch_f8<true, 256, 128>(up, stream);
    } else if (f32) {
        up.n_blocks = (int)(ws.inter_max / 64);
        if (bm == 16) launch_one<ET_F32, true, false, 16, 64, 1, 4>(up, stream);
        else launch_one<ET_F32, true, false, 128, 64, 2, 2>(up, stream);
    } else if (bm == 16) {
        up.n_blocks = (int)(ws.inter_max / SMALL_UP_BN);
        launch_one<ET_BF16, true, true, 16, SMALL_UP_BN, 1, SMALL_UP_WAVES, 2, SMALL_UP_MINW>(up, stream);
    } else {
        up.n_blocks = (int)(ws.inter_max / 128);
        launch_w<true>(up, stream);
    }
    return hipGetLastError();
}

hipError_t launch_down_gemm(const moe_shape_t& s, const void* W2, const float* W2s, const void* S2, const float* S2s,
                            const Workspace& ws, hipStream_t stream, int e_base, int n_shared)
{
    const bool fp8 = s.w_dtype == MOE_FP8_E4M3, f32 = s.act_dtype == MOE_F32;
    const int64_t act = f32 ? 4 : 2;
    GemmArgs dn = base_args(s, ws, e_base);
    dn.A = (const uint8_t*)ws.h;
    dn.As = ws.hs;
    dn.lda = ws.inter_max * (fp8 ? 1 : act);
    dn.ldas = ws.inter_max / 128;
    dn.B1 = (const uint8_t*)W2;
    dn.B1s = W2s;
    // shared expert: S2 is [d, n_shared]
    dn.S1 = (const uint8_t*)S2;
    dn.S1s = S2s;
    dn.ld_s = n_shared;
    dn.nkb_s = n_shared / 128;
    dn.out = (uint8_t*)ws.y_rows;
    dn.ldo = s.d;
    dn.N_r = dn.N_s = (int)s.d;
    dn.K_r = (int)s.inter;
    dn.K_s = n_shared;
    dn.krot = KROT_DN;
    const int bm = tile_rows(s);
    // With at most one tile per expert on average no weight panel is shared between tiles: walk each
    // tile's n-blocks together instead, so its h rows are fetched once into L2.
    if (bm > 16 && s.T * s.k <= (int64_t)s.E * bm) dn.group_m = 1;
    else if (fp8 && bm > 16) dn.group_m = GROUP_M_F8_DN;
    // 256-wide n-blocks where d allows (d is a multiple of 128; an odd multiple takes 128-wide ones)
    const bool wide = s.d % 256 == 0;
    if (bm == 16) {
        dn.n_blocks = (int)(s.d / 64);
        if (fp8) launch_one<ET_FP8, false, true, 16, 64, 1, 4>(dn, stream);
        else if (f32) launch_one<ET_F32, false, false, 16, 64, 1, 4>(dn, stream);
        else if (s.d % SMALL_DN_BN == 0) {
            dn.n_blocks = (int)(s.d / SMALL_DN_BN);
            launch_one<ET_BF16, false, true, 16, SMALL_DN_BN, 1, SMALL_DN_WAVES, 2, SMALL_DN_MINW>(dn, stream);
        } else launch_one<ET_BF16, false, true, 16, 64, 1, 4>(dn, stream);
    } else if (fp8) {
        dn.n_blocks = (int)(s.d / (wide ? 256 : 128));
        if (bm == 128) wide ? launch_f8<false, 128, 256>(dn, stream) : launch_f8<false, 128, 128>(dn, stream);
        else wide ? launch_f8<false, 256, 256>(dn, stream) : launch_f8<false, 256, 128>(dn, stream);
    } else if (f32) {
        dn.n_blocks = (int)(s.d / 128);
        launch_one<ET_F32, false, false, 128, 128, 2, 2>(dn, stream);
    } else if (wide) {
        dn.n_blocks = (int)(s.d / 256);
        dn.krot = KROT_WDN;
        launch_w<false>(dn, stream);
    } else {
        dn.n_blocks = (int)(s.d / 128);
        launch_one<ET_BF16, false, true, 256, 128, 2, 2, 2, 1>(dn, stream);
    }
    return hipGetLastError();
}

}  // namespace moe
