/*
 * moe_oracle.c -- plain CPU oracle for one DeepSeek-V3-style mixture-of-experts feed-forward layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or load this file: only the
 * test suite, the smoke check and the benchmark's CPU-baseline leg do.  It shares no source, header,
 * table or helper with the HIP library; its bf16 and OCP-E4M3 converters are written here from the
 * IEEE-754 and OCP 8-bit floating point definitions.
 *
 * Sources (the pages this follows, cited by title and section):
 *   [P1] "DeepSeek-V3's mixture-of-experts architecture explained" (n4n.ai), "The architecture in one
 *        diagram", block pseudocode: router_logits = gate(x); (weights, indices) = topk(router_logits, 8);
 *        weights = softmax(weights) over the selected values only.
 *   [P5] "DeepSeek-V3.2-Exp / Mixture of experts / Shared expert" (atlas.klimoza.dev):
 *        - "All 5 steps": g = x W1, u = x W3, a = g sigma(g), h = a (.) u, y = h W2;
 *        - MLP forward excerpt: silu(w1(x).float()) * w3(x).float() is formed in fp32 and cast back to
 *          the activation dtype before w2;
 *        - MoE forward excerpt: y starts as an fp32 zero tensor; bincount of the indices; a loop over the
 *          experts in ascending order that skips empty ones; y[idx] += expert(x[idx]) * weights[idx, top];
 *          then y += shared_experts(x);
 *        - "Exact per-instance accounting": the three projections are 7168 x 2048 each.
 *
 * Readings taken where the pages are silent (each listed in the design notes):
 *   - logits: one fp32 fused-multiply-add chain per (token, expert), i ascending from +0.0f, then one
 *     fp32 add of an optional per-expert bias.  This fixes the rounding of every logit, so the routing
 *     decision (an integer) is taken in the same fp32 precision the router is specified in.
 *   - top-k order: descending logit, equal logits ordered by ascending expert index; +0 == -0.
 *   - softmax over the k selected logits, evaluated in fp64 from the fp32 logits, stored as fp32.
 *   - every linear (w1, w3, w2) accumulates in fp64 and rounds once to the activation dtype, as a
 *     bf16 linear returns bf16; silu(g)*u is formed in fp32 as the MLP excerpt states.
 *   - fp8 weights: (code, fp32 block scale) per 128x128 block define the weight; activations entering an
 *     fp8 linear are quantised per 1x128 group: s = amax/448 (fp32, s = 1 when amax = 0),
 *     q = e4m3_rne_saturating(v / s) with IEEE fp32 division.
 *
 * Precision: everything not fixed above is computed in fp64.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_F32 0
#define ORACLE_BF16 1
#define ORACLE_FP8_E4M3 2

/* ------------------------------------------------------------------------------------------------ */
/* bf16: IEEE-754 binary32 with the low 16 fraction bits dropped; round to nearest, ties to even.     */
/* ------------------------------------------------------------------------------------------------ */

static float f32_from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t bits_from_f32(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

float oracle_bf16_to_float(uint16_t b) { return f32_from_bits((uint32_t)b << 16); }

/* Round a double to the nearest bf16 value (ties to even), returned as a float (exact).  bf16 keeps
 * 8 significant bits; the smallest normal is 2^-126 and subnormals are multiples of 2^-133. */
float oracle_round_bf16_from_double(double v)
{
    if (v == 0.0 || isnan(v) || isinf(v)) return (float)v;
    int ex;
    frexp(v, &ex);                      /* |v| = m * 2^ex, m in [0.5, 1) */
    int q = ex - 8;                     /* quantum exponent for 8 significant bits */
    if (q < -133) q = -133;             /* subnormal quantum */
    double r = rint(ldexp(v, -q));      /* exact scaling, then round half to even */
    double out = ldexp(r, q);
    if (fabs(out) > 3.38953138925153547590470800371487866e38) return v > 0 ? INFINITY : -INFINITY;
    return (float)out;                  /* exact: out has at most 8 significant bits */
}

uint16_t oracle_bf16_bits_from_double(double v)
{
    return (uint16_t)(bits_from_f32(oracle_round_bf16_from_double(v)) >> 16);
}

/* ------------------------------------------------------------------------------------------------ */
/* OCP 8-bit floating point, E4M3 ("FN"): bias 7, no infinities, 0x7F/0xFF are NaN, max normal 448.   */
/* ------------------------------------------------------------------------------------------------ */

double oracle_e4m3_decode(uint8_t c)
{
    int sign = c >> 7, e = (c >> 3) & 15, m = c & 7;
    double mag;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) mag = ldexp((double)m, -9);                 /* subnormal: m * 2^-6 / 8 */
    else mag = ldexp(1.0 + m / 8.0, e - 7);
    return sign ? -mag : mag;
}

/* Round to the nearest E4M3 value, ties to even; magnitudes above 448 saturate to 448. */
uint8_t oracle_e4m3_encode(double v)
{
    if (isnan(v)) return 0x7F;
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double a = fabs(v);
    if (a > 448.0) return sign | 0x7E;
    if (a == 0.0) return sign;
    int ex;
    frexp(a, &ex);                      /* a = m * 2^ex, m in [0.5,1): unbiased exponent of a is ex-1 */
    int q = (ex - 1) - 3;               /* 4 significant bits */
    if (q < -9) q = -9;                 /* subnormal quantum 2^-9 */
    double r = ldexp(rint(ldexp(a, -q)), q);
    if (r == 0.0) return sign;
    if (r < ldexp(1.0, -6)) return sign | (uint8_t)ldexp(r, 9);      /* subnormal code 1..7 */
    int er;
    frexp(r, &er);
    int E = er - 1;                     /* r = 1.f * 2^E, -6 <= E <= 8 */
    int mant = (int)ldexp(r, 3 - E) - 8;                           /* (r / 2^E - 1) * 8 */
    return sign | (uint8_t)(((E + 7) << 3) | mant);
}

/* Quantise one group of n values (n <= 128) per the 1x128 activation rule; returns the scale. */
static float quantize_group(const float* v, int n, uint8_t* q)
{
    float amax = 0.0f;
    for (int i = 0; i < n; i++) {
        float a = fabsf(v[i]);
        if (a > amax) amax = a;
    }
    float s = amax > 0.0f ? amax / 448.0f : 1.0f;
    for (int i = 0; i < n; i++) q[i] = oracle_e4m3_encode((double)(v[i] / s));
    return s;
}

/* Quantise a [rows x cols] fp32 matrix per 1x128 group along each row; scales are [rows x cols/128]. */
int oracle_quantize_rows_e4m3(int64_t rows, int64_t cols, const float* v, uint8_t* q, float* s)
{
    if (cols % 128) return 1;
    for (int64_t r = 0; r < rows; r++)
        for (int64_t g = 0; g < cols / 128; g++)
            s[r * (cols / 128) + g] = quantize_group(v + r * cols + g * 128, 128, q + r * cols + g * 128);
    return 0;
}

/* ------------------------------------------------------------------------------------------------ */
/* Router [P1 block pseudocode]: logits = gate(x), topk(8), softmax over the selected values.          */
/* ------------------------------------------------------------------------------------------------ */

static float act_value(int act_dtype, const void* x, int64_t i)
{
    if (act_dtype == ORACLE_F32) return ((const float*)x)[i];
    return oracle_bf16_to_float(((const uint16_t*)x)[i]);
}

/* logits[t][e] = sum_i x[t][i] * Wg[e][i] as one fp32 FMA chain, i ascending, then + bias[e].  Wg is the
 * gate's nn.Linear(hidden, n_experts) weight, [E, d] [P1 block pseudocode: self.gate(x)]. */
int oracle_router_logits(int64_t T, int64_t d, int64_t E, int act_dtype, const void* x,
                         const float* Wg, const float* bias, float* logits)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; t++) {
        for (int64_t e = 0; e < E; e++) {
            float acc = 0.0f;
            for (int64_t i = 0; i < d; i++) acc = fmaf(act_value(act_dtype, x, t * d + i), Wg[e * d + i], acc);
            if (bias) acc = acc + bias[e];
            logits[t * E + e] = acc;
        }
    }
    return 0;
}

/* Does expert a rank above expert b?  Larger logit first; equal logits: lower index first. */
static int ranks_above(const float* L, int64_t a, int64_t b)
{
    return L[a] > L[b] || (L[a] == L[b] && a < b);
}

/* Top-k of one token's logits, in rank order, by repeatedly taking the best remaining expert. */
static void topk_one(const float* L, int64_t E, int64_t k, int32_t* idx)
{
    for (int64_t j = 0; j < k; j++) {
        int64_t best = -1;
        for (int64_t e = 0; e < E; e++) {
            int taken = 0;
            for (int64_t jj = 0; jj < j; jj++) taken |= (idx[jj] == e);
            if (taken) continue;
            if (best < 0 || ranks_above(L, e, best)) best = e;
        }
        idx[j] = (int32_t)best;
    }
}

/*
 * Group-limited top-k ["Technical Architecture and Core Innovations", "Architectural Breakthroughs", item 1,
 * "Hierarchical Dynamic Routing": tokens are first distributed over 8 expert groups by a softmax, then 2
 * experts per group are selected].  Reading (the one under which 2 experts per group agree with top-k):
 * the E experts form G groups of E / G consecutive experts; a group's candidates are its two best
 * experts (ranks_above); its score is the fp32 sum of their two logits; the k / 2 groups with the largest
 * scores are kept (a softmax over the group scores keeps their order), equal scores ordered by ascending
 * group index; the token's k experts are the kept groups' pairs, listed in rank order.
 */
static void topk_grouped_one(const float* L, int64_t E, int64_t k, int64_t G, int32_t* idx)
{
    const int64_t gs = E / G, keep = k / 2;
    int64_t first[64], second[64];
    float score[64];
    int kept[64];
    for (int64_t g = 0; g < G; g++) {
        int64_t a = -1, b = -1;
        for (int64_t e = g * gs; e < (g + 1) * gs; e++) {
            if (a < 0 || ranks_above(L, e, a)) {
                b = a;
                a = e;
            } else if (b < 0 || ranks_above(L, e, b)) {
                b = e;
            }
        }
        first[g] = a;
        second[g] = b;
        score[g] = L[a] + L[b];                                  /* one fp32 add */
        kept[g] = 0;
    }
    for (int64_t r = 0; r < keep; r++) {
        int64_t best = -1;
        for (int64_t g = 0; g < G; g++)
            if (!kept[g] && (best < 0 || score[g] > score[best])) best = g;   /* ties: the lower group */
        kept[best] = 1;
    }
    /* the kept pairs in rank order, by repeatedly taking the best remaining candidate */
    for (int64_t j = 0; j < k; j++) {
        int64_t best = -1;
        for (int64_t g = 0; g < G; g++) {
            if (!kept[g]) continue;
            const int64_t cand[2] = {first[g], second[g]};
            for (int c = 0; c < 2; c++) {
                int taken = 0;
                for (int64_t jj = 0; jj < j; jj++) taken |= (idx[jj] == cand[c]);
                if (!taken && (best < 0 || ranks_above(L, cand[c], best))) best = cand[c];
            }
        }
        idx[j] = (int32_t)best;
    }
}

/* Softmax over the k selected logits (fp64 from the fp32 logits; the max is the first one). */
static void softmax_selected(const float* L, const int32_t* idx, int64_t k, float* w)
{
    double m = L[idx[0]], z[64], sum = 0.0;
    for (int64_t j = 0; j < k; j++) {
        z[j] = exp((double)L[idx[j]] - m);
        sum += z[j];
    }
    for (int64_t j = 0; j < k; j++) w[j] = (float)(z[j] / sum);
}

/*
 * Routing artefacts [P5 MoE forward: bincount of the indices, torch.where(indices == i)]:
 *   counts[e]       number of (token, slot) pairs routed to e;
 *   offsets[e]      exclusive prefix sum of counts, offsets[E] = T*k;
 *   sorted_slots[p] slot ids s = t*k + j listed expert by expert, tokens ascending within an expert
 *                   (torch.where scans row-major);
 *   pos[s]          inverse: the position of slot s in sorted_slots.
 * Any output pointer may be NULL except idx and w.
 */
static int route_impl(int64_t T, int64_t d, int64_t E, int64_t k, int act_dtype, const void* x,
                      const float* Wg, const float* bias, const uint8_t* allowed, int64_t n_group, float* logits_out,
                      int32_t* idx, float* w, int32_t* counts, int32_t* offsets, int32_t* sorted_slots,
                      int32_t* pos)
{
    if (k < 1 || k > E || k > 64) return 1;
    /* group-limited: G groups of at least two experts, k even, k / 2 groups kept */
    if (n_group && (n_group < 1 || n_group > 64 || E % n_group || E / n_group < 2 || k % 2 || k / 2 > n_group))
        return 1;
    if (allowed) {   /* at least one allowed expert; with fewer than k, the rest come at -inf, weight 0 */
        int64_t n_allowed = 0;
        for (int64_t e = 0; e < E; e++) n_allowed += allowed[e] != 0;
        if (n_allowed < 1) return 1;
    }
    float* L = logits_out ? logits_out : (float*)malloc(sizeof(float) * (size_t)(T * E));
    if (!L) return 2;
    oracle_router_logits(T, d, E, act_dtype, x, Wg, bias, L);
    /* Device-limited routing ["DeepSeek-V3's mixture-of-experts architecture explained", "Why 256
     * experts with top-8 routing?", device_limited_routing]: a mask of -inf outside the allowed experts
     * and 0 inside is added to the logits before top-k. */
    if (allowed)
        for (int64_t t = 0; t < T; t++)
            for (int64_t e = 0; e < E; e++) L[t * E + e] = L[t * E + e] + (allowed[e] ? 0.0f : -INFINITY);
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; t++) {
        if (n_group) topk_grouped_one(L + t * E, E, k, n_group, idx + t * k);
        else topk_one(L + t * E, E, k, idx + t * k);
        softmax_selected(L + t * E, idx + t * k, k, w + t * k);
    }
    if (!logits_out) free(L);

    int32_t* c = counts ? counts : (int32_t*)calloc((size_t)E, sizeof(int32_t));
    if (!c) return 2;
    memset(c, 0, sizeof(int32_t) * (size_t)E);
    for (int64_t s = 0; s < T * k; s++) c[idx[s]]++;
    if (offsets) {
        offsets[0] = 0;
        for (int64_t e = 0; e < E; e++) offsets[e + 1] = offsets[e] + c[e];
    }
    if (sorted_slots || pos) {
        int64_t p = 0;
        for (int64_t e = 0; e < E; e++)
            for (int64_t t = 0; t < T; t++)
                for (int64_t j = 0; j < k; j++)
                    if (idx[t * k + j] == e) {
                        if (sorted_slots) sorted_slots[p] = (int32_t)(t * k + j);
                        if (pos) pos[t * k + j] = (int32_t)p;
                        p++;
                    }
    }
    if (!counts) free(c);
    return 0;
}

int oracle_route(int64_t T, int64_t d, int64_t E, int64_t k, int act_dtype, const void* x,
                 const float* Wg, const float* bias, float* logits_out, int32_t* idx, float* w,
                 int32_t* counts, int32_t* offsets, int32_t* sorted_slots, int32_t* pos)
{
    return route_impl(T, d, E, k, act_dtype, x, Wg, bias, NULL, 0, logits_out, idx, w, counts, offsets,
                      sorted_slots, pos);
}

/* Group-limited routing (topk_grouped_one) over n_group groups. */
int oracle_route_grouped(int64_t T, int64_t d, int64_t E, int64_t k, int64_t n_group, int act_dtype, const void* x,
                         const float* Wg, const float* bias, float* logits_out, int32_t* idx, float* w,
                         int32_t* counts, int32_t* offsets, int32_t* sorted_slots, int32_t* pos)
{
    if (n_group < 1) return 1;
    return route_impl(T, d, E, k, act_dtype, x, Wg, bias, NULL, n_group, logits_out, idx, w, counts, offsets,
                      sorted_slots, pos);
}

/* Routing restricted to the experts with allowed[e] != 0 (at least one of them). */
int oracle_route_limited(int64_t T, int64_t d, int64_t E, int64_t k, int act_dtype, const void* x,
                         const float* Wg, const float* bias, const uint8_t* allowed, float* logits_out,
                         int32_t* idx, float* w, int32_t* counts, int32_t* offsets, int32_t* sorted_slots,
                         int32_t* pos)
{
    return route_impl(T, d, E, k, act_dtype, x, Wg, bias, allowed, 0, logits_out, idx, w, counts, offsets,
                      sorted_slots, pos);
}

/*
 * Expert utilisation ["DeepSeek-V3's mixture-of-experts architecture explained", "Where the
 * architecture struggles", log_expert_utilization]: utilization = counts.float() / counts.sum() (fp32
 * division), with an alert for experts above 2x or below 0.1x the mean utilisation 1/E.  The alert
 * thresholds are taken on the exact rationals: over <=> counts[e] * E > 2 * total,
 * under <=> 10 * counts[e] * E < total.  flags[e] = +1 over, -1 under, 0 otherwise; summary = (#over,
 * #under).
 */
int oracle_expert_utilization(int64_t E, const int32_t* counts, float* util, int32_t* flags, int32_t* summary)
{
    int64_t total = 0;
    for (int64_t e = 0; e < E; e++) total += counts[e];
    int32_t n_over = 0, n_under = 0;
    for (int64_t e = 0; e < E; e++) {
        util[e] = total > 0 ? (float)counts[e] / (float)total : 0.0f;
        const int64_t c = counts[e];
        const int over = total > 0 && c * E > 2 * total, under = total > 0 && 10 * c * E < total;
        flags[e] = over ? 1 : under ? -1 : 0;
        n_over += over;
        n_under += under;
    }
    summary[0] = n_over;
    summary[1] = n_under;
    return 0;
}

/* ------------------------------------------------------------------------------------------------ */
/* Experts [P5 "All 5 steps" and MLP forward].                                                         */
/* ------------------------------------------------------------------------------------------------ */

typedef struct {
    int64_t T, d, E, k, inter, inter_shared;
    int32_t act_dtype, w_dtype;
} oracle_shape_t;

/* One SwiGLU weight set: W1, W3 are [.][d] and W2 is [d][ld2] (nn.Linear [out][in]).  The expert uses
 * the n_inter hidden features starting at row0 of W1/W3 and column row0 of W2 (a tensor-parallel
 * slice of a wider expert; row0 = 0 and ld2 = n_inter for a whole expert). */
typedef struct {
    const void* w1; const void* w3; const void* w2;
    const float* s1; const float* s3; const float* s2;   /* fp8 block scales, else NULL */
    int64_t n_inter;
    int64_t row0, ld2;
} swiglu_weights_t;

/* Values of all 256 E4M3 codes, filled from oracle_e4m3_decode before any parallel region. */
static double e4m3_value[256];
static void fill_e4m3_values(void)
{
    for (int c = 0; c < 256; c++) e4m3_value[c] = oracle_e4m3_decode((uint8_t)c);
}

/* The exact real value of weight element (r, c) of a [rows][cols] matrix. */
static inline double weight_value(int w_dtype, const void* W, const float* S, int64_t cols, int64_t r, int64_t c)
{
    if (w_dtype == ORACLE_F32) return ((const float*)W)[r * cols + c];
    if (w_dtype == ORACLE_BF16) return oracle_bf16_to_float(((const uint16_t*)W)[r * cols + c]);
    return e4m3_value[((const uint8_t*)W)[r * cols + c]] * (double)S[(r / 128) * (cols / 128) + c / 128];
}

/* Round a value to the activation dtype (fp32 or bf16), returned as float. */
static float round_act(int act_dtype, double v)
{
    return act_dtype == ORACLE_F32 ? (float)v : oracle_round_bf16_from_double(v);
}
static float round_act_f(int act_dtype, float v)
{
    return act_dtype == ORACLE_F32 ? v : oracle_round_bf16_from_double((double)v);
}

/* The value an fp8 linear sees for an activation row: per-128-group quantise-dequantise. */
static void fp8_activation_view(const float* v, int64_t n, double* out)
{
    uint8_t q[128];
    for (int64_t g = 0; g < n / 128; g++) {
        float s = quantize_group(v + g * 128, 128, q);
        for (int i = 0; i < 128; i++) out[g * 128 + i] = e4m3_value[q[i]] * (double)s;
    }
}

/* Columns [c0, c0 + n) of row r of a [rows][cols] weight matrix as exact fp64 values. */
static void weight_row(int w_dtype, const void* W, const float* S, int64_t cols, int64_t r, int64_t c0, int64_t n,
                       double* out)
{
    for (int64_t c = 0; c < n; c++) out[c] = weight_value(w_dtype, W, S, cols, r, c0 + c);
}

static double dot(const double* a, const double* b, int64_t n)
{
    double acc = 0.0;
    for (int64_t i = 0; i < n; i++) acc += a[i] * b[i];
    return acc;
}

/* y_out[m] (activation dtype, as float) = SwiGLU of one token row xv (activation values, length d). */
static void swiglu_row(const oracle_shape_t* sh, const swiglu_weights_t* W, const float* xv, float* y_out)
{
    const int64_t d = sh->d, n_inter = W->n_inter;
    const int fp8 = sh->w_dtype == ORACLE_FP8_E4M3;
    double* xin = (double*)malloc(sizeof(double) * (size_t)d);
    double* row1 = (double*)malloc(sizeof(double) * (size_t)(d > n_inter ? d : n_inter));
    double* row3 = (double*)malloc(sizeof(double) * (size_t)d);
    float* h = (float*)malloc(sizeof(float) * (size_t)n_inter);
    double* hin = (double*)malloc(sizeof(double) * (size_t)n_inter);

    if (fp8) fp8_activation_view(xv, d, xin);
    else for (int64_t i = 0; i < d; i++) xin[i] = xv[i];

    for (int64_t n = 0; n < n_inter; n++) {
        weight_row(sh->w_dtype, W->w1, W->s1, d, W->row0 + n, 0, d, row1);
        weight_row(sh->w_dtype, W->w3, W->s3, d, W->row0 + n, 0, d, row3);
        float g = round_act(sh->act_dtype, dot(xin, row1, d));      /* g = x W1 */
        float u = round_act(sh->act_dtype, dot(xin, row3, d));      /* u = x W3 */
        float sig = 1.0f / (1.0f + expf(-g));                        /* sigma(g), fp32 */
        float a = g * sig;                                           /* a = g sigma(g) */
        h[n] = round_act_f(sh->act_dtype, a * u);                    /* h = a (.) u, cast back */
    }

    if (fp8) fp8_activation_view(h, n_inter, hin);
    else for (int64_t n = 0; n < n_inter; n++) hin[n] = h[n];

    for (int64_t m = 0; m < d; m++) {                                /* y = h W2 */
        weight_row(sh->w_dtype, W->w2, W->s2, W->ld2, m, W->row0, n_inter, row1);
        y_out[m] = round_act(sh->act_dtype, dot(hin, row1, n_inter));
    }
    free(xin); free(row1); free(row3); free(h); free(hin);
}

static size_t w_elem_bytes(int w_dtype) { return w_dtype == ORACLE_F32 ? 4 : w_dtype == ORACLE_BF16 ? 2 : 1; }

/*
 * Layer output for a list of tokens [P5 MoE forward]:
 *   acc = 0 (fp32); for each expert e ascending that token t selected (slot j):
 *       acc += float(expert_e(x[t]) * w[t][j]);
 *   acc += shared(x[t]);  y[t] = acc rounded to the activation dtype.
 * No residual is added: the residual belongs to the transformer block, not to this layer.
 * tokens: n_tok token ids (a sample, or all T); out_f32 and y are [n_tok][d].
 * idx, w: the [T][k] routing from oracle_route.
 */
int oracle_forward(const oracle_shape_t* sh, const void* x,
                   const void* W1, const void* W3, const void* W2,
                   const float* W1s, const float* W3s, const float* W2s,
                   const void* S1, const void* S3, const void* S2,
                   const float* S1s, const float* S3s, const float* S2s,
                   const int32_t* idx, const float* w,
                   int64_t n_tok, const int32_t* tokens, float* out_f32, void* y)
{
    const int64_t d = sh->d, E = sh->E, k = sh->k, inter = sh->inter;
    const int fp8 = sh->w_dtype == ORACLE_FP8_E4M3;
    if (fp8 && (d % 128 || inter % 128 || sh->inter_shared % 128)) return 1;
    if (!fp8 && sh->w_dtype != sh->act_dtype) return 1;
    const size_t eb = w_elem_bytes(sh->w_dtype);
    const int64_t nb_in = d / 128, nb_mid = inter / 128;   /* fp8 block counts */
    fill_e4m3_values();

#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < n_tok; r++) {
        const int64_t t = tokens[r];
        float* xv = (float*)malloc(sizeof(float) * (size_t)d);
        float* ye = (float*)malloc(sizeof(float) * (size_t)d);
        float* acc = out_f32 + r * d;
        for (int64_t i = 0; i < d; i++) xv[i] = act_value(sh->act_dtype, x, t * d + i);
        for (int64_t m = 0; m < d; m++) acc[m] = 0.0f;

        for (int64_t e = 0; e < E; e++) {
            int64_t j = -1;
            for (int64_t jj = 0; jj < k; jj++) if (idx[t * k + jj] == e) j = jj;
            if (j < 0) continue;
            swiglu_weights_t we = {
                (const char*)W1 + (size_t)e * inter * d * eb,
                (const char*)W3 + (size_t)e * inter * d * eb,
                (const char*)W2 + (size_t)e * d * inter * eb,
                fp8 ? W1s + e * nb_mid * nb_in : NULL,
                fp8 ? W3s + e * nb_mid * nb_in : NULL,
                fp8 ? W2s + e * nb_in * nb_mid : NULL,
                inter, 0, inter};
            swiglu_row(sh, &we, xv, ye);
            const float wj = w[t * k + j];
            for (int64_t m = 0; m < d; m++) {
                float p = ye[m] * wj;            /* expert(x) * weight, fp32 */
                acc[m] = acc[m] + p;
            }
        }
        swiglu_weights_t ws = {S1, S3, S2, S1s, S3s, S2s, sh->inter_shared, 0, sh->inter_shared};
        swiglu_row(sh, &ws, xv, ye);
        for (int64_t m = 0; m < d; m++) acc[m] = acc[m] + ye[m];

        for (int64_t m = 0; m < d; m++) {
            if (sh->act_dtype == ORACLE_F32) ((float*)y)[r * d + m] = acc[m];
            else ((uint16_t*)y)[r * d + m] = oracle_bf16_bits_from_double((double)acc[m]);
        }
        free(xv); free(ye);
    }
    return 0;
}

/*
 * One expert-parallel rank's share of the layer [P5 MoE __init__/forward: the rank owns experts
 * [experts_start_idx, experts_end_idx) and a slice of the shared expert built with
 * reduce_output=False; the fp32 partial y is what dist.all_reduce(y) sums over ranks]:
 *   partial[t] = sum over the token's experts e in [e0, e1), ascending, of float(expert_e(x[t]) * w)
 *              + (if s0 < s1) the shared expert's hidden features [s0, s1): its W2 partial product
 *                rounded to the activation dtype, as a row-parallel linear returns it;
 * no final rounding.  With e0 = 0, e1 = E, s0 = 0, s1 = inter_shared this is oracle_forward's fp32 out.
 */
int oracle_forward_shard(const oracle_shape_t* sh, const void* x,
                         const void* W1, const void* W3, const void* W2,
                         const float* W1s, const float* W3s, const float* W2s,
                         const void* S1, const void* S3, const void* S2,
                         const float* S1s, const float* S3s, const float* S2s,
                         const int32_t* idx, const float* w, int64_t e0, int64_t e1, int64_t s0, int64_t s1,
                         int64_t n_tok, const int32_t* tokens, float* partial)
{
    const int64_t d = sh->d, E = sh->E, k = sh->k, inter = sh->inter, is = sh->inter_shared;
    const int fp8 = sh->w_dtype == ORACLE_FP8_E4M3;
    if (fp8 && (d % 128 || inter % 128 || is % 128 || s0 % 128 || s1 % 128)) return 1;
    if (!fp8 && sh->w_dtype != sh->act_dtype) return 1;
    if (e0 < 0 || e1 > E || e0 > e1 || s0 < 0 || s1 > is || s0 > s1) return 1;
    const size_t eb = w_elem_bytes(sh->w_dtype);
    const int64_t nb_in = d / 128, nb_mid = inter / 128;
    fill_e4m3_values();

#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < n_tok; r++) {
        const int64_t t = tokens[r];
        float* xv = (float*)malloc(sizeof(float) * (size_t)d);
        float* ye = (float*)malloc(sizeof(float) * (size_t)d);
        float* acc = partial + r * d;
        for (int64_t i = 0; i < d; i++) xv[i] = act_value(sh->act_dtype, x, t * d + i);
        for (int64_t m = 0; m < d; m++) acc[m] = 0.0f;
        for (int64_t e = e0; e < e1; e++) {
            int64_t j = -1;
            for (int64_t jj = 0; jj < k; jj++) if (idx[t * k + jj] == e) j = jj;
            if (j < 0) continue;
            swiglu_weights_t we = {
                (const char*)W1 + (size_t)e * inter * d * eb,
                (const char*)W3 + (size_t)e * inter * d * eb,
                (const char*)W2 + (size_t)e * d * inter * eb,
                fp8 ? W1s + e * nb_mid * nb_in : NULL,
                fp8 ? W3s + e * nb_mid * nb_in : NULL,
                fp8 ? W2s + e * nb_in * nb_mid : NULL,
                inter, 0, inter};
            swiglu_row(sh, &we, xv, ye);
            const float wj = w[t * k + j];
            for (int64_t m = 0; m < d; m++) {
                float p = ye[m] * wj;
                acc[m] = acc[m] + p;
            }
        }
        if (s0 < s1) {
            swiglu_weights_t ws = {S1, S3, S2, S1s, S3s, S2s, s1 - s0, s0, is};
            swiglu_row(sh, &ws, xv, ye);
            for (int64_t m = 0; m < d; m++) acc[m] = acc[m] + ye[m];
        }
        free(xv); free(ye);
    }
    return 0;
}

/* One SwiGLU expert applied to rows of activations, exposed for the dense-reduction check. */
int oracle_swiglu_rows(const oracle_shape_t* sh, const void* w1, const void* w3, const void* w2,
                       const float* s1, const float* s3, const float* s2, int64_t n_inter,
                       int64_t rows, const float* xv, float* y)
{
    swiglu_weights_t W = {w1, w3, w2, s1, s3, s2, n_inter, 0, n_inter};
    fill_e4m3_values();
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < rows; r++) swiglu_row(sh, &W, xv + r * sh->d, y + r * sh->d);
    return 0;
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}
