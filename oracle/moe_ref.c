/*
 * moe_ref.c -- CPU oracle for the fused MoE expert layer (TEST INFRASTRUCTURE;
 * never linked or called by the product library).
 *
 * Plain loops, written as the definitions read.  OpenMP splits only the
 * outermost loop over independent rows/tokens; it changes no arithmetic.
 * Built with gcc -O2 -fopenmp -ffp-contract=off -fno-fast-math so that every
 * fp32 operation written here is one IEEE operation (fmaf only where written).
 *
 * Page references are to the vLLM pull-request pages named in moe_ref.h.
 */
#include "moe_ref.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define GROUP 128

static uint32_t f32_bits(float v) { uint32_t u; memcpy(&u, &v, 4); return u; }
static float bits_f32(uint32_t u) { float v; memcpy(&v, &u, 4); return v; }

/* ======================================================================== *
 * Numerics.  bf16 and OCP E4M3FN (the float8_e4m3fn dtype PR #20903 profiles
 * with, Optimizations) are defined as "nearest representable value, ties to
 * the even significand"; E4M3FN saturates at +-448 before rounding.
 * ======================================================================== */

float moe_ref_f32_from_bf16(uint16_t b) { return bits_f32((uint32_t)b << 16); }

/* fp32 -> bf16: pick the nearer of the two bf16 neighbours of v; on a tie the
 * one whose last significand bit is 0.  The two neighbours are v with its low
 * 16 bits cleared (toward zero) and the next bf16 away from zero (which is
 * +-inf past the largest finite bf16, so overflow rounds to inf). */
uint16_t moe_ref_bf16_from_f32(float v) {
    uint32_t u = f32_bits(v);
    if (isnan(v)) return (uint16_t)((u >> 16) | 0x0040u);
    if (isinf(v)) return (uint16_t)(u >> 16);
    uint32_t lo_bits = u & 0xFFFF0000u;
    uint32_t hi_bits = lo_bits + 0x00010000u;
    double dv = (double)v;
    double lo = (double)bits_f32(lo_bits);
    double hi = (double)bits_f32(hi_bits);   /* may be +-inf */
    /* past the largest finite bf16 the upper neighbour is +-2^128, which
     * stands for infinity as in IEEE overflow rounding */
    if (isinf(hi)) hi = copysign(ldexp(1.0, 128), dv);
    double d_lo = fabs(dv - lo);
    double d_hi = fabs(hi - dv);
    uint32_t pick;
    if (d_lo < d_hi) pick = lo_bits;
    else if (d_hi < d_lo) pick = hi_bits;
    else pick = ((lo_bits >> 16) & 1u) ? hi_bits : lo_bits;
    return (uint16_t)(pick >> 16);
}

/* double -> bf16 with a single rounding: 8 significant bits, nearest, ties
 * to even; the bf16 exponent range is fp32's (subnormal step 2^-133). */
uint16_t moe_ref_bf16_from_f64(double v) {
    if (isnan(v)) return 0x7FC0u;
    if (v == 0.0) return signbit(v) ? 0x8000u : 0x0000u;
    double a = fabs(v);
    double r;
    if (a < ldexp(1.0, -126)) {
        r = nearbyint(a / ldexp(1.0, -133)) * ldexp(1.0, -133);
    } else {
        int e;
        frexp(a, &e);                 /* a = f * 2^e, f in [0.5, 1) */
        double step = ldexp(1.0, e - 8);
        r = nearbyint(a / step) * step;
    }
    float f = (r >= ldexp(1.0, 128)) ? INFINITY : (float)r;  /* exact if finite */
    if (signbit(v)) f = -f;
    return (uint16_t)(f32_bits(f) >> 16);
}

/* exact value of an E4M3FN code: sign, 4-bit exponent (bias 7), 3-bit
 * mantissa; exponent 0 is subnormal (m * 2^-9); S.1111.111 is NaN. */
double moe_ref_e4m3_value(uint8_t q) {
    int s = q >> 7, E = (q >> 3) & 15, m = q & 7;
    double v;
    if (E == 15 && m == 7) return NAN;
    if (E == 0) v = ldexp((double)m, -9);
    else v = ldexp((double)(8 + m), E - 10);
    return s ? -v : v;
}

/* fp32 -> E4M3FN: NaN -> 0x7F with the sign; otherwise clamp to [-448, 448]
 * and round |v| to the nearest multiple of the E4M3 spacing at its binade
 * (2^-9 below 2^-6, else 2^(e-3) for |v| in [2^e, 2^(e+1))), ties to even. */
uint8_t moe_ref_e4m3_from_f32(float v) {
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    if (isnan(v)) return (uint8_t)(0x7F | sign);
    double a = fabs((double)v);
    if (a > 448.0) a = 448.0;
    if (a < ldexp(1.0, -6)) {
        double r = nearbyint(a / ldexp(1.0, -9));   /* 0..8; 8 is 2^-6 = code 0x08 */
        return (uint8_t)(sign | (uint8_t)r);
    }
    int x;
    frexp(a, &x);           /* a = f * 2^x, f in [0.5,1): binade e = x - 1 */
    int e = x - 1;
    double r = nearbyint(a / ldexp(1.0, e - 3));    /* 8..16 */
    if (r == 16.0) { e += 1; r = 8.0; }
    return (uint8_t)(sign | (uint8_t)(((e + 7) << 3) | ((int)r - 8)));
}

/* exp(x) for SiLU, pinned step by step so that a GPU can reproduce it bit
 * for bit: Cody-Waite reduction x = n*ln2 + r with a two-part ln2, then the
 * degree-7 Taylor polynomial of exp(r) by Horner's rule, then scale by 2^n.
 * Constants: fp32(1/ln2); ln2 cut to 16 significant bits; fp32 of the
 * remainder; fp32(1/k!) for k = 0..7. */
float moe_ref_exp_spec(float x) {
    const float L2E = bits_f32(0x3fb8aa3bu);
    const float LN2_HI = bits_f32(0x3f317200u);
    const float LN2_LO = bits_f32(0x35bfbe8eu);
    const uint32_t C[8] = {0x3f800000u, 0x3f800000u, 0x3f000000u, 0x3e2aaaabu,
                           0x3d2aaaabu, 0x3c088889u, 0x3ab60b61u, 0x39500d01u};
    float xc = fminf(fmaxf(x, -86.0f), 88.0f);
    float t = xc * L2E;
    float n = rintf(t);
    float r = fmaf(-n, LN2_HI, xc);
    r = fmaf(-n, LN2_LO, r);
    float p = bits_f32(C[7]);
    for (int i = 6; i >= 0; --i) p = fmaf(p, r, bits_f32(C[i]));
    return ldexpf(p, (int)n);
}

/* One 1x128 group: amax = the largest non-NaN |v| (quiet and signalling
 * NaNs alike are skipped), d = max(amax, 1e-10),
 * scale s = d/448, codes e4m3(v * (448/d)).  Reading: fp8 per-128-group
 * activation scales as in PR #20903 (Optimizations, block 128). */
void moe_ref_quant_group(const float* v, uint8_t* q, float* s) {
    float amax = 0.0f;
    for (int i = 0; i < GROUP; ++i) {
        float a = fabsf(v[i]);
        if (a > amax) amax = a;   /* false for NaN */
    }
    float d = fmaxf(amax, 1e-10f);
    float scale = d / 448.0f;
    float inv = 448.0f / d;
    for (int i = 0; i < GROUP; ++i) {
        float t = v[i] * inv;
        q[i] = moe_ref_e4m3_from_f32(t);
    }
    *s = scale;
}

int moe_ref_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ======================================================================== *
 * Routing bookkeeping.
 * ======================================================================== */

/* Local expert of a global id: -1 for the "not routed here" id -1, for ids
 * outside [0, Eg), and for ids the expert map sends to -1 (non-local
 * experts, PR #20392 review: count over topk_ids with local_num_experts and
 * expert_map).  With no map, ids are local iff < El. */
int moe_ref_loc(int32_t id, const int32_t* expert_map, int32_t Eg, int32_t El) {
    if (id < 0 || id >= Eg) return -1;
    int e = expert_map ? expert_map[id] : id;
    if (e < 0 || e >= El) return -1;
    return e;
}

static int id_invalid(int32_t id, int32_t Eg) { return id < -1 || id >= Eg; }

/* counts[e] = number of (token, k) pairs whose id is local expert e
 * (count_expert_num_tokens, PR #20392 Purpose, Bug 2).  invalid_ids (if
 * given) receives the number of ids outside [-1, Eg). */
int moe_ref_count(const int32_t* topk_ids, int64_t num_pairs, const int32_t* expert_map,
                  int32_t Eg, int32_t El, int32_t* counts, int32_t* invalid_ids) {
    if (!topk_ids && num_pairs > 0) return MOE_REF_ERR_ARG;
    if (!counts || Eg <= 0 || El <= 0 || num_pairs < 0) return MOE_REF_ERR_ARG;
    if (!expert_map && El > Eg) return MOE_REF_ERR_ARG;
    for (int e = 0; e < El; ++e) counts[e] = 0;
    int32_t bad = 0;
    for (int64_t f = 0; f < num_pairs; ++f) {
        int e = moe_ref_loc(topk_ids[f], expert_map, Eg, El);
        if (e >= 0) counts[e] += 1;
        if (id_invalid(topk_ids[f], Eg)) bad += 1;
    }
    if (invalid_ids) *invalid_ids = bad;
    return MOE_REF_OK;
}

static int64_t ceil_div64(int64_t a, int64_t b) { return (a + b - 1) / b; }

/* An upper bound on the padded row count that holds for any routing: at
 * most Mc*topk local pairs, and each nonempty expert adds at most align-1
 * padding rows. */
int64_t moe_ref_max_rows(int64_t Mc, int32_t topk, int32_t El, int32_t align) {
    int64_t p = Mc * (int64_t)topk;
    int64_t ne = p < El ? p : El;
    return p + ne * (int64_t)(align - 1);
}

/* ======================================================================== *
 * Activation quantisation (prepare side).  Each row of n values (n a
 * multiple of 128) splits into n/128 groups quantised independently.
 * ======================================================================== */
int moe_ref_act_quant_identity(const uint16_t* x, int64_t rows, int32_t n, uint8_t* q, float* q_s) {
    if (n <= 0 || n % GROUP || rows < 0) return MOE_REF_ERR_SHAPE;
    int ng = n / GROUP;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        float v[GROUP];
        for (int g = 0; g < ng; ++g) {
            for (int i = 0; i < GROUP; ++i) v[i] = moe_ref_f32_from_bf16(x[r * n + g * GROUP + i]);
            moe_ref_quant_group(v, q + r * n + g * GROUP, q_s + r * ng + g);
        }
    }
    return MOE_REF_OK;
}

/* ======================================================================== *
 * Permute (the ep_scatter of PR #20903, Purpose item 2).
 *  - expert_offsets[e+1] = expert_offsets[e] + align*ceil(counts[e]/align)
 *  - pairs visited in flat order f = t*topk + k; a local pair of expert e
 *    takes the next free row of e's segment (stable order by f)
 *  - a_perm[row] = a_q[t], a_perm_s[row] = a_s[t] (times the pair's router
 *    weight when it is applied on the input, PR #20725 Purpose/Changes)
 *  - inv_perm[t,k] = row or -1; row_src[row] = t, -1 for padding and for
 *    rows past the last segment.  Padding rows of a_perm/a_perm_s are 0.
 * ======================================================================== */
int moe_ref_permute(const uint8_t* a_q, const float* a_s, const int32_t* topk_ids,
                    const float* topk_weights, int32_t apply_on_input, int64_t Mc, int32_t K,
                    int32_t topk, const int32_t* expert_map, int32_t Eg, int32_t El, int32_t align,
                    int64_t cap_rows, uint8_t* a_perm, float* a_perm_s, int32_t* counts,
                    int32_t* expert_offsets, int32_t* inv_perm, int32_t* row_src) {
    if (K <= 0 || K % GROUP || topk <= 0 || Mc < 0) return MOE_REF_ERR_SHAPE;
    if (!(align == 16 || align == 32 || align == 64 || align == 128)) return MOE_REF_ERR_SHAPE;
    if (apply_on_input && !topk_weights) return MOE_REF_ERR_ARG;
    if (cap_rows < moe_ref_max_rows(Mc, topk, El, align)) return MOE_REF_ERR_CAPACITY;
    int kg = K / GROUP;
    int rc = moe_ref_count(topk_ids, Mc * topk, expert_map, Eg, El, counts, NULL);
    if (rc) return rc;
    expert_offsets[0] = 0;
    for (int e = 0; e < El; ++e)
        expert_offsets[e + 1] = expert_offsets[e] + (int32_t)(align * ceil_div64(counts[e], align));
    for (int64_t r = 0; r < cap_rows; ++r) row_src[r] = -1;
    memset(a_perm, 0, (size_t)cap_rows * K);
    memset(a_perm_s, 0, (size_t)cap_rows * kg * sizeof(float));
    int32_t* fill = (int32_t*)calloc((size_t)El, sizeof(int32_t));
    if (!fill) return MOE_REF_ERR_ARG;
    for (int64_t t = 0; t < Mc; ++t) {
        for (int k = 0; k < topk; ++k) {
            int64_t f = t * topk + k;
            int e = moe_ref_loc(topk_ids[f], expert_map, Eg, El);
            if (e < 0) { inv_perm[f] = -1; continue; }
            int32_t row = expert_offsets[e] + fill[e];
            fill[e] += 1;
            inv_perm[f] = row;
            row_src[row] = (int32_t)t;
            memcpy(a_perm + (int64_t)row * K, a_q + t * K, (size_t)K);
            for (int g = 0; g < kg; ++g) {
                float s = a_s[t * kg + g];
                if (apply_on_input) s = s * topk_weights[f];
                a_perm_s[(int64_t)row * kg + g] = s;
            }
        }
    }
    free(fill);
    return MOE_REF_OK;
}

/* ======================================================================== *
 * Block-scaled fp8 GEMM, one row at a time (the DeepGEMM grouped GEMM of PR
 * #20903, Optimizations: e4m3 with 128x128 blocks):
 *   out[r,n] = bf16( sum_g a_s[r,g] * w_s[e, n/128, g] * S_g ),
 *   S_g = sum_{k in group g} e4m3(a[r,k]) * e4m3(w[e,n,k]).
 * Every e4m3 value is an integer multiple of 2^-9 below 2^9 in magnitude,
 * so S_g is exact in double; the scaled sum is formed in double and rounded
 * once to bf16.
 * ======================================================================== */
int moe_ref_gemm_rows(const uint8_t* a, const float* a_s, const int32_t* row_expert, int64_t rows,
                      const uint8_t* w, const float* w_s, int32_t El, int32_t n_out, int32_t k_in,
                      uint16_t* out) {
    if (n_out <= 0 || k_in <= 0 || n_out % GROUP || k_in % GROUP) return MOE_REF_ERR_SHAPE;
    for (int64_t r = 0; r < rows; ++r)
        if (row_expert[r] < 0 || row_expert[r] >= El) return MOE_REF_ERR_ARG;
    double dec[256];
    for (int c = 0; c < 256; ++c) dec[c] = moe_ref_e4m3_value((uint8_t)c);
    int kg = k_in / GROUP, ng = n_out / GROUP;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < rows; ++r) {
        int e = row_expert[r];
        const uint8_t* ar = a + r * k_in;
        for (int n = 0; n < n_out; ++n) {
            const uint8_t* wr = w + ((int64_t)e * n_out + n) * k_in;
            double acc = 0.0;
            for (int g = 0; g < kg; ++g) {
                double S = 0.0;
                for (int k = g * GROUP; k < (g + 1) * GROUP; ++k) S += dec[ar[k]] * dec[wr[k]];
                double sc = (double)a_s[r * kg + g] * (double)w_s[((int64_t)e * ng + n / GROUP) * kg + g];
                acc += sc * S;
            }
            out[r * n_out + n] = moe_ref_bf16_from_f64(acc);
        }
    }
    return MOE_REF_OK;
}

/* Grouped form: rows [off[e], off[e]+counts[e]) belong to expert e; every
 * other row of out (padding) is written as 0. */
int moe_ref_grouped_gemm(const uint8_t* a, const float* a_s, const uint8_t* w, const float* w_s,
                         const int32_t* expert_offsets, const int32_t* counts, int32_t El,
                         int64_t cap_rows, int32_t n_out, int32_t k_in, uint16_t* out) {
    if (n_out <= 0 || k_in <= 0 || n_out % GROUP || k_in % GROUP) return MOE_REF_ERR_SHAPE;
    if (expert_offsets[El] > cap_rows) return MOE_REF_ERR_CAPACITY;
    memset(out, 0, (size_t)cap_rows * n_out * sizeof(uint16_t));
    for (int e = 0; e < El; ++e) {
        int64_t r0 = expert_offsets[e], c = counts[e];
        if (c <= 0) continue;
        if (r0 + c > expert_offsets[e + 1]) return MOE_REF_ERR_ARG;
        int32_t* ex = (int32_t*)malloc((size_t)c * sizeof(int32_t));
        if (!ex) return MOE_REF_ERR_ARG;
        for (int64_t i = 0; i < c; ++i) ex[i] = e;
        int rc = moe_ref_gemm_rows(a + r0 * k_in, a_s + r0 * (k_in / GROUP), ex, c, w, w_s, El,
                                   n_out, k_in, out + r0 * n_out);
        free(ex);
        if (rc) return rc;
    }
    return MOE_REF_OK;
}

/* ======================================================================== *
 * SiLU-and-mul with per-token-group fp8 requant (between the two grouped
 * GEMMs).  Reading: columns [0, n) of h are the gate, [n, 2n) the up
 * projection; act = bf16(silu(gate) * up) with silu(g) = g / (1 + exp(-g)),
 * then act is quantised per 1x128 group like the input.  Only valid rows
 * (off[e] <= r < off[e]+counts[e]) are written; others are zeroed.
 * ======================================================================== */
int moe_ref_silu_mul_quant(const uint16_t* h, int64_t rows, int32_t n, const int32_t* expert_offsets,
                           const int32_t* counts, int32_t El, uint8_t* q, float* q_s) {
    if (n <= 0 || n % GROUP || rows < 0) return MOE_REF_ERR_SHAPE;
    int ng = n / GROUP;
    memset(q, 0, (size_t)rows * n);
    memset(q_s, 0, (size_t)rows * ng * sizeof(float));
    char* valid = (char*)calloc((size_t)(rows > 0 ? rows : 1), 1);
    if (!valid) return MOE_REF_ERR_ARG;
    if (expert_offsets) {
        for (int e = 0; e < El; ++e)
            for (int64_t r = expert_offsets[e]; r < (int64_t)expert_offsets[e] + counts[e] && r < rows; ++r)
                valid[r] = 1;
    } else {
        memset(valid, 1, (size_t)rows);
    }
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        if (!valid[r]) continue;
        float act[GROUP];
        for (int g = 0; g < ng; ++g) {
            for (int i = 0; i < GROUP; ++i) {
                int j = g * GROUP + i;
                float gate = moe_ref_f32_from_bf16(h[r * 2 * (int64_t)n + j]);
                float up = moe_ref_f32_from_bf16(h[r * 2 * (int64_t)n + n + j]);
                float ex = moe_ref_exp_spec(-gate);
                float s = gate / (1.0f + ex);
                float prod = s * up;
                act[i] = moe_ref_f32_from_bf16(moe_ref_bf16_from_f32(prod));
            }
            moe_ref_quant_group(act, q + r * n + g * GROUP, q_s + r * ng + g);
        }
    }
    free(valid);
    return MOE_REF_OK;
}

/* ======================================================================== *
 * Unpermute + topk weight + reduce (the ep_gather of PR #20903; weight and
 * reduce inside the experts per PR #20725 Purpose, output (M, K)):
 *   acc = +0; for k ascending with inv_perm[t,k] >= 0:
 *       acc = fmaf(w', y[inv_perm[t,k], c], acc)
 *   out[t,c] = bf16(acc); w' = 1 when the weight was applied on the input.
 * ======================================================================== */
int moe_ref_unpermute(const uint16_t* y, const int32_t* inv_perm, const float* topk_weights,
                      int64_t Mc, int32_t K, int32_t topk, int32_t apply_on_input, uint16_t* out) {
    if (K <= 0 || topk <= 0 || Mc < 0) return MOE_REF_ERR_SHAPE;
    if (!apply_on_input && !topk_weights) return MOE_REF_ERR_ARG;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < Mc; ++t) {
        for (int c = 0; c < K; ++c) {
            float acc = 0.0f;
            for (int k = 0; k < topk; ++k) {
                int32_t row = inv_perm[t * topk + k];
                if (row < 0) continue;
                float wk = apply_on_input ? 1.0f : topk_weights[t * topk + k];
                acc = fmaf(wk, moe_ref_f32_from_bf16(y[(int64_t)row * K + c]), acc);
            }
            out[t * K + c] = moe_ref_bf16_from_f32(acc);
        }
    }
    return MOE_REF_OK;
}

/* ======================================================================== *
 * Whole layer, chunked over M (PR #20392: chunks of the chunk size, the last
 * one short; counts and workspace shapes taken per chunk).  chunk_size <= 0
 * or >= M means one chunk.  per_chunk_counts, if given, is
 * [num_chunks, El].
 * ======================================================================== */
int moe_ref_forward_chunked(int64_t M, int32_t K, int32_t N, int32_t topk, int32_t Eg, int32_t El,
                            int32_t align, int32_t apply_on_input, int64_t chunk_size,
                            const uint16_t* x, const int32_t* topk_ids, const float* topk_weights,
                            const int32_t* expert_map, const uint8_t* w13, const float* w13_s,
                            const uint8_t* w2, const float* w2_s, uint16_t* out,
                            int32_t* per_chunk_counts) {
    if (M < 0 || K <= 0 || N <= 0 || K % GROUP || N % GROUP || topk <= 0) return MOE_REF_ERR_SHAPE;
    if (!(align == 16 || align == 32 || align == 64 || align == 128)) return MOE_REF_ERR_SHAPE;
    if (Eg <= 0 || El <= 0 || (!expert_map && El > Eg)) return MOE_REF_ERR_ARG;
    if (!topk_weights) return MOE_REF_ERR_ARG;
    if (M == 0) return MOE_REF_OK;
    int64_t cs = (chunk_size <= 0 || chunk_size >= M) ? M : chunk_size;
    int64_t nchunks = ceil_div64(M, cs);
    int64_t cap = moe_ref_max_rows(cs, topk, El, align);
    int kg = K / GROUP, ng = N / GROUP;

    uint8_t* a_q = (uint8_t*)malloc((size_t)cs * K);
    float* a_s = (float*)malloc((size_t)cs * kg * sizeof(float));
    uint8_t* a_perm = (uint8_t*)malloc((size_t)cap * K);
    float* a_perm_s = (float*)malloc((size_t)cap * kg * sizeof(float));
    int32_t* counts = (int32_t*)malloc((size_t)El * sizeof(int32_t));
    int32_t* offs = (int32_t*)malloc((size_t)(El + 1) * sizeof(int32_t));
    int32_t* inv = (int32_t*)malloc((size_t)cs * topk * sizeof(int32_t));
    int32_t* rsrc = (int32_t*)malloc((size_t)cap * sizeof(int32_t));
    uint16_t* h = (uint16_t*)malloc((size_t)cap * 2 * N * sizeof(uint16_t));
    uint8_t* act_q = (uint8_t*)malloc((size_t)cap * N);
    float* act_s = (float*)malloc((size_t)cap * ng * sizeof(float));
    uint16_t* y = (uint16_t*)malloc((size_t)cap * K * sizeof(uint16_t));
    int rc = MOE_REF_OK;
    if (!a_q || !a_s || !a_perm || !a_perm_s || !counts || !offs || !inv || !rsrc || !h || !act_q ||
        !act_s || !y) {
        rc = MOE_REF_ERR_ARG;
        goto done;
    }
    for (int64_t c = 0; c < nchunks && rc == MOE_REF_OK; ++c) {
        int64_t t0 = c * cs;
        int64_t Mc = (t0 + cs <= M) ? cs : (M - t0);
        const int32_t* ids_c = topk_ids + t0 * topk;
        const float* w_c = topk_weights + t0 * topk;
        rc = moe_ref_act_quant_identity(x + t0 * K, Mc, K, a_q, a_s);
        if (rc) break;
        rc = moe_ref_permute(a_q, a_s, ids_c, w_c, apply_on_input, Mc, K, topk, expert_map, Eg, El,
                             align, cap, a_perm, a_perm_s, counts, offs, inv, rsrc);
        if (rc) break;
        if (per_chunk_counts) memcpy(per_chunk_counts + c * El, counts, (size_t)El * sizeof(int32_t));
        rc = moe_ref_grouped_gemm(a_perm, a_perm_s, w13, w13_s, offs, counts, El, cap, 2 * N, K, h);
        if (rc) break;
        rc = moe_ref_silu_mul_quant(h, cap, N, offs, counts, El, act_q, act_s);
        if (rc) break;
        rc = moe_ref_grouped_gemm(act_q, act_s, w2, w2_s, offs, counts, El, cap, K, N, y);
        if (rc) break;
        rc = moe_ref_unpermute(y, inv, w_c, Mc, K, topk, apply_on_input, out + t0 * K);
    }
done:
    free(a_q); free(a_s); free(a_perm); free(a_perm_s); free(counts); free(offs);
    free(inv); free(rsrc); free(h); free(act_q); free(act_s); free(y);
    return rc;
}
