/*
 * CPU oracle for the MoE token path: the parts whose result must be
 * reproduced bit for bit.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load this library. It shares no source
 * with the GPU library and is written from the definitions below, not from
 * any kernel.
 *
 * Built with plain gcc, -O2 -ffp-contract=off, so that every multiply-add
 * written as `a*b + c` stays two roundings and every fused step is an
 * explicit fmaf().
 *
 * What the pages fix and what is our reading:
 *  - A router picks a few experts per token and only those run (Megatron
 *    Core MoE summary, "O essencial" and technical summary section 1).
 *    Top-k of 8 (Mixtral flags, skill page "Workflow 2: MoE") and of 256
 *    experts top-8 (Megatron Core summary section 4; Hybrid-EP article,
 *    results list). The pages give no router formula, no tie rule and no
 *    precision; we take:
 *      * logits in fp32 as a sequential fused multiply-add over the hidden
 *        index in ascending order (one rounding per step), plus an optional
 *        per-expert bias added once in fp32;
 *      * ranking by logit, larger first, equal logits broken by the lower
 *        expert index; -0 equals +0; NaN ranks below every number;
 *      * DeepSeek-style group limit: contiguous groups, group score = sum of
 *        the two best sigmoid scores of the group (or the best one), keep
 *        the best groups (ties to the lower group index), then top-k inside;
 *      * sigmoid scores s = 1 / (1 + exp_spec(-L)) with an fp32 exponential
 *        exp_spec that is fully specified here (Cody-Waite reduction by
 *        ln 2 split in two parts, degree-7 Taylor polynomial in Horner form,
 *        scaling by 2^n) so that group choice is reproducible bit for bit.
 *  - FP8 (Megatron Core summary section 2.2 and contribution 4: reduced
 *    precision FP8/FP4; Hybrid-EP article: low-precision dispatch). The
 *    format is not stated; we take OCP E4M3FN (max 448, no infinities),
 *    round to nearest with ties to the even code, saturating at +-448, with
 *    one fp32 scale per block: scale = amax / 448 (1 when amax is 0) and
 *    q = e4m3(v / scale).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- exp_spec */

#define EXPS_LOG2E 0x1.715476p+0f   /* log2(e) rounded to fp32 */
#define EXPS_LN2_HI 0x1.62e4p-1f    /* leading 15 bits of ln 2: n*LN2_HI is exact */
#define EXPS_LN2_LO 0x1.7f7d1cp-20f /* ln 2 - LN2_HI, rounded to fp32 */

float orc_exp_spec(float x)
{
    if (x != x) return x;
    if (x > 88.0f) return INFINITY;
    if (x < -86.0f) return 0.0f; /* keeps every result a normal number */
    float n = rintf(x * EXPS_LOG2E);
    float r = fmaf(-n, EXPS_LN2_HI, x);
    r = fmaf(-n, EXPS_LN2_LO, r);
    /* sum_{i=0..7} r^i / i!, coefficients 1/i! rounded to fp32 */
    float p = 0x1.a01a02p-13f;
    p = fmaf(p, r, 0x1.6c16c2p-10f);
    p = fmaf(p, r, 0x1.111112p-7f);
    p = fmaf(p, r, 0x1.555556p-5f);
    p = fmaf(p, r, 0x1.555556p-3f);
    p = fmaf(p, r, 0x1p-1f);
    p = fmaf(p, r, 1.0f);
    p = fmaf(p, r, 1.0f);
    return ldexpf(p, (int)n);
}

float orc_sigmoid_spec(float L)
{
    return 1.0f / (1.0f + orc_exp_spec(-L));
}

void orc_exp_spec_array(const float *x, float *out, int64_t n)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = orc_exp_spec(x[i]);
}

void orc_sigmoid_spec_array(const float *x, float *out, int64_t n)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = orc_sigmoid_spec(x[i]);
}

/* Worst error of exp_spec in ulps of the fp32 result, against libm's double
 * exp, over every fp32 bit pattern in [lo_bits, hi_bits) whose value lies in
 * [-86, 88]. Returns the maximum; *count receives how many inputs were
 * checked. */
double orc_exp_spec_max_ulp(uint32_t lo_bits, uint32_t hi_bits, int64_t *count)
{
    double worst = 0.0;
    int64_t cnt = 0;
#pragma omp parallel for schedule(static) reduction(max : worst) reduction(+ : cnt)
    for (int64_t b = lo_bits; b < (int64_t)hi_bits; ++b) {
        uint32_t u = (uint32_t)b;
        float x;
        memcpy(&x, &u, 4);
        if (!(x >= -86.0f && x <= 88.0f)) continue;
        double ref = exp((double)x);
        float got = orc_exp_spec(x);
        int e;
        frexp(ref, &e);                 /* ref in [2^(e-1), 2^e) */
        double ulp = ldexp(1.0, e - 24); /* ulp of fp32 in that binade */
        double err = fabs((double)got - ref) / ulp;
        if (err > worst) worst = err;
        cnt += 1;
    }
    if (count) *count = cnt;
    return worst;
}

/* ----------------------------------------------------------- router logits */

/* logits[t,e] = fp32 sequential fused multiply-add of x[t,i]*wr[e,i] over
 * i = 0..d-1 starting from +0, then + bias[e] (one fp32 add) if bias != NULL.
 * x is passed widened to fp32 (exact for bf16 inputs). */
void orc_router_logits(int64_t T, int64_t d, int64_t E, const float *x,
                       const float *wr, const float *bias, float *logits)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        const float *xr = x + t * d;
        for (int64_t e = 0; e < E; ++e) {
            const float *w = wr + e * d;
            float acc = 0.0f;
            for (int64_t i = 0; i < d; ++i) acc = fmaf(xr[i], w[i], acc);
            if (bias) acc = acc + bias[e];
            logits[t * E + e] = acc;
        }
    }
}

/* --------------------------------------------------------------- selection */

/* 1 if (La, a) ranks strictly above (Lb, b). */
static int ranks_above(float La, int64_t a, float Lb, int64_t b)
{
    int na = (La != La), nb = (Lb != Lb);
    if (na != nb) return nb; /* a number ranks above NaN */
    if (!na && La != Lb) return La > Lb; /* -0 == +0 falls through */
    return a < b;
}

static int score_above(float Sa, int64_t a, float Sb, int64_t b)
{
    return ranks_above(Sa, a, Sb, b);
}

/* Top-k selection for every token.
 *   logits [T,E] fp32 (bias already added), idx [T,k] out.
 *   num_groups > 1 with topk_groups < num_groups turns on the group limit:
 *   experts are split into num_groups contiguous groups of E/num_groups;
 *   a group's score is the sigmoid score of its best expert plus that of its
 *   second best (group_score 0) or the best alone (group_score 1); the
 *   topk_groups best groups are kept and top-k is taken inside them.
 * Slot j of a token holds its j-th ranked expert. Returns 0, or -1 on bad
 * arguments. */
int orc_route_select(int64_t T, int64_t E, int64_t k, const float *logits,
                     int64_t num_groups, int64_t topk_groups, int group_score,
                     int32_t *idx)
{
    if (k < 1 || k > E || num_groups < 1 || E % num_groups != 0 ||
        topk_groups < 1 || topk_groups > num_groups ||
        topk_groups * (E / num_groups) < k)
        return -1;
    int grouped = (num_groups > 1 && topk_groups < num_groups);
    int64_t gsize = E / num_groups;
    int bad = 0;
#pragma omp parallel
    {
        unsigned char *allowed = (unsigned char *)malloc((size_t)E);
        unsigned char *taken = (unsigned char *)malloc((size_t)E);
        float *gscore = (float *)malloc(sizeof(float) * (size_t)num_groups);
        unsigned char *gkeep = (unsigned char *)malloc((size_t)num_groups);
#pragma omp for schedule(static)
        for (int64_t t = 0; t < T; ++t) {
            const float *L = logits + t * E;
            for (int64_t e = 0; e < E; ++e) allowed[e] = 1, taken[e] = 0;
            if (grouped) {
                for (int64_t g = 0; g < num_groups; ++g) {
                    int64_t b1 = -1, b2 = -1;
                    for (int64_t e = g * gsize; e < (g + 1) * gsize; ++e) {
                        if (b1 < 0 || ranks_above(L[e], e, L[b1], b1)) {
                            b2 = b1;
                            b1 = e;
                        } else if (b2 < 0 || ranks_above(L[e], e, L[b2], b2)) {
                            b2 = e;
                        }
                    }
                    float s = orc_sigmoid_spec(L[b1]);
                    if (group_score == 0 && b2 >= 0) s = s + orc_sigmoid_spec(L[b2]);
                    gscore[g] = s;
                    gkeep[g] = 0;
                }
                for (int64_t r = 0; r < topk_groups; ++r) {
                    int64_t best = -1;
                    for (int64_t g = 0; g < num_groups; ++g)
                        if (!gkeep[g] && (best < 0 || score_above(gscore[g], g, gscore[best], best)))
                            best = g;
                    gkeep[best] = 1;
                }
                for (int64_t e = 0; e < E; ++e) allowed[e] = gkeep[e / gsize];
            }
            for (int64_t j = 0; j < k; ++j) {
                int64_t best = -1;
                for (int64_t e = 0; e < E; ++e)
                    if (allowed[e] && !taken[e] && (best < 0 || ranks_above(L[e], e, L[best], best)))
                        best = e;
                taken[best] = 1;
                idx[t * k + j] = (int32_t)best;
            }
        }
        free(allowed);
        free(taken);
        free(gscore);
        free(gkeep);
    }
    return bad;
}

/* -------------------------------------------------------------- FP8 E4M3FN */

/* Value of a non-negative E4M3FN code 0x00..0x7E: exponent field e (bias 7),
 * mantissa m; e == 0 is subnormal m/8 * 2^-6. */
static double e4m3_value_def(int c)
{
    int e = c >> 3, m = c & 7;
    if (e == 0) return ldexp((double)m / 8.0, -6);
    return ldexp(1.0 + (double)m / 8.0, e - 7);
}

static double e4m3_table[127];

__attribute__((constructor)) static void e4m3_table_init(void)
{
    for (int c = 0; c < 127; ++c) e4m3_table[c] = e4m3_value_def(c);
}

static double e4m3_value(int c) { return e4m3_table[c]; }

float orc_e4m3_decode(uint8_t c)
{
    int mag = c & 0x7F;
    if (mag == 0x7F) return NAN;
    double v = e4m3_value(mag);
    return (float)((c & 0x80) ? -v : v);
}

/* Nearest E4M3FN code, ties to the code with an even last bit, |v| >= 448
 * saturating to 448, NaN to 0x7F; the sign bit is kept (also for zero). */
uint8_t orc_e4m3_encode(float v)
{
    if (v != v) return 0x7F;
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double a = fabs((double)v);
    if (a >= 448.0) return (uint8_t)(sign | 0x7E);
    /* largest code whose value is <= a */
    int lo = 0, hi = 0x7E;
    while (lo < hi) {
        int mid = (lo + hi + 1) / 2;
        if (e4m3_value(mid) <= a) lo = mid; else hi = mid - 1;
    }
    int c = lo;
    double vlo = e4m3_value(c);
    if (vlo == a) return (uint8_t)(sign | c);
    double vhi = e4m3_value(c + 1);
    double dlo = a - vlo, dhi = vhi - a; /* exact in double */
    int pick;
    if (dlo < dhi) pick = c;
    else if (dhi < dlo) pick = c + 1;
    else pick = (c & 1) ? c + 1 : c;
    return (uint8_t)(sign | pick);
}

void orc_e4m3_encode_array(const float *v, uint8_t *out, int64_t n)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3_encode(v[i]);
}

void orc_e4m3_decode_array(const uint8_t *c, float *out, int64_t n)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3_decode(c[i]);
}

/* Block quantisation of src [R,C] (fp32) in blocks of br x bc (the last
 * block row/column may be partial): per block amax = max |v|,
 * scale = amax / 448 (fp32 divide; 1 when amax == 0), q = e4m3(v / scale).
 * scale is [ceil(R/br), ceil(C/bc)]. */
void orc_quant_blocks(int64_t R, int64_t C, const float *src, int64_t br,
                      int64_t bc, uint8_t *q, float *scale)
{
    int64_t nbr = (R + br - 1) / br, nbc = (C + bc - 1) / bc;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t I = 0; I < nbr; ++I) {
        for (int64_t J = 0; J < nbc; ++J) {
            int64_t r1 = (I + 1) * br < R ? (I + 1) * br : R;
            int64_t c1 = (J + 1) * bc < C ? (J + 1) * bc : C;
            float amax = 0.0f;
            for (int64_t r = I * br; r < r1; ++r)
                for (int64_t c = J * bc; c < c1; ++c) {
                    float a = fabsf(src[r * C + c]);
                    if (a > amax) amax = a;
                }
            float s = (amax == 0.0f) ? 1.0f : amax / 448.0f;
            scale[I * nbc + J] = s;
            for (int64_t r = I * br; r < r1; ++r)
                for (int64_t c = J * bc; c < c1; ++c)
                    q[r * C + c] = orc_e4m3_encode(src[r * C + c] / s);
        }
    }
}

/* MXFP8 (OCP Microscaling Formats v1.0, the MXFP8 E4M3 format the Hybrid-EP
 * article's results use): one power-of-two scale X = 2^x per block of 32
 * consecutive elements of a row, stored as an E8M0 byte x + 127. The MX
 * definition fixes the format, not how x is chosen. Here x is the smallest
 * integer with amax * 2^-x <= 448 (the largest E4M3 magnitude), so that no
 * element saturates; x = 0 when amax = 0, and x >= -127 (E8M0's range).
 * With amax = m * 2^e, m in [0.5, 1): amax * 2^-x = m * 2^(e-x), which is
 * <= 448 = 0.875 * 2^9 exactly when e - x <= 9 (m <= 0.875) or e - x <= 8
 * (m > 0.875). Elements are v * 2^-x (a power-of-two rescaling) encoded to
 * E4M3 with round-to-nearest-even (orc_e4m3_encode). */
int orc_mx_scale_exp(float amax)
{
    if (amax == 0.0f) return 0;
    int e;
    float m = frexpf(amax, &e);
    int x = (m > 0.875f) ? e - 8 : e - 9;
    if (x < -127) x = -127;
    if (x > 127) x = 127;
    return x;
}

/* src [R,C] fp32, C a multiple of 32: q [R,C] E4M3 codes, e8m0 [R, C/32]. */
void orc_quant_mx_rows(int64_t R, int64_t C, const float *src, uint8_t *q, uint8_t *e8m0)
{
    int64_t nb = C / 32;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t r = 0; r < R; ++r) {
        for (int64_t b = 0; b < nb; ++b) {
            const float *v = src + r * C + b * 32;
            float amax = 0.0f;
            for (int i = 0; i < 32; ++i) {
                float a = fabsf(v[i]);
                if (a > amax) amax = a;
            }
            int x = orc_mx_scale_exp(amax);
            e8m0[r * nb + b] = (uint8_t)(x + 127);
            for (int i = 0; i < 32; ++i) q[r * C + b * 32 + i] = orc_e4m3_encode(ldexpf(v[i], -x));
        }
    }
}

/* The same MXFP8 rule in 32 x 1 blocks: src [R,C] fp32, R a multiple of 32,
 * each block 32 consecutive rows of one column (the row rule applied to the
 * transpose): q [R,C] E4M3 codes, e8m0 [R/32, C]. */
void orc_quant_mx_cols(int64_t R, int64_t C, const float *src, uint8_t *q, uint8_t *e8m0)
{
    int64_t nb = R / 32;
#pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < nb; ++b) {
        for (int64_t c = 0; c < C; ++c) {
            float amax = 0.0f;
            for (int i = 0; i < 32; ++i) {
                float a = fabsf(src[(b * 32 + i) * C + c]);
                if (a > amax) amax = a;
            }
            int x = orc_mx_scale_exp(amax);
            e8m0[b * C + c] = (uint8_t)(x + 127);
            for (int i = 0; i < 32; ++i)
                q[(b * 32 + i) * C + c] = orc_e4m3_encode(ldexpf(src[(b * 32 + i) * C + c], -x));
        }
    }
}
