/*
 * kvq_oracle.c -- CPU oracle for the int4 group-wise KV cache and the
 * decode-phase attention that reads it.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or
 * load this code: only the tests, the smoke check and the benchmark's CPU
 * baseline leg use it.  It shares no source, header, table or helper with
 * the HIP library; the only thing both sides receive is the same input
 * bytes.
 *
 * Plain, scalar, slow on purpose.  Every step follows the text it cites:
 *
 *  [FG-blog]   "FlexGen: High-Throughput Generative Inference of Large
 *              Language Models with a Single GPU [ICML'23]" (qingweiji blog),
 *              sections "P/D阶段计算 / 解码阶段" (decode-phase KV update and
 *              attention), "预填充阶段" (prefill attention) and "KV Cache"
 *              (the [b, s, a, h/a] cache shape).
 *  [FG-report] "FlexGen研究学术报告" (fmread), section 三.2(C) "近似方法的应用":
 *              group-wise asymmetric 4-bit quantisation, 64 contiguous
 *              elements per group, tensors dequantised to FP16 before
 *              compute; and top-10% sparse attention (load only the KV
 *              entries with the highest attention values).
 *  [Survey]    notes on "A Survey on Efficient Inference for Large Language
 *              Models" (gumorming), eq. (2): Softmax(Q K^T / sqrt(d_k)) V
 *              with d_k the query/key dimension.
 *
 * Precision.  The codec decides integers (the 4-bit codes), so it runs in
 * binary32 with one rounding per operation (built with -ffp-contract=off,
 * no fast-math), in the order listed at oracle_quantize_group.  Attention
 * runs in binary64 over the dequantised values min + code*scale taken
 * exactly (oracle_dequant_value).  The report's "dequantised to FP16 before
 * compute" describes the data type of FlexGen's own GPU compute; that form
 * is oracle_dequant_elem_f16, and oracle_attend_rows runs the same attention
 * over it (the second reference the GPU output is compared with).  It is not
 * the primary reference: with the OPT-30B style outlier channels (queries
 * and keys x8) the FP16 rounding of a dequantised key alone moves a logit by
 * ~1e-2, more than the tolerance the GPU path is held to, so there an
 * FP16-rounded reference measures rounding noise rather than the method.
 *
 * Readings taken where the pages are silent (each one is listed in the
 * design notes with its reason):
 *   - the group runs along head_dim (64 contiguous head_dim elements);
 *   - asymmetric = min/max affine code: scale = (max-min)/15, 16 levels
 *     min + c*scale, code = round_half_even((x-min)*(15/(max-min))),
 *     clamped to 0..15;
 *   - a constant group (max == min) stores scale 0 and codes 0;
 *   - metadata planes in binary32 (oracle_quantize_group) or binary16
 *     (oracle_quantize_group_m16: min exact, scale rounded to nearest, codes
 *     taken against the stored scale);
 *   - a stored min/max of -0 is canonicalised to +0;
 *   - two codes per byte, the even element in the low nibble;
 *   - attention scale 1/sqrt(d), d = head_dim = h/a (the survey's d_k);
 *   - top-k ranks tokens by score (softmax is monotone), larger score
 *     first, ties to the smaller token index; the softmax is renormalised
 *     over the kept tokens;
 *   - prefill attention is causal and runs over the fp16 K and V (the
 *     quantised copy is what the cache keeps for the decode steps).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_GROUP 64

/* ------------------------------------------------------------------------
 * IEEE 754 binary16 <-> binary32, from the format's definition:
 * 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits; exponent 0 holds
 * the subnormals (fraction * 2^-24), exponent 31 holds inf/NaN.
 * --------------------------------------------------------------------- */
float oracle_f16_to_f32(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 31;
    int frac = h & 1023;
    float v;
    if (e == 0)
        v = ldexpf((float)frac, -24);
    else if (e == 31)
        v = frac ? NAN : INFINITY;
    else
        v = ldexpf((float)(1024 + frac), e - 25);
    return sign ? -v : v;
}

/* Round a binary32 value to the nearest binary16 value, ties to even. */
uint16_t oracle_f32_to_f16(float f)
{
    uint16_t sign = signbit(f) ? 0x8000u : 0u;
    if (isnan(f))
        return 0x7e00u;
    double a = fabs((double)f);
    if (a == 0.0)
        return sign;
    /* Quantum (spacing of binary16 values) in the binade of a. */
    int e;
    frexp(a, &e); /* a = m * 2^e, m in [0.5, 1): binade [2^(e-1), 2^e) */
    int unbiased = e - 1;
    double quantum = (unbiased < -14) ? ldexp(1.0, -24) : ldexp(1.0, unbiased - 10);
    double r = nearbyint(a / quantum) * quantum; /* exact scaling; ties to even */
    if (r > 65504.0)
        return (uint16_t)(sign | 0x7c00u); /* rounds beyond the largest finite: inf */
    if (r < ldexp(1.0, -14)) {
        /* subnormal (or zero): fraction counts units of 2^-24 */
        return (uint16_t)(sign | (uint16_t)(r / ldexp(1.0, -24)));
    }
    int er;
    double m = frexp(r, &er); /* r = m * 2^er, m in [0.5, 1) */
    uint16_t exp_field = (uint16_t)(er - 1 + 15);
    uint16_t frac = (uint16_t)((2.0 * m - 1.0) * 1024.0);
    return (uint16_t)(sign | (exp_field << 10) | frac);
}

/* ------------------------------------------------------------------------
 * Codec: one group of 64 consecutive head_dim elements ([FG-report] 三.2(C)).
 * --------------------------------------------------------------------- */

/* Quantise 64 fp16 values.  Writes 32 code bytes, the group min and scale.
 * Steps, each a single binary32 rounding:
 *   widen to binary32 (exact);
 *   mn = min, mx = max (exact), then -0 -> +0 by adding +0;
 *   rng = mx - mn;
 *   rng == 0: scale = 0, every code 0;
 *   else scale = rng / 15, inv = 15 / rng (correctly rounded divisions),
 *        code = clamp(rint_half_even((x - mn) * inv), 0, 15);
 *   byte j = code[2j] | code[2j+1] << 4.                                   */
/* Widen a group to binary32 and find its min and max, -0 stored as +0. */
static void group_minmax(const uint16_t *x, float *f, float *out_mn, float *out_mx)
{
    for (int i = 0; i < ORACLE_GROUP; ++i)
        f[i] = oracle_f16_to_f32(x[i]);
    float mn = f[0], mx = f[0];
    for (int i = 1; i < ORACLE_GROUP; ++i) {
        if (f[i] < mn)
            mn = f[i];
        if (f[i] > mx)
            mx = f[i];
    }
    *out_mn = mn + 0.0f;
    *out_mx = mx + 0.0f;
}

static void pack_codes(const int *c, uint8_t *codes)
{
    for (int j = 0; j < ORACLE_GROUP / 2; ++j)
        codes[j] = (uint8_t)(c[2 * j] | (c[2 * j + 1] << 4));
}

void oracle_quantize_group(const uint16_t *x, uint8_t *codes, float *out_min, float *out_scale)
{
    float f[ORACLE_GROUP];
    int c[ORACLE_GROUP];
    float mn, mx;
    group_minmax(x, f, &mn, &mx);
    float rng = mx - mn;
    float scale;
    if (rng == 0.0f) {
        scale = 0.0f;
        for (int i = 0; i < ORACLE_GROUP; ++i)
            c[i] = 0;
    } else {
        scale = rng / 15.0f;
        float inv = 15.0f / rng;
        for (int i = 0; i < ORACLE_GROUP; ++i) {
            float t = f[i] - mn;
            t = t * inv;
            float r = rintf(t); /* default rounding mode: nearest, ties to even */
            if (r < 0.0f)
                r = 0.0f;
            if (r > 15.0f)
                r = 15.0f;
            c[i] = (int)r;
        }
    }
    pack_codes(c, codes);
    *out_min = mn;
    *out_scale = scale;
}

/* The same codec with binary16 min and scale planes (half the metadata
 * bytes).  The pages fix no metadata type; this variant stores:
 *   min   = the group minimum, which is one of the fp16 inputs, so exact;
 *   scale = the binary32 quotient rng/15 rounded to the nearest binary16
 *           value, ties to even;
 * and takes the codes against the stored pair, so that min + code*scale is
 * the nearest of the 16 levels it can reconstruct:
 *   inv = 1/scale (binary32, correctly rounded),
 *   code = clamp(rint_half_even((x - min) * inv), 0, 15).
 * A group whose stored scale is 0 (a constant group, or a range below
 * 15 * 2^-25 whose scale underflows binary16) gets codes 0.                */
void oracle_quantize_group_m16(const uint16_t *x, uint8_t *codes, uint16_t *out_min, uint16_t *out_scale)
{
    float f[ORACLE_GROUP];
    int c[ORACLE_GROUP];
    float mn, mx;
    group_minmax(x, f, &mn, &mx);
    float rng = mx - mn;
    uint16_t s16 = 0;
    if (rng != 0.0f)
        s16 = oracle_f32_to_f16(rng / 15.0f);
    float scale = oracle_f16_to_f32(s16);
    if (scale == 0.0f) {
        for (int i = 0; i < ORACLE_GROUP; ++i)
            c[i] = 0;
    } else {
        float inv = 1.0f / scale;
        for (int i = 0; i < ORACLE_GROUP; ++i) {
            float t = f[i] - mn;
            t = t * inv;
            float r = rintf(t);
            if (r < 0.0f)
                r = 0.0f;
            if (r > 15.0f)
                r = 15.0f;
            c[i] = (int)r;
        }
    }
    pack_codes(c, codes);
    *out_min = oracle_f32_to_f16(mn);
    *out_scale = s16;
}

/* The stored scale and the inverse the codes are taken with, for n group
 * ranges rng[i] > 0: binary32 metadata (meta16 = 0) as in
 * oracle_quantize_group (scale = rng/15, inv = 15/rng), binary16 metadata
 * (meta16 = 1) as in oracle_quantize_group_m16 (scale = rng/15 rounded to
 * binary16, inv = 1/scale); inv = 0 where the stored scale is 0.  The stored
 * scale is returned widened to binary32.                                   */
void oracle_codec_params(int meta16, int64_t n, const float *rng, float *scale, float *inv)
{
    for (int64_t i = 0; i < n; ++i) {
        float r = rng[i];
        float s, v;
        if (!meta16) {
            s = r / 15.0f;
            v = 15.0f / r;
        } else {
            s = oracle_f16_to_f32(oracle_f32_to_f16(r / 15.0f));
            v = s != 0.0f ? 1.0f / s : 0.0f;
        }
        scale[i] = s;
        inv[i] = v;
    }
}

/* Quantise one token row of d fp16 values (d a multiple of 64): group g
 * covers elements 64g..64g+63; codes[d/2], mins[d/64], scales[d/64].      */
void oracle_quantize_row(int d, const uint16_t *x, uint8_t *codes, float *mins, float *scales)
{
    for (int g = 0; g < d / ORACLE_GROUP; ++g)
        oracle_quantize_group(x + g * ORACLE_GROUP, codes + g * (ORACLE_GROUP / 2), mins + g, scales + g);
}

/* nrows independent rows, packed back to back (row r at x + r*d). */
void oracle_quantize_rows(int nrows, int d, const uint16_t *x, uint8_t *codes, float *mins, float *scales)
{
    int G = d / ORACLE_GROUP;
    for (int r = 0; r < nrows; ++r)
        oracle_quantize_row(d, x + (size_t)r * d, codes + (size_t)r * (d / 2), mins + (size_t)r * G,
                            scales + (size_t)r * G);
}

/* Rows with binary16 metadata: mins[d/64], scales[d/64] as binary16 bits. */
void oracle_quantize_rows_m16(int nrows, int d, const uint16_t *x, uint8_t *codes, uint16_t *mins,
                              uint16_t *scales)
{
    int G = d / ORACLE_GROUP;
    for (int r = 0; r < nrows; ++r)
        for (int g = 0; g < G; ++g)
            oracle_quantize_group_m16(x + (size_t)r * d + g * ORACLE_GROUP,
                                      codes + (size_t)r * (d / 2) + g * (ORACLE_GROUP / 2), mins + (size_t)r * G + g,
                                      scales + (size_t)r * G + g);
}

/* Code of element i of a row (low nibble = even element). */
int oracle_code_at(const uint8_t *row_codes, int i)
{
    uint8_t byte = row_codes[i / 2];
    return (i % 2 == 0) ? (byte & 15) : (byte >> 4);
}

/* Dequantised value of element i of a row: min + code * scale, the affine
 * map of the asymmetric code, taken exactly (binary64 holds the product of a
 * 4-bit integer and a binary32 scale, and the sum with the binary32 min, to
 * far below the tolerances used here).  This is the value attention uses.  */
double oracle_dequant_value(const uint8_t *row_codes, const float *row_mins, const float *row_scales, int i)
{
    int g = i / ORACLE_GROUP;
    return (double)oracle_code_at(row_codes, i) * (double)row_scales[g] + (double)row_mins[g];
}

/* The same value as the report writes it for its GPU: dequantised to FP16
 * ([FG-report] 三.2(C)): v = code*scale, then v + min (two binary32
 * roundings), then rounded to binary16.  Kept as a reference: the attention
 * functions below use oracle_dequant_value (see the header note).          */
uint16_t oracle_dequant_elem_f16(const uint8_t *row_codes, const float *row_mins, const float *row_scales, int i)
{
    int g = i / ORACLE_GROUP;
    float v = (float)oracle_code_at(row_codes, i) * row_scales[g];
    v = v + row_mins[g];
    return oracle_f32_to_f16(v);
}

void oracle_dequant_rows(int nrows, int d, const uint8_t *codes, const float *mins, const float *scales,
                         double *out)
{
    int G = d / ORACLE_GROUP;
    for (int r = 0; r < nrows; ++r)
        for (int i = 0; i < d; ++i)
            out[(size_t)r * d + i] = oracle_dequant_value(codes + (size_t)r * (d / 2), mins + (size_t)r * G,
                                                          scales + (size_t)r * G, i);
}

void oracle_dequant_rows_f16(int nrows, int d, const uint8_t *codes, const float *mins, const float *scales,
                             uint16_t *out)
{
    int G = d / ORACLE_GROUP;
    for (int r = 0; r < nrows; ++r)
        for (int i = 0; i < d; ++i)
            out[(size_t)r * d + i] = oracle_dequant_elem_f16(codes + (size_t)r * (d / 2), mins + (size_t)r * G,
                                                             scales + (size_t)r * G, i);
}

/* ------------------------------------------------------------------------
 * Decode attention for one (batch row, head) over a quantised cache
 * ([FG-blog] 解码阶段: t_out = softmax(t_Q x_K^T / sqrt(.)) x_V, stopping
 * before W_O; scale 1/sqrt(d) per [Survey] eq. (2)).
 * Cache of one (batch row, head): codes [T][d/2], mins/scales [T][d/64].
 * --------------------------------------------------------------------- */

static double kdot(int d, const uint16_t *q, const uint8_t *kc, const float *kmin, const float *ksc, int t)
{
    int G = d / ORACLE_GROUP;
    double acc = 0.0;
    for (int i = 0; i < d; ++i) {
        double qi = (double)oracle_f16_to_f32(q[i]);
        double ki = oracle_dequant_value(kc + (size_t)t * (d / 2), kmin + (size_t)t * G, ksc + (size_t)t * G, i);
        acc += qi * ki;
    }
    return acc;
}

/* Scores s_t = (q . k_t) / sqrt(d) for t = 0..T-1. */
void oracle_scores(int d, int T, const uint16_t *q, const uint8_t *kc, const float *kmin, const float *ksc,
                   double *scores)
{
    double c = 1.0 / sqrt((double)d);
    for (int t = 0; t < T; ++t)
        scores[t] = kdot(d, q, kc, kmin, ksc, t) * c;
}

/* Dense decode attention: out[i] = sum_t p_t v_t[i] / sum_t p_t,
 * p_t = exp(s_t - max_s).                                                  */
void oracle_attend(int d, int T, const uint16_t *q, const uint8_t *kc, const float *kmin, const float *ksc,
                   const uint8_t *vc, const float *vmin, const float *vsc, double *out)
{
    int G = d / ORACLE_GROUP;
    if (T < 1)
        return;
    double *s = (double *)malloc(sizeof(double) * (size_t)T);
    oracle_scores(d, T, q, kc, kmin, ksc, s);
    double m = s[0];
    for (int t = 1; t < T; ++t)
        if (s[t] > m)
            m = s[t];
    double l = 0.0;
    for (int t = 0; t < T; ++t) {
        s[t] = exp(s[t] - m);
        l += s[t];
    }
    for (int i = 0; i < d; ++i) {
        double acc = 0.0;
        for (int t = 0; t < T; ++t) {
            double vi = oracle_dequant_value(vc + (size_t)t * (d / 2), vmin + (size_t)t * G, vsc + (size_t)t * G, i);
            acc += s[t] * vi;
        }
        out[i] = acc / l;
    }
    free(s);
}

/* Attention restricted to the token set idx[0..nidx-1]: the softmax is
 * taken over those tokens' scores only.                                    */
void oracle_attend_subset(int d, int nidx, const int32_t *idx, const uint16_t *q, const uint8_t *kc,
                          const float *kmin, const float *ksc, const uint8_t *vc, const float *vmin,
                          const float *vsc, double *out)
{
    int G = d / ORACLE_GROUP;
    double c = 1.0 / sqrt((double)d);
    if (nidx < 1)
        return;
    double *p = (double *)malloc(sizeof(double) * (size_t)nidx);
    for (int j = 0; j < nidx; ++j)
        p[j] = kdot(d, q, kc, kmin, ksc, idx[j]) * c;
    double m = p[0];
    for (int j = 1; j < nidx; ++j)
        if (p[j] > m)
            m = p[j];
    double l = 0.0;
    for (int j = 0; j < nidx; ++j) {
        p[j] = exp(p[j] - m);
        l += p[j];
    }
    for (int i = 0; i < d; ++i) {
        double acc = 0.0;
        for (int j = 0; j < nidx; ++j) {
            int t = idx[j];
            double vi = oracle_dequant_value(vc + (size_t)t * (d / 2), vmin + (size_t)t * G, vsc + (size_t)t * G, i);
            acc += p[j] * vi;
        }
        out[i] = acc / l;
    }
    free(p);
}

/* Top-k selection: the k tokens with the largest scores, larger score
 * first and ties to the smaller index; returned in ascending token order.
 * Plain selection by repeated scans (k passes over T) -- slow and obvious.  */
void oracle_select_topk(int T, const double *scores, int k, int32_t *sel)
{
    unsigned char *taken = (unsigned char *)calloc((size_t)T, 1);
    for (int j = 0; j < k; ++j) {
        int best = -1;
        for (int t = 0; t < T; ++t) {
            if (taken[t])
                continue;
            if (best < 0 || scores[t] > scores[best])
                best = t; /* strict '>' keeps the smaller index on ties */
        }
        taken[best] = 1;
    }
    int n = 0;
    for (int t = 0; t < T; ++t)
        if (taken[t])
            sel[n++] = t;
    free(taken);
}

/* Sparse decode attention ([FG-report] 三.2(C)): rank all T scores, keep the
 * top k, softmax and P.V over the kept tokens only.  sel (may be NULL)
 * receives the kept token indices in ascending order.                      */
void oracle_attend_topk(int d, int T, int k, const uint16_t *q, const uint8_t *kc, const float *kmin,
                        const float *ksc, const uint8_t *vc, const float *vmin, const float *vsc, double *out,
                        int32_t *sel)
{
    double *s = (double *)malloc(sizeof(double) * (size_t)T);
    int32_t *idx = (int32_t *)malloc(sizeof(int32_t) * (size_t)k);
    oracle_scores(d, T, q, kc, kmin, ksc, s);
    oracle_select_topk(T, s, k, idx);
    oracle_attend_subset(d, k, idx, q, kc, kmin, ksc, vc, vmin, vsc, out);
    if (sel)
        memcpy(sel, idx, sizeof(int32_t) * (size_t)k);
    free(idx);
    free(s);
}

/* Decode attention of one query over T dequantised rows given explicitly
 * (binary64, row t of K^ at khat + t*d, of V^ at vhat + t*d): the same
 * scores (scale 1/sqrt(d)), max-subtracted softmax and P.V as oracle_attend.
 * With the rows in the FP16 form (oracle_dequant_rows_f16, widened exactly)
 * this is attention over the cache "dequantised to FP16 before compute" as
 * [FG-report] 三.2(C) writes it; with a chosen subset of rows it is the
 * sparse variant over those rows.                                          */
void oracle_attend_rows(int d, int T, const uint16_t *q, const double *khat, const double *vhat, double *out)
{
    double c = 1.0 / sqrt((double)d);
    if (T < 1)
        return;
    double *p = (double *)malloc(sizeof(double) * (size_t)T);
    for (int t = 0; t < T; ++t) {
        double acc = 0.0;
        for (int i = 0; i < d; ++i)
            acc += (double)oracle_f16_to_f32(q[i]) * khat[(size_t)t * d + i];
        p[t] = acc * c;
    }
    double m = p[0];
    for (int t = 1; t < T; ++t)
        if (p[t] > m)
            m = p[t];
    double l = 0.0;
    for (int t = 0; t < T; ++t) {
        p[t] = exp(p[t] - m);
        l += p[t];
    }
    for (int i = 0; i < d; ++i) {
        double acc = 0.0;
        for (int t = 0; t < T; ++t)
            acc += p[t] * vhat[(size_t)t * d + i];
        out[i] = acc / l;
    }
    free(p);
}

/* ------------------------------------------------------------------------
 * Prefill attention for one (batch row, head) over the prompt ([FG-blog]
 * 预填充阶段: x_out = softmax(x_Q x_K^T / sqrt(.)) x_V, stopping before W_O
 * and the residual; scale 1/sqrt(d) per [Survey] eq. (2)).
 * Readings: causal -- prompt token i attends to tokens 0..i, the tokens a
 * decode step at position i would see ([FG-blog]: each generated token
 * depends on the tokens before it), so prefill row i equals that decode
 * step's attention; and over the fp16 K and V as the projections produced
 * them (the quantised copy is what the cache keeps for the decode steps).
 * q, k, v: fp16 bits, row t at + t*stride elements (stride >= d lets the
 * caller pass one head of a [s][a][d] batch row); out: binary64 [s][d].
 * --------------------------------------------------------------------- */
/* Row i of the causal prefill attention (0 <= i < s): query i over keys
 * 0..i; p holds at least i + 1 doubles of scratch.                          */
static void prefill_row(int d, int s, int i, int stride, const uint16_t *q, const uint16_t *k, const uint16_t *v,
                        double *p, double *out_row)
{
    if (i < 0 || i >= s)
        return;
    double c = 1.0 / sqrt((double)d);
    const uint16_t *qi = q + (size_t)i * stride;
    double m = -INFINITY;
    for (int t = 0; t <= i; ++t) {
        const uint16_t *kt = k + (size_t)t * stride;
        double acc = 0.0;
        for (int e = 0; e < d; ++e)
            acc += (double)oracle_f16_to_f32(qi[e]) * (double)oracle_f16_to_f32(kt[e]);
        p[t] = acc * c;
        if (p[t] > m)
            m = p[t];
    }
    double l = 0.0;
    for (int t = 0; t <= i; ++t) {
        p[t] = exp(p[t] - m);
        l += p[t];
    }
    for (int e = 0; e < d; ++e) {
        double acc = 0.0;
        for (int t = 0; t <= i; ++t)
            acc += p[t] * (double)oracle_f16_to_f32(v[(size_t)t * stride + e]);
        out_row[e] = acc / l;
    }
}

void oracle_prefill_attend(int d, int s, int stride, const uint16_t *q, const uint16_t *k, const uint16_t *v,
                           double *out)
{
    double *p = (double *)malloc(sizeof(double) * (size_t)(s > 0 ? s : 1));
    for (int i = 0; i < s; ++i)
        prefill_row(d, s, i, stride, q, k, v, p, out + (size_t)i * d);
    free(p);
}

/* The same attention for the query rows rows[0..nrows-1] only (each in
 * 0..s-1): out[j][d] is row rows[j].  The cost of row i grows with i, so a
 * few rows of every head cost far less than every row of a few heads.     */
void oracle_prefill_attend_rows(int d, int s, int stride, const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                int nrows, const int32_t *rows, double *out)
{
    double *p = (double *)malloc(sizeof(double) * (size_t)(s > 0 ? s : 1));
    for (int j = 0; j < nrows; ++j)
        prefill_row(d, s, rows[j], stride, q, k, v, p, out + (size_t)j * d);
    free(p);
}

/* ------------------------------------------------------------------------
 * Group-wise int4 weights ([FG-report] 三.2(C): the weights are compressed
 * with the same group-wise asymmetric 4-bit code as the KV cache and
 * dequantised to FP16 before compute).  A weight matrix W [N][K] (output
 * row n, input column k; the [FG-blog] 解码阶段 projections t W_Q, t W_K,
 * t W_V and t_out W_O) is quantised row by row with the binary16-metadata
 * codec (oracle_quantize_rows_m16): groups of 64 contiguous k.
 * --------------------------------------------------------------------- */

/* The FP16 form of a dequantised weight: the binary16 value nearest to
 * min + code*scale (ties to even), the sum taken exactly.  With binary16 min
 * and scale every term is an integer multiple of 2^-24, so the sum is an
 * exact 64-bit integer count of 2^-24 units.                               */
uint16_t oracle_w_dequant(int code, uint16_t min16, uint16_t scale16)
{
    double mn = (double)oracle_f16_to_f32(min16), sc = (double)oracle_f16_to_f32(scale16);
    int64_t units = (int64_t)llround(ldexp(mn, 24)) + (int64_t)code * (int64_t)llround(ldexp(sc, 24));
    int neg = units < 0;
    uint64_t a = (uint64_t)(neg ? -units : units);
    if (a == 0)
        return 0; /* +0 */
    /* binary16 spacing at a * 2^-24: 2^(e-10) for 2^e <= value < 2^(e+1), at least 2^-24 */
    int e = 63 - __builtin_clzll(a) - 24;
    int qshift = (e - 10 > -24 ? e - 10 : -24) + 24; /* spacing in units, log2 */
    uint64_t q = (uint64_t)1 << qshift;
    uint64_t lo = a / q * q, rem = a - lo;
    uint64_t r = lo;
    if (rem * 2 > q || (rem * 2 == q && ((lo / q) & 1)))
        r = lo + q;
    double v = ldexp((double)r, -24); /* exact: r is representable in binary16 (or overflows it) */
    if (v > 65504.0)
        return neg ? 0xfc00u : 0x7c00u;
    uint16_t h = oracle_f32_to_f16((float)v); /* exact, v is a binary16 value */
    return neg ? (uint16_t)(h | 0x8000u) : h;
}

/* y[m][n] = sum_k x[m][k] * W^[n][k] (binary64, k ascending), W^ the FP16
 * form of the dequantised weights: the linear layer y = x W^T of a decode
 * projection.  x fp16 [M][K]; codes [N][K/2]; mins, scales binary16
 * [N][K/64].                                                               */
void oracle_gemm_w4a16(int M, int N, int K, const uint16_t *x, const uint8_t *codes, const uint16_t *mins,
                       const uint16_t *scales, double *y)
{
    int G = K / ORACLE_GROUP;
    double *wrow = (double *)malloc(sizeof(double) * (size_t)K);
    for (int n = 0; n < N; ++n) {
        for (int k = 0; k < K; ++k) {
            int g = k / ORACLE_GROUP;
            int c = oracle_code_at(codes + (size_t)n * (K / 2), k);
            wrow[k] = (double)oracle_f16_to_f32(
                oracle_w_dequant(c, mins[(size_t)n * G + g], scales[(size_t)n * G + g]));
        }
        for (int m = 0; m < M; ++m) {
            double acc = 0.0;
            for (int k = 0; k < K; ++k)
                acc += (double)oracle_f16_to_f32(x[(size_t)m * K + k]) * wrow[k];
            y[(size_t)m * N + n] = acc;
        }
    }
    free(wrow);
}
