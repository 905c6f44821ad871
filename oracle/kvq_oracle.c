/*
 * kvq_oracle.c -- plain CPU reference for the compressed-KV decode path.
 *
 * TEST INFRASTRUCTURE ONLY (see kvq_oracle.h).  Built with -O2
 * -ffp-contract=off and no fast-math so every fp32 operation below is one IEEE
 * operation in source order.
 */
#include "kvq_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------- */
/* Number formats                                                             */
/* ------------------------------------------------------------------------- */

/* binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
 * Finite values are (-1)^s * 2^(e-15) * (1 + f/1024) for e in 1..30 and
 * (-1)^s * 2^-14 * (f/1024) for e == 0.  Rounding to nearest, ties to even,
 * is done by scaling |x| to an integer count of the target quantum in double
 * (exact: a power-of-two scale) and calling nearbyint in the default mode.  */
uint16_t kvo_f32_to_f16(float x)
{
    uint32_t bits;
    memcpy(&bits, &x, sizeof bits);
    uint16_t sign = (uint16_t)((bits >> 16) & 0x8000u);
    double a = fabs((double)x);
    if (isnan(x))
        return (uint16_t)(sign | 0x7E00u);
    if (isinf(x))
        return (uint16_t)(sign | 0x7C00u);
    if (a == 0.0)
        return sign;
    int e2;
    frexp(a, &e2);           /* a = m * 2^e2, m in [0.5, 1) -> floor(log2 a) = e2-1 */
    int e = e2 - 1;
    if (e < -14)
        e = -14;             /* subnormal range shares the quantum 2^-24 */
    double quantum = ldexp(1.0, e - 10);
    double n = nearbyint(a / quantum);   /* integer count of quanta, ties to even */
    if (n >= 2048.0) {       /* rounding carried into the next binade */
        n /= 2.0;
        e += 1;
    }
    if (e > 15)
        return (uint16_t)(sign | 0x7C00u);  /* overflow to infinity */
    if (n < 1024.0)          /* subnormal (only possible with e == -14) */
        return (uint16_t)(sign | (uint16_t)n);
    return (uint16_t)(sign | (uint16_t)((e + 15) << 10) | (uint16_t)(n - 1024.0));
}

float kvo_f16_to_f32(uint16_t h)
{
    int s = (h >> 15) & 1;
    int e = (h >> 10) & 0x1F;
    int f = h & 0x3FF;
    double v;
    if (e == 0x1F)
        v = f ? NAN : INFINITY;
    else if (e == 0)
        v = ldexp((double)f, -24);
    else
        v = ldexp(1024.0 + f, e - 25);
    return (float)(s ? -v : v);
}

float kvo_bf16_to_f32(uint16_t b)
{
    uint32_t bits = (uint32_t)b << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return f;
}

void kvo_f32_to_f16_n(const float* x, int64_t n, uint16_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = kvo_f32_to_f16(x[i]);
}

void kvo_f16_to_f32_n(const uint16_t* h, int64_t n, float* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = kvo_f16_to_f32(h[i]);
}

/* ------------------------------------------------------------------------- */
/* Affine quantization ([P1] "Affine quantisation formula")                  */
/* ------------------------------------------------------------------------- */

static const float KVO_EPS = 1e-5f;   /* [P1] eps = 1e-5 */

/* Scale and zero of one slice of n values spaced by `stride`.
 * scale = max(eps, (max - min) / (qMax - qMin)), zero = min, both stored as
 * fp16 (the pages store scales and zeros as fp16).  qMax - qMin = 2^bits - 1:
 * 255 for int8 (-128..127) and 15 for int4 (-8..7).                          */
static void affine_params(const float* x, int n, int64_t stride, int bits,
                          uint16_t* scale16, uint16_t* zero16)
{
    float mn = x[0], mx = x[0];
    for (int i = 1; i < n; ++i) {
        float v = x[(int64_t)i * stride];
        if (v < mn) mn = v;
        if (v > mx) mx = v;
    }
    float levels = (float)((1 << bits) - 1);
    float range = mx - mn;
    float s = range / levels;
    if (s < KVO_EPS) s = KVO_EPS;
    *scale16 = kvo_f32_to_f16(s);
    *zero16 = kvo_f32_to_f16(mn);
}

/* Code of one value against the stored (fp16) scale and zero:
 * u = clamp(rint((x - zero) / scale), 0, 2^bits - 1), the offset code q - qMin.
 * Subtract, divide and round are single IEEE fp32 operations.                */
static uint8_t affine_code(float x, uint16_t scale16, uint16_t zero16, int bits)
{
    float s = kvo_f16_to_f32(scale16);
    float z = kvo_f16_to_f32(zero16);
    float diff = x - z;
    float ratio = diff / s;
    float y = rintf(ratio);
    float top = (float)((1 << bits) - 1);
    if (!(y >= 0.0f)) y = 0.0f;       /* also maps NaN to 0 */
    if (y > top) y = top;
    return (uint8_t)y;
}

void kvo_quant_tok_affine(const float* x, int64_t rows, int D, int G, int bits,
                          uint8_t* u, uint16_t* meta)
{
    int ng = D / G;
    for (int64_t r = 0; r < rows; ++r) {
        for (int g = 0; g < ng; ++g) {
            const float* xs = x + r * D + (int64_t)g * G;
            uint16_t s16, z16;
            affine_params(xs, G, 1, bits, &s16, &z16);
            meta[(r * ng + g) * 2 + 0] = s16;
            meta[(r * ng + g) * 2 + 1] = z16;
            for (int i = 0; i < G; ++i)
                u[r * D + (int64_t)g * G + i] = affine_code(xs[i], s16, z16, bits);
        }
    }
}

void kvo_quant_channel_group(const float* x, int Gt, int D, int bits,
                             uint8_t* u, uint16_t* meta)
{
    for (int d = 0; d < D; ++d) {
        uint16_t s16, z16;
        affine_params(x + d, Gt, D, bits, &s16, &z16);
        meta[d * 2 + 0] = s16;
        meta[d * 2 + 1] = z16;
        for (int t = 0; t < Gt; ++t)
            u[(int64_t)t * D + d] = affine_code(x[(int64_t)t * D + d], s16, z16, bits);
    }
}

/* ------------------------------------------------------------------------- */
/* Symmetric 4-bit blocks with optional mean-centering ([P3] "The idea")     */
/* ------------------------------------------------------------------------- */

/* Per block of 32 channels: x' = x - bias, d = max(eps, max|x'| / 7) stored as
 * fp16, q = clamp(rint(x' / d), -8, 7), code u = q + 8.  qMax = 7 is the
 * int4 constant of [P1]; the block size 32 with an fp16 scale is the Q4_0
 * shape.  A NULL bias means no centering.                                     */
void kvo_quant_sym4(const float* x, int64_t rows, int D, const float* bias,
                    uint8_t* u, uint16_t* scale)
{
    int nb = D / 32;
    float xc[32];
    for (int64_t r = 0; r < rows; ++r) {
        for (int b = 0; b < nb; ++b) {
            float amax = 0.0f;
            for (int i = 0; i < 32; ++i) {
                int d = b * 32 + i;
                float v = x[r * D + d];
                if (bias) v = v - bias[d];
                xc[i] = v;
                float av = fabsf(v);
                if (av > amax) amax = av;
            }
            float dd = amax / 7.0f;
            if (dd < KVO_EPS) dd = KVO_EPS;
            uint16_t d16 = kvo_f32_to_f16(dd);
            float df = kvo_f16_to_f32(d16);
            scale[r * nb + b] = d16;
            for (int i = 0; i < 32; ++i) {
                float y = rintf(xc[i] / df);
                if (!(y >= -8.0f)) y = -8.0f;
                if (y > 7.0f) y = 7.0f;
                u[r * D + b * 32 + i] = (uint8_t)(int)(y + 8.0f);
            }
        }
    }
}

/* ------------------------------------------------------------------------- */
/* Dequantization and decode attention (fp64)                                */
/* ------------------------------------------------------------------------- */

double kvo_dequant(const kvo_view* v, int t, int d)
{
    int D = v->D;
    switch (v->kind) {
    case KVO_PLAIN:
        return (double)v->plain[(int64_t)t * D + d];
    case KVO_CHANNEL: {
        if (t >= v->n_coded)
            return (double)v->plain[(int64_t)(t - v->n_coded) * D + d];
        int r = v->row[t];
        double s = kvo_f16_to_f32(v->meta[((int64_t)r * D + d) * 2 + 0]);
        double z = kvo_f16_to_f32(v->meta[((int64_t)r * D + d) * 2 + 1]);
        return (double)v->u[(int64_t)t * D + d] * s + z;
    }
    case KVO_TOK_AFFINE: {
        int ng = D / v->G;
        int g = d / v->G;
        double s = kvo_f16_to_f32(v->meta[((int64_t)t * ng + g) * 2 + 0]);
        double z = kvo_f16_to_f32(v->meta[((int64_t)t * ng + g) * 2 + 1]);
        return (double)v->u[(int64_t)t * D + d] * s + z;
    }
    case KVO_SYM4: {
        int nb = D / 32;
        double s = kvo_f16_to_f32(v->meta[(int64_t)t * nb + d / 32]);
        return ((double)v->u[(int64_t)t * D + d] - 8.0) * s;
    }
    }
    return NAN;
}

/* Softmax attention of one query over T cached slots, all in fp64:
 * logits l_t = scale * sum_d q_d k_t[d]; p_t = exp(l_t - max l) / sum exp(...);
 * out[d] = sum_t p_t v_t[d].  Keys and values are the dequantized cache
 * entries, so no full-precision copy of K or V is stored.                     */
void kvo_decode_head(const kvo_view* K, const kvo_view* V, int T,
                     const float* q, double scale, double* out)
{
    int D = K->D;
    for (int d = 0; d < D; ++d) out[d] = 0.0;
    if (T <= 0) return;
    double* logit = (double*)malloc(sizeof(double) * (size_t)T);
    double m = -INFINITY;
    for (int t = 0; t < T; ++t) {
        double acc = 0.0;
        for (int d = 0; d < D; ++d)
            acc += (double)q[d] * kvo_dequant(K, t, d);
        logit[t] = scale * acc;
        if (logit[t] > m) m = logit[t];
    }
    double denom = 0.0;
    for (int t = 0; t < T; ++t) {
        logit[t] = exp(logit[t] - m);
        denom += logit[t];
    }
    for (int t = 0; t < T; ++t) {
        double p = logit[t] / denom;
        for (int d = 0; d < D; ++d)
            out[d] += p * kvo_dequant(V, t, d);
    }
    free(logit);
}

/* ------------------------------------------------------------------------- */
/* RoPE on read ("StreamingLLM + KIVI", "RoPE caveat": keys stored before the  */
/* rotation, rotated at their slot index in the compressed cache)             */
/* ------------------------------------------------------------------------- */

void kvo_rope_rotate(double* x, int D, double base, int pos)
{
    int half = D / 2;
    for (int j = 0; j < half; ++j) {
        double theta = pow(base, -2.0 * (double)j / (double)D);
        double angle = (double)pos * theta;
        double c = cos(angle), s = sin(angle);
        double a = x[j], b = x[j + half];
        x[j] = a * c - b * s;
        x[j + half] = a * s + b * c;
    }
}

void kvo_decode_head_rope(const kvo_view* K, const kvo_view* V, int T,
                          const float* q, double scale, double base, int q_pos,
                          double* out)
{
    int D = K->D;
    for (int d = 0; d < D; ++d) out[d] = 0.0;
    if (T <= 0) return;
    double* qr = (double*)malloc(sizeof(double) * (size_t)D);
    double* kr = (double*)malloc(sizeof(double) * (size_t)D);
    double* logit = (double*)malloc(sizeof(double) * (size_t)T);
    for (int d = 0; d < D; ++d) qr[d] = (double)q[d];
    kvo_rope_rotate(qr, D, base, q_pos);
    double m = -INFINITY;
    for (int t = 0; t < T; ++t) {
        for (int d = 0; d < D; ++d) kr[d] = kvo_dequant(K, t, d);
        kvo_rope_rotate(kr, D, base, t);
        double acc = 0.0;
        for (int d = 0; d < D; ++d) acc += qr[d] * kr[d];
        logit[t] = scale * acc;
        if (logit[t] > m) m = logit[t];
    }
    double denom = 0.0;
    for (int t = 0; t < T; ++t) {
        logit[t] = exp(logit[t] - m);
        denom += logit[t];
    }
    for (int t = 0; t < T; ++t) {
        double p = logit[t] / denom;
        for (int d = 0; d < D; ++d)
            out[d] += p * kvo_dequant(V, t, d);
    }
    free(qr);
    free(kr);
    free(logit);
}

/* ------------------------------------------------------------------------- */
/* SnapKV ([P2] "How it works")                                              */
/* ------------------------------------------------------------------------- */

void kvo_snapkv_scores(const float* K, int S, int D, int w, double* score)
{
    for (int j = 0; j < S; ++j) score[j] = 0.0;
    if (S <= 0) return;
    int wc = w < S ? w : S;            /* obs_window clamped to S */
    if (wc <= 0) return;
    double inv_sqrt_d = 1.0 / sqrt((double)D);
    double* row = (double*)malloc(sizeof(double) * (size_t)S);
    for (int i = S - wc; i < S; ++i) {
        double m = -INFINITY;
        for (int j = 0; j < S; ++j) {
            double acc = 0.0;
            for (int d = 0; d < D; ++d)
                acc += (double)K[(int64_t)i * D + d] * (double)K[(int64_t)j * D + d];
            row[j] = acc * inv_sqrt_d;
            if (row[j] > m) m = row[j];
        }
        double denom = 0.0;
        for (int j = 0; j < S; ++j) {
            row[j] = exp(row[j] - m);
            denom += row[j];
        }
        for (int j = 0; j < S; ++j)
            score[j] += row[j] / denom;
    }
    for (int j = 0; j < S; ++j)
        score[j] /= (double)wc;
    free(row);
}

void kvo_snapkv_scores_rows(const float* Q, int n_rows, const float* K, int S, int D, double* score)
{
    for (int j = 0; j < S; ++j) score[j] = 0.0;
    if (S <= 0 || n_rows <= 0) return;
    double inv_sqrt_d = 1.0 / sqrt((double)D);
    double* row = (double*)malloc(sizeof(double) * (size_t)S);
    for (int r = 0; r < n_rows; ++r) {
        double m = -INFINITY;
        for (int j = 0; j < S; ++j) {
            double acc = 0.0;
            for (int d = 0; d < D; ++d)
                acc += (double)Q[(int64_t)r * D + d] * (double)K[(int64_t)j * D + d];
            row[j] = acc * inv_sqrt_d;
            if (row[j] > m) m = row[j];
        }
        double denom = 0.0;
        for (int j = 0; j < S; ++j) {
            row[j] = exp(row[j] - m);
            denom += row[j];
        }
        for (int j = 0; j < S; ++j)
            score[j] += row[j] / denom;
    }
    for (int j = 0; j < S; ++j)
        score[j] /= (double)n_rows;
    free(row);
}

void kvo_maxpool1d(const float* in, int S, int kernel, float* out)
{
    int r = (kernel - 1) / 2;
    for (int j = 0; j < S; ++j) {
        int lo = j - r < 0 ? 0 : j - r;
        int hi = j + r > S - 1 ? S - 1 : j + r;
        float m = in[lo];
        for (int t = lo + 1; t <= hi; ++t)
            if (in[t] > m) m = in[t];
        out[j] = m;
    }
}

typedef struct { float s; int32_t i; } kvo_cand;

/* Higher score first; equal scores: lower position first. */
static int cand_cmp(const void* a, const void* b)
{
    const kvo_cand* x = (const kvo_cand*)a;
    const kvo_cand* y = (const kvo_cand*)b;
    if (x->s > y->s) return -1;
    if (x->s < y->s) return 1;
    return (x->i > y->i) - (x->i < y->i);
}

static int int_cmp(const void* a, const void* b)
{
    int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
    return (x > y) - (x < y);
}

int kvo_snapkv_select(const float* score, int S, int n_sink, int budget, int32_t* kept)
{
    if (S <= 0 || budget <= 0) return 0;
    int n_keep = budget < S ? budget : S;
    int n_s = n_sink < n_keep ? n_sink : n_keep;
    if (n_s < 0) n_s = 0;
    int n_cand = S - n_s;
    kvo_cand* c = (kvo_cand*)malloc(sizeof(kvo_cand) * (size_t)(n_cand > 0 ? n_cand : 1));
    for (int j = 0; j < n_cand; ++j) {
        c[j].s = score[n_s + j];
        c[j].i = n_s + j;
    }
    qsort(c, (size_t)n_cand, sizeof(kvo_cand), cand_cmp);
    int k = 0;
    for (int j = 0; j < n_s; ++j) kept[k++] = j;          /* sink guarantee */
    for (int j = 0; j < n_keep - n_s; ++j) kept[k++] = c[j].i;
    qsort(kept, (size_t)k, sizeof(int32_t), int_cmp);     /* keep original order */
    free(c);
    return k;
}
