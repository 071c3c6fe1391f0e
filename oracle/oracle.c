/*
 * oracle.c -- plain, slow CPU reference of one batch-1 decode step of a
 * pre-norm Llama-style decoder.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the GPU path.
 *
 * What the step computes follows the third-party MegaBake article ("MegaBake:
 * a PyTorch model compiled into one CUDA kernel", section "What a megakernel
 * is, and why small models want one"): per layer an RMSNorm, the Q/K/V
 * projections, RoPE, attention, the output projection, a residual add, a
 * second RMSNorm, the gate and up projections, SiLU, the down projection and
 * a second residual add.  The MegaBake README mirror (section "Current
 * status") adds the embedding, the final norm, the vocabulary projection and
 * the KV-cache update inside the step.  Greedy argmax of the logits ends it.
 *
 * Precision: weights and the KV cache are bf16 (used as their exact fp32
 * values); every other tensor is stored fp32.  Each dot product, sum and
 * softmax accumulates in double and is rounded to fp32 once per named output
 * (xn, q, k, v after bias, q/k after rotation, o, x after each residual add,
 * the SiLU*up product, logits).  The result is therefore independent of
 * summation order and at least as accurate as any fp32 implementation.
 *
 * Readings of points the pages leave open (all Hugging Face Llama/Qwen2
 * conventions): RMSNorm is x * (mean(x^2) + eps)^-1/2 * w; RoPE rotates the
 * pairs (i, i + hd/2) of every query and key head by pos * theta^(-2i/hd);
 * keys are cached after rotation; the cache holds bf16 (round to nearest
 * even) and attention reads the rounded values, the current position
 * included; attention is causal over 0..pos with scale 1/sqrt(hd) and query
 * head h reads KV head floor(h / (n_heads / n_kv_heads)); the LM head is the
 * tied embedding; argmax returns the lowest index among equal maxima.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "oracle.h"

#ifdef _OPENMP
#include <omp.h>
#endif

/* ---- bf16 <-> fp32 -------------------------------------------------------- */

float orc_bf16_to_f32(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* Round-to-nearest-even truncation of an fp32 to its top 16 bits. */
uint16_t orc_f32_to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return (uint16_t)((u >> 16) | 0x40);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7fffu + lsb;
    return (uint16_t)(u >> 16);
}

#define W(p) ((double)orc_bf16_to_f32(p))

/* ---- building blocks -------------------------------------------------------- */

/* RMSNorm (article, "What a megakernel is"; folded into its consumer in the
 * section "How a model gets in", step 4): out = x / sqrt(mean(x^2) + eps) * w. */
void orc_rmsnorm(const float *x, const uint16_t *w, int n, double eps, float *out) {
    double ss = 0.0;
    for (int i = 0; i < n; ++i) ss += (double)x[i] * (double)x[i];
    double r = 1.0 / sqrt(ss / (double)n + eps);
    for (int i = 0; i < n; ++i) out[i] = (float)((double)x[i] * r * W(w[i]));
}

/* y[r] = sum_k W[r][k] x[k] (+ b[r]) for a row-major [M][K] bf16 matrix.
 * The projections and the vocabulary head are all this product at batch 1
 * (article, section "How a model gets in", step 3; README "Current status":
 * bias added to the addmm result). */
void orc_matvec(const uint16_t *Wm, const uint16_t *b, int M, int K, const float *x, float *y) {
#pragma omp parallel for schedule(static)
    for (int r = 0; r < M; ++r) {
        const uint16_t *row = Wm + (size_t)r * (size_t)K;
        double acc = 0.0;
        for (int k = 0; k < K; ++k) acc += W(row[k]) * (double)x[k];
        if (b) acc += W(b[r]);
        y[r] = (float)acc;
    }
}

/* x[r] += sum_k W[r][k] v[k]: a projection followed by the residual add,
 * rounded once (article, "What a megakernel is": output projection then
 * residual add; down projection then another add). */
void orc_matvec_residual(const uint16_t *Wm, int M, int K, const float *v, float *x) {
#pragma omp parallel for schedule(static)
    for (int r = 0; r < M; ++r) {
        const uint16_t *row = Wm + (size_t)r * (size_t)K;
        double acc = (double)x[r];
        for (int k = 0; k < K; ++k) acc += W(row[k]) * (double)v[k];
        x[r] = (float)acc;
    }
}

/* Rotary position embedding of n_heads heads of size hd, in place.  Pair
 * (i, i + hd/2) of each head turns by angle pos * theta^(-2i/hd). */
void orc_rope(float *v, int n_heads, int hd, int pos, double theta) {
    int half = hd / 2;
    for (int i = 0; i < half; ++i) {
        double ang = (double)pos * pow(theta, -2.0 * (double)i / (double)hd);
        double c = cos(ang), s = sin(ang);
        for (int h = 0; h < n_heads; ++h) {
            float *p = v + (size_t)h * hd;
            double u = p[i], w = p[i + half];
            p[i] = (float)(u * c - w * s);
            p[i + half] = (float)(w * c + u * s);
        }
    }
}

/* Causal decode attention of one query token over cached positions 0..Lc-1.
 * K and V point at one layer's [n_kv][cap][hd] bf16 blocks.  Query head h
 * uses KV head h / (nq / nkv) (grouped-query attention, README "Current
 * status": query heads sharing a KV head).  Softmax of q.k / sqrt(hd), max
 * subtracted, then the weighted sum of V.  The split-context merge of the GPU
 * path is not modelled here: this is the unsplit definition. */
void orc_attention(const float *q, const uint16_t *K, const uint16_t *V, int nq, int nkv, int hd,
                   int cap, int Lc, float *o) {
    int g = nq / nkv;
    double scale = 1.0 / sqrt((double)hd);
#pragma omp parallel for schedule(static)
    for (int h = 0; h < nq; ++h) {
        int j = h / g;
        const uint16_t *Kj = K + (size_t)j * cap * hd;
        const uint16_t *Vj = V + (size_t)j * cap * hd;
        const float *qh = q + (size_t)h * hd;
        double *s = (double *)malloc(sizeof(double) * (size_t)Lc);
        double m = -INFINITY;
        for (int t = 0; t < Lc; ++t) {
            double d = 0.0;
            for (int e = 0; e < hd; ++e) d += (double)qh[e] * W(Kj[(size_t)t * hd + e]);
            s[t] = d * scale;
            if (s[t] > m) m = s[t];
        }
        double den = 0.0;
        for (int t = 0; t < Lc; ++t) {
            s[t] = exp(s[t] - m);
            den += s[t];
        }
        for (int e = 0; e < hd; ++e) {
            double acc = 0.0;
            for (int t = 0; t < Lc; ++t) acc += s[t] * W(Vj[(size_t)t * hd + e]);
            o[(size_t)h * hd + e] = (float)(acc / den);
        }
        free(s);
    }
}

/* SwiGLU activation: silu(g) * u, silu(z) = z / (1 + exp(-z)) (article,
 * "What a megakernel is": gate and up projections, SiLU). */
void orc_silu_mul(const float *g, const float *u, int n, float *out) {
    for (int i = 0; i < n; ++i) {
        double z = g[i];
        out[i] = (float)(z / (1.0 + exp(-z)) * (double)u[i]);
    }
}

/* Index of the largest value; the lowest index wins ties. */
int orc_argmax(const float *v, int n) {
    int best = 0;
    for (int i = 1; i < n; ++i)
        if (v[i] > v[best]) best = i;
    return best;
}

/* ---- one decode step -------------------------------------------------------- */

size_t orc_kv_bytes(const orc_config *c) {
    return (size_t)c->n_layers * 2 * c->n_kv_heads * c->kv_capacity * c->head_dim * sizeof(uint16_t);
}

static uint16_t *kv_block(const orc_config *c, uint16_t *kv, int layer, int which) {
    size_t blk = (size_t)c->n_kv_heads * c->kv_capacity * c->head_dim;
    return kv + ((size_t)layer * 2 + which) * blk;
}

int orc_decode_step(const orc_config *c, const orc_weights *w, uint16_t *kv, int token, int pos,
                    float *logits, int *argmax, orc_trace *tr) {
    const int H = c->hidden, hd = c->head_dim, nq = c->n_heads, nkv = c->n_kv_heads;
    const int Q = nq * hd, KV = nkv * hd, I = c->intermediate;
    if (token < 0 || token >= c->vocab || pos < 0 || pos >= c->kv_capacity) return -1;
    if (nkv <= 0 || nq % nkv != 0 || hd % 2 != 0) return -2;

    float *x = (float *)malloc(sizeof(float) * H);
    float *xn = (float *)malloc(sizeof(float) * H);
    float *q = (float *)malloc(sizeof(float) * Q);
    float *k = (float *)malloc(sizeof(float) * KV);
    float *v = (float *)malloc(sizeof(float) * KV);
    float *o = (float *)malloc(sizeof(float) * Q);
    float *gt = (float *)malloc(sizeof(float) * I);
    float *up = (float *)malloc(sizeof(float) * I);
    float *a = (float *)malloc(sizeof(float) * I);

    /* Embedding gather (README mirror, "Current status": the kernel covers the embedding). */
    for (int i = 0; i < H; ++i) x[i] = orc_bf16_to_f32(w->embed[(size_t)token * H + i]);

    for (int l = 0; l < c->n_layers; ++l) {
        if (tr && tr->x_in) memcpy(tr->x_in + (size_t)l * H, x, sizeof(float) * H);
        orc_rmsnorm(x, w->attn_norm[l], H, c->rms_eps, xn);
        orc_matvec(w->wq[l], c->qkv_bias ? w->bq[l] : NULL, Q, H, xn, q);
        orc_matvec(w->wk[l], c->qkv_bias ? w->bk[l] : NULL, KV, H, xn, k);
        orc_matvec(w->wv[l], c->qkv_bias ? w->bv[l] : NULL, KV, H, xn, v);
        orc_rope(q, nq, hd, pos, c->rope_theta);
        orc_rope(k, nkv, hd, pos, c->rope_theta);
        if (tr && tr->q) memcpy(tr->q + (size_t)l * Q, q, sizeof(float) * Q);
        if (tr && tr->k) memcpy(tr->k + (size_t)l * KV, k, sizeof(float) * KV);
        if (tr && tr->v) memcpy(tr->v + (size_t)l * KV, v, sizeof(float) * KV);
        /* KV-cache update: slot pos of layer l receives bf16(k), bf16(v). */
        uint16_t *Kl = kv_block(c, kv, l, 0), *Vl = kv_block(c, kv, l, 1);
        for (int j = 0; j < nkv; ++j)
            for (int e = 0; e < hd; ++e) {
                Kl[((size_t)j * c->kv_capacity + pos) * hd + e] = orc_f32_to_bf16(k[j * hd + e]);
                Vl[((size_t)j * c->kv_capacity + pos) * hd + e] = orc_f32_to_bf16(v[j * hd + e]);
            }
        orc_attention(q, Kl, Vl, nq, nkv, hd, c->kv_capacity, pos + 1, o);
        if (tr && tr->o) memcpy(tr->o + (size_t)l * Q, o, sizeof(float) * Q);
        orc_matvec_residual(w->wo[l], H, Q, o, x);
        if (tr && tr->x_mid) memcpy(tr->x_mid + (size_t)l * H, x, sizeof(float) * H);
        orc_rmsnorm(x, w->mlp_norm[l], H, c->rms_eps, xn);
        orc_matvec(w->wgate[l], NULL, I, H, xn, gt);
        orc_matvec(w->wup[l], NULL, I, H, xn, up);
        orc_silu_mul(gt, up, I, a);
        if (tr && tr->a) memcpy(tr->a + (size_t)l * I, a, sizeof(float) * I);
        orc_matvec_residual(w->wdown[l], H, I, a, x);
    }
    if (tr && tr->x_final) memcpy(tr->x_final, x, sizeof(float) * H);
    /* Final norm, tied vocabulary projection, greedy argmax. */
    orc_rmsnorm(x, w->final_norm, H, c->rms_eps, xn);
    orc_matvec(w->lm_head ? w->lm_head : w->embed, NULL, c->vocab, H, xn, logits);
    if (argmax) *argmax = orc_argmax(logits, c->vocab);

    free(x); free(xn); free(q); free(k); free(v); free(o); free(gt); free(up); free(a);
    return 0;
}

int orc_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ---- FP8 weights ------------------------------------------------------------------------------------
 * The pages name FP8 only as a direction of the project (MegaBake project site, "Next"); the format and
 * the scaling are this implementation's readings, stated here once:
 *  - codes are OCP 8-bit floating point, E4M3 variant: sign bit, 4 exponent bits with bias 7, 3 mantissa
 *    bits; exponent field 0 holds the subnormals (m / 8) * 2^-6; the patterns S.1111.111 are NaN, so the
 *    largest finite magnitude is 1.75 * 2^8 = 448; there are no infinities;
 *  - every output row r of a weight matrix has one power-of-two scale 2^e_r, e_r the smallest integer
 *    not below -126 with max_k |W[r][k]| / 2^e_r <= 448 (0 for an all-zero row), so no weight saturates;
 *  - code[r][k] is W[r][k] / 2^e_r (exact: a power-of-two scaling) rounded to the nearest E4M3 value,
 *    ties to the even code; the sign of the weight is kept, zero included.
 * The weight a code stands for, value(code) * 2^e_r, has at most 4 significant bits and an exponent
 * well inside bf16's range, so it is exactly a bf16 value: the quantised model is a bf16 model that
 * orc_decode_step runs unchanged. */

double orc_e4m3_value(int code) {
    const int s = (code >> 7) & 1, e = (code >> 3) & 15, m = code & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) v = ldexp((double)m / 8.0, -6);
    else v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -v : v;
}

/* Nearest E4M3 code of a finite x with |x| <= 448, ties to even: the spacing of the binade |x| falls in
 * (2^-9 below 2^-6, else 2^(E-3) for |x| in [2^E, 2^(E+1))), the multiple of it nearest to |x| (the
 * division is exact; nearbyint rounds halves to even), then the fields of that value. */
uint8_t orc_e4m3_encode(double x) {
    const int s = signbit(x) ? 1 : 0;
    const double a = fabs(x);
    if (a == 0.0) return (uint8_t)(s << 7);
    int E2;
    (void)frexp(a, &E2);          /* a = f * 2^E2, f in [0.5, 1): a in [2^(E2-1), 2^E2) */
    const int E = E2 - 1;
    int code;
    if (E < -6) {
        const double n = nearbyint(ldexp(a, 9));     /* multiples of 2^-9: 0 .. 8 */
        code = (int)n;                                /* 8 is 2^-6, the smallest normal (field 1) */
    } else {
        double n = nearbyint(ldexp(a, 3 - E));        /* 8 .. 16 multiples of 2^(E-3) */
        int Ex = E;
        if (n >= 16.0) { n = 8.0; ++Ex; }
        code = ((Ex + 7) << 3) | ((int)n - 8);
    }
    return (uint8_t)((s << 7) | code);
}

int orc_fp8_row_exponent(const uint16_t *w, int n) {
    double amax = 0.0;
    for (int i = 0; i < n; ++i) amax = fmax(amax, fabs((double)orc_bf16_to_f32(w[i])));
    if (amax == 0.0) return 0;
    int e = -126;
    while (ldexp(amax, -e) > 448.0) ++e;
    return e;
}

void orc_quantize_rows_e4m3(const uint16_t *W, int rows, int K, uint8_t *codes, int32_t *exps) {
#pragma omp parallel for schedule(static)
    for (int r = 0; r < rows; ++r) {
        const uint16_t *w = W + (size_t)r * K;
        const int e = orc_fp8_row_exponent(w, K);
        exps[r] = e;
        for (int k = 0; k < K; ++k) codes[(size_t)r * K + k] = orc_e4m3_encode(ldexp((double)orc_bf16_to_f32(w[k]), -e));
    }
}

/* The bf16 weights the codes stand for (exact; see above). */
void orc_dequantize_rows_e4m3(const uint8_t *codes, const int32_t *exps, int rows, int K, uint16_t *W) {
#pragma omp parallel for schedule(static)
    for (int r = 0; r < rows; ++r)
        for (int k = 0; k < K; ++k)
            W[(size_t)r * K + k] = orc_f32_to_bf16((float)ldexp(orc_e4m3_value(codes[(size_t)r * K + k]), exps[r]));
}
