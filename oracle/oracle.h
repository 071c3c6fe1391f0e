/*
 * oracle.h -- C interface of the CPU oracle (test infrastructure only).
 *
 * Layouts: matrices are row-major [out][in] bf16 (uint16 bit patterns); the
 * KV cache is [n_layers][2 (K, V)][n_kv_heads][kv_capacity][head_dim] bf16.
 */
#ifndef ORC_ORACLE_H
#define ORC_ORACLE_H
#include <stddef.h>
#include <stdint.h>

typedef struct {
    int n_layers, hidden, n_heads, n_kv_heads, head_dim, intermediate, vocab, kv_capacity, qkv_bias;
    double rms_eps, rope_theta;
} orc_config;

typedef struct {
    const uint16_t *embed;      /* [vocab][hidden], also the LM head */
    const uint16_t *final_norm; /* [hidden] */
    /* per-layer arrays of n_layers pointers */
    const uint16_t *const *attn_norm, *const *wq, *const *wk, *const *wv;
    const uint16_t *const *bq, *const *bk, *const *bv; /* used when qkv_bias != 0 */
    const uint16_t *const *wo, *const *mlp_norm, *const *wgate, *const *wup, *const *wdown;
    const uint16_t *lm_head;    /* [vocab][hidden] vocabulary projection; NULL: the tied embedding */
} orc_weights;

/* Optional per-layer intermediates (any pointer may be NULL). */
typedef struct {
    float *x_in;    /* [n_layers][hidden]  residual stream entering the layer */
    float *q;       /* [n_layers][n_heads*hd] rotated queries */
    float *k;       /* [n_layers][n_kv*hd]   rotated keys (before bf16 rounding) */
    float *v;       /* [n_layers][n_kv*hd] */
    float *o;       /* [n_layers][n_heads*hd] attention output */
    float *x_mid;   /* [n_layers][hidden]  after the attention residual add */
    float *a;       /* [n_layers][intermediate] silu(gate)*up */
    float *x_final; /* [hidden] before the final norm */
} orc_trace;

float orc_bf16_to_f32(uint16_t h);
uint16_t orc_f32_to_bf16(float f);
void orc_rmsnorm(const float *x, const uint16_t *w, int n, double eps, float *out);
void orc_matvec(const uint16_t *W, const uint16_t *b, int M, int K, const float *x, float *y);
void orc_matvec_residual(const uint16_t *W, int M, int K, const float *v, float *x);
void orc_rope(float *v, int n_heads, int hd, int pos, double theta);
void orc_attention(const float *q, const uint16_t *K, const uint16_t *V, int nq, int nkv, int hd, int cap,
                   int Lc, float *o);
void orc_silu_mul(const float *g, const float *u, int n, float *out);
int orc_argmax(const float *v, int n);
size_t orc_kv_bytes(const orc_config *c);
/* Returns 0, or -1 for token/pos out of range, -2 for unsupported dims. */
int orc_decode_step(const orc_config *c, const orc_weights *w, uint16_t *kv, int token, int pos, float *logits,
                    int *argmax, orc_trace *tr);
int orc_num_threads(void);

/* FP8 (OCP E4M3) weight quantisation; see oracle.c. */
double orc_e4m3_value(int code);
uint8_t orc_e4m3_encode(double x);
int orc_fp8_row_exponent(const uint16_t *w, int n);
void orc_quantize_rows_e4m3(const uint16_t *W, int rows, int K, uint8_t *codes, int32_t *exps);
void orc_dequantize_rows_e4m3(const uint8_t *codes, const int32_t *exps, int rows, int K, uint16_t *W);

#endif
