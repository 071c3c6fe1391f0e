/*
 * oracle_driver.c -- host sanitizer run of the CPU oracle and the seeded input generator (test
 * infrastructure: built with -fsanitize=address,undefined by tests/test_sanitizers.py).
 *
 * Generates the tiny decoder's weights (2 layers, hidden 64, 4/2 heads of 16, SwiGLU 176, vocabulary 512,
 * 32 KV slots) from the generator, steps the oracle through every slot, and calls each building block on
 * edge sizes, so that any out-of-bounds access or undefined operation in either is reported.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "oracle.h"

uint64_t syn_key(uint64_t seed, const char *name);
void syn_normal_bf16(uint64_t key, double mean, double std, int64_t n, uint16_t *out);
void syn_tokens(uint64_t key, int64_t n, int32_t vocab, int32_t *out);
void syn_uniform(uint64_t key, int64_t n, double *out);

static uint16_t *drawn[64];
static int n_drawn;

static uint16_t *draw(const char *name, int64_t n, double mean, double std) {
    uint16_t *p = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)n);
    syn_normal_bf16(syn_key(0, name), mean, std, n, p);
    drawn[n_drawn++] = p;
    return p;
}

int main(void) {
    enum { NL = 2, H = 64, NQ = 4, NKV = 2, HD = 16, I = 176, V = 512, S = 32 };
    const orc_config c = {NL, H, NQ, NKV, HD, I, V, S, 1, 1e-5, 1e4};
    const uint16_t *attn_norm[NL], *wq[NL], *wk[NL], *wv[NL], *bq[NL], *bk[NL], *bv[NL], *wo[NL], *mlp_norm[NL],
        *wgate[NL], *wup[NL], *wdown[NL];
    for (int l = 0; l < NL; ++l) {
        attn_norm[l] = draw("attn_norm", H, 1.0, 0.02);
        wq[l] = draw("wq", (int64_t)NQ * HD * H, 0.0, 0.02);
        wk[l] = draw("wk", (int64_t)NKV * HD * H, 0.0, 0.02);
        wv[l] = draw("wv", (int64_t)NKV * HD * H, 0.0, 0.02);
        bq[l] = draw("bq", NQ * HD, 0.0, 0.02);
        bk[l] = draw("bk", NKV * HD, 0.0, 0.02);
        bv[l] = draw("bv", NKV * HD, 0.0, 0.02);
        wo[l] = draw("wo", (int64_t)H * NQ * HD, 0.0, 0.02);
        mlp_norm[l] = draw("mlp_norm", H, 1.0, 0.02);
        wgate[l] = draw("wgate", (int64_t)I * H, 0.0, 0.02);
        wup[l] = draw("wup", (int64_t)I * H, 0.0, 0.02);
        wdown[l] = draw("wdown", (int64_t)H * I, 0.0, 0.02);
    }
    const orc_weights w = {draw("embed", (int64_t)V * H, 0.0, 0.02), draw("final_norm", H, 1.0, 0.02),
                           attn_norm, wq, wk, wv, bq, bk, bv, wo, mlp_norm, wgate, wup, wdown};
    uint16_t *kv = (uint16_t *)calloc(orc_kv_bytes(&c), 1);
    float *logits = (float *)malloc(sizeof(float) * V);
    int32_t toks[S];
    syn_tokens(syn_key(1, "prompt"), S, V, toks);
    double u[4];
    syn_uniform(syn_key(2, "u"), 4, u);
    float x[H], xn[H], q[NQ * HD], o[NQ * HD], g[I], up[I], a[I];
    orc_trace tr = {0};
    float *tq = (float *)malloc(sizeof(float) * NL * NQ * HD);
    tr.q = tq;
    int bad = 0;
    for (int pos = 0; pos < S; ++pos) {
        int am = -1;
        const int tok = pos == 0 ? 0 : (pos == 1 ? V - 1 : toks[pos]);
        if (orc_decode_step(&c, &w, kv, tok, pos, logits, &am, &tr) != 0) bad = 1;
        for (int i = 0; i < V; ++i) bad |= !isfinite(logits[i]);
        bad |= am < 0 || am >= V;
    }
    /* out-of-range arguments are rejected, not read */
    int am;
    bad |= orc_decode_step(&c, &w, kv, V, 0, logits, &am, NULL) == 0;
    bad |= orc_decode_step(&c, &w, kv, 0, S, logits, &am, NULL) == 0;
    for (int i = 0; i < H; ++i) x[i] = (float)(i - 32) * 0.1f;
    orc_rmsnorm(x, w.final_norm, H, 1e-5, xn);
    orc_matvec(wq[0], bq[0], NQ * HD, H, xn, q);
    orc_rope(q, NQ, HD, S - 1, 1e4);
    orc_attention(q, kv, kv + (size_t)NKV * S * HD, NQ, NKV, HD, S, S, o);
    orc_attention(q, kv, kv + (size_t)NKV * S * HD, NQ, NKV, HD, S, 1, o);
    orc_matvec_residual(wo[0], H, NQ * HD, o, x);
    orc_matvec(wgate[0], NULL, I, H, xn, g);
    orc_matvec(wup[0], NULL, I, H, xn, up);
    orc_silu_mul(g, up, I, a);
    bad |= orc_argmax(a, 1) != 0 || orc_argmax(a, I) < 0;
    bad |= orc_f32_to_bf16(orc_bf16_to_f32(0x3f80)) != 0x3f80;
    printf("oracle driver: %s (%d threads)\n", bad ? "FAILED" : "ok", orc_num_threads());
    free(tq);
    free(logits);
    free(kv);
    for (int i = 0; i < n_drawn; ++i) free(drawn[i]);
    return bad;
}
