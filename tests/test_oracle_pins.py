"""Pins of the CPU oracle against facts fixed by the pages and by mathematics.

Each test is chosen so that a plausible mistake in the oracle (a dropped term,
a wrong sign or index, a transposed operand, eps outside the root, the wrong
RoPE pairing, the wrong GQA head mapping, a cache read before the append)
fails at least one of them.
"""
import os

import numpy as np
import pytest
from scipy.special import expit, softmax

import oracle
import synth
from synth import bf16_to_f32

from fullseq import forward as fullseq_forward

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
ONE_BF16 = 0x3F80


def _golden_int(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return int([l for l in f if l.strip() and not l.startswith("#")][0])


def _rng(seed=0):
    return np.random.default_rng(seed)


def _rand_bf16(shape, std, seed):
    return synth.normal_bf16(seed, "pin/%s" % (shape,), shape, 0.0, std)


# ---- configuration arithmetic -------------------------------------------------------------

def test_param_count_matches_page():
    assert synth.get("smollm135m-kv128").param_count() == _golden_int("smollm135m_param_count.txt")


# ---- bf16 --------------------------------------------------------------------------------------

def test_bf16_round_to_nearest_even():
    f = lambda bits: np.array([bits], np.uint32).view(np.float32)[0]
    assert oracle.f32_to_bf16(f(0x3F808000)) == 0x3F80          # tie -> even (down)
    assert oracle.f32_to_bf16(f(0x3F818000)) == 0x3F82          # tie -> even (up)
    assert oracle.f32_to_bf16(f(0x3F808001)) == 0x3F81          # above tie -> up
    assert oracle.f32_to_bf16(f(0xBF807FFF)) == 0xBF80          # below tie -> down (negative)
    assert oracle.f32_to_bf16(1.0) == ONE_BF16


# ---- RMSNorm -----------------------------------------------------------------------------------

def test_rmsnorm_constant_vector_closed_form():
    n, eps = 64, 1e-5
    w = _rand_bf16((n,), 0.5, 1)
    for c in [3.0, -0.25, 1e-3]:
        out = oracle.rmsnorm(np.full(n, c, np.float32), w, eps)
        want = c * bf16_to_f32(w).astype(np.float64) / np.sqrt(c * c + eps)
        np.testing.assert_allclose(out, want, rtol=1e-6)


def test_rmsnorm_unit_rms_and_scale_invariance():
    x = _rng(1).normal(size=576).astype(np.float32)
    ones = np.full(576, ONE_BF16, np.uint16)
    y = oracle.rmsnorm(x, ones, 0.0)
    assert abs(np.sqrt(np.mean(y.astype(np.float64) ** 2)) - 1.0) < 1e-6
    y2 = oracle.rmsnorm(x * np.float32(8.0), ones, 0.0)
    np.testing.assert_allclose(y2, y, rtol=1e-6)


# ---- matrix-vector product ---------------------------------------------------------------------

@pytest.mark.parametrize("M,K", [(7, 13), (192, 576), (64, 1536)])
def test_matvec_matches_numpy_float64(M, K):
    W = _rand_bf16((M, K), 0.02, 2)
    b = _rand_bf16((M,), 0.02, 3)
    x = _rng(2).normal(size=K).astype(np.float32)
    Wd = bf16_to_f32(W).astype(np.float64)
    np.testing.assert_allclose(oracle.matvec(W, x), Wd @ x.astype(np.float64), rtol=1e-6, atol=1e-7)
    np.testing.assert_allclose(oracle.matvec(W, x, b), Wd @ x + bf16_to_f32(b), rtol=1e-6, atol=1e-7)
    x0 = _rng(3).normal(size=M).astype(np.float32)
    np.testing.assert_allclose(oracle.matvec_residual(W, x, x0), x0 + Wd @ x, rtol=1e-6, atol=1e-7)


# ---- RoPE --------------------------------------------------------------------------------------

HD = 16


def test_rope_identity_at_position_zero():
    v = _rng(4).normal(size=3 * HD).astype(np.float32)
    assert np.array_equal(oracle.rope(v, 3, HD, 0, 1e4), v)


def test_rope_preserves_norm_of_each_head():
    v = _rng(5).normal(size=4 * 64).astype(np.float32)
    r = oracle.rope(v, 4, 64, 1234, 1e4)
    np.testing.assert_allclose(np.linalg.norm(r.reshape(4, 64), axis=1), np.linalg.norm(v.reshape(4, 64), axis=1),
                               rtol=1e-6)


def test_rope_relative_position_dot_product():
    q = _rng(6).normal(size=64).astype(np.float32)
    k = _rng(7).normal(size=64).astype(np.float32)
    for theta in [1e4, 1e6]:
        d = [float(np.dot(oracle.rope(q, 1, 64, m + s, theta).astype(np.float64),
                          oracle.rope(k, 1, 64, n + s, theta).astype(np.float64)))
             for (m, n, s) in [(10, 3, 0), (10, 3, 100), (10, 3, 2000)]]
        np.testing.assert_allclose(d[1:], [d[0]] * 2, rtol=2e-5, atol=2e-5)


def test_rope_composition():
    v = _rng(8).normal(size=2 * HD).astype(np.float32)
    a = oracle.rope(oracle.rope(v, 2, HD, 5, 1e4), 2, HD, 11, 1e4)
    np.testing.assert_allclose(a, oracle.rope(v, 2, HD, 16, 1e4), rtol=1e-5, atol=1e-6)


def test_rope_pairs_and_angles():
    """Unit vector e_i moves only within (i, i + hd/2) and turns by pos * theta^(-2i/hd)."""
    pos, theta, half = 3, 1e4, HD // 2
    for i in range(HD):
        e = np.zeros(HD, np.float32)
        e[i] = 1.0
        r = oracle.rope(e, 1, HD, pos, theta).astype(np.float64)
        base = i % half
        assert np.all(np.delete(r, [base, base + half]) == 0.0)
        ang = pos * theta ** (-2.0 * base / HD)
        start = 0.0 if i < half else np.pi / 2                          # e_i = angle 0 or pi/2 in the pair plane
        got = np.arctan2(r[base + half], r[base])
        assert abs(np.angle(np.exp(1j * (got - start - ang)))) < 1e-6


# ---- attention ---------------------------------------------------------------------------------

def _kv(nkv, cap, hd, seed, std=1.0):
    return synth.normal_bf16(seed, "pin/kv", (nkv, cap, hd), 0.0, std)


def test_attention_matches_softmax_brute_force():
    nq, nkv, hd, cap, Lc = 6, 2, 16, 40, 29
    K, V = _kv(nkv, cap, hd, 10), _kv(nkv, cap, hd, 11)
    q = _rng(9).normal(size=nq * hd).astype(np.float32)
    o = oracle.attention(q, K, V, nq, nkv, hd, Lc)
    Kf, Vf = bf16_to_f32(K).astype(np.float64), bf16_to_f32(V).astype(np.float64)
    for h in range(nq):
        j = h // (nq // nkv)
        p = softmax(Kf[j, :Lc] @ q[h * hd:(h + 1) * hd].astype(np.float64) / np.sqrt(hd))
        np.testing.assert_allclose(o[h * hd:(h + 1) * hd], p @ Vf[j, :Lc], rtol=1e-6, atol=1e-7)


def test_attention_single_position_returns_v0():
    nq, nkv, hd = 4, 2, 16
    K, V = _kv(nkv, 8, hd, 12), _kv(nkv, 8, hd, 13)
    q = _rng(10).normal(size=nq * hd).astype(np.float32)
    o = oracle.attention(q, K, V, nq, nkv, hd, 1).reshape(nq, hd)
    for h in range(nq):
        assert np.array_equal(o[h], bf16_to_f32(V[h // 2, 0]))


def test_attention_equal_keys_or_zero_query_gives_mean_of_v():
    nq, nkv, hd, Lc = 3, 1, 64, 4033
    V = _kv(nkv, Lc, hd, 14)
    K = np.repeat(_kv(nkv, 1, hd, 15), Lc, axis=1)
    q = _rng(11).normal(size=nq * hd).astype(np.float32)
    mean_v = bf16_to_f32(V[0]).astype(np.float64).mean(axis=0)
    np.testing.assert_allclose(oracle.attention(q, K, V, nq, nkv, hd, Lc).reshape(nq, hd), np.tile(mean_v, (nq, 1)),
                               rtol=1e-5, atol=1e-7)
    K2 = _kv(nkv, Lc, hd, 16)
    np.testing.assert_allclose(oracle.attention(np.zeros(nq * hd, np.float32), K2, V, nq, nkv, hd, Lc).reshape(nq, hd),
                               np.tile(mean_v, (nq, 1)), rtol=1e-5, atol=1e-7)


def test_attention_gqa_equals_mha_with_repeated_heads_and_maps_heads_in_blocks():
    nq, nkv, hd, cap, Lc = 6, 2, 16, 20, 17
    K, V = _kv(nkv, cap, hd, 17), _kv(nkv, cap, hd, 18)
    q = _rng(12).normal(size=nq * hd).astype(np.float32)
    g = nq // nkv
    o_gqa = oracle.attention(q, K, V, nq, nkv, hd, Lc)
    o_mha = oracle.attention(q, np.repeat(K, g, axis=0), np.repeat(V, g, axis=0), nq, nq, hd, Lc)
    assert np.array_equal(o_gqa, o_mha)
    # constant V per KV head: head h must see KV head h // g (not h % nkv)
    Vc = np.stack([np.full((cap, hd), 0x3F80 + 0x80 * j, np.uint16) for j in range(nkv)])
    o = oracle.attention(q, K, Vc, nq, nkv, hd, Lc).reshape(nq, hd)
    for h in range(nq):
        assert np.all(o[h] == bf16_to_f32(Vc[h // g, 0, 0]))


# ---- SwiGLU ------------------------------------------------------------------------------------

def test_silu_mul():
    g = np.array([0.0, 30.0, -30.0, 1.5, -0.7], np.float32)
    u = np.array([5.0, 1.0, 1.0, 2.0, 3.0], np.float32)
    out = oracle.silu_mul(g, u).astype(np.float64)
    assert out[0] == 0.0
    assert abs(out[1] - 30.0) < 1e-6 and abs(out[2]) < 1e-10
    np.testing.assert_allclose(out, g * expit(g.astype(np.float64)) * u, rtol=1e-6)


# ---- argmax ------------------------------------------------------------------------------------

def test_argmax_lowest_index_on_ties():
    v = np.array([1.0, 3.0, -2.0, 3.0, 3.0], np.float32)
    assert oracle.argmax(v) == 1
    x = _rng(13).normal(size=49152).astype(np.float32)
    assert oracle.argmax(x) == int(np.argmax(x))


# ---- whole decode step -------------------------------------------------------------------------

def _greedy_oracle_run(wl, W, positions, first_tokens, kv_prefix=None):
    m = oracle.Model(wl, W)
    if kv_prefix is not None:
        m.prefill_kv(kv_prefix)
    toks, logits = [], []
    tok = None
    for i, p in enumerate(positions):
        tok = first_tokens[i] if i < len(first_tokens) else tok
        lg, am, _ = m.step(tok, p)
        toks.append(tok)
        logits.append(lg.astype(np.float64))
        tok = am
    return toks, np.array(logits)


def test_stepwise_decode_equals_full_sequence_tiny():
    wl = synth.get("tiny-2L-h64-kv32")
    W = synth.make_weights(wl)
    prompt = list(synth.prompt_tokens(wl))
    toks, lg = _greedy_oracle_run(wl, W, list(range(24)), prompt)
    ref = fullseq_forward(wl, W, toks)
    std = lg.std(axis=1)
    assert np.all(np.max(np.abs(lg - ref), axis=1) <= 1e-3 * std)


def test_stepwise_decode_equals_full_sequence_smollm_slice_with_bias_variant():
    """Two layers at SmolLM-135M dims (and a biased, Qwen2-like eps/theta variant)."""
    base = synth.get("smollm135m-kv128").replace(n_layers=2, vocab=4096, kv_capacity=16)
    for wl in [base, base.replace(qkv_bias=True, rms_eps=1e-6, rope_theta=1e6)]:
        W = synth.make_weights(wl)
        toks = list(synth.tokens(9, "pin/slice", 6, wl.vocab))
        _, lg = _greedy_oracle_run(wl, W, list(range(6)), toks)
        ref = fullseq_forward(wl, W, toks)
        assert np.all(np.max(np.abs(lg - ref), axis=1) <= 1e-3 * lg.std(axis=1))


def test_stepwise_decode_over_prefilled_cache_equals_full_sequence():
    wl = synth.get("tiny-2L-h64-kv32").replace(kv_prefill=20, n_prompt=0)
    W = synth.make_weights(wl)
    pre = synth.kv_prefill(wl)
    toks = list(synth.tokens(4, "pin/pre", 5, wl.vocab))
    _, lg = _greedy_oracle_run(wl, W, list(range(20, 25)), toks, kv_prefix=pre)
    ref = fullseq_forward(wl, W, toks, start_pos=20, kv_prefix=pre)
    assert np.all(np.max(np.abs(lg - ref), axis=1) <= 1e-3 * lg.std(axis=1))


def test_cache_append_is_visible_to_the_same_step():
    """The step attends its own bf16-rounded key/value: with one position, o == bf16(v)."""
    wl = synth.get("tiny-2L-h64-kv32")
    W = synth.make_weights(wl)
    m = oracle.Model(wl, W)
    _, _, tr = m.step(7, 0, trace=True)
    for l in range(wl.n_layers):
        v = tr["v"][l].reshape(wl.n_kv_heads, wl.head_dim)
        vb = bf16_to_f32(np.array([oracle.f32_to_bf16(float(a)) for a in v.ravel()], np.uint16)).reshape(v.shape)
        o = tr["o"][l].reshape(wl.n_heads, wl.head_dim)
        for h in range(wl.n_heads):
            assert np.array_equal(o[h], vb[h // (wl.n_heads // wl.n_kv_heads)])
        assert np.array_equal(m.kv[l, 1, :, 0, :], np.array([[oracle.f32_to_bf16(float(a)) for a in r] for r in v]))


@pytest.mark.parametrize("name", ["tiny-2L-h64-kv32", "smollm135m-kv128"])
def test_zero_projections_give_closed_form_logits(name):
    """With W_o = W_down = 0 the residual stream stays E[t]: logits = E (w_f * E_t / rms(E_t))."""
    wl = synth.get(name)
    if wl.n_layers > 2:
        wl = wl.replace(n_layers=2)
    W = synth.make_weights(wl)
    for Lw in W["layers"]:
        Lw["wo"] = np.zeros_like(Lw["wo"])
        Lw["wdown"] = np.zeros_like(Lw["wdown"])
    t = 321
    m = oracle.Model(wl, W)
    lg, am, _ = m.step(t, 0)
    E = bf16_to_f32(W["embed"]).astype(np.float64)
    e = E[t]
    xf = e / np.sqrt(np.mean(e * e) + wl.rms_eps) * bf16_to_f32(W["final_norm"])
    np.testing.assert_allclose(lg, E @ xf, rtol=2e-5, atol=2e-5 * np.abs(E @ xf).max())
    assert am == t
