"""Pins of the oracle's FP8 (OCP E4M3) weight quantiser.

The format facts come from the OCP 8-bit floating point specification (E4M3: bias 7, 3 mantissa bits,
subnormals at exponent field 0, S.1111.111 the only NaN patterns, largest finite 448); the encoder is
checked against those facts, against a nearest-value brute force over every code, and against PyTorch's
own float8_e4m3fn conversion (an independent implementation of the same format).  A plausible mistake in
the oracle -- a wrong bias, subnormal spacing, rounding that is not ties-to-even, a dropped sign, a scale
that saturates -- fails one of them."""
import numpy as np
import pytest
import torch

import oracle
import synth
from synth import bf16_to_f32

FINITE = [c for c in range(256) if (c & 0x7F) != 0x7F]


def _values(codes):
    return np.array([oracle.e4m3_value(c) for c in codes])


def test_format_fixed_points():
    assert oracle.e4m3_value(0x7E) == 448.0            # largest finite
    assert oracle.e4m3_value(0x08) == 2.0 ** -6        # smallest normal
    assert oracle.e4m3_value(0x01) == 2.0 ** -9        # smallest subnormal
    assert oracle.e4m3_value(0x07) == 7 * 2.0 ** -9    # largest subnormal
    assert oracle.e4m3_value(0x38) == 1.0
    assert oracle.e4m3_value(0xB8) == -1.0
    assert np.isnan(oracle.e4m3_value(0x7F)) and np.isnan(oracle.e4m3_value(0xFF))
    assert oracle.e4m3_value(0x80) == 0.0 and np.signbit(oracle.e4m3_value(0x80))
    pos = _values(range(0x7F))
    assert np.all(np.diff(pos) > 0), "positive codes are ordered by value"
    assert len(set(pos.tolist())) == 127


def test_values_match_torch_float8_e4m3fn():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = _values(range(256))
    both_nan = np.isnan(ref) & np.isnan(mine)
    assert np.all(both_nan | (ref == mine))


def test_every_finite_code_encodes_to_itself():
    for c in FINITE:
        assert oracle.e4m3_encode(oracle.e4m3_value(c)) == c, hex(c)


def test_midpoints_round_to_the_even_code():
    for c in range(0x7E):                      # neighbours c, c + 1 among the positive finite codes
        lo, hi = oracle.e4m3_value(c), oracle.e4m3_value(c + 1)
        mid = (lo + hi) / 2
        even = c if c % 2 == 0 else c + 1
        assert oracle.e4m3_encode(mid) == even, hex(c)
        assert oracle.e4m3_encode(-mid) == 0x80 | even
        assert oracle.e4m3_encode(np.nextafter(mid, 0)) == c
        assert oracle.e4m3_encode(np.nextafter(mid, 1e9)) == c + 1
    # below half the smallest subnormal: zero; exactly half: ties to the even code 0
    assert oracle.e4m3_encode(2.0 ** -10) == 0
    assert oracle.e4m3_encode(np.nextafter(2.0 ** -10, 1)) == 1


def test_encoder_is_the_nearest_value_by_brute_force():
    rng = np.random.default_rng(5)
    pos = _values(range(0x7F))
    x = np.concatenate([rng.uniform(-448, 448, 3000), rng.standard_normal(3000) * 0.05,
                        np.exp(rng.uniform(np.log(2.0 ** -12), np.log(448), 3000)) * rng.choice([-1, 1], 3000)])
    for v in x:
        d = np.abs(pos - abs(v))
        best = np.flatnonzero(d == d.min())
        c = int(best[0]) if len(best) == 1 else int([b for b in best if b % 2 == 0][0])
        want = c | (0x80 if np.signbit(v) else 0)
        assert oracle.e4m3_encode(v) == want, (v, hex(want))


def test_encoder_matches_torch_conversion():
    rng = np.random.default_rng(6)
    x = np.concatenate([rng.uniform(-448, 448, 20000), rng.standard_normal(20000) * 0.01]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    mine = np.array([oracle.e4m3_encode(float(v)) for v in x], dtype=np.uint8)
    assert np.array_equal(ref, mine)


def _bf16(vals):
    return np.array([oracle.f32_to_bf16(v) for v in vals], dtype=np.uint16)


def test_row_exponent_is_the_smallest_that_fits():
    rng = np.random.default_rng(7)
    rows = [rng.standard_normal(64) * s for s in (1e-3, 0.02, 1.0, 300.0, 1e5)]
    rows += [np.full(8, 448.0), np.full(8, 449.0), np.full(8, 896.0), np.full(8, 897.0), np.zeros(8)]
    for r in rows:
        w = _bf16(r)
        e = oracle.fp8_row_exponent(w)
        amax = np.abs(bf16_to_f32(w).astype(np.float64)).max()
        if amax == 0:
            assert e == 0
            continue
        assert amax / 2.0 ** e <= 448.0
        assert e == -126 or amax / 2.0 ** (e - 1) > 448.0
    assert oracle.fp8_row_exponent(_bf16([448.0])) == 0
    assert oracle.fp8_row_exponent(_bf16([896.0])) == 1
    assert oracle.fp8_row_exponent(_bf16([1e-38])) == -126     # the lower clamp


def test_quantised_rows_dequantise_exactly_to_bf16():
    W = synth.normal_bf16(9, "fp8/pin", (48, 96), 0.0, 0.05)
    W[3] = 0
    W[5, 7] = _bf16([-0.0])[0]
    codes, exps = oracle.quantize_e4m3_rows(W)
    assert exps[3] == 0 and not codes[3].any()
    assert codes[5, 7] == 0x80                         # the sign of zero is kept
    D = oracle.dequantize_e4m3_rows(codes, exps)
    want = _values(range(256))[codes] * np.ldexp(1.0, exps)[:, None]
    assert np.array_equal(bf16_to_f32(D).astype(np.float64), want)
    # every weight moved by at most half the spacing of its binade: 2^-4 of its magnitude, or 2^-10 * 2^e
    w = bf16_to_f32(W).astype(np.float64)
    err = np.abs(want - w)
    bound = np.maximum(np.abs(w) * 2.0 ** -4, np.ldexp(2.0 ** -10, exps)[:, None])
    assert np.all(err <= bound)
    # no code is NaN, and every nonzero row's largest magnitude, scaled into (224, 448] before rounding,
    # rounds into [224, 448]: the scale uses the top of the range and never saturates
    assert not np.any((codes & 0x7F) == 0x7F)
    amax_codes = np.abs(_values(range(256))[codes]).max(axis=1)
    nz = np.abs(bf16_to_f32(W)).max(axis=1) > 0
    assert np.all((amax_codes[nz] >= 224) & (amax_codes[nz] <= 448))


def test_lm_head_pointer():
    """A separate vocabulary projection equal to the embedding gives the tied result bit for bit; a zero
    one gives zero logits (argmax 0, the lowest index)."""
    wl = synth.get("tiny-2L-h64-kv32")
    W = synth.make_weights(wl)
    a, b = oracle.Model(wl, W), oracle.Model(wl, dict(W, lm_head=W["embed"].copy()))
    c = oracle.Model(wl, dict(W, lm_head=np.zeros_like(W["embed"])))
    for pos, t in enumerate((3, 9, 27)):
        la, ia, _ = a.step(t, pos)
        lb, ib, _ = b.step(t, pos)
        lc, ic, _ = c.step(t, pos)
        assert np.array_equal(la.view(np.uint32), lb.view(np.uint32)) and ia == ib
        assert not lc.any() and ic == 0


@pytest.mark.parametrize("name", ["tiny-2L-h64-kv32", "smollm135m-kv128"])
def test_fp8_model_stays_close_to_bf16(name):
    """The quantised model is a perturbation of the bf16 one of relative size about 2^-5 per weight:
    its logits after a few steps stay within a few percent of the bf16 model's (relative L2)."""
    wl = synth.get(name)
    if name != "tiny-2L-h64-kv32":
        wl = wl.replace(n_layers=2, vocab=4096, kv_capacity=16)
    W = synth.make_weights(wl)
    Wq, q = oracle.fp8_weights(W)
    for l, L in enumerate(q["layers"]):
        for n, (codes, exps) in L.items():
            assert codes.shape == W["layers"][l][n].shape and exps.shape == (codes.shape[0],)
    a, b = oracle.Model(wl, W), oracle.Model(wl, Wq)
    toks = synth.tokens(3, "fp8-close", 6, wl.vocab)
    for pos, t in enumerate(toks):
        la, _, _ = a.step(int(t), pos)
        lb, _, _ = b.step(int(t), pos)
    rel = np.linalg.norm(la - lb) / np.linalg.norm(la)
    assert 0 < rel < 0.1, rel
