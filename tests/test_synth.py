"""The seeded input generator: definition, determinism and distribution."""
import math

import numpy as np
import pytest

import synth


def _mix64(z):
    m = (1 << 64) - 1
    z ^= z >> 30
    z = (z * 0xBF58476D1CE4E5B9) & m
    z ^= z >> 27
    z = (z * 0x94D049BB133111EB) & m
    z ^= z >> 31
    return z


def _key(seed, name):
    h = 0xcbf29ce484222325
    for b in name.encode():
        h = ((h ^ b) * 0x100000001b3) & ((1 << 64) - 1)
    return _mix64(_mix64((seed + 0x9E3779B97F4A7C15) & ((1 << 64) - 1)) ^ h)


def _uniform(key, i):
    x = _mix64((key + (i + 1) * 0x9E3779B97F4A7C15) & ((1 << 64) - 1))
    return ((x >> 11) + 0.5) * 2.0 ** -53


def test_key_and_uniform_match_python_definition():
    for seed, name in [(0, "a"), (7, "L3/wq"), (123456789, "x" * 40)]:
        k = _key(seed, name)
        assert synth.key(seed, name) == k
        u = synth.uniform(seed, name, 16)
        assert np.array_equal(u, np.array([_uniform(k, i) for i in range(16)]))


def test_normal_matches_box_muller_definition():
    n = 4001
    k = synth.key(5, "bm")
    got = synth.bf16_to_f32(synth.normal_bf16(5, "bm", (n,), 0.0, 1.0)).astype(np.float64)
    want = []
    for j in range((n + 1) // 2):
        ua, ub = _uniform(k, 2 * j), _uniform(k, 2 * j + 1)
        r = math.sqrt(-2.0 * math.log(ua))
        want += [r * math.cos(2 * math.pi * ub), r * math.sin(2 * math.pi * ub)]
    want = np.array(want[:n])
    # bf16 keeps 8 significant bits: allow one bf16 ulp for libm rounding differences.
    assert np.all(np.abs(got - want) <= np.abs(want) * 2.0 ** -7 + 1e-30)


def test_deterministic_and_prefix_stable():
    a = synth.normal_bf16(0, "t", (1000,), 0.0, 0.02)
    b = synth.normal_bf16(0, "t", (1000,), 0.0, 0.02)
    c = synth.normal_bf16(0, "t", (400,), 0.0, 0.02)
    d = synth.normal_bf16(1, "t", (1000,), 0.0, 0.02)
    assert np.array_equal(a, b)
    assert np.array_equal(a[:400], c)
    assert not np.array_equal(a, d)


def test_distribution_moments():
    x = synth.bf16_to_f32(synth.normal_bf16(0, "moments", (1 << 20,), 1.0, 0.02)).astype(np.float64)
    assert abs(x.mean() - 1.0) < 1e-4
    assert abs(x.std() - 0.02) < 2e-4
    # shape moments on a zero-mean draw (near 1.0 the bf16 step is 0.4 sigma and skews them)
    z = synth.bf16_to_f32(synth.normal_bf16(0, "moments0", (1 << 20,), 0.0, 1.0)).astype(np.float64)
    assert abs(z.mean()) < 5e-3 and abs(z.std() - 1.0) < 5e-3
    assert abs(np.mean(z ** 3)) < 0.02 and abs(np.mean(z ** 4) - 3.0) < 0.05


def test_tokens_in_range_and_spread():
    t = synth.tokens(1, "tok", 20000, 512)
    assert t.min() >= 0 and t.max() < 512
    counts = np.bincount(t, minlength=512)
    assert counts.min() > 0


def test_workload_weights_shapes_and_sharing():
    w = synth.get("tiny-2L-h64-kv32")
    W = synth.make_weights(w)
    assert W["embed"].shape == (512, 64) and len(W["layers"]) == 2
    L0 = W["layers"][0]
    assert L0["wq"].shape == (64, 64) and L0["wk"].shape == (32, 64) and L0["wdown"].shape == (64, 176)
    # the two SmolLM-135M workloads share one weight stream
    a, b = synth.get("smollm135m-kv128"), synth.get("smollm135m-kv4096")
    assert synth._shape_key(a) == synth._shape_key(b)


def test_kv_prefill_prefix_stable():
    w = synth.get("tiny-2L-h64-kv32").replace(kv_prefill=12)
    a = synth.kv_prefill(w, 12)
    b = synth.kv_prefill(w, 5)
    assert a.shape == (2, 2, 2, 12, 16)
    assert np.array_equal(a[:, :, :, :5], b)
