"""Independent float64 full-sequence forward of the decoder, used to pin the oracle.

Written in matrix form over all positions at once (causal mask, scipy
softmax, RoPE as multiplication of complex numbers), so it shares neither
structure nor code with the oracle's step-at-a-time C implementation.  Keys
and values are rounded to bf16 before attention, as the cache stores them.
"""
from __future__ import annotations

import numpy as np
from scipy.special import expit, softmax

from synth import bf16_to_f32


def bf16_round(a: np.ndarray) -> np.ndarray:
    """float64 -> float32 -> bf16 (round to nearest even) -> float64."""
    f = np.asarray(a, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return bf16_to_f32(u.astype(np.uint16)).astype(np.float64)


def _norm(X, w, eps):
    return X / np.sqrt(np.mean(X * X, axis=-1, keepdims=True) + eps) * w


def _rotate(Z, positions, theta):
    """Z: [T, n_heads, hd]. Pairs (i, i+hd/2) are the real/imag parts of a complex number."""
    hd = Z.shape[-1]
    half = hd // 2
    inv = theta ** (-np.arange(half, dtype=np.float64) * 2.0 / hd)
    ang = np.outer(np.asarray(positions, dtype=np.float64), inv)          # [T, half]
    c = (Z[..., :half] + 1j * Z[..., half:]) * np.exp(1j * ang)[:, None, :]
    return np.concatenate([c.real, c.imag], axis=-1)


def forward(wl, weights, tokens, start_pos=0, kv_prefix=None):
    """Logits [T][V] (float64) for tokens at positions start_pos..start_pos+T-1.

    kv_prefix: optional bf16 [NL][2][nkv][start_pos][hd] cache contents for the
    earlier positions (already rotated keys).
    """
    f = lambda a: bf16_to_f32(a).astype(np.float64)
    T = len(tokens)
    H, hd, nq, nkv = wl.hidden, wl.head_dim, wl.n_heads, wl.n_kv_heads
    g = nq // nkv
    E = f(weights["embed"])
    X = E[np.asarray(tokens)]
    positions = np.arange(start_pos, start_pos + T)
    for l, Lw in enumerate(weights["layers"]):
        Xn = _norm(X, f(Lw["attn_norm"]), wl.rms_eps)
        Q = Xn @ f(Lw["wq"]).T
        K = Xn @ f(Lw["wk"]).T
        V = Xn @ f(Lw["wv"]).T
        if wl.qkv_bias:
            Q, K, V = Q + f(Lw["bq"]), K + f(Lw["bk"]), V + f(Lw["bv"])
        Q = _rotate(Q.reshape(T, nq, hd), positions, wl.rope_theta)
        K = bf16_round(_rotate(K.reshape(T, nkv, hd), positions, wl.rope_theta))
        V = bf16_round(V.reshape(T, nkv, hd))
        if kv_prefix is not None and start_pos > 0:
            K = np.concatenate([f(kv_prefix[l, 0]).transpose(1, 0, 2), K], axis=0)
            V = np.concatenate([f(kv_prefix[l, 1]).transpose(1, 0, 2), V], axis=0)
        S = K.shape[0]                                                     # all positions 0..start+T-1
        Kr = np.repeat(K, g, axis=1)                                       # [S, nq, hd]
        Vr = np.repeat(V, g, axis=1)
        scores = np.einsum("thd,shd->hts", Q, Kr) / np.sqrt(hd)            # [nq, T, S]
        allowed = np.arange(S)[None, :] <= positions[:, None]              # causal
        scores = np.where(allowed[None], scores, -np.inf)
        P = softmax(scores, axis=-1)
        O = np.einsum("hts,shd->thd", P, Vr).reshape(T, nq * hd)
        X = X + O @ f(Lw["wo"]).T
        Xn = _norm(X, f(Lw["mlp_norm"]), wl.rms_eps)
        G = Xn @ f(Lw["wgate"]).T
        U = Xn @ f(Lw["wup"]).T
        X = X + (G * expit(G) * U) @ f(Lw["wdown"]).T
    return _norm(X, f(weights["final_norm"]), wl.rms_eps) @ E.T
