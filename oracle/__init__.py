"""CPU oracle for one batch-1 decode step -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU product path never touches it.
The arithmetic lives in ``oracle.c`` (plain C, fp64 accumulation); this file
only marshals numpy arrays through ctypes.

Pins (each checked by a ``-m "not gpu"`` test):
  * parameter count of the SmolLM-135M shape = 134,515,008, the figure the
    MegaBake article prints (section "What a megakernel is");
  * RMSNorm: closed form on constant vectors, unit RMS, scale invariance;
  * matvec: numpy's float64 matrix product;
  * RoPE: identity at position 0, norm preservation, relative-position
    dot products, composition, pair structure and per-pair angle;
  * attention: scipy softmax brute force, one position gives V_0, equal keys
    or a zero query give the mean of V, GQA == MHA with repeated KV heads;
  * SiLU: silu(0) = 0, silu(z) -> z for large z, scipy expit;
  * decode step: stepwise decode equals an independent float64 full-sequence
    causal forward; zero output projections give a closed-form logit vector
    whose argmax is the input token.
  * FP8 (E4M3) quantiser: every finite code encodes back to itself, every
    midpoint of neighbouring codes goes to the even one, nearest-value brute
    force over all codes on random inputs, the OCP format's fixed points (448,
    2^-6, 2^-9, the NaN patterns), the row exponent against its defining
    inequality, and the dequantised weights exactly representable in bf16.
Nothing here is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Dict, Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_HDR = os.path.join(_HERE, "oracle.h")
_SO = os.path.join(_HERE, "liboracle.so")


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so (gcc -O2, OpenMP)."""
    newest = max(os.path.getmtime(_SRC), os.path.getmtime(_HDR))
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < newest:
        tmp = _SO + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _SO)
    return _SO


class Config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in (
        "n_layers", "hidden", "n_heads", "n_kv_heads", "head_dim", "intermediate", "vocab", "kv_capacity",
        "qkv_bias")] + [("rms_eps", ctypes.c_double), ("rope_theta", ctypes.c_double)]


_PP = ctypes.POINTER(ctypes.c_void_p)


class Weights(ctypes.Structure):
    _fields_ = [("embed", ctypes.c_void_p), ("final_norm", ctypes.c_void_p)] + [
        (n, _PP) for n in ("attn_norm", "wq", "wk", "wv", "bq", "bk", "bv", "wo", "mlp_norm", "wgate", "wup",
                           "wdown")] + [("lm_head", ctypes.c_void_p)]


class Trace(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("x_in", "q", "k", "v", "o", "x_mid", "a", "x_final")]


_lib = None


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_SO)
        vp, i, d = ctypes.c_void_p, ctypes.c_int, ctypes.c_double
        lib.orc_rmsnorm.argtypes = [vp, vp, i, d, vp]
        lib.orc_matvec.argtypes = [vp, vp, i, i, vp, vp]
        lib.orc_matvec_residual.argtypes = [vp, i, i, vp, vp]
        lib.orc_rope.argtypes = [vp, i, i, i, d]
        lib.orc_attention.argtypes = [vp, vp, vp, i, i, i, i, i, vp]
        lib.orc_silu_mul.argtypes = [vp, vp, i, vp]
        lib.orc_argmax.argtypes = [vp, i]
        lib.orc_argmax.restype = i
        lib.orc_bf16_to_f32.argtypes = [ctypes.c_uint16]
        lib.orc_bf16_to_f32.restype = ctypes.c_float
        lib.orc_f32_to_bf16.argtypes = [ctypes.c_float]
        lib.orc_f32_to_bf16.restype = ctypes.c_uint16
        lib.orc_decode_step.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(Weights), vp, i, i, vp,
                                        ctypes.POINTER(ctypes.c_int), ctypes.POINTER(Trace)]
        lib.orc_decode_step.restype = i
        lib.orc_num_threads.restype = i
        lib.orc_e4m3_value.argtypes = [i]
        lib.orc_e4m3_value.restype = d
        lib.orc_e4m3_encode.argtypes = [d]
        lib.orc_e4m3_encode.restype = ctypes.c_uint8
        lib.orc_fp8_row_exponent.argtypes = [vp, i]
        lib.orc_fp8_row_exponent.restype = i
        lib.orc_quantize_rows_e4m3.argtypes = [vp, i, i, vp, vp]
        lib.orc_dequantize_rows_e4m3.argtypes = [vp, vp, i, i, vp]
        _lib = lib
    return _lib


def _f32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32)


def _u16(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.uint16)


def num_threads() -> int:
    return int(_load().orc_num_threads())


def f32_to_bf16(x: float) -> int:
    return int(_load().orc_f32_to_bf16(float(x)))


def rmsnorm(x, w_bf16, eps: float) -> np.ndarray:
    x, w = _f32(x), _u16(w_bf16)
    out = np.empty_like(x)
    _load().orc_rmsnorm(x.ctypes.data, w.ctypes.data, x.size, eps, out.ctypes.data)
    return out


def matvec(W_bf16, x, b_bf16=None) -> np.ndarray:
    W, x = _u16(W_bf16), _f32(x)
    M, K = W.shape
    assert x.size == K
    b = None if b_bf16 is None else _u16(b_bf16)
    y = np.empty(M, dtype=np.float32)
    _load().orc_matvec(W.ctypes.data, None if b is None else b.ctypes.data, M, K, x.ctypes.data, y.ctypes.data)
    return y


def matvec_residual(W_bf16, v, x) -> np.ndarray:
    W, v = _u16(W_bf16), _f32(v)
    out = _f32(x).copy()
    M, K = W.shape
    _load().orc_matvec_residual(W.ctypes.data, M, K, v.ctypes.data, out.ctypes.data)
    return out


def rope(v, n_heads: int, head_dim: int, pos: int, theta: float) -> np.ndarray:
    out = _f32(v).copy()
    assert out.size == n_heads * head_dim
    _load().orc_rope(out.ctypes.data, n_heads, head_dim, pos, theta)
    return out


def attention(q, K_bf16, V_bf16, n_heads: int, n_kv: int, head_dim: int, Lc: int) -> np.ndarray:
    """q [nq*hd] fp32; K, V [n_kv][cap][hd] bf16 of one layer; attends positions 0..Lc-1."""
    q, K, V = _f32(q), _u16(K_bf16), _u16(V_bf16)
    cap = K.shape[1]
    o = np.empty(n_heads * head_dim, dtype=np.float32)
    _load().orc_attention(q.ctypes.data, K.ctypes.data, V.ctypes.data, n_heads, n_kv, head_dim, cap, Lc,
                          o.ctypes.data)
    return o


def silu_mul(g, u) -> np.ndarray:
    g, u = _f32(g), _f32(u)
    out = np.empty_like(g)
    _load().orc_silu_mul(g.ctypes.data, u.ctypes.data, g.size, out.ctypes.data)
    return out


def argmax(v) -> int:
    v = _f32(v)
    return int(_load().orc_argmax(v.ctypes.data, v.size))


def e4m3_value(code: int) -> float:
    """Value of an OCP E4M3 code (NaN for the two NaN patterns)."""
    return float(_load().orc_e4m3_value(int(code)))


def e4m3_encode(x: float) -> int:
    """Nearest E4M3 code of a finite x with |x| <= 448, ties to the even code."""
    return int(_load().orc_e4m3_encode(float(x)))


def fp8_row_exponent(w_bf16) -> int:
    w = _u16(w_bf16)
    return int(_load().orc_fp8_row_exponent(w.ctypes.data, w.size))


def quantize_e4m3_rows(W_bf16) -> Tuple[np.ndarray, np.ndarray]:
    """Per-row power-of-two scaled E4M3 codes of a [rows][K] bf16 matrix: (codes uint8, exponents int32)."""
    W = _u16(W_bf16)
    rows, K = W.shape
    codes = np.empty((rows, K), dtype=np.uint8)
    exps = np.empty(rows, dtype=np.int32)
    _load().orc_quantize_rows_e4m3(W.ctypes.data, rows, K, codes.ctypes.data, exps.ctypes.data)
    return codes, exps


def dequantize_e4m3_rows(codes, exps) -> np.ndarray:
    """The bf16 weights the codes stand for, value(code) * 2^e (exact)."""
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    e = np.ascontiguousarray(exps, dtype=np.int32)
    rows, K = c.shape
    W = np.empty((rows, K), dtype=np.uint16)
    _load().orc_dequantize_rows_e4m3(c.ctypes.data, e.ctypes.data, rows, K, W.ctypes.data)
    return W


FP8_MATRICES = ("wq", "wk", "wv", "wo", "wgate", "wup", "wdown")


def fp8_weights(weights: Dict[str, object]) -> Tuple[Dict[str, object], Dict[str, object]]:
    """The FP8 form of a bf16 weight set: every projection matrix and the vocabulary projection (the tied
    embedding) quantised row by row.  Returns (the quantised model as bf16 weights -- the embedding row
    gather keeps the bf16 table, the vocabulary projection is "lm_head" --, the codes and exponents)."""
    q = {"layers": [], "lm_head": quantize_e4m3_rows(weights["embed"])}
    out = {"embed": weights["embed"], "final_norm": weights["final_norm"], "layers": [],
           "lm_head": dequantize_e4m3_rows(*q["lm_head"])}
    for L in weights["layers"]:
        ql, ol = {}, dict(L)
        for n in FP8_MATRICES:
            ql[n] = quantize_e4m3_rows(L[n])
            ol[n] = dequantize_e4m3_rows(*ql[n])
        q["layers"].append(ql)
        out["layers"].append(ol)
    return out, q


class Model:
    """Holds a workload's config, its bf16 weights and an oracle-side KV cache."""

    def __init__(self, wl, weights: Dict[str, object]):
        self.wl = wl
        self.cfg = Config(wl.n_layers, wl.hidden, wl.n_heads, wl.n_kv_heads, wl.head_dim, wl.intermediate,
                          wl.vocab, wl.kv_capacity, int(wl.qkv_bias), wl.rms_eps, wl.rope_theta)
        self._keep = []
        self.weights = weights
        L = wl.n_layers
        arrs = {}
        names = ["attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "wgate", "wup", "wdown"]
        if wl.qkv_bias:
            names += ["bq", "bk", "bv"]
        for n in names:
            a = (ctypes.c_void_p * L)()
            for l in range(L):
                t = _u16(weights["layers"][l][n])
                self._keep.append(t)
                a[l] = t.ctypes.data
            self._keep.append(a)
            arrs[n] = ctypes.cast(a, _PP)
        emb, fn = _u16(weights["embed"]), _u16(weights["final_norm"])
        self._keep += [emb, fn]
        w = Weights()
        w.embed, w.final_norm = emb.ctypes.data, fn.ctypes.data
        if weights.get("lm_head") is not None:
            lm = _u16(weights["lm_head"])
            self._keep.append(lm)
            w.lm_head = lm.ctypes.data
        for n, p in arrs.items():
            setattr(w, n, p)
        self.w = w
        self.kv = np.zeros((L, 2, wl.n_kv_heads, wl.kv_capacity, wl.head_dim), dtype=np.uint16)

    def prefill_kv(self, kv_prefix: np.ndarray) -> None:
        """Copy [NL][2][nkv][P][hd] bf16 values into slots 0..P-1."""
        P = kv_prefix.shape[3]
        self.kv[:, :, :, :P, :] = kv_prefix

    def step(self, token: int, pos: int, trace: bool = False) -> Tuple[np.ndarray, int, Optional[dict]]:
        wl = self.wl
        logits = np.empty(wl.vocab, dtype=np.float32)
        am = ctypes.c_int(-1)
        tr, trd = None, None
        if trace:
            L, H, Q, KV, I = wl.n_layers, wl.hidden, wl.n_heads * wl.head_dim, wl.n_kv_heads * wl.head_dim, wl.intermediate
            trd = {"x_in": np.empty((L, H), np.float32), "q": np.empty((L, Q), np.float32),
                   "k": np.empty((L, KV), np.float32), "v": np.empty((L, KV), np.float32),
                   "o": np.empty((L, Q), np.float32), "x_mid": np.empty((L, H), np.float32),
                   "a": np.empty((L, I), np.float32), "x_final": np.empty(H, np.float32)}
            tr = Trace(*[trd[n].ctypes.data for n in ("x_in", "q", "k", "v", "o", "x_mid", "a", "x_final")])
        rc = _load().orc_decode_step(ctypes.byref(self.cfg), ctypes.byref(self.w), self.kv.ctypes.data,
                                     int(token), int(pos), logits.ctypes.data, ctypes.byref(am),
                                     ctypes.byref(tr) if tr is not None else None)
        if rc != 0:
            raise ValueError("orc_decode_step failed with %d (token=%d pos=%d)" % (rc, token, pos))
        return logits, int(am.value), trd
