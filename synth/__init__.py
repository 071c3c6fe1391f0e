"""Seeded synthetic inputs for batch-1 decoder workloads.

This module holds shapes, seeds and random draws only -- none of the decode
method's arithmetic.  Both the CPU oracle and the GPU path are fed from here,
so each side sees the same bytes.  The generator is defined in ``synth.c``
(SplitMix64 finaliser over a counter, Box-Muller for normals, bf16
round-to-nearest-even of the fp32 sample).

Workload shapes are those of the pages' decode leaderboard models
(SmolLM-135M, Qwen2-0.5B, SmolLM-1.7B; "MegaBake" project site, section
"Decode leaderboard"; third-party article, section "What a megakernel is")
with random-init weights in place of the trained checkpoints, plus a tiny
2-layer decoder small enough for pure-Python checks.

Value recipe:
  * matrices and the tied embedding: bf16(N(0, 0.02))
  * RMSNorm weights: bf16(1 + N(0, 0.02))
  * Q/K/V biases (when the model has them): bf16(N(0, 0.02))
  * prompt / first-decode token ids: uniform in [0, vocab)
  * long-context key/value prefill: bf16(N(0, 1)), stored (post-rotation) keys
Seeds: weights 0, prompt ids 1, KV prefill 2, first decode token 3.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
import subprocess
from typing import Dict, List, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libsynth.so")
_SRC = os.path.join(_HERE, "synth.c")

SEED_WEIGHTS = 0
SEED_PROMPT = 1
SEED_KV = 2
SEED_FIRST_TOKEN = 3


def build(force: bool = False) -> str:
    """Compile synth.c into libsynth.so next to it (gcc, OpenMP)."""
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
        tmp = _SO + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _SO)
    return _SO


_lib = None


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_SO)
        lib.syn_key.restype = ctypes.c_uint64
        lib.syn_key.argtypes = [ctypes.c_uint64, ctypes.c_char_p]
        lib.syn_normal_bf16.restype = None
        lib.syn_normal_bf16.argtypes = [ctypes.c_uint64, ctypes.c_double, ctypes.c_double, ctypes.c_int64, ctypes.c_void_p]
        lib.syn_tokens.restype = None
        lib.syn_tokens.argtypes = [ctypes.c_uint64, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p]
        lib.syn_uniform.restype = None
        lib.syn_uniform.argtypes = [ctypes.c_uint64, ctypes.c_int64, ctypes.c_void_p]
        _lib = lib
    return _lib


def key(seed: int, name: str) -> int:
    return int(_load().syn_key(seed, name.encode()))


def normal_bf16(seed: int, name: str, shape, mean: float = 0.0, std: float = 1.0) -> np.ndarray:
    """bf16 bit patterns (uint16) of mean + std * N(0,1), drawn from stream (seed, name)."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    _load().syn_normal_bf16(key(seed, name), float(mean), float(std), n, out.ctypes.data)
    return out.reshape(shape)


def tokens(seed: int, name: str, n: int, vocab: int) -> np.ndarray:
    out = np.empty(n, dtype=np.int32)
    _load().syn_tokens(key(seed, name), n, vocab, out.ctypes.data)
    return out


def uniform(seed: int, name: str, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.float64)
    _load().syn_uniform(key(seed, name), n, out.ctypes.data)
    return out


def bf16_to_f32(a: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.asarray(a, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass(frozen=True)
class Workload:
    """Decoder shape plus the decode schedule run on it."""
    name: str
    n_layers: int
    hidden: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    intermediate: int
    vocab: int
    kv_capacity: int
    qkv_bias: bool
    rms_eps: float
    rope_theta: float
    n_prompt: int       # prompt tokens stepped one at a time from position 0
    kv_prefill: int     # positions 0..kv_prefill-1 pre-filled with N(0,1) keys/values
    n_decode: int       # greedy decode steps after the prompt / prefill

    @property
    def first_pos(self) -> int:
        return self.kv_prefill

    @property
    def greedy_start(self) -> int:
        return self.kv_prefill + self.n_prompt

    def param_count(self) -> int:
        """Number of parameters (tied embedding counted once)."""
        H, hd = self.hidden, self.head_dim
        q, kv = self.n_heads * hd, self.n_kv_heads * hd
        per_layer = (q * H + 2 * kv * H + H * q + 3 * self.intermediate * H + 2 * H)
        if self.qkv_bias:
            per_layer += q + 2 * kv
        return self.n_layers * per_layer + self.vocab * H + H

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads: a tiny decoder, then the leaderboard model shapes.
WORKLOADS: Dict[str, Workload] = {
    w.name: w for w in [
        Workload("tiny-2L-h64-kv32", 2, 64, 4, 2, 16, 176, 512, 32, False, 1e-5, 1e4,
                 n_prompt=8, kv_prefill=0, n_decode=16),
        Workload("smollm135m-kv128", 30, 576, 9, 3, 64, 1536, 49152, 128, False, 1e-5, 1e4,
                 n_prompt=64, kv_prefill=0, n_decode=64),
        Workload("smollm135m-kv4096", 30, 576, 9, 3, 64, 1536, 49152, 4096, False, 1e-5, 1e4,
                 n_prompt=0, kv_prefill=4032, n_decode=64),
        Workload("qwen2-0.5b-kv128", 24, 896, 14, 2, 64, 4864, 151936, 128, True, 1e-6, 1e6,
                 n_prompt=64, kv_prefill=0, n_decode=64),
        Workload("smollm1.7b-kv4096", 24, 2048, 32, 32, 64, 8192, 49152, 4096, False, 1e-5, 1e4,
                 n_prompt=0, kv_prefill=4032, n_decode=64),
    ]
}
WORKLOAD_ORDER: List[str] = list(WORKLOADS)

# A measurement shape, not a parity workload: one SmolLM-1.7B-sized layer and a
# 262,144-row tied vocabulary projection (1.07 GB of bf16), so a step is
# dominated by the GEMV body streaming a packed matrix of more than 1 GB.
MEASUREMENT_WORKLOADS: Dict[str, Workload] = {
    w.name: w for w in [
        Workload("stream-1l-v262144", 1, 2048, 32, 32, 64, 8192, 262144, 128, False, 1e-5, 1e4,
                 n_prompt=8, kv_prefill=0, n_decode=64),
    ]
}


def get(name: str) -> Workload:
    return WORKLOADS[name] if name in WORKLOADS else MEASUREMENT_WORKLOADS[name]


def _shape_key(w: Workload) -> str:
    # Streams are named by the model shape, not the cache size, so the two
    # SmolLM-135M workloads share weights.
    return "L%d-H%d-nq%d-nkv%d-hd%d-I%d-V%d-b%d" % (
        w.n_layers, w.hidden, w.n_heads, w.n_kv_heads, w.head_dim, w.intermediate, w.vocab, int(w.qkv_bias))


def make_weights(w: Workload, seed: int = SEED_WEIGHTS) -> Dict[str, object]:
    """bf16 weights in Hugging Face layout ([out][in], row-major) as uint16 arrays.

    Returns {"embed": [V,H], "final_norm": [H], "layers": [ {name: array} ] }.
    """
    s = _shape_key(w)
    H, hd, I = w.hidden, w.head_dim, w.intermediate
    q, kv = w.n_heads * hd, w.n_kv_heads * hd
    out: Dict[str, object] = {
        "embed": normal_bf16(seed, s + "/embed", (w.vocab, H), 0.0, 0.02),
        "final_norm": normal_bf16(seed, s + "/final_norm", (H,), 1.0, 0.02),
    }
    layers = []
    for l in range(w.n_layers):
        p = "%s/L%d/" % (s, l)
        d = {
            "attn_norm": normal_bf16(seed, p + "attn_norm", (H,), 1.0, 0.02),
            "wq": normal_bf16(seed, p + "wq", (q, H), 0.0, 0.02),
            "wk": normal_bf16(seed, p + "wk", (kv, H), 0.0, 0.02),
            "wv": normal_bf16(seed, p + "wv", (kv, H), 0.0, 0.02),
            "wo": normal_bf16(seed, p + "wo", (H, q), 0.0, 0.02),
            "mlp_norm": normal_bf16(seed, p + "mlp_norm", (H,), 1.0, 0.02),
            "wgate": normal_bf16(seed, p + "wgate", (I, H), 0.0, 0.02),
            "wup": normal_bf16(seed, p + "wup", (I, H), 0.0, 0.02),
            "wdown": normal_bf16(seed, p + "wdown", (H, I), 0.0, 0.02),
        }
        if w.qkv_bias:
            d["bq"] = normal_bf16(seed, p + "bq", (q,), 0.0, 0.02)
            d["bk"] = normal_bf16(seed, p + "bk", (kv,), 0.0, 0.02)
            d["bv"] = normal_bf16(seed, p + "bv", (kv,), 0.0, 0.02)
        layers.append(d)
    out["layers"] = layers
    return out


def prompt_tokens(w: Workload, seed: int = SEED_PROMPT) -> np.ndarray:
    return tokens(seed, _shape_key(w) + "/prompt", w.n_prompt, w.vocab)


def first_token(w: Workload, seed: int = SEED_FIRST_TOKEN) -> int:
    return int(tokens(seed, _shape_key(w) + "/first", 1, w.vocab)[0])


def kv_prefill(w: Workload, npos: Optional[int] = None, seed: int = SEED_KV) -> np.ndarray:
    """bf16 N(0,1) keys/values for positions 0..npos-1: array [NL][2][nkv][npos][hd] (uint16).

    Drawn per (layer, K|V, kv head) stream so any prefix length gives the same values.
    """
    npos = w.kv_prefill if npos is None else npos
    out = np.empty((w.n_layers, 2, w.n_kv_heads, npos, w.head_dim), dtype=np.uint16)
    s = _shape_key(w)
    for l in range(w.n_layers):
        for c in range(2):
            for j in range(w.n_kv_heads):
                out[l, c, j] = normal_bf16(seed, "%s/kv/L%d/%s/h%d" % (s, l, "KV"[c], j),
                                           (npos, w.head_dim), 0.0, 1.0)
    return out


def kv_cache_bytes(w: Workload) -> int:
    """Bytes of a static bf16 cache laid out [NL][2][nkv][capacity][hd]."""
    return w.n_layers * 2 * w.n_kv_heads * w.kv_capacity * w.head_dim * 2


def decode_schedule(w: Workload) -> List[int]:
    """Positions stepped by the workload, in order."""
    return list(range(w.first_pos, w.greedy_start + w.n_decode))
