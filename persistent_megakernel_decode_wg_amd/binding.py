"""ctypes binding with the same names as the C ABI in include/mbk.h."""
from __future__ import annotations

import atexit
import ctypes
import os
import sys
import weakref
from typing import Dict, Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_HERE, "libmbk.so")

MBK_OK, MBK_ERR_ARG, MBK_ERR_RANGE, MBK_ERR_SIZE, MBK_ERR_UNSUPPORTED = 0, 1, 2, 3, 4
MBK_ERR_HIP, MBK_ERR_TIMEOUT, MBK_ERR_STATE = 5, 6, 7
MBK_TOKEN_PREV = -1
MBK_SYNC_DATAFLOW = 0
MBK_SYNC_BARRIER = 1
MBK_LAUNCH_PLAIN = 0
MBK_LAUNCH_COOPERATIVE = 1
MBK_WEIGHTS_BF16 = 0
MBK_WEIGHTS_FP8_E4M3 = 1


class MbkError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__("libmbk error %d: %s" % (code, msg))
        self.code = code


class mbk_config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "n_layers", "hidden", "n_heads", "n_kv_heads", "head_dim", "intermediate", "vocab", "kv_capacity",
        "qkv_bias")] + [("rms_eps", ctypes.c_float), ("rope_theta", ctypes.c_float)]


_PP = ctypes.POINTER(ctypes.c_void_p)


class mbk_weights(ctypes.Structure):
    _fields_ = [("embed", ctypes.c_void_p), ("final_norm", ctypes.c_void_p)] + [
        (n, _PP) for n in ("attn_norm", "wq", "wk", "wv", "bq", "bk", "bv", "wo", "mlp_norm", "wgate", "wup",
                           "wdown")]


class mbk_matrix_layout(ctypes.Structure):
    _fields_ = [("offset", ctypes.c_uint64)] + [(n, ctypes.c_int32) for n in (
        "rows", "cols", "lanes_per_row", "rows_per_tile", "steps", "tiles", "kind", "format", "values_per_group",
        "tile_bytes", "scale_offset")]


_lib = None


def lib():
    """Load libmbk.so (built by __graft_entry__.build()); raises if it is missing.

    torch is imported first: its HIP runtime is then the one libmbk.so binds to (both name the same
    runtime library), so the library and the tensors it is handed share one device context."""
    global _lib
    if _lib is None:
        if not os.path.exists(lib_path):
            raise RuntimeError("libmbk.so is not built (%s); run __graft_entry__.build()" % lib_path)
        import torch  # noqa: F401  (loads the HIP runtime the library then shares)
        L = ctypes.CDLL(lib_path)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        P = ctypes.POINTER
        L.mbk_create.argtypes = [P(mbk_config), P(vp)]
        L.mbk_destroy.argtypes = [vp]
        L.mbk_destroy.restype = None
        L.mbk_pack_weights.argtypes = [vp, P(mbk_weights), vp, P(sz), vp]
        L.mbk_alloc_kv.argtypes = [vp, vp, P(sz), vp, P(sz), vp]
        L.mbk_decode_step.argtypes = [vp, i32, i32, vp, vp, vp]
        L.mbk_decode_step_ablation.argtypes = [vp, i32, i32, vp, vp, i32, vp]
        L.mbk_decode_step_static.argtypes = [vp, vp, i32, i32, vp, vp, vp]
        L.mbk_check.argtypes = [vp, vp]
        L.mbk_barrier_bench.argtypes = [vp, i32, vp, P(ctypes.c_float)]
        L.mbk_barrier_stress.argtypes = [vp, i32, vp, P(i32)]
        L.mbk_get_matrix_layout.argtypes = [vp, i32, i32, P(mbk_matrix_layout)]
        L.mbk_prefill.argtypes = [vp, P(i32), i32, i32, vp, sz, vp, vp, vp]
        L.mbk_prefill_scratch_bytes.argtypes = [vp, i32, P(sz)]
        L.mbk_num_intervals.argtypes = [vp, P(i32)]
        L.mbk_set_debug.argtypes = [vp, i32, i32, i32]
        L.mbk_set_phase_trace.argtypes = [vp, vp, sz]
        L.mbk_set_attention_split.argtypes = [vp, i32]
        L.mbk_set_sync_mode.argtypes = [vp, i32]
        L.mbk_set_launch_mode.argtypes = [vp, i32]
        L.mbk_set_workgroups.argtypes = [vp, i32]
        L.mbk_set_attention_items.argtypes = [vp, i32]
        L.mbk_set_weight_format.argtypes = [vp, i32]
        L.mbk_describe.argtypes = [vp, ctypes.c_char_p, sz]
        L.mbk_last_error.argtypes = []
        L.mbk_last_error.restype = ctypes.c_char_p
        for n in ("mbk_create", "mbk_pack_weights", "mbk_alloc_kv", "mbk_decode_step", "mbk_decode_step_ablation",
                  "mbk_decode_step_static", "mbk_check", "mbk_barrier_bench", "mbk_barrier_stress", "mbk_get_matrix_layout", "mbk_prefill", "mbk_prefill_scratch_bytes", "mbk_num_intervals", "mbk_set_debug", "mbk_set_phase_trace",
                  "mbk_set_attention_split", "mbk_set_sync_mode", "mbk_set_launch_mode", "mbk_set_workgroups", "mbk_set_attention_items", "mbk_set_weight_format", "mbk_describe"):
            getattr(L, n).restype = ctypes.c_int
        _lib = L
    return _lib


def _chk(rc: int) -> None:
    if rc != MBK_OK:
        raise MbkError(rc, lib().mbk_last_error().decode())


def _stream(stream=None):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def make_config(wl) -> mbk_config:
    """mbk_config from any object with the decoder shape attributes."""
    return mbk_config(wl.n_layers, wl.hidden, wl.n_heads, wl.n_kv_heads, wl.head_dim, wl.intermediate, wl.vocab,
                      wl.kv_capacity, int(wl.qkv_bias), wl.rms_eps, wl.rope_theta)


# Handles still open when the interpreter exits are closed by an atexit hook, which runs before the HIP
# runtime's own exit-time teardown; after it no handle makes a library (and so HIP) call, so nothing
# reaches HIP from a finalizer or garbage collection during interpreter shutdown.
_live = weakref.WeakSet()
_shutting_down = False


def _close_all() -> None:
    global _shutting_down
    for d in list(_live):
        try:
            d.close()
        except Exception:
            pass
    _shutting_down = True


atexit.register(_close_all)


class Decoder:
    """One handle: packed weights, KV cache and workspace (torch tensors), decode steps.

    Call close() when done (or let the atexit hook do it); the destructor closes only while the
    interpreter is not shutting down."""

    def __init__(self, cfg):
        self.cfg = cfg
        self._c = make_config(cfg)
        h = ctypes.c_void_p()
        _chk(lib().mbk_create(ctypes.byref(self._c), ctypes.byref(h)))
        self.h = h
        self.packed = self.kv = self.ws = None
        self._keep = []
        _live.add(self)

    def close(self):
        if getattr(self, "h", None) and not _shutting_down:
            lib().mbk_destroy(self.h)
        self.h = None

    def __del__(self, _finalizing=sys.is_finalizing):
        # during interpreter teardown module globals may already be None: then (and once the atexit hook
        # has run) nothing is called
        try:
            if _shutting_down is not False or _finalizing():
                return
            self.close()
        except Exception:
            pass

    # -- setup ------------------------------------------------------------------------------------
    def pack_weights(self, weights: Dict[str, object], stream=None) -> None:
        """weights: {"embed", "final_norm", "layers": [{"attn_norm","wq","wk","wv","wo","mlp_norm","wgate",
        "wup","wdown"[,"bq","bk","bv"]}]} of contiguous bf16 (or int16/uint16 bit pattern) CUDA tensors."""
        import torch
        L = self.cfg.n_layers
        arrays = {}
        names = ["attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "wgate", "wup", "wdown"]
        if self.cfg.qkv_bias:
            names += ["bq", "bk", "bv"]
        for n in names:
            a = (ctypes.c_void_p * L)(*[weights["layers"][l][n].data_ptr() for l in range(L)])
            self._keep.append(a)
            arrays[n] = ctypes.cast(a, _PP)
        w = mbk_weights()
        w.embed = weights["embed"].data_ptr()
        w.final_norm = weights["final_norm"].data_ptr()
        for n, p in arrays.items():
            setattr(w, n, p)
        nbytes = ctypes.c_size_t(0)
        _chk(lib().mbk_pack_weights(self.h, ctypes.byref(w), None, ctypes.byref(nbytes), _stream(stream)))
        self.packed = torch.empty(nbytes.value, dtype=torch.uint8, device="cuda")
        _chk(lib().mbk_pack_weights(self.h, ctypes.byref(w), ctypes.c_void_p(self.packed.data_ptr()),
                                    ctypes.byref(nbytes), _stream(stream)))

    def matrix_layout(self, layer: int, which: int) -> dict:
        """Layout of one packed matrix (include/mbk.h, mbk_get_matrix_layout) as a dict."""
        g = mbk_matrix_layout()
        _chk(lib().mbk_get_matrix_layout(self.h, int(layer), int(which), ctypes.byref(g)))
        return {n: getattr(g, n) for n, _ in mbk_matrix_layout._fields_}

    def packed_bytes(self) -> int:
        nbytes = ctypes.c_size_t(0)
        _chk(lib().mbk_pack_weights(self.h, None, None, ctypes.byref(nbytes), None))
        return nbytes.value

    def alloc_kv(self, stream=None) -> None:
        import torch
        kvb, wsb = ctypes.c_size_t(0), ctypes.c_size_t(0)
        _chk(lib().mbk_alloc_kv(self.h, None, ctypes.byref(kvb), None, ctypes.byref(wsb), _stream(stream)))
        c = self.cfg
        self.kv = torch.empty((c.n_layers, 2, c.n_kv_heads, c.kv_capacity, c.head_dim), dtype=torch.int16,
                              device="cuda")
        assert self.kv.numel() * 2 == kvb.value
        self.ws = torch.empty(wsb.value, dtype=torch.uint8, device="cuda")
        self.rebind(stream)

    def rebind(self, stream=None) -> None:
        """Zero-fills and re-binds the KV cache and workspace (after a watchdog error)."""
        kvb, wsb = ctypes.c_size_t(self.kv.numel() * 2), ctypes.c_size_t(self.ws.numel())
        _chk(lib().mbk_alloc_kv(self.h, ctypes.c_void_p(self.kv.data_ptr()), ctypes.byref(kvb),
                                ctypes.c_void_p(self.ws.data_ptr()), ctypes.byref(wsb), _stream(stream)))

    # -- decode -----------------------------------------------------------------------------------
    def decode_step(self, token: int, pos: int, logits=None, argmax=None, stream=None):
        _chk(lib().mbk_decode_step(self.h, int(token), int(pos),
                                   ctypes.c_void_p(logits.data_ptr()) if logits is not None else None,
                                   ctypes.c_void_p(argmax.data_ptr()) if argmax is not None else None,
                                   _stream(stream)))
        return logits, argmax

    def prefill_scratch_bytes(self, n_tokens: int) -> int:
        n = ctypes.c_size_t(0)
        _chk(lib().mbk_prefill_scratch_bytes(self.h, int(n_tokens), ctypes.byref(n)))
        return n.value

    def prefill(self, tokens, pos0: int = 0, logits=None, argmax=None, scratch=None, stream=None):
        """Prompt tokens (a host sequence of ints) at positions pos0 .. pos0 + len - 1 in one call; logits and
        argmax of the last position.  scratch: a uint8 device tensor of at least prefill_scratch_bytes(len)
        bytes (allocated here when None)."""
        import torch
        toks = (ctypes.c_int32 * len(tokens))(*[int(t) for t in tokens])
        need = self.prefill_scratch_bytes(len(tokens))
        if scratch is None or scratch.numel() < need:
            scratch = torch.empty(need, dtype=torch.uint8, device="cuda")
        _chk(lib().mbk_prefill(self.h, toks, len(tokens), int(pos0), ctypes.c_void_p(scratch.data_ptr()),
                               scratch.numel(), ctypes.c_void_p(logits.data_ptr()) if logits is not None else None,
                               ctypes.c_void_p(argmax.data_ptr()) if argmax is not None else None, _stream(stream)))
        return scratch

    def decode_step_static(self, kv, token: int, pos: int, logits=None, argmax=None, stream=None):
        """The step on the library's static scratch (no workspace): `kv` is a cache tensor in the layout of
        alloc_kv(), which this call does not need."""
        _chk(lib().mbk_decode_step_static(self.h, ctypes.c_void_p(kv.data_ptr()) if kv is not None else None,
                                          int(token), int(pos),
                                          ctypes.c_void_p(logits.data_ptr()) if logits is not None else None,
                                          ctypes.c_void_p(argmax.data_ptr()) if argmax is not None else None,
                                          _stream(stream)))
        return logits, argmax

    def decode_step_ablation(self, token: int, pos: int, logits=None, argmax=None, use_graph: bool = False,
                             stream=None):
        _chk(lib().mbk_decode_step_ablation(self.h, int(token), int(pos),
                                            ctypes.c_void_p(logits.data_ptr()) if logits is not None else None,
                                            ctypes.c_void_p(argmax.data_ptr()) if argmax is not None else None,
                                            int(bool(use_graph)), _stream(stream)))
        return logits, argmax

    def check(self, stream=None) -> None:
        _chk(lib().mbk_check(self.h, _stream(stream)))

    def barrier_bench(self, n: int, stream=None) -> float:
        us = ctypes.c_float(0)
        _chk(lib().mbk_barrier_bench(self.h, int(n), _stream(stream), ctypes.byref(us)))
        return us.value

    def barrier_stress(self, n: int, stream=None):
        """Validated grid barriers: returns (round, reader, writer, value) of the first failed check, round 0
        when all passed."""
        out = (ctypes.c_int32 * 4)()
        _chk(lib().mbk_barrier_stress(self.h, int(n), _stream(stream), out))
        return tuple(out)

    def num_intervals(self) -> int:
        n = ctypes.c_int32(0)
        _chk(lib().mbk_num_intervals(self.h, ctypes.byref(n)))
        return n.value

    def set_debug(self, spin_limit: int = 0, skip_wg: int = -1, skip_interval: int = -1) -> None:
        _chk(lib().mbk_set_debug(self.h, spin_limit, skip_wg, skip_interval))

    def set_workgroups(self, n: int) -> None:
        _chk(lib().mbk_set_workgroups(self.h, n))

    def set_attention_items(self, heads_per_item: int) -> None:
        """0 (automatic), 1 (one query head per item) or n_heads / n_kv_heads (a KV head's query heads
        packed); before the schedule is planned."""
        _chk(lib().mbk_set_attention_items(self.h, int(heads_per_item)))

    def set_weight_format(self, fmt: int) -> None:
        """MBK_WEIGHTS_BF16 (default) or MBK_WEIGHTS_FP8_E4M3; before the schedule is planned."""
        _chk(lib().mbk_set_weight_format(self.h, int(fmt)))

    def describe(self) -> dict:
        import json
        buf = ctypes.create_string_buffer(8192)
        _chk(lib().mbk_describe(self.h, buf, len(buf)))
        return json.loads(buf.value.decode())

    def set_sync_mode(self, mode: int) -> None:
        """MBK_SYNC_DATAFLOW (0, default) or MBK_SYNC_BARRIER (1)."""
        _chk(lib().mbk_set_sync_mode(self.h, int(mode)))

    def set_launch_mode(self, mode: int) -> None:
        """MBK_LAUNCH_PLAIN (0, default) or MBK_LAUNCH_COOPERATIVE (1)."""
        _chk(lib().mbk_set_launch_mode(self.h, int(mode)))

    def set_attention_split(self, min_positions: int) -> None:
        _chk(lib().mbk_set_attention_split(self.h, int(min_positions)))

    def set_phase_trace(self, enable: bool = True):
        """Returns the int64 [intervals][n_wg][4] trace tensor (device wall clock) or None."""
        import torch
        if not enable:
            _chk(lib().mbk_set_phase_trace(self.h, None, 0))
            return None
        n_wg = torch.cuda.get_device_properties(torch.cuda.current_device()).multi_processor_count
        buf = torch.zeros((self.num_intervals(), n_wg, 4), dtype=torch.int64, device="cuda")
        _chk(lib().mbk_set_phase_trace(self.h, ctypes.c_void_p(buf.data_ptr()), buf.numel() * 8))
        self._trace = buf
        return buf
