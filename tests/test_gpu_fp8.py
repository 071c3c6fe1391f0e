"""FP8 (OCP E4M3) weight streaming on the GPU, against the oracle.

* The packer's codes and row scales equal the oracle quantiser's bit for bit (byte work), read back from
  the packed blob through the documented layout.
* The decode step of an FP8 handle matches the oracle run on the quantised model -- the bf16 weights the
  codes stand for, value(code) * 2^e, which are exact -- to the same bar as the bf16 path: logits within
  2e-2 of the oracle's standard deviation, the argmax rule, and the cache slot each step writes (layer 0
  within one bf16 step plus 2^-10 of the RMS, every layer within 2e-2 relative L2).
* Prefill on an FP8 handle matches the same oracle to the same bar, and a prompt taken in two calls gives the
  one-call bits."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import LOGIT_TOL, Pair, compare, kv_slot_check, log, teacher_forced, upload

pytestmark = pytest.mark.gpu


def _fp8_setup(d):
    from persistent_megakernel_decode_wg_amd import MBK_WEIGHTS_FP8_E4M3
    d.set_weight_format(MBK_WEIGHTS_FP8_E4M3)


@pytest.fixture
def fp8_pair():
    made = []

    def make(wl, kv_prefix=None):
        W = synth.make_weights(wl)
        Wq, _ = oracle.fp8_weights(W)
        p = Pair(wl, W, kv_prefix=kv_prefix, setup=_fp8_setup, oracle_W=Wq)
        made.append(p)
        return p
    yield make
    for p in made:
        p.close()


def _unpack_fp8(blob: np.ndarray, g: dict):
    """Codes [rows][cols] (packed row order) and row scales of an fp8 matrix, from the layout record;
    checks that padding rows, padding groups and scale padding are zero."""
    T, S, RT, L, tb, so = g["tiles"], g["steps"], g["rows_per_tile"], g["lanes_per_row"], g["tile_bytes"], g["scale_offset"]
    assert g["format"] == 1 and g["values_per_group"] == 16 and so == S * 1024
    raw = blob[g["offset"]:g["offset"] + T * tb].reshape(T, tb)
    codes = raw[:, :so].reshape(T, S, RT, L, 16).transpose(0, 2, 1, 3, 4).reshape(T * RT, S * L * 16)
    sblk = raw[:, so:].copy().view(np.float32).reshape(T, -1)
    scales = sblk[:, :RT].reshape(-1)
    assert not sblk[:, RT:].any(), "nonzero scale padding"
    assert not codes[g["rows"]:].any() and not scales[g["rows"]:].any(), "nonzero padding rows"
    assert not codes[:, g["cols"]:].any(), "nonzero padding groups"
    return codes[:g["rows"], :g["cols"]], scales[:g["rows"]]


def _rope_pairs(M: np.ndarray, heads: int, hd: int) -> np.ndarray:
    perm = np.empty(hd, dtype=np.int64)
    perm[0::2] = np.arange(hd // 2)
    perm[1::2] = np.arange(hd // 2) + hd // 2
    return M.reshape(heads, hd, *M.shape[1:])[:, perm].reshape(heads * hd, *M.shape[1:])


@pytest.mark.parametrize("name,layers", [("tiny-2L-h64-kv32", None), ("smollm135m-kv128", [0, 29]),
                                         ("qwen2-0.5b-kv128", [0, 23]), ("smollm1.7b-kv4096", [5])])
def test_fp8_packed_codes_and_scales_equal_the_oracle_quantiser(name, layers):
    from persistent_megakernel_decode_wg_amd import Decoder
    wl = synth.get(name)
    W = synth.make_weights(wl)
    d = Decoder(wl)
    try:
        _fp8_setup(d)
        d.pack_weights(upload(W))
        blob = d.packed.cpu().numpy()
        hd = wl.head_dim
        for l in (range(wl.n_layers) if layers is None else layers):
            L = W["layers"][l]
            q = {n: oracle.quantize_e4m3_rows(L[n]) for n in oracle.FP8_MATRICES}
            want = {
                0: (np.concatenate([_rope_pairs(q["wq"][0], wl.n_heads, hd), _rope_pairs(q["wk"][0], wl.n_kv_heads, hd),
                                    q["wv"][0]]),
                    np.concatenate([_rope_pairs(q["wq"][1], wl.n_heads, hd), _rope_pairs(q["wk"][1], wl.n_kv_heads, hd),
                                    q["wv"][1]])),
                1: q["wo"],
                2: (np.stack([q["wgate"][0], q["wup"][0]], axis=1).reshape(2 * wl.intermediate, wl.hidden),
                    np.stack([q["wgate"][1], q["wup"][1]], axis=1).reshape(-1)),
                3: q["wdown"],
            }
            for which, (codes, exps) in want.items():
                got_c, got_s = _unpack_fp8(blob, d.matrix_layout(l, which))
                assert np.array_equal(got_c, codes), "layer %d matrix %d codes" % (l, which)
                assert np.array_equal(got_s, np.ldexp(np.float32(1), exps).astype(np.float32)), \
                    "layer %d matrix %d scales" % (l, which)
        codes, exps = oracle.quantize_e4m3_rows(W["embed"])
        got_c, got_s = _unpack_fp8(blob, d.matrix_layout(-1, 1))
        assert np.array_equal(got_c, codes) and np.array_equal(got_s, np.ldexp(np.float32(1), exps).astype(np.float32))
        g = d.matrix_layout(-1, 0)
        assert g["format"] == 0   # the embedding row gather keeps the bf16 table
    finally:
        d.close()


def test_fp8_tiny_full_schedule_and_executors(fp8_pair):
    wl = synth.get("tiny-2L-h64-kv32")
    p = fp8_pair(wl)
    worst = teacher_forced(p, synth.decode_schedule(wl), list(synth.prompt_tokens(wl)), label="fp8 tiny")
    log("fp8 tiny worst max|dlogit|/std = %.3g" % worst)
    tok = int(synth.prompt_tokens(wl)[2])
    for pos in (0, 5, wl.kv_capacity - 1):
        a, ia = p.gpu_step(tok, pos, "mega")
        for mode in ("cooperative", "barrier", "ablation", "graph"):
            b, ib = p.gpu_step(tok, pos, mode)
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32)) and ia == ib, "pos %d %s" % (pos, mode)


def test_fp8_smollm135m_kv128_full_schedule(fp8_pair):
    """All 128 steps (64 prompt positions, 64 greedy steps to the last slot), every step checked."""
    wl = synth.get("smollm135m-kv128")
    p = fp8_pair(wl)
    worst = teacher_forced(p, synth.decode_schedule(wl), list(synth.prompt_tokens(wl)), label="fp8 smollm135m")
    log("fp8 smollm135m-kv128 worst max|dlogit|/std = %.3g" % worst)


def test_fp8_qwen2_bias_kv128(fp8_pair):
    """Biases stay bf16 on an fp8 handle: all 128 steps, every 2nd checked, and the last slot."""
    wl = synth.get("qwen2-0.5b-kv128")
    p = fp8_pair(wl)
    positions = synth.decode_schedule(wl)
    worst = teacher_forced(p, positions, list(synth.prompt_tokens(wl)), check_every=2, label="fp8 qwen2")
    log("fp8 qwen2-0.5b-kv128 worst max|dlogit|/std = %.3g" % worst)


def test_fp8_smollm1p7b_kv4096_prefilled(fp8_pair):
    """The 4096-slot cache pre-filled at 0..4031: all 64 steps to the last slot, every 8th checked and
    the last one."""
    wl = synth.get("smollm1.7b-kv4096")
    p = fp8_pair(wl, kv_prefix=synth.kv_prefill(wl))
    positions = synth.decode_schedule(wl)
    assert positions[-1] == wl.kv_capacity - 1
    worst = teacher_forced(p, positions, [synth.first_token(wl)], check_every=8, label="fp8 smollm1.7b-4k")
    log("fp8 smollm1.7b-kv4096 worst max|dlogit|/std = %.3g" % worst)


def test_fp8_maximum_sizes_to_the_last_slot(fp8_pair):
    """The largest shape the kernel takes (every GEMV input 8,192 wide: fp8 tiles of 8,192 codes per row;
    G = 8 at head size 128), one layer, the 8,192-slot cache pre-filled to 8,188 and stepped to slot 8,191."""
    wl = synth.Workload("max-h8192-kv8192", 1, 8192, 64, 8, 128, 8192, 4096, 8192, False, 1e-5, 1e4,
                        n_prompt=0, kv_prefill=8189, n_decode=3)
    p = fp8_pair(wl, kv_prefix=synth.kv_prefill(wl))
    positions = synth.decode_schedule(wl)
    assert positions[-1] == wl.kv_capacity - 1
    worst = teacher_forced(p, positions, [synth.first_token(wl)], label="fp8 max sizes")
    log("fp8 max sizes worst max|dlogit|/std = %.3g" % worst)


def test_fp8_handle_rejects_late_format_change():
    from persistent_megakernel_decode_wg_amd import MBK_ERR_STATE, MBK_WEIGHTS_BF16, Decoder, MbkError
    wl = synth.get("tiny-2L-h64-kv32")
    d = Decoder(wl)
    try:
        _fp8_setup(d)
        d.pack_weights(upload(synth.make_weights(wl)))
        d.alloc_kv()
        with pytest.raises(MbkError) as e:
            d.set_weight_format(MBK_WEIGHTS_BF16)
        assert e.value.code == MBK_ERR_STATE
    finally:
        d.close()


class _Fp8Prefill:
    """An FP8 handle and the oracle on the quantised model, for prefill."""

    def __init__(self, wl, W):
        import torch
        from persistent_megakernel_decode_wg_amd import Decoder
        Wq, _ = oracle.fp8_weights(W)
        self.dec = Decoder(wl)
        _fp8_setup(self.dec)
        self.dec.pack_weights(upload(W))
        self.dec.alloc_kv()
        self.ref = oracle.Model(wl, Wq)
        self.logits = torch.empty(wl.vocab, dtype=torch.float32, device="cuda")
        self.am = torch.empty(1, dtype=torch.int32, device="cuda")

    def prefill(self, toks, pos0):
        self.dec.prefill(toks, pos0, self.logits, self.am)
        self.dec.check()
        return self.logits.cpu().numpy().copy(), int(self.am.item())

    def check(self, toks, pos0, label):
        lg, am = self.prefill(toks, pos0)
        lo = ao = None
        for i, t in enumerate(toks):
            lo, ao, _ = self.ref.step(int(t), pos0 + i)
        assert np.all(np.isfinite(lg)), label
        rel, margin = compare(lg, am, lo, ao)
        assert rel <= LOGIT_TOL, "%s: max|dlogit| = %.4g std" % (label, rel)
        kv = self.dec.kv.cpu().numpy().view(np.uint16)
        for slot in range(pos0, pos0 + len(toks)):
            x0, r = kv_slot_check(kv[:, :, :, slot, :], self.ref.kv[:, :, :, slot, :])
            assert x0.max() <= 1.0 and r.max() <= LOGIT_TOL, "%s slot %d" % (label, slot)
        log("%s: max|dlogit|/std %.3g, margin %.3g" % (label, rel, margin))

    def close(self):
        self.dec.close()


@pytest.mark.parametrize("name", ["tiny-2L-h64-kv32", "smollm135m-kv128"])
def test_fp8_prefill_against_the_quantised_oracle(name):
    """Prefill on an FP8 handle (every GEMM widens its weight codes to bf16 exactly and scales the output
    rows; the vocabulary projection reads the fp8 copy of the embedding) against the oracle stepped on the
    quantised model: the tiny model's whole cache, the SmolLM-135M 64-token prompt; then the prompt again
    as two calls, bit for bit."""
    import torch
    wl = synth.get(name)
    W = synth.make_weights(wl)
    n = wl.kv_capacity if name.startswith("tiny") else wl.n_prompt
    toks = [int(t) for t in synth.tokens(21, "fp8-prefill", n, wl.vocab)]
    a, b = _Fp8Prefill(wl, W), _Fp8Prefill(wl, W)
    try:
        a.check(toks, 0, "fp8 prefill %s 0..%d" % (name, n - 1))
        la, ia = a.logits.cpu().numpy().copy(), int(a.am.item())
        cut = n // 3
        b.prefill(toks[:cut], 0)
        lb, ib = b.prefill(toks[cut:], cut)
        assert np.array_equal(la.view(np.uint32), lb.view(np.uint32)) and ia == ib
        assert torch.equal(a.dec.kv, b.dec.kv)
    finally:
        a.close()
        b.close()


def test_fp8_prefill_1p7b_shape_kernel_forms_agree_bitwise():
    """Two layers of the SmolLM-1.7B shape on an FP8 handle: a 256-token prompt in one call (every projection
    with four row blocks and two position blocks per workgroup) and in four calls of 64 tokens (query/key/value
    two row blocks and two position blocks, the 4M-weight output projection two row blocks and one position
    block, gate/up four and two, down one and two) give the same logits, argmax and cache bit for bit; the first
    64-token call is also checked against the oracle on the quantised model."""
    import torch
    wl = synth.Workload("smollm1.7b-2L-kv512", 2, 2048, 32, 32, 64, 8192, 49152, 512, False, 1e-5, 1e4,
                        n_prompt=0, kv_prefill=0, n_decode=0)
    W = synth.make_weights(wl)
    toks = [int(t) for t in synth.tokens(31, "fp8-prefill-forms", 256, wl.vocab)]
    a, b = _Fp8Prefill(wl, W), _Fp8Prefill(wl, W)
    try:
        la, ia = a.prefill(toks, 0)
        b.check(toks[:64], 0, "fp8 smollm1.7b shape, 2 layers, prefill 0..63")
        for c in range(64, 256, 64):
            lb, ib = b.prefill(toks[c:c + 64], c)
        assert np.array_equal(la.view(np.uint32), lb.view(np.uint32)) and ia == ib
        assert torch.equal(a.dec.kv, b.dec.kv)
    finally:
        a.close()
        b.close()
