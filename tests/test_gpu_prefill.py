"""Multi-token prefill (mbk_prefill) against the oracle stepped over the same positions, on the GPU.

The oracle for a prefill of positions p0 .. p0 + n - 1 is the decode-step oracle run over those positions
(itself pinned by stepwise decode = full-sequence recomputation).  Checked: the last position's logits
(max |dlogit| <= 2e-2 * std) and argmax (the lowest-index maximum of the GPU's own logits; the oracle's where
its margin exceeds 5e-2, else one of its near-ties), and every cache slot the prefill wrote, per layer, as for
the decode step (layer 0 within one bf16 step plus 2^-10 of the RMS, every layer within 2e-2 in relative L2)."""
import numpy as np
import pytest

import synth
from gpu_util import LOGIT_TOL, compare, kv_slot_check, log, upload

pytestmark = pytest.mark.gpu


class PrefillPair:
    def __init__(self, wl, W=None):
        import torch
        import oracle
        from persistent_megakernel_decode_wg_amd import Decoder
        self.wl = wl
        self.W = synth.make_weights(wl) if W is None else W
        self.dec = Decoder(wl)
        self.dec.pack_weights(upload(self.W))
        self.dec.alloc_kv()
        self.ref = oracle.Model(wl, self.W)
        self.logits = torch.empty(wl.vocab, dtype=torch.float32, device="cuda")
        self.am = torch.empty(1, dtype=torch.int32, device="cuda")

    def close(self):
        self.dec.close()

    def prefill(self, tokens, pos0):
        self.dec.prefill(tokens, pos0, self.logits, self.am)
        self.dec.check()
        return self.logits.cpu().numpy().copy(), int(self.am.item())

    def oracle_steps(self, tokens, pos0):
        lo = ao = None
        for i, t in enumerate(tokens):
            lo, ao, _ = self.ref.step(int(t), pos0 + i)
        return lo, ao

    def check(self, tokens, pos0, label):
        lg, am = self.prefill(tokens, pos0)
        lo, ao = self.oracle_steps(tokens, pos0)
        assert np.all(np.isfinite(lg)), label
        rel, margin = compare(lg, am, lo, ao)
        assert rel <= LOGIT_TOL, "%s: max|dlogit| = %.4g std" % (label, rel)
        kv = self.dec.kv.cpu().numpy().view(np.uint16)
        worst0 = worst_rel = 0.0
        for slot in range(pos0, pos0 + len(tokens)):
            x0, r = kv_slot_check(kv[:, :, :, slot, :], self.ref.kv[:, :, :, slot, :])
            assert x0.max() <= 1.0, "%s slot %d: layer-0 cache entry off by %.3g x the tolerance" % (label, slot, x0.max())
            assert r.max() <= LOGIT_TOL, "%s slot %d: layer %d cache off by %.3g (relative L2)" % (
                label, slot, int(np.unravel_index(r.argmax(), r.shape)[0]), r.max())
            worst0, worst_rel = max(worst0, float(x0.max())), max(worst_rel, float(r.max()))
        log("%s: max|dlogit|/std %.3g, margin %.3g; cache: layer 0 %.3g of the tolerance, worst relative L2 %.3g"
            % (label, rel, margin, worst0, worst_rel))
        return lg, am, lo, ao


@pytest.fixture
def make():
    made = []

    def f(*a, **kw):
        p = PrefillPair(*a, **kw)
        made.append(p)
        return p
    yield f
    for p in made:
        p.close()


def test_prefill_tiny_whole_cache(make):
    wl = synth.get("tiny-2L-h64-kv32")
    p = make(wl)
    toks = [int(t) for t in synth.tokens(11, "prefill", wl.kv_capacity, wl.vocab)]
    p.check(toks, 0, "tiny prefill 0..31")


def test_prefill_after_decode_steps_and_in_chunks(make):
    """Decode steps at 0..4, then prefill 5..20 and 21..30 on the same cache: both match the oracle."""
    wl = synth.get("tiny-2L-h64-kv32")
    p = make(wl)
    toks = [int(t) for t in synth.tokens(12, "prefill", 31, wl.vocab)]
    for pos in range(5):
        p.dec.decode_step(toks[pos], pos, p.logits, p.am)
        p.dec.check()
        p.ref.step(toks[pos], pos)
    p.check(toks[5:21], 5, "tiny prefill 5..20 after decode 0..4")
    p.check(toks[21:31], 21, "tiny prefill 21..30")


def test_prefill_single_tokens_at_the_cache_edges(make):
    """The degenerate prompt of one token (63 padding rows in the GEMMs): at position 0, then 1..30 in one call,
    then one token into the last slot, 31 -- each against the oracle."""
    wl = synth.get("tiny-2L-h64-kv32")
    p = make(wl)
    toks = [int(t) for t in synth.tokens(14, "prefill-single", wl.kv_capacity, wl.vocab)]
    p.check(toks[:1], 0, "tiny prefill of one token at 0")
    p.check(toks[1:31], 1, "tiny prefill 1..30")
    p.check(toks[31:32], 31, "tiny prefill of one token at the last slot")


def test_prefill_chunked_equals_one_shot_bitwise(make):
    """Every position's projections are independent rows of the GEMMs and its attention reads the same
    cache slots, so prefilling 0..63 in one call or as 0..23, 24..63 gives the same bits (logits, argmax
    and every cache slot)."""
    import torch
    wl = synth.get("smollm135m-kv128")
    W = synth.make_weights(wl)
    a, b = make(wl, W), make(wl, W)
    toks = [int(t) for t in synth.prompt_tokens(wl)]
    la, ia = a.prefill(toks, 0)
    b.prefill(toks[:24], 0)
    lb, ib = b.prefill(toks[24:], 24)
    assert np.array_equal(la.view(np.uint32), lb.view(np.uint32)) and ia == ib
    assert torch.equal(a.dec.kv, b.dec.kv)


def test_prefill_smollm135m_prompt_then_decode(make):
    """The SmolLM-135M-shaped 64-token prompt in one prefill, then greedy decode steps 64..79 (the first
    one fed the prefill's argmax through MBK_TOKEN_PREV), all against the oracle."""
    from persistent_megakernel_decode_wg_amd import MBK_TOKEN_PREV
    wl = synth.get("smollm135m-kv128")
    p = make(wl)
    toks = [int(t) for t in synth.prompt_tokens(wl)]
    lg, am, lo, ao = p.check(toks, 0, "smollm135m prefill 0..63")
    tok = ao
    for pos in range(64, 80):
        g_in = MBK_TOKEN_PREV if pos == 64 and am == ao else tok
        p.dec.decode_step(g_in, pos, p.logits, p.am)
        p.dec.check()
        lg = p.logits.cpu().numpy()
        lo, ao2, _ = p.ref.step(tok, pos)
        rel, _ = compare(lg, int(p.am.item()), lo, ao2)
        assert rel <= LOGIT_TOL, "decode after prefill, pos %d" % pos
        tok = ao2


def test_prefill_long_prompt_on_4096_slot_cache(make):
    """512 seeded tokens at positions 0..511 of the 4096-slot SmolLM-135M-shaped cache."""
    wl = synth.get("smollm135m-kv4096")
    p = make(wl)
    toks = [int(t) for t in synth.tokens(13, "long-prompt", 512, wl.vocab)]
    p.check(toks, 0, "smollm135m-kv4096 prefill 0..511")


def test_prefill_qwen2_bias(make):
    """Q/K/V biases and a 7-way query group: the 64-token prompt of the Qwen2-0.5B-shaped decoder."""
    wl = synth.get("qwen2-0.5b-kv128")
    p = make(wl)
    p.check([int(t) for t in synth.prompt_tokens(wl)], 0, "qwen2 prefill 0..63")


def test_prefill_argument_errors(make):
    from persistent_megakernel_decode_wg_amd import MBK_ERR_ARG, MBK_ERR_RANGE, MbkError
    wl = synth.get("tiny-2L-h64-kv32")
    p = make(wl)
    for toks, pos0, code in (([1, 2], wl.kv_capacity - 1, MBK_ERR_RANGE), ([1, wl.vocab], 0, MBK_ERR_ARG),
                             ([-1], 0, MBK_ERR_ARG), ([1], -1, MBK_ERR_RANGE)):
        with pytest.raises(MbkError) as e:
            p.dec.prefill(toks, pos0, p.logits, p.am)
        assert e.value.code == code


# (query heads, KV heads, head size): the matrix-core attention at head size 128 (per-head KV and G = 8), and the
# VALU attention at head size 32 (G = 5); 2-layer decoders on a 256-slot cache
PREFILL_SHAPES = [(6, 6, 128), (16, 2, 128), (10, 2, 32)]


@pytest.mark.parametrize("shape", PREFILL_SHAPES, ids=["nq%d-nkv%d-hd%d" % s for s in PREFILL_SHAPES])
def test_prefill_head_sizes_and_group_sizes(make, shape):
    """A 77-token prompt (a ragged last block of queries and keys) against the stepped oracle, then the same
    prompt as 0..40 and 41..76 giving the one-shot bits."""
    import torch
    nq, nkv, hd = shape
    wl = synth.Workload("pf-%d-%d-hd%d" % shape, 2, 256, nq, nkv, hd, 512, 1024, 256, False, 1e-5, 1e4,
                        n_prompt=0, kv_prefill=0, n_decode=0)
    W = synth.make_weights(wl)
    a, b = make(wl, W), make(wl, W)
    toks = [int(t) for t in synth.tokens(13, "prefill-shapes", 77, wl.vocab)]
    la, ia, _, _ = a.check(toks, 0, "prefill nq %d nkv %d hd %d" % shape)
    b.prefill(toks[:41], 0)
    lb, ib = b.prefill(toks[41:], 41)
    assert np.array_equal(la.view(np.uint32), lb.view(np.uint32)) and ia == ib
    assert torch.equal(a.dec.kv, b.dec.kv)


def test_prefill_maximum_sizes_to_the_last_slot(make):
    """The largest shape taken (hidden, query heads x head size and intermediate all 8,192, G = 8 at head size
    128), one layer: the cache pre-filled at 0..8,091 and a 100-token prompt prefilled at 8,092..8,191, the
    last slot, against the oracle stepped over the same positions."""
    import torch
    wl = synth.Workload("max-h8192-kv8192", 1, 8192, 64, 8, 128, 8192, 4096, 8192, False, 1e-5, 1e4,
                        n_prompt=0, kv_prefill=8092, n_decode=0)
    p = make(wl)
    kv = synth.kv_prefill(wl)
    P = kv.shape[3]
    p.dec.kv[:, :, :, :P, :] = torch.from_numpy(np.ascontiguousarray(kv).view(np.int16)).cuda()
    p.ref.prefill_kv(kv)
    toks = [int(t) for t in synth.tokens(17, "prefill-max", 100, wl.vocab)]
    assert P + len(toks) == wl.kv_capacity
    p.check(toks, P, "prefill max sizes")


def test_prefill_long_prompt_equals_short_chunks_bitwise(make):
    """A 512-token prompt on the SmolLM-135M shape in one call (its gate/up projection then runs with operand
    tiles shared through LDS by four waves) and in eight calls of 64 tokens (every projection with per-wave
    operands): the same logits, argmax and cache, bit for bit -- both forms add each row's products in the
    same order."""
    import torch
    wl = synth.get("smollm135m-kv4096")
    W = synth.make_weights(wl)
    a, b = make(wl, W), make(wl, W)
    toks = [int(t) for t in synth.tokens(19, "prefill-long", 512, wl.vocab)]
    la, ia = a.prefill(toks, 0)
    for c in range(0, 512, 64):
        lb, ib = b.prefill(toks[c:c + 64], c)
    assert np.array_equal(la.view(np.uint32), lb.view(np.uint32)) and ia == ib
    assert torch.equal(a.dec.kv, b.dec.kv)


def test_prefill_1p7b_shape_kernel_forms_agree_bitwise(make):
    """Two layers of the SmolLM-1.7B shape: a 256-token prompt in one call (every projection with operand tiles
    shared through LDS; query/key/value, output and down projections with their k-step quarters on separate
    workgroups, summed in order by a second kernel) and in four calls of 64 tokens (gate/up still through LDS; query/key/value
    with two row blocks and two position blocks, the 4M-weight output projection two row blocks and one
    position block, down one row block and two position blocks) give the same logits, argmax and cache bit for
    bit; the first 64-token call is also checked against the oracle."""
    import torch
    wl = synth.Workload("smollm1.7b-2L-kv512", 2, 2048, 32, 32, 64, 8192, 49152, 512, False, 1e-5, 1e4,
                        n_prompt=0, kv_prefill=0, n_decode=0)
    W = synth.make_weights(wl)
    a, b = make(wl, W), make(wl, W)
    toks = [int(t) for t in synth.tokens(23, "prefill-forms", 256, wl.vocab)]
    la, ia = a.prefill(toks, 0)
    b.check(toks[:64], 0, "smollm1.7b shape, 2 layers, prefill 0..63")
    for c in range(64, 256, 64):
        lb, ib = b.prefill(toks[c:c + 64], c)
    assert np.array_equal(la.view(np.uint32), lb.view(np.uint32)) and ia == ib
    assert torch.equal(a.dec.kv, b.dec.kv)


def test_prefill_inputs_not_a_multiple_of_32(make):
    """Hidden 200, query heads x head size 5 x 16 = 80 and intermediate 528 (each a multiple of 8 but not of
    32, so every GEMM's last k step of 32 inputs runs past the row's end onto cleared entries), vocabulary 1,030
    (a ragged last row block, and the argmax's one-logit-at-a-time scan): a 45-token prompt against the stepped
    oracle, and the same prompt as 0..20 and 21..44 giving the one-shot bits."""
    import torch
    wl = synth.Workload("pf-ragged-k-h200", 2, 200, 5, 1, 16, 528, 1030, 128, False, 1e-5, 1e4,
                        n_prompt=0, kv_prefill=0, n_decode=0)
    W = synth.make_weights(wl)
    a, b = make(wl, W), make(wl, W)
    toks = [int(t) for t in synth.tokens(29, "prefill-ragged-k", 45, wl.vocab)]
    la, ia, _, _ = a.check(toks, 0, "prefill hidden 200, Q 80, intermediate 528")
    b.prefill(toks[:21], 0)
    lb, ib = b.prefill(toks[21:], 21)
    assert np.array_equal(la.view(np.uint32), lb.view(np.uint32)) and ia == ib
    assert torch.equal(a.dec.kv, b.dec.kv)
