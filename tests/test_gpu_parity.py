"""Parity of the HIP decode step (through the C ABI) with the CPU oracle, on the GPU.

Every checked step compares the logits (max |dlogit| <= 2e-2 * std of the oracle's logits), the argmax
(exactly the lowest-index maximum of the GPU's own logits; the oracle's where its top-1/top-2 margin
exceeds 5e-2, else one of its near-ties) and the cache slot the step wrote (every layer's key and value
within one bf16 step of the oracle's; no other slot changed)."""
import numpy as np
import pytest

import synth

from gpu_util import LOGIT_TOL, MARGIN, Pair, compare, log, teacher_forced

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tiny():
    p = Pair(synth.get("tiny-2L-h64-kv32"))
    yield p
    p.close()


@pytest.fixture
def pair_factory():
    """Pairs made through this fixture are closed when the test ends."""
    made = []

    def make(*a, **kw):
        p = Pair(*a, **kw)
        made.append(p)
        return p
    yield make
    for p in made:
        p.close()


def _bitwise(a, ia, b, ib):
    return np.array_equal(a.view(np.uint32), b.view(np.uint32)) and ia == ib


def test_tiny_full_schedule_teacher_forced(tiny):
    wl = tiny.wl
    log("tiny: prompt %d + %d greedy steps" % (wl.n_prompt, wl.n_decode))
    worst = teacher_forced(tiny, synth.decode_schedule(wl), list(synth.prompt_tokens(wl)), label="tiny")
    log("tiny worst max|dlogit|/std = %.3g" % worst)


@pytest.mark.parametrize("mode", ["cooperative", "barrier", "ablation", "graph"])
def test_tiny_executors_are_bitwise_equal(tiny, mode):
    wl = tiny.wl
    prompt = list(synth.prompt_tokens(wl))
    for pos in range(12):
        tok = prompt[pos % len(prompt)]
        a, ia = tiny.gpu_step(tok, pos, "mega")
        b, ib = tiny.gpu_step(tok, pos, mode)
        assert _bitwise(a, ia, b, ib), "pos %d" % pos


def test_tiny_rerun_same_position_is_idempotent_and_deterministic(tiny):
    wl = tiny.wl
    prompt = list(synth.prompt_tokens(wl))
    for pos in range(6):
        tiny.gpu_step(prompt[pos], pos)
    a, ia = tiny.gpu_step(prompt[5], 5)
    b, ib = tiny.gpu_step(prompt[5], 5)
    assert _bitwise(a, ia, b, ib)


def test_tiny_edge_tokens_and_last_slot(pair_factory):
    wl = synth.get("tiny-2L-h64-kv32")
    p = pair_factory(wl)
    toks = [0, wl.vocab - 1] + [int(t) for t in synth.tokens(5, "edge", wl.kv_capacity - 2, wl.vocab)]
    # positions 0 .. capacity-1: the last step fills the final slot
    teacher_forced(p, list(range(wl.kv_capacity)), toks, check_every=1, label="tiny-edge")


def test_tiny_pipelined_previous_token_matches_oracle_greedy(pair_factory):
    from persistent_megakernel_decode_wg_amd import MBK_TOKEN_PREV
    wl = synth.get("tiny-2L-h64-kv32")
    p = pair_factory(wl)
    prompt = list(synth.prompt_tokens(wl))
    tok = None
    for pos in synth.decode_schedule(wl):
        t_gpu = prompt[pos] if pos < len(prompt) else MBK_TOKEN_PREV
        t_ref = prompt[pos] if pos < len(prompt) else tok
        lg, am = p.gpu_step(t_gpu, pos)
        lo, ao, _ = p.ref.step(t_ref, pos)
        lo64 = lo.astype(np.float64)
        rel = float(np.max(np.abs(lg - lo64))) / float(lo64.std())
        assert rel <= LOGIT_TOL
        assert am == int(np.argmax(lg))
        if am != ao:
            top = np.sort(lo64)[-2:]
            margin = float(top[1] - top[0])
            assert margin <= MARGIN, "free-running greedy diverged at pos %d with margin %.3g" % (pos, margin)
            break
        tok = ao


def test_zero_projections_closed_form_on_gpu(pair_factory):
    """W_o = W_down = 0 keeps the residual at E[t]: argmax must be t and logits E (w_f * E_t / rms)."""
    wl = synth.get("tiny-2L-h64-kv32")
    W = synth.make_weights(wl)
    for L in W["layers"]:
        L["wo"] = np.zeros_like(L["wo"])
        L["wdown"] = np.zeros_like(L["wdown"])
    p = pair_factory(wl, W)
    for t in [3, 321, 511]:
        lg, am = p.gpu_step(t, 0)
        assert am == t
        E = synth.bf16_to_f32(W["embed"]).astype(np.float64)
        e = E[t]
        want = E @ (e / np.sqrt(np.mean(e * e) + wl.rms_eps) * synth.bf16_to_f32(W["final_norm"]))
        np.testing.assert_allclose(lg, want, rtol=1e-4, atol=1e-4 * np.abs(want).max())


def test_smollm135m_kv128_full_schedule(pair_factory):
    """All 128 steps (64 prompt positions, then 64 greedy steps to the last slot), every step checked;
    then the cooperative launch, the barrier mode and both ablations give the persistent kernel's bits at
    this size."""
    wl = synth.get("smollm135m-kv128")
    p = pair_factory(wl)
    sched = synth.decode_schedule(wl)
    log("smollm135m-kv128: %d steps, positions %d..%d" % (len(sched), sched[0], sched[-1]))
    worst = teacher_forced(p, sched, list(synth.prompt_tokens(wl)), label="smollm135m")
    log("smollm135m-kv128 worst max|dlogit|/std = %.3g" % worst)
    tok = int(synth.prompt_tokens(wl)[7])
    for pos in (3, 64, 127):
        a, ia = p.gpu_step(tok, pos, "mega")
        for mode in ("cooperative", "barrier", "ablation", "graph"):
            b, ib = p.gpu_step(tok, pos, mode)
            assert _bitwise(a, ia, b, ib), "pos %d %s" % (pos, mode)


def test_smollm135m_kv4096_prefilled_long_context(pair_factory):
    """The 4096-slot cache pre-filled at 0..4031: all 64 steps 4032..4095 (the last slot), every step
    checked; split-context attention gives the same bits in every executor, although the persistent
    kernel merges the splits in all of them at once (each a slice of the head) and a one-interval launch
    merges them in the last split to arrive."""
    wl = synth.get("smollm135m-kv4096")
    p = pair_factory(wl, kv_prefix=synth.kv_prefill(wl))
    positions = synth.decode_schedule(wl)
    assert positions[-1] == wl.kv_capacity - 1
    log("smollm135m-kv4096: positions %d..%d" % (positions[0], positions[-1]))
    worst = teacher_forced(p, positions, [synth.first_token(wl)], label="smollm135m-4k")
    log("smollm135m-kv4096 worst max|dlogit|/std = %.3g" % worst)
    tok = synth.first_token(wl)
    for pos in (positions[8], positions[-1]):
        a, ia = p.gpu_step(tok, pos, "mega")
        for mode in ("cooperative", "barrier", "ablation", "graph"):
            b, ib = p.gpu_step(tok, pos, mode)
            assert _bitwise(a, ia, b, ib), "pos %d %s" % (pos, mode)


def test_smollm135m_kv128_split_attention_merged_by_output_projection(pair_factory):
    """A 32-position attention split on the 128-slot cache (up to 4 splits per query head): the split
    partials are tagged and merged by the output projection's workgroups while they load their input.
    Every position 0..127 is checked (so every split count 1..4 and every split boundary: attended lengths
    32, 33, 64, 65, 96, 97, 128); every executor gives the same bits."""
    wl = synth.get("smollm135m-kv128")
    p = pair_factory(wl)
    p.dec.set_attention_split(32)
    d = p.dec.describe()
    assert d["max_splits"] >= 4
    positions = list(range(wl.kv_capacity))
    worst = teacher_forced(p, positions, list(synth.prompt_tokens(wl)), label="smollm135m-split32")
    log("smollm135m-kv128 split 32: worst max|dlogit|/std = %.3g" % worst)
    tok = int(synth.prompt_tokens(wl)[5])
    for pos in (31, 32, 64, 100):
        a, ia = p.gpu_step(tok, pos, "mega")
        for mode in ("barrier", "ablation", "graph"):
            b, ib = p.gpu_step(tok, pos, mode)
            assert _bitwise(a, ia, b, ib), "pos %d %s" % (pos, mode)


def test_smollm135m_kv4096_packed_gqa_items(pair_factory):
    """The query heads of a KV head packed into one attention item (each cached key and value read
    once), the split merge spread over the splits (persistent kernel) or done by the last split to arrive
    (ablation): all 64 steps to the last slot (every 4th checked, and the last), and equal bits across
    executors."""
    wl = synth.get("smollm135m-kv4096")
    G = wl.n_heads // wl.n_kv_heads
    p = pair_factory(wl, kv_prefix=synth.kv_prefill(wl), setup=lambda d: d.set_attention_items(G))
    assert p.dec.describe()["attention_heads_per_item"] == G
    positions = synth.decode_schedule(wl)
    worst = teacher_forced(p, positions, [synth.first_token(wl)], check_every=4, label="smollm135m-4k-packed")
    log("smollm135m-kv4096 packed items: worst max|dlogit|/std = %.3g" % worst)
    pos, tok = positions[8], synth.first_token(wl)
    a, ia = p.gpu_step(tok, pos, "mega")
    for mode in ("barrier", "ablation"):
        b, ib = p.gpu_step(tok, pos, mode)
        assert _bitwise(a, ia, b, ib), mode


def test_phase_timer_stamps(tiny):
    """The phase timer: a workgroup with work in an interval stamps start <= inputs loaded <= body done; the
    launch clears every workgroup's entries first (stale values never survive); the results are the same
    bits as without the timer."""
    import torch
    wl = tiny.wl
    tok = int(synth.prompt_tokens(wl)[0])
    a, ia = tiny.gpu_step(tok, 0)
    tr = tiny.dec.set_phase_trace(True)
    try:
        tr.fill_(-1)       # stale values: the launch clears this workgroup's entries first
        b, ib = tiny.gpu_step(tok, 0)
        torch.cuda.synchronize()
        t = tr.cpu().numpy()
    finally:
        tiny.dec.set_phase_trace(False)
    assert _bitwise(a, ia, b, ib)
    assert not (t == -1).any()
    work = t[:, :, 1] > 0
    assert work.any(axis=1).all(), "every interval has a working workgroup"
    tw = t[work]
    assert (tw[:, 0] > 0).all() and (tw[:, 0] <= tw[:, 1]).all() and (tw[:, 1] <= tw[:, 2]).all()
    # no work: nothing stamped, or (only split items beyond this step's split count) start and done
    idle = t[~work]
    assert (((idle[:, 0] == 0) & (idle[:, 2] == 0)) | ((idle[:, 0] > 0) & (idle[:, 2] >= idle[:, 0]))).all()


@pytest.mark.parametrize("mode", ["mega", "barrier"])
def test_watchdog_expires_and_recovers(pair_factory, mode):
    """Workgroup 0 leaves the persistent kernel before interval 0 (host-set debug switch, tiny spin
    limit): the waits that need its results expire, every workgroup exits, the step reports
    MBK_ERR_TIMEOUT, and after re-binding the workspace the next step is correct again."""
    from persistent_megakernel_decode_wg_amd import MBK_ERR_TIMEOUT, MbkError
    wl = synth.get("tiny-2L-h64-kv32")
    p = pair_factory(wl)
    tok = int(synth.prompt_tokens(wl)[0])
    p.dec.set_debug(spin_limit=1 << 14, skip_wg=0, skip_interval=0)
    with pytest.raises(MbkError) as e:
        p.gpu_step(tok, 0, mode)
    assert e.value.code == MBK_ERR_TIMEOUT
    p.dec.set_debug(0, -1, -1)
    p.dec.rebind()
    teacher_forced(p, [0, 1, 2], list(synth.prompt_tokens(wl)), mode=mode, label="after-watchdog")


def test_qwen2_0p5b_bias_kv128(pair_factory):
    """Q/K/V biases and a 7-way query group: all 128 steps (64 prompt positions, 64 greedy steps to the
    last slot), every step checked."""
    wl = synth.get("qwen2-0.5b-kv128")
    p = pair_factory(wl)
    positions = synth.decode_schedule(wl)
    assert positions[-1] == wl.kv_capacity - 1
    worst = teacher_forced(p, positions, list(synth.prompt_tokens(wl)), label="qwen2")
    log("qwen2-0.5b-kv128 worst max|dlogit|/std = %.3g" % worst)


def test_smollm1p7b_kv4096_prefilled(pair_factory):
    """No query grouping (32/32 heads), 4096-slot cache pre-filled at 0..4031: all 64 steps to the last
    slot, every 4th step checked, and the last one."""
    wl = synth.get("smollm1.7b-kv4096")
    p = pair_factory(wl, kv_prefix=synth.kv_prefill(wl))
    positions = synth.decode_schedule(wl)
    assert positions[-1] == wl.kv_capacity - 1
    worst = teacher_forced(p, positions, [synth.first_token(wl)], check_every=4, label="smollm1.7b-4k")
    log("smollm1.7b-kv4096 worst max|dlogit|/std = %.3g" % worst)
