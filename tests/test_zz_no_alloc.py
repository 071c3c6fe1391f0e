"""The allocation-free entry point (mbk_decode_step_static, the step on the library's static scratch)
against mbk_decode_step with a caller workspace, through the C ABI: bitwise equal logits, argmax and cache
on calls in a row whose shapes (and workspaces) differ, the second call of each pair the smaller one."""
import numpy as np
import pytest

import synth
from gpu_util import log, upload

pytestmark = pytest.mark.gpu


class _Side:
    """Two handles on the same weights: `ref` steps with its own workspace (mbk_decode_step), `st` on the
    static scratch (mbk_decode_step_static) with a cache tensor of its own and no workspace bound."""

    def __init__(self, wl):
        import torch
        from persistent_megakernel_decode_wg_amd import Decoder
        self.wl = wl
        W = synth.make_weights(wl)
        Wd = upload(W)
        self.ref = Decoder(wl)
        self.ref.pack_weights(Wd)
        self.ref.alloc_kv()
        self.st = Decoder(wl)
        self.st.pack_weights(Wd)
        self.kv = torch.zeros_like(self.ref.kv)
        self.lg = [torch.empty(wl.vocab, dtype=torch.float32, device="cuda") for _ in range(2)]
        self.am = [torch.empty(1, dtype=torch.int32, device="cuda") for _ in range(2)]

    def step_static(self, token, pos):
        self.st.decode_step_static(self.kv, token, pos, self.lg[1], self.am[1])
        self.st.check()

    def step_ref(self, token, pos):
        self.ref.decode_step(token, pos, self.lg[0], self.am[0])
        self.ref.check()

    def assert_equal(self, what):
        import torch
        a, b = self.lg[0].cpu().numpy(), self.lg[1].cpu().numpy()
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), "%s: logits differ" % what
        assert int(self.am[0].item()) == int(self.am[1].item()), "%s: argmax differs" % what
        assert torch.equal(self.ref.kv, self.kv), "%s: cache differs" % what

    def close(self):
        self.ref.close()
        self.st.close()


def test_static_scratch_equals_workspace_step_on_calls_in_a_row():
    from persistent_megakernel_decode_wg_amd import MBK_TOKEN_PREV
    big = _Side(synth.get("smollm135m-kv128"))      # 55,552-byte workspace, 151 intervals
    small = _Side(synth.get("tiny-2L-h64-kv32"))    # 10,240-byte workspace, 11 intervals
    try:
        pb, ps = synth.prompt_tokens(big.wl), synth.prompt_tokens(small.wl)
        for pos in range(6):
            log("static scratch: pos %d, SmolLM-135M shape then the tiny shape" % pos)
            # first call: the larger shape
            big.step_static(int(pb[pos]), pos)
            big.step_ref(int(pb[pos]), pos)
            big.assert_equal("SmolLM-135M pos %d" % pos)
            # second call: the smaller shape, on the scratch the larger one just left
            small.step_static(int(ps[pos]), pos)
            small.step_ref(int(ps[pos]), pos)
            small.assert_equal("tiny pos %d" % pos)
        # the previous device argmax of the static scratch is the last static step's (the tiny shape's)
        small.step_static(MBK_TOKEN_PREV, 6)
        small.step_ref(MBK_TOKEN_PREV, 6)
        small.assert_equal("tiny pos 6, previous token")
        # the grid-barrier ordering on the static scratch (its barrier counters start from its own epoch)
        big.st.set_sync_mode(1)
        big.step_static(int(pb[6]), 6)
        big.st.set_sync_mode(0)
        big.step_ref(int(pb[6]), 6)
        big.assert_equal("SmolLM-135M pos 6, barrier mode")
        small.step_static(int(ps[7]), 7)
        small.step_ref(int(ps[7]), 7)
        small.assert_equal("tiny pos 7 after a barrier-mode step")
    finally:
        big.close()
        small.close()
