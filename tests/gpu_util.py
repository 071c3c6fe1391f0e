"""Helpers of the GPU parity tests: upload synthetic weights, run the HIP path and the oracle side by side."""
from __future__ import annotations

import sys

import numpy as np

import oracle
import synth

# Acceptance: per step, max |logit_gpu - logit_oracle| <= LOGIT_TOL * std(oracle logits); greedy tokens
# equal wherever the oracle's top-1/top-2 margin exceeds MARGIN.
LOGIT_TOL = 2e-2
MARGIN = 5e-2
# The cache slot written by a step, checked per layer and per K / V:
#  * layer 0 reads the same input on both sides (the embedding row), so there every bf16 entry lies within
#    one bf16 step (of the larger magnitude) plus KV_REL times the RMS of the layer's key (or value) vector
#    of the oracle's: both sides round an fp32 value to bf16, and those values differ by the GPU's own
#    arithmetic (its ~16-bit input representation, fp32 accumulation order), which in entries much smaller
#    than the RMS (cancellation) can exceed the entry's own bf16 step;
#  * every layer's key and value vectors lie within LOGIT_TOL of the oracle's in relative L2 norm.  From
#    layer 1 on the inputs differ by what earlier layers carried forward: bf16 cache roundings that land on
#    neighbouring values move later layers by far more than their own rounding.  An emulation of the GPU's
#    input representation on the CPU (SmolLM-135M shape, positions 0..23) stays at <= 3.1e-3; a wrong
#    rotation pair or sign, head, slot or bias moves a vector by a sizeable fraction of its norm.
KV_REL = 2.0 ** -10


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()


def upload(W):
    return {"embed": to_dev(W["embed"]), "final_norm": to_dev(W["final_norm"]),
            "layers": [{k: to_dev(v) for k, v in L.items()} for L in W["layers"]]}


def bf16_step(m: np.ndarray) -> np.ndarray:
    """The spacing of bf16 values at magnitude m (8 significant bits)."""
    m = np.maximum(np.abs(m), np.finfo(np.float32).tiny)
    return np.exp2(np.floor(np.log2(m)) - 7)


def kv_slot_check(gpu: np.ndarray, want: np.ndarray):
    """For bf16 bit patterns [NL][2][nkv][hd]: (layer-0 |gpu - want| / (bf16 step + KV_REL * rms) per entry
    [2][nkv][hd], relative L2 difference per layer and K/V [NL][2])."""
    a = synth.bf16_to_f32(gpu).astype(np.float64)
    b = synth.bf16_to_f32(want).astype(np.float64)
    rms = np.sqrt(np.mean(b * b, axis=(2, 3), keepdims=True))
    tol0 = bf16_step(np.maximum(np.abs(a[0]), np.abs(b[0]))) + KV_REL * rms[0]
    rel = np.sqrt(np.sum((a - b) ** 2, axis=(2, 3)) / np.maximum(np.sum(b * b, axis=(2, 3)), 1e-300))
    return np.abs(a[0] - b[0]) / tol0, rel


class Pair:
    """A GPU decoder and the oracle on the same workload, weights and KV prefix."""

    def __init__(self, wl, W=None, kv_prefix=None, setup=None, oracle_W=None):
        """setup(decoder), if given, runs before the weights are packed (plan-time settings); oracle_W,
        if given, are the weights the oracle runs (the model the packed weights stand for)."""
        import torch
        from persistent_megakernel_decode_wg_amd import Decoder
        from persistent_megakernel_decode_wg_amd import build as mbk_build
        mbk_build.ensure_built()
        self.wl = wl
        self.W = synth.make_weights(wl) if W is None else W
        self.dec = Decoder(wl)
        if setup is not None:
            setup(self.dec)
        self.dec.pack_weights(upload(self.W))
        self.dec.alloc_kv()
        self.ref = oracle.Model(wl, self.W if oracle_W is None else oracle_W)
        if kv_prefix is not None:
            P = kv_prefix.shape[3]
            self.dec.kv[:, :, :, :P, :] = torch.from_numpy(np.ascontiguousarray(kv_prefix).view(np.int16)).cuda()
            self.ref.prefill_kv(kv_prefix)
        self.logits = torch.empty(wl.vocab, dtype=torch.float32, device="cuda")
        self.am = torch.empty(1, dtype=torch.int32, device="cuda")
        self.kv_slot = None
        torch.cuda.synchronize()

    def close(self):
        """Releases the handle (no HIP call is left for interpreter exit)."""
        if self.dec is not None:
            self.dec.close()
            self.dec = None

    def gpu_step(self, token, pos, mode="mega", kv_check=False):
        """mode: mega (persistent kernel, dataflow), cooperative (the same, cooperative launch),
        barrier (persistent kernel, grid barriers), ablation (one launch per interval) or graph
        (the ablation replayed as a hipGraph).  kv_check: assert that the step changed no cache slot
        but `pos` and keep that slot (bf16 bits [NL][2][nkv][hd]) in self.kv_slot."""
        import torch
        before = self.dec.kv.clone() if kv_check else None
        if mode == "mega":
            self.dec.decode_step(token, pos, self.logits, self.am)
        elif mode == "cooperative":
            self.dec.set_launch_mode(1)
            try:
                self.dec.decode_step(token, pos, self.logits, self.am)
            finally:
                self.dec.set_launch_mode(0)
        elif mode == "barrier":
            self.dec.set_sync_mode(1)
            try:
                self.dec.decode_step(token, pos, self.logits, self.am)
            finally:
                self.dec.set_sync_mode(0)
        elif mode == "ablation":
            self.dec.decode_step_ablation(token, pos, self.logits, self.am, use_graph=False)
        else:
            self.dec.decode_step_ablation(token, pos, self.logits, self.am, use_graph=True)
        self.dec.check()
        if kv_check:
            after = self.dec.kv
            self.kv_slot = after[:, :, :, pos, :].cpu().numpy().view(np.uint16).copy()
            a = after.clone()
            a[:, :, :, pos, :] = 0
            before[:, :, :, pos, :] = 0
            assert torch.equal(a, before), "pos %d: the step changed cache slots other than its own" % pos
            del a, before
        return self.logits.cpu().numpy().copy(), int(self.am.item())

    def check_kv_slot(self, pos, label=""):
        """The slot the last kv_check step wrote, every layer, K and V, against the oracle's cache.
        Returns (layer-0 worst |difference| / tolerance, worst relative L2 difference over the layers)."""
        want = self.ref.kv[:, :, :, pos, :]
        x0, rel = kv_slot_check(self.kv_slot, want)
        if x0.max() > 1.0:
            c, j, e = np.unravel_index(int(x0.argmax()), x0.shape)
            g, o = synth.bf16_to_f32(self.kv_slot[0, c, j, e]), synth.bf16_to_f32(want[0, c, j, e])
            raise AssertionError("%s pos %d: cache slot layer 0 %s head %d dim %d: GPU %.6g oracle %.6g (%.3g x the "
                                 "tolerance)" % (label, pos, "KV"[c], j, e, g, o, x0.max()))
        if rel.max() > LOGIT_TOL:
            l, c = np.unravel_index(int(rel.argmax()), rel.shape)
            raise AssertionError("%s pos %d: cache slot layer %d %s differs from the oracle's by %.3g in relative L2 "
                                 "norm (> %.3g)" % (label, pos, l, "KV"[c], rel.max(), LOGIT_TOL))
        return float(x0.max()), float(rel.max())


def compare(lg, am, lo, ao):
    """Checks one step's logits and argmax against the oracle; returns (max|dlogit| / std, margin).

    * the GPU argmax is the lowest index attaining the maximum of the GPU's own logits (index work:
      exact at every step);
    * where the oracle's top-1/top-2 margin exceeds MARGIN it is the oracle's argmax;
    * elsewhere it is one of the oracle's near-ties: its oracle logit lies within the two-sided logit
      tolerance (2 * LOGIT_TOL * std) of the oracle's maximum.
    """
    lo64 = lo.astype(np.float64)
    std = float(lo64.std())
    err = float(np.max(np.abs(lg.astype(np.float64) - lo64)))
    top = np.sort(lo64)[-2:]
    margin = float(top[1] - top[0])
    own = int(np.argmax(lg))   # numpy returns the first (lowest) index among equal maxima
    assert am == own, "GPU argmax %d is not the lowest-index maximum %d of the GPU's own logits" % (am, own)
    if margin > MARGIN:
        assert am == ao, "argmax %d != oracle %d with margin %.3g" % (am, ao, margin)
    else:
        assert lo64[am] >= top[1] - 2 * LOGIT_TOL * std, (
            "low-margin step: GPU argmax %d has oracle logit %.5g, below the oracle maximum %.5g by more than "
            "2 * %.3g * std" % (am, lo64[am], top[1], LOGIT_TOL))
    return err / std, margin


def teacher_forced(pair: Pair, positions, first_tokens, mode="mega", check_every=1, label="", kv_check=True):
    """Runs both sides over `positions`, feeding the GPU the oracle's tokens. Every step at index
    i % check_every == 0, and the last one, compares logits, argmax and (kv_check) the cache slot the
    step wrote. Returns the worst max|dlogit|/std."""
    worst = kv0 = kvrel = 0.0
    tok = None
    n = len(positions)
    for i, pos in enumerate(positions):
        t_in = int(first_tokens[i]) if i < len(first_tokens) else tok
        checked = i % check_every == 0 or i == n - 1
        lg, am = pair.gpu_step(t_in, pos, mode, kv_check=kv_check and checked)
        lo, ao, _ = pair.ref.step(t_in, pos)
        if checked:
            assert np.all(np.isfinite(lg)), "%s pos %d: non-finite logits" % (label, pos)
            rel, margin = compare(lg, am, lo, ao)
            worst = max(worst, rel)
            assert rel <= LOGIT_TOL, "%s pos %d: max|dlogit| = %.4g std > %.3g" % (label, pos, rel, LOGIT_TOL)
            if kv_check:
                x0, rel = pair.check_kv_slot(pos, label)
                kv0, kvrel = max(kv0, x0), max(kvrel, rel)
        tok = ao
    if kv_check:
        log("%s: cache slots: layer 0 worst difference / tolerance %.3g; worst relative L2 over layers %.3g"
            % (label, kv0, kvrel))
    return worst
