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


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()


def upload(W):
    return {"embed": to_dev(W["embed"]), "final_norm": to_dev(W["final_norm"]),
            "layers": [{k: to_dev(v) for k, v in L.items()} for L in W["layers"]]}


class Pair:
    """A GPU decoder and the oracle on the same workload, weights and KV prefix."""

    def __init__(self, wl, W=None, kv_prefix=None, setup=None):
        """setup(decoder), if given, runs before the weights are packed (plan-time settings)."""
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
        self.ref = oracle.Model(wl, self.W)
        if kv_prefix is not None:
            P = kv_prefix.shape[3]
            self.dec.kv[:, :, :, :P, :] = torch.from_numpy(np.ascontiguousarray(kv_prefix).view(np.int16)).cuda()
            self.ref.prefill_kv(kv_prefix)
        self.logits = torch.empty(wl.vocab, dtype=torch.float32, device="cuda")
        self.am = torch.empty(1, dtype=torch.int32, device="cuda")
        torch.cuda.synchronize()

    def gpu_step(self, token, pos, mode="mega"):
        """mode: mega (persistent kernel, dataflow), cooperative (the same, cooperative launch),
        barrier (persistent kernel, grid barriers), ablation (one launch per interval) or graph
        (the ablation replayed as a hipGraph)."""
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
        return self.logits.cpu().numpy().copy(), int(self.am.item())


def compare(lg, am, lo, ao):
    """Returns (max|dlogit| / std, margin, argmax_ok)."""
    lo64 = lo.astype(np.float64)
    std = float(lo64.std())
    err = float(np.max(np.abs(lg.astype(np.float64) - lo64)))
    top = np.sort(lo64)[-2:]
    margin = float(top[1] - top[0])
    return err / std, margin, (am == ao) or margin <= MARGIN


def teacher_forced(pair: Pair, positions, first_tokens, mode="mega", check_every=1, label=""):
    """Runs both sides over `positions`, feeding the GPU the oracle's tokens. Returns worst err/std."""
    worst = 0.0
    tok = None
    for i, pos in enumerate(positions):
        t_in = int(first_tokens[i]) if i < len(first_tokens) else tok
        lg, am = pair.gpu_step(t_in, pos, mode)
        lo, ao, _ = pair.ref.step(t_in, pos)
        if i % check_every == 0 or i == len(positions) - 1:
            rel, margin, ok = compare(lg, am, lo, ao)
            worst = max(worst, rel)
            assert np.all(np.isfinite(lg)), "%s pos %d: non-finite logits" % (label, pos)
            assert rel <= LOGIT_TOL, "%s pos %d: max|dlogit| = %.4g std > %.3g" % (label, pos, rel, LOGIT_TOL)
            assert ok, "%s pos %d: argmax %d != oracle %d with margin %.3g" % (label, pos, am, ao, margin)
        tok = ao
    return worst
