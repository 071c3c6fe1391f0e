"""Auxiliary checks on the GPU through the C ABI: validated grid barriers, KV checkpoint/resume, and the
packed weight layout read back byte for byte."""
import numpy as np
import pytest

import synth
from gpu_util import log, upload

pytestmark = pytest.mark.gpu


def _decoder(wl, W=None):
    from persistent_megakernel_decode_wg_amd import Decoder
    W = synth.make_weights(wl) if W is None else W
    d = Decoder(wl)
    d.pack_weights(upload(W))
    d.alloc_kv()
    return d, W


def test_grid_barrier_validated_over_100k_rounds():
    """10^5 counting grid barriers on every compute unit; after each, every workgroup reads every
    workgroup's epoch slot, which must already hold that round's value."""
    d, _ = _decoder(synth.get("tiny-2L-h64-kv32"))
    try:
        bad = d.barrier_stress(100000)
        assert bad[0] == 0, "first failed check: round %d, reader %d, writer %d, value %d" % bad
        # the decode step still works on the same workspace afterwards (barrier epochs continue)
        import torch
        lg = torch.empty(d.cfg.vocab, dtype=torch.float32, device="cuda")
        am = torch.empty(1, dtype=torch.int32, device="cuda")
        d.set_sync_mode(1)
        d.decode_step(3, 0, lg, am)
        d.check()
    finally:
        d.close()


def test_grid_barrier_missing_workgroup_times_out_and_recovers():
    """A workgroup that never arrives (host-set debug switch, small spin limit): every other workgroup's
    bounded wait expires, the call reports MBK_ERR_TIMEOUT, and after re-binding the workspace the
    validated barriers pass again."""
    from persistent_megakernel_decode_wg_amd import MBK_ERR_TIMEOUT, MbkError
    d, _ = _decoder(synth.get("tiny-2L-h64-kv32"))
    try:
        d.set_debug(spin_limit=1 << 12, skip_wg=3)
        with pytest.raises(MbkError) as e:
            d.barrier_stress(64)
        assert e.value.code == MBK_ERR_TIMEOUT
        d.set_debug(0, -1, -1)
        d.rebind()
        assert d.barrier_stress(1000)[0] == 0
    finally:
        d.close()


def test_kv_checkpoint_resume_is_bitwise():
    """Decode to position P, copy the cache to the host, destroy the handle, build a new one, restore the
    cache and continue: every later step's logits and argmax equal those of an uninterrupted run, bit for
    bit (the step's state is the bounded contiguous KV cache; the workspace holds none across steps)."""
    import torch
    wl = synth.get("smollm135m-kv128")
    W = synth.make_weights(wl)
    prompt = [int(t) for t in synth.prompt_tokens(wl)]
    P, N = 72, 24

    def run(d, positions, token_at):
        lg = torch.empty(wl.vocab, dtype=torch.float32, device="cuda")
        am = torch.empty(1, dtype=torch.int32, device="cuda")
        out = []
        for pos in positions:
            d.decode_step(token_at(pos, out), pos, lg, am)
            d.check()
            out.append((lg.cpu().numpy().copy(), int(am.item())))
        return out

    # uninterrupted: the prompt, then greedy tokens (each step's argmax is the next step's token)
    a, _ = _decoder(wl, W)
    try:
        full = run(a, list(range(P + N)), lambda pos, out: prompt[pos] if pos < len(prompt) else out[-1][1])
    finally:
        a.close()
    token = lambda pos, out: prompt[pos] if pos < len(prompt) else full[pos - 1][1]
    b, _ = _decoder(wl, W)
    try:
        head = run(b, list(range(P)), token)
        saved = b.kv.cpu().numpy().copy()
    finally:
        b.close()
    for i in range(P):
        assert np.array_equal(full[i][0].view(np.uint32), head[i][0].view(np.uint32)), "step %d" % i
    c, _ = _decoder(wl, W)
    try:
        c.kv.copy_(torch.from_numpy(saved).cuda())
        tail = run(c, list(range(P, P + N)), token)
    finally:
        c.close()
    for i, (x, y) in enumerate(zip(full[P:], tail)):
        assert np.array_equal(x[0].view(np.uint32), y[0].view(np.uint32)) and x[1] == y[1], "step %d" % (P + i)
    log("KV checkpoint/resume: %d steps after position %d bitwise equal" % (N, P))


def _unpack(blob: np.ndarray, g: dict) -> np.ndarray:
    """Inverse of the packed layout (include/mbk.h, mbk_get_matrix_layout), written from its description:
    returns the [rows][cols] bf16 matrix in packed row order, after checking that every padding row and
    group is zero."""
    T, S, RT, L = g["tiles"], g["steps"], g["rows_per_tile"], g["lanes_per_row"]
    n = T * S * 64 * 8
    raw = blob[g["offset"]:g["offset"] + 2 * n].view(np.uint16).reshape(T, S, RT, L, 8)
    M = raw.transpose(0, 2, 1, 3, 4).reshape(T * RT, S * L * 8)
    assert not M[g["rows"]:].any(), "nonzero padding rows"
    assert not M[:, g["cols"]:].any(), "nonzero padding groups"
    return M[:g["rows"], :g["cols"]]


def _rope_pairs(Wh: np.ndarray, heads: int, hd: int) -> np.ndarray:
    """Rows of each head reordered so that rows 2m, 2m+1 are head dims m, m + hd/2."""
    perm = np.empty(hd, dtype=np.int64)
    perm[0::2] = np.arange(hd // 2)
    perm[1::2] = np.arange(hd // 2) + hd // 2
    return Wh.reshape(heads, hd, -1)[:, perm, :].reshape(heads * hd, -1)


@pytest.mark.parametrize("name,layers", [("tiny-2L-h64-kv32", None), ("smollm135m-kv128", [0, 17, 29]),
                                         ("qwen2-0.5b-kv128", [0, 23]), ("smollm1.7b-kv4096", [5])])
def test_packed_weights_round_trip_bit_exact(name, layers):
    """Every packed matrix read back from the blob on the host (layout from mbk_get_matrix_layout) equals
    its source bf16 matrix bit for bit, with the Q/K/V rotation pairs and the gate/up interleave undone,
    and every padding row and group zero."""
    wl = synth.get(name)
    W = synth.make_weights(wl)
    d, _ = _decoder(wl, W)
    try:
        blob = d.packed.cpu().numpy()
        hd = wl.head_dim
        for l in (range(wl.n_layers) if layers is None else layers):
            L = W["layers"][l]
            want = {
                0: np.concatenate([_rope_pairs(L["wq"], wl.n_heads, hd), _rope_pairs(L["wk"], wl.n_kv_heads, hd),
                                   L["wv"]]),
                1: L["wo"],
                2: np.stack([L["wgate"], L["wup"]], axis=1).reshape(2 * wl.intermediate, wl.hidden),
                3: L["wdown"],
            }
            for which, w in want.items():
                g = d.matrix_layout(l, which)
                assert g["kind"] == (1 if which == 0 else 2 if which == 2 else 0)
                got = _unpack(blob, g)
                assert got.shape == w.shape and np.array_equal(got, w), "layer %d matrix %d" % (l, which)
        g = d.matrix_layout(-1, 0)
        assert np.array_equal(_unpack(blob, g), W["embed"]), "tied embedding"
    finally:
        d.close()
