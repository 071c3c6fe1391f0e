"""Decode parity for every query-head group size G the kernel is built for (1..8 query heads per KV head)
and head sizes 32, 64 and 128, on small 2-layer decoders with a 600-position prefilled cache.

The decode step is compiled once per G, and its attention folds 4, 2 or 1 cached positions per lane and
round depending on G; the model shapes of the other tests cover G = 1, 2, 3 and 7 only.  Each case runs
16 teacher-forced steps from position 600 with every step checked against the oracle (logits, argmax and
the cache slot written), once with one attention item per query head and once with the query heads of a KV
head packed into one item, with the split partials merged by the output projection (few partials) or by the
splits themselves (many: a 32-position split), and checks that the one-launch-per-interval executor gives
the persistent kernel's bits.  The largest shape the kernel takes (every GEMV input 8,192 wide, G = 8 at head
size 128, a one-layer decoder whose 8,192-slot cache is pre-filled to position 8,188) is stepped to the last
slot the same way.  Shapes and values are synthetic (seeded random-init weights)."""
import pytest

import synth

from gpu_util import Pair, log, teacher_forced

pytestmark = pytest.mark.gpu

# (query heads, KV heads, head size): G = 1, 4, 5, 6, 8, and G = 1 at head size 128
SHAPES = [(8, 8, 32), (8, 2, 64), (10, 2, 32), (12, 2, 64), (16, 2, 128), (6, 6, 128)]
CASES = [(s, packed, split) for s in SHAPES for packed in (False, True) for split in (0, 32)
         if not (packed and s[0] == s[1])]


def _workload(nq, nkv, hd):
    return synth.Workload("gqa-%d-%d-hd%d" % (nq, nkv, hd), 2, 256, nq, nkv, hd, 512, 1024, 1024, False, 1e-5, 1e4,
                          n_prompt=0, kv_prefill=600, n_decode=16)


@pytest.mark.parametrize("shape,packed,split", CASES,
                         ids=["nq%d-nkv%d-hd%d-%s-split%s" % (s + ("packed" if p else "perhead", sp or "default"))
                              for s, p, sp in CASES])
def test_gqa_group_sizes_and_head_sizes(shape, packed, split):
    nq, nkv, hd = shape
    wl = _workload(nq, nkv, hd)
    G = nq // nkv

    def setup(d):
        if packed:
            d.set_attention_items(G)
        if split:
            d.set_attention_split(split)

    p = Pair(wl, kv_prefix=synth.kv_prefill(wl), setup=setup)
    try:
        d = p.dec.describe()
        assert d["attention_heads_per_item"] == (G if packed else 1)
        positions = synth.decode_schedule(wl)
        label = "G=%d hd=%d %s split %s" % (G, hd, "packed" if packed else "per-head", split or "default")
        log("%s: positions %d..%d, max_splits %d" % (label, positions[0], positions[-1], d["max_splits"]))
        worst = teacher_forced(p, positions, [synth.first_token(wl)], label=label)
        log("%s: worst max|dlogit|/std = %.3g" % (label, worst))
        tok, pos = synth.first_token(wl), positions[-1]
        a, ia = p.gpu_step(tok, pos, "mega")
        b, ib = p.gpu_step(tok, pos, "ablation")
        assert (a.view("u4") == b.view("u4")).all() and ia == ib, label
    finally:
        p.close()


# the largest shape the kernel takes: every GEMV input 8,192 wide (hidden, query heads x head size,
# intermediate), G = 8 at head size 128, and the 8,192-slot cache filled to its last slot
MAX_WL = synth.Workload("max-h8192-kv8192", 1, 8192, 64, 8, 128, 8192, 4096, 8192, False, 1e-5, 1e4,
                        n_prompt=0, kv_prefill=8189, n_decode=3)


@pytest.mark.parametrize("packed", [False, True], ids=["perhead", "packed"])
def test_maximum_sizes_to_the_last_slot(packed):
    wl = MAX_WL
    G = wl.n_heads // wl.n_kv_heads
    p = Pair(wl, kv_prefix=synth.kv_prefill(wl), setup=(lambda d: d.set_attention_items(G)) if packed else None)
    try:
        positions = synth.decode_schedule(wl)
        assert positions[-1] == wl.kv_capacity - 1
        label = "max sizes %s" % ("packed" if packed else "per-head")
        log("%s: positions %d..%d, %s" % (label, positions[0], positions[-1], p.dec.describe()))
        worst = teacher_forced(p, positions, [synth.first_token(wl)], label=label)
        log("%s: worst max|dlogit|/std = %.3g" % (label, worst))
        tok, pos = synth.first_token(wl), positions[-1]
        a, ia = p.gpu_step(tok, pos, "mega")
        b, ib = p.gpu_step(tok, pos, "ablation")
        assert (a.view("u4") == b.view("u4")).all() and ia == ib, label
    finally:
        p.close()
