"""Decode parity for every query-head group size G the kernel is built for (1..8 query heads per KV head)
and head sizes 32, 64 and 128, on small 2-layer decoders with a 600-position prefilled cache.

The decode step is compiled once per G, and its attention folds 4, 2 or 1 cached positions per lane and
round depending on G; the model shapes of the other tests cover G = 1, 2, 3 and 7 only.  Each case runs
16 teacher-forced steps from position 600 with every step checked against the oracle (logits, argmax and
the cache slot written), once with one attention item per query head and once with the query heads of a KV
head packed into one item, with the split partials merged by the output projection (few partials) or by the
splits themselves (many: a 32-position split), and checks that the one-launch-per-interval executor gives
the persistent kernel's bits.  Shapes and values are synthetic (seeded random-init weights)."""
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
