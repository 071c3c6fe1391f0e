"""C ABI checks that need no GPU: exported symbols and host-side validation."""
import ctypes
import os
import re

import pytest

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    from persistent_megakernel_decode_wg_amd import build as mbk_build
    mbk_build.ensure_built()
    import persistent_megakernel_decode_wg_amd as pkg
    return pkg.lib()


def _declared_functions():
    with open(os.path.join(ROOT, "include", "mbk.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mbk_[a-z_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(L):
    names = _declared_functions()
    assert "mbk_decode_step" in names and "mbk_pack_weights" in names and "mbk_alloc_kv" in names
    for n in names:
        assert hasattr(L, n), "libmbk.so does not export %s" % n


def _create(cfg):
    from persistent_megakernel_decode_wg_amd.binding import make_config
    c = make_config(cfg)
    h = ctypes.c_void_p()
    import persistent_megakernel_decode_wg_amd as pkg
    rc = pkg.lib().mbk_create(ctypes.byref(c), ctypes.byref(h))
    return rc, h


@pytest.mark.parametrize("change,code", [
    (dict(head_dim=48), 4), (dict(n_heads=9, n_kv_heads=2), 4), (dict(n_heads=18, n_kv_heads=2), 4),
    (dict(hidden=100), 4), (dict(kv_capacity=16384), 4), (dict(intermediate=16384), 4),
    (dict(n_layers=0), 1), (dict(vocab=-5), 1), (dict(rms_eps=0.0), 1), (dict(qkv_bias=2), 1),
])
def test_create_rejects_unsupported_or_bad_shapes(L, change, code):
    wl = synth.get("tiny-2L-h64-kv32").replace(**change)
    rc, h = _create(wl)
    assert rc == code, L.mbk_last_error()
    assert L.mbk_last_error()


@pytest.mark.parametrize("name", synth.WORKLOAD_ORDER)
def test_create_accepts_every_workload_and_counts_intervals(L, name):
    wl = synth.get(name)
    rc, h = _create(wl)
    assert rc == 0, L.mbk_last_error()
    n = ctypes.c_int32()
    assert L.mbk_num_intervals(h, ctypes.byref(n)) == 0
    assert n.value == 5 * wl.n_layers + 1
    L.mbk_destroy(h)


def test_step_before_pack_is_a_state_error_and_args_are_checked(L):
    rc, h = _create(synth.get("tiny-2L-h64-kv32"))
    assert rc == 0
    am = ctypes.c_int32()
    assert L.mbk_decode_step(h, 1, 0, None, ctypes.byref(am), None) == 7           # MBK_ERR_STATE
    assert L.mbk_decode_step(None, 1, 0, None, ctypes.byref(am), None) == 1        # MBK_ERR_ARG
    assert L.mbk_decode_step_ablation(h, 1, 0, None, ctypes.byref(am), 0, None) == 7
    assert L.mbk_set_debug(h, -1, 0, 0) == 1
    assert L.mbk_set_launch_mode(h, 2) == 1                                       # unknown mode
    assert L.mbk_set_launch_mode(h, 1) == 0 and L.mbk_set_launch_mode(h, 0) == 0
    assert L.mbk_set_launch_mode(None, 0) == 1
    assert L.mbk_pack_weights(h, None, None, None, None) == 1
    L.mbk_destroy(h)
    L.mbk_destroy(None)


def test_no_device_is_reported_as_hip_error(L):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    rc, h = _create(synth.get("tiny-2L-h64-kv32"))
    n = ctypes.c_size_t()
    assert L.mbk_pack_weights(h, None, None, ctypes.byref(n), None) == 5          # MBK_ERR_HIP
    L.mbk_destroy(h)


@pytest.mark.parametrize("name", ["tiny-2L-h64-kv32", "smollm135m-kv128", "smollm135m-kv4096", "qwen2-0.5b-kv128",
                                  "smollm1.7b-kv4096", "stream-1l-v262144"])
def test_plan_fits_lds_and_ring_rules(name):
    """The host planner (no device: workgroups fixed) keeps every workgroup inside the 160 KiB of LDS, every
    GEMV task run within a third of the ring, every attention piece within a third (60 % where one piece holds a whole
    split), and the packed payload at
    2 bytes per parameter."""
    from persistent_megakernel_decode_wg_amd import Decoder
    wl = synth.get(name)
    d = Decoder(wl)
    d.set_workgroups(256)
    info = d.describe()
    assert info["workgroups"] == 256 and info["intervals"] == 5 * wl.n_layers + 1
    assert info["lds_bytes"] + 512 <= 160 * 1024
    assert info["max_task_bytes"] * 3 <= info["ring_bytes"]
    assert info["max_tile_bytes"] * 3 <= info["ring_bytes"]
    assert info["piece_positions"] >= 1
    seg = (info["piece_positions"] * wl.head_dim * 2 + 1023) // 1024 * 1024   # keys (or values) of one piece
    # a third of the ring; up to 60 % where every split (at least 128 positions) fits in one piece of 256
    longest = max(-(-wl.kv_capacity // info["max_splits"]), 128)
    if longest <= 256:
        assert 2 * seg * 10 <= info["ring_bytes"] * 6 and info["piece_positions"] <= 256
    else:
        assert 2 * seg * 3 <= info["ring_bytes"] and info["piece_positions"] <= 128
    # packed matrices are exactly 2 bytes per parameter (plus norms, RoPE table and schedule tables)
    assert info["packed_bytes"] >= 2 * wl.param_count()
    d.close()


def test_planner_reports_a_tile_too_large_for_the_ring():
    """An input width whose 8-value groups number an odd 65 (intermediate 520) packs 64 rows to a tile, 66.5 KB,
    more than a third of the ring: planning fails with MBK_ERR_UNSUPPORTED and says why; 528 (66 groups, 32 rows
    to a tile) plans."""
    from persistent_megakernel_decode_wg_amd import Decoder, MbkError, MBK_ERR_UNSUPPORTED
    for inter, ok in ((520, False), (528, True)):
        wl = synth.Workload("ragged-%d" % inter, 2, 200, 5, 1, 16, inter, 1024, 128, False, 1e-5, 1e4,
                            n_prompt=0, kv_prefill=0, n_decode=0)
        d = Decoder(wl)
        d.set_workgroups(256)
        if ok:
            assert d.describe()["max_tile_bytes"] * 3 <= d.describe()["ring_bytes"]
        else:
            with pytest.raises(MbkError) as e:
                d.describe()
            assert e.value.code == MBK_ERR_UNSUPPORTED and "ring" in str(e.value)
        d.close()


def test_set_workgroups_after_planning_is_a_state_error():
    from persistent_megakernel_decode_wg_amd import Decoder, MbkError, MBK_ERR_STATE
    d = Decoder(synth.get("tiny-2L-h64-kv32"))
    d.set_workgroups(128)
    d.describe()
    with pytest.raises(MbkError) as e:
        d.set_workgroups(64)
    assert e.value.code == MBK_ERR_STATE
    d.close()


def test_attention_items_policy():
    """One query head per attention item by default (fewer query heads than workgroups); the packed
    choice (a KV head's G query heads per item) on request; other values are argument errors, and a
    change after planning is a state error."""
    from persistent_megakernel_decode_wg_amd import Decoder, MbkError, MBK_ERR_ARG, MBK_ERR_STATE
    wl = synth.get("smollm135m-kv4096")
    G = wl.n_heads // wl.n_kv_heads
    d = Decoder(wl)
    d.set_workgroups(256)
    for bad in (-1, 2, G + 1):
        with pytest.raises(MbkError) as e:
            d.set_attention_items(bad)
        assert e.value.code == MBK_ERR_ARG
    assert d.describe()["attention_heads_per_item"] == 1
    with pytest.raises(MbkError) as e:
        d.set_attention_items(G)
    assert e.value.code == MBK_ERR_STATE
    d.set_attention_items(0)      # unchanged: allowed
    d.close()
    d = Decoder(wl)
    d.set_workgroups(256)
    d.set_attention_items(G)
    info = d.describe()
    assert info["attention_heads_per_item"] == G and info["max_splits"] >= 1
    d.close()


def test_static_scratch_step_rejects_oversized_workspace_and_checks_state(L):
    """mbk_decode_step_static: a shape whose workspace exceeds the 512 KiB static scratch is a size error
    before anything runs; a shape that fits but has no packed weights is a state error; every workload
    of the repository fits."""
    from persistent_megakernel_decode_wg_amd import Decoder, MBK_ERR_ARG, MBK_ERR_SIZE, MBK_ERR_STATE
    am = ctypes.c_int32()
    big = synth.get("smollm1.7b-kv4096").replace(hidden=4096, n_heads=64, n_kv_heads=64, head_dim=128,
                                                 intermediate=8192, vocab=1024, n_layers=1)
    d = Decoder(big)
    d.set_workgroups(256)
    assert d.describe()["workspace_bytes"] > 512 * 1024
    assert L.mbk_decode_step_static(d.h, None, 0, 0, None, ctypes.byref(am), None) == MBK_ERR_SIZE
    assert b"static scratch" in L.mbk_last_error()
    d.close()
    for name in synth.WORKLOAD_ORDER:
        d = Decoder(synth.get(name))
        d.set_workgroups(256)
        assert d.describe()["workspace_bytes"] <= 512 * 1024, name
        assert L.mbk_decode_step_static(d.h, None, 0, 0, None, ctypes.byref(am), None) == MBK_ERR_STATE
        d.close()
    assert L.mbk_decode_step_static(None, None, 0, 0, None, ctypes.byref(am), None) == MBK_ERR_ARG
