#!/usr/bin/env python3
"""Batch-1 decode benchmark of the persistent megakernel on one MI355X.

Workload: the SmolLM-135M-shaped decoder (30 layers, hidden 576, 9/3 heads of
64, SwiGLU 1536, vocabulary 49152, tied embeddings) with seeded random bf16
weights and a static 128-slot KV cache: the 64 prompt tokens are stepped at
positions 0..63 (setup), then greedy steps run at positions 64..127 with the
token fed back on the device (MBK_TOKEN_PREV), cycling over that range.
One timed step = one launch of the persistent kernel (plain launch, one
workgroup per compute unit) = the whole decode step.

Prints ONE JSON line (rank 0).  `value` is tok/s over the K timed steps.
`roofline.achieved` = algorithmic bytes per step / mean kernel duration from
HIP events recorded on the launch stream.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0


def algorithmic_bytes(wl, pos: int, fp8: bool = False) -> int:
    """Bytes one step must move: every weight once (tied embedding once), the embedding row,
    the KV read over 0..pos and the append at pos, the fp32 logits, and the RoPE table row.
    fp8: the projection matrices and the vocabulary projection at one byte per weight plus a 4-byte
    scale per row; norms and biases stay bf16."""
    kv_pos = wl.n_layers * 2 * wl.n_kv_heads * wl.head_dim * 2
    rest = 2 * wl.hidden + (pos + 1) * kv_pos + kv_pos + 4 * wl.vocab + 4 * wl.head_dim
    if not fp8:
        return 2 * wl.param_count() + rest
    H, Q, KV, I, V, L = (wl.hidden, wl.n_heads * wl.head_dim, wl.n_kv_heads * wl.head_dim, wl.intermediate,
                         wl.vocab, wl.n_layers)
    mats = L * ((Q + 2 * KV) * H + H * Q + 2 * I * H + H * I) + V * H
    rows = L * ((Q + 2 * KV) + H + 2 * I + H) + V
    small = 2 * (2 * L + 1) * H + (2 * L * (Q + 2 * KV) if wl.qkv_bias else 0)
    return mats + 4 * rows + small + rest


OPS = ["qkv", "attn", "o", "gateup", "down"]


def phase_breakdown(dec, wl, positions, logits, am, steps=8, dump=""):
    """Per-operator means (us) from the device phase timer (100 MHz wall clock; stamps [0] interval start,
    [1] inputs loaded -- only on workgroups with work --, [2] body done).  Per interval: done = last working
    workgroup's [2]; span = done - previous interval's done (the step's critical path); wait = median
    working workgroup's [1] - previous done (input hand-over latency); comp = median [2] - [1] over working
    workgroups and comp_max its maximum; n_work = working workgroups."""
    import numpy as np
    import torch
    from persistent_megakernel_decode_wg_amd import MBK_TOKEN_PREV
    tr = dec.set_phase_trace(True)
    acc = {}
    raw = []
    for i in range(steps):
        tr.zero_()
        dec.decode_step(MBK_TOKEN_PREV, positions(i), logits, am)
        torch.cuda.synchronize()
        t = tr.cpu().numpy().astype(np.int64)          # [iv][wg][4]
        raw.append(t.copy())
        n_iv = t.shape[0]
        prev_done = t[0, t[0, :, 0] > 0, 0].min()
        for iv in range(n_iv):
            op = "lmhead" if iv == n_iv - 1 else OPS[iv % 5]
            work = t[iv, :, 1] > 0
            if not work.any():
                continue
            t1, t2 = t[iv, work, 1], t[iv, work, 2]
            done = t2.max()
            a = acc.setdefault(op, np.zeros(6))
            a += [(done - prev_done) * 0.01, (np.median(t1) - prev_done) * 0.01, np.median(t2 - t1) * 0.01,
                  (t2 - t1).max() * 0.01, work.sum(), 1]
            prev_done = done
    dec.set_phase_trace(False)
    if dump:
        np.save(dump, np.stack(raw))
    out = {op: {"span_us": round(a[0] / a[5], 3), "wait_us": round(a[1] / a[5], 3), "comp_us": round(a[2] / a[5], 3),
                "comp_max_us": round(a[3] / a[5], 3), "n_work": int(a[4] / a[5]),
                "count_per_step": int(a[5]) // steps} for op, a in acc.items()}
    print("phase breakdown (us, mean per interval): " + json.dumps(out), file=sys.stderr, flush=True)
    return out


def pct(xs, q):
    xs = sorted(xs)
    return xs[min(len(xs) - 1, int(q * (len(xs) - 1) + 0.5))]


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def setup_workload(wl, W=None, fp8=False):
    """Packs the workload's seeded weights into a Decoder and runs its setup (the prompt stepped from position 0,
    or the N(0,1) KV prefix and the step after it).  Returns (dec, W, logits, argmax, g0, g1): greedy positions
    g0 .. g1 - 1 follow."""
    import numpy as np
    import torch

    import synth
    from persistent_megakernel_decode_wg_amd import Decoder
    W = synth.make_weights(wl) if W is None else W
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()
    Wt = {"embed": dev(W["embed"]), "final_norm": dev(W["final_norm"]),
          "layers": [{k: dev(v) for k, v in L.items()} for L in W["layers"]]}
    dec = Decoder(wl)
    if fp8:
        from persistent_megakernel_decode_wg_amd import MBK_WEIGHTS_FP8_E4M3
        dec.set_weight_format(MBK_WEIGHTS_FP8_E4M3)
    dec.pack_weights(Wt)
    del Wt
    dec.alloc_kv()
    logits = torch.empty(wl.vocab, dtype=torch.float32, device="cuda")
    am = torch.empty(1, dtype=torch.int32, device="cuda")
    if wl.kv_prefill:
        pre = synth.kv_prefill(wl)
        dec.kv[:, :, :, :wl.kv_prefill, :] = torch.from_numpy(pre.view(np.int16)).cuda()
        del pre
        dec.decode_step(synth.first_token(wl), wl.kv_prefill, logits, am)
        g0 = wl.kv_prefill + 1
    else:
        for p, t in enumerate(synth.prompt_tokens(wl)):
            dec.decode_step(int(t), p, logits, am)
        g0 = wl.greedy_start
    dec.check()
    return dec, W, logits, am, g0, wl.greedy_start + wl.n_decode


def timed_steps(dec, positions, n, logits, am, stream, fn=None):
    """Kernel time (us) of n steps at positions(i), each bracketed by HIP events on the launch stream."""
    import torch
    from persistent_megakernel_decode_wg_amd import MBK_TOKEN_PREV
    fn = fn or (lambda pos: dec.decode_step(MBK_TOKEN_PREV, pos, logits, am))
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for i in range(n):
        ev[i][0].record(stream)
        fn(positions(i))
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    dec.check()
    return [a.elapsed_time(b) * 1e3 for a, b in ev]


def prefill_flops(wl, n: int, pos0: int = 0) -> float:
    """Algorithmic flops of a prefill of n tokens at positions pos0 .. pos0 + n - 1: every projection matrix
    applied to every position (multiply-add = 2 flops), causal attention (scores and weighted values over
    each position's pos + 1 cached positions), the vocabulary projection of the last position."""
    H, hd, nq, nkv, I = wl.hidden, wl.head_dim, wl.n_heads, wl.n_kv_heads, wl.intermediate
    per_layer = (nq * hd + 2 * nkv * hd) * H + H * nq * hd + 3 * I * H
    attended = sum(pos0 + i + 1 for i in range(n))
    return 2.0 * n * per_layer * wl.n_layers + 2.0 * 2 * hd * nq * attended * wl.n_layers + 2.0 * wl.vocab * H


def prefill_summary(wl, n: int, decode_us: float, reps: int = 21, fp8: bool = False):
    """p50 time of one prefill of n seeded tokens at position 0 (HIP events on the stream), against n decode
    steps of the same model (decode_us per step), and its algorithmic TFLOP/s against the bf16 matrix-core
    peak (the hi/lo input pairs double the products actually executed); fp8: on the E4M3-quantised weights."""
    import torch
    import synth
    from persistent_megakernel_decode_wg_amd import Decoder
    W = synth.make_weights(wl)
    dev = lambda a: torch.from_numpy(a.view("int16")).cuda()
    dec = Decoder(wl)
    if fp8:
        from persistent_megakernel_decode_wg_amd import MBK_WEIGHTS_FP8_E4M3
        dec.set_weight_format(MBK_WEIGHTS_FP8_E4M3)
    dec.pack_weights({"embed": dev(W["embed"]), "final_norm": dev(W["final_norm"]),
                      "layers": [{k: dev(v) for k, v in L.items()} for L in W["layers"]]})
    del W
    dec.alloc_kv()
    toks = [int(t) for t in synth.tokens(13, "bench-prompt", n, wl.vocab)]
    logits = torch.empty(wl.vocab, dtype=torch.float32, device="cuda")
    am = torch.empty(1, dtype=torch.int32, device="cuda")
    scratch = dec.prefill(toks, 0, logits, am)
    stream = torch.cuda.current_stream()
    us = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        dec.prefill(toks, 0, logits, am, scratch=scratch)
        e1.record(stream)
        torch.cuda.synchronize()
        us.append(e0.elapsed_time(e1) * 1e3)
    dec.check()
    dec.close()
    del dec, scratch
    torch.cuda.empty_cache()
    t = pct(us, 0.5)
    fl = prefill_flops(wl, n)
    res = {"tokens": n, "us_p50": round(t, 1), "us_per_token": round(t / n, 2), "tok_s": round(n / t * 1e6, 1)}
    if decode_us is not None:
        res.update({"decode_steps_us": round(decode_us * n, 1), "speedup_over_decode_steps": round(decode_us * n / t, 2)})
    return {**res,
            "algorithmic_tflops": round(fl / t * 1e-6, 2), "frac_of_bf16_mfma_peak": round(fl / t * 1e-6 / 2500.0, 4)}


def fp8_summary(wl, steps: int = 64):
    """The workload with FP8 (OCP E4M3) weights, measured like the headline: p50 us/token and the fraction
    of the 8 TB/s roofline for the bytes an fp8 step moves."""
    import torch
    dec, W, logits, am, g0, g1 = setup_workload(wl, fp8=True)
    del W
    stream = torch.cuda.current_stream()
    span = g1 - g0
    positions = lambda i: g0 + (i % span)
    timed_steps(dec, positions, 8, logits, am, stream)
    us = timed_steps(dec, positions, steps, logits, am, stream)
    dec.check()
    dec.close()
    del dec, logits, am
    torch.cuda.empty_cache()
    p50 = pct(us, 0.5)
    nb = sum(algorithmic_bytes(wl, positions(i), fp8=True) for i in range(steps)) / steps
    return {"us_per_token_p50": round(p50, 2), "tok_s": round(1e6 / p50, 1), "bytes_per_token": int(nb),
            "roofline_frac": round(nb / (p50 * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}


def config_summary(wl, steps: int = 64):
    """One workload measured the way the headline is (its greedy positions, the token fed back on the device):
    p50 us/token of the persistent kernel, its fraction of the 8 TB/s roofline, the same kernel with a grid
    barrier after every interval, and the per-operator ablation (plain launches and hipGraph replay)."""
    import torch
    from persistent_megakernel_decode_wg_amd import MBK_SYNC_BARRIER, MBK_SYNC_DATAFLOW, MBK_TOKEN_PREV
    dec, W, logits, am, g0, g1 = setup_workload(wl)
    del W
    stream = torch.cuda.current_stream()
    span = g1 - g0
    positions = lambda i: g0 + (i % span)
    timed_steps(dec, positions, 8, logits, am, stream)
    us = timed_steps(dec, positions, steps, logits, am, stream)
    p50 = pct(us, 0.5)
    nb = sum(algorithmic_bytes(wl, positions(i)) for i in range(steps)) / steps
    dec.set_sync_mode(MBK_SYNC_BARRIER)
    timed_steps(dec, positions, 4, logits, am, stream)
    bar = pct(timed_steps(dec, positions, min(steps, 32), logits, am, stream), 0.5)
    dec.set_sync_mode(MBK_SYNC_DATAFLOW)
    abl = {}
    for mode, use_graph in (("plain", False), ("graph", True)):
        f = lambda pos: dec.decode_step_ablation(MBK_TOKEN_PREV, pos, logits, am, use_graph=use_graph)
        timed_steps(dec, positions, 4, logits, am, stream, f)
        abl[mode] = pct(timed_steps(dec, positions, min(steps, 32), logits, am, stream, f), 0.5)
    dec.close()
    del dec, logits, am
    torch.cuda.empty_cache()
    return {"us_per_token_p50": round(p50, 2), "tok_s": round(1e6 / p50, 1),
            "roofline_frac": round(nb / (p50 * 1e-6) / 1e9 / PEAK_HBM_GBS, 4), "bytes_per_token": int(nb),
            "positions": "%d-%d" % (positions(0), positions(steps - 1)) if steps <= span else "%d-%d cycled" % (g0, g1 - 1),
            "barrier_mode_us_per_token": round(bar, 2), "ablation_plain_us_per_token": round(abl["plain"], 2),
            "ablation_graph_us_per_token": round(abl["graph"], 2),
            "faster_than_both_ablations": bool(p50 < abl["plain"] and p50 < abl["graph"])}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=640)
    ap.add_argument("--warmup", type=int, default=64)
    ap.add_argument("--workload", default="smollm135m-kv128")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ablation", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--sync", choices=["dataflow", "barrier"], default="dataflow",
                    help="interval ordering of the persistent kernel (the other mode is timed as an extra)")
    ap.add_argument("--phase", action="store_true", help="print a per-operator phase-timer breakdown to stderr")
    ap.add_argument("--phase-dump", default="", help="also save the raw phase-timer arrays (.npy) to this path")
    ap.add_argument("--attn-split", type=int, default=0, help="attention split size in positions (0: library default)")
    ap.add_argument("--no-other-mode", action="store_true", help="skip timing the other sync mode")
    ap.add_argument("--cold", type=int, default=0, metavar="N",
                    help="also time N steps each preceded by a 1 GiB device write (caches cold: extra.cold_us_per_token_p50)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-config summary of every workload (extra.configs)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="after the timed steps, run one device-to-device copy of this many MiB (counter calibration)")
    ap.add_argument("--weights", choices=["bf16", "fp8"], default="bf16",
                    help="weight storage of the timed decoder: bf16, or OCP E4M3 codes with per-row scales")
    ap.add_argument("--prefill-tokens", type=int, default=0, metavar="N",
                    help="time only a prefill of N tokens of the workload (one JSON line, no decode steps)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (--gpus %d requested)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    from persistent_megakernel_decode_wg_amd import MBK_SYNC_BARRIER, MBK_SYNC_DATAFLOW, MBK_TOKEN_PREV, Decoder
    from persistent_megakernel_decode_wg_amd import build as mbk_build

    mbk_build.ensure_built()
    torch.cuda.set_device(0)
    wl = synth.get(args.workload)
    if args.prefill_tokens:
        res = prefill_summary(wl, args.prefill_tokens, None, fp8=args.weights == "fp8")
        print(json.dumps({"metric": "prefill us (one call)", "workload": wl.name, "weights": args.weights, **res}),
              flush=True)
        return
    fp8 = args.weights == "fp8"
    dec, W, logits, am, g0, g1 = setup_workload(wl, fp8=fp8)
    if args.attn_split:
        dec.set_attention_split(args.attn_split)
    sync_modes = {"dataflow": MBK_SYNC_DATAFLOW, "barrier": MBK_SYNC_BARRIER}
    dec.set_sync_mode(sync_modes[args.sync])
    stream = torch.cuda.current_stream()
    span = g1 - g0                              # greedy positions g0 .. g1 - 1, cycled
    positions = lambda i: g0 + (i % span)

    for i in range(args.warmup):
        dec.decode_step(MBK_TOKEN_PREV, positions(i), logits, am)
    dec.check()

    K = args.steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        ev[i][0].record(stream)
        dec.decode_step(MBK_TOKEN_PREV, positions(i), logits, am)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    dec.check()
    kern_us = [a.elapsed_time(b) * 1e3 for a, b in ev]
    if args.calib_copy_mib:
        n = args.calib_copy_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    mean_kern_us = sum(kern_us) / K
    bytes_mean = sum(algorithmic_bytes(wl, positions(i), fp8=fp8) for i in range(K)) / K
    achieved = bytes_mean / (mean_kern_us * 1e-6) / 1e9

    # complete synchronized call (host + GPU), as the pages' leaderboard measures
    call_us = []
    for i in range(min(64, K)):
        torch.cuda.synchronize()
        c0 = time.perf_counter()
        dec.decode_step(MBK_TOKEN_PREV, positions(i), logits, am)
        torch.cuda.synchronize()
        call_us.append((time.perf_counter() - c0) * 1e6)

    extra = {
        "us_per_token_p10": round(pct(kern_us, 0.1), 2), "us_per_token_p50": round(pct(kern_us, 0.5), 2),
        "us_per_token_p90": round(pct(kern_us, 0.9), 2), "complete_call_us_p50": round(pct(call_us, 0.5), 2),
        "bytes_per_token": int(bytes_mean), "intervals_per_step": dec.num_intervals(),
    }
    # the other interval ordering of the same persistent kernel
    extra["sync_mode"] = args.sync
    extra["launch"] = "plain launch, one workgroup per compute unit"
    if not args.no_other_mode:
        other = "barrier" if args.sync == "dataflow" else "dataflow"
        dec.set_sync_mode(sync_modes[other])
        for i in range(8):
            dec.decode_step(MBK_TOKEN_PREV, positions(i), logits, am)
        ev2 = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(128)]
        for i in range(128):
            ev2[i][0].record(stream)
            dec.decode_step(MBK_TOKEN_PREV, positions(i), logits, am)
            ev2[i][1].record(stream)
        torch.cuda.synchronize()
        dec.check()
        extra[other + "_mode_us_per_token"] = round(sum(a.elapsed_time(b) for a, b in ev2) / 128 * 1e3, 2)
        dec.set_sync_mode(sync_modes[args.sync])

    if not args.no_ablation:
        for mode, use_graph in (("ablation_plain", False), ("ablation_graph", True)):
            f = lambda pos: dec.decode_step_ablation(MBK_TOKEN_PREV, pos, logits, am, use_graph=use_graph)
            timed_steps(dec, positions, 8, logits, am, stream, f)
            us = timed_steps(dec, positions, min(K, 128), logits, am, stream, f)
            extra[mode + "_us_per_token"] = round(pct(us, 0.5), 2)
        extra["ablation_launches_per_token"] = dec.num_intervals()
        # what one launch boundary costs the ablation over the persistent kernel (the pages' per-kernel gap)
        extra["ablation_graph_us_per_launch_over_persistent"] = round(
            (extra["ablation_graph_us_per_token"] - extra["us_per_token_p50"]) / dec.num_intervals(), 3)
        extra["barrier_us"] = round(dec.barrier_bench(10000), 3)
        dec.check()

    if args.cold:
        # every timed step follows a 1 GiB write, which leaves neither the weights nor the KV cache in L2 or the
        # last-level cache; the step alone is timed
        flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
        cold = []
        for i in range(args.cold):
            flush.fill_(float(i))
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            dec.decode_step(MBK_TOKEN_PREV, positions(i), logits, am)
            e1.record(stream)
            torch.cuda.synchronize()
            cold.append(e0.elapsed_time(e1) * 1e3)
        dec.check()
        del flush
        extra["cold_us_per_token_p50"] = round(pct(cold, 0.5), 2)

    if args.phase:
        ph = phase_breakdown(dec, wl, positions, logits, am, dump=args.phase_dump)
        extra["phase"] = ph
        # the step as hops x (hand-over + body) against bytes / peak bandwidth
        hops = sum(v["count_per_step"] for v in ph.values())
        sync = sum(v["wait_us"] * v["count_per_step"] for v in ph.values())
        body = sum(v["comp_us"] * v["count_per_step"] for v in ph.values())
        extra["decomposition"] = {
            "hops": hops, "handover_us_per_hop": round(sync / hops, 3), "body_us_per_hop": round(body / hops, 3),
            "hops_x_handover_plus_body_us": round(sync + body, 1),
            "bytes_over_peak_us": round(bytes_mean / (PEAK_HBM_GBS * 1e3), 1)}

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        ref = oracle.Model(wl, W)
        if wl.kv_prefill:
            ref.prefill_kv(synth.kv_prefill(wl))
            tok = synth.first_token(wl)
            _, tok, _ = ref.step(tok, wl.kv_prefill)
        else:
            tok = 0
            for p, t in enumerate(synth.prompt_tokens(wl)):
                _, tok, _ = ref.step(int(t), p)
        n, c0 = 0, time.perf_counter()
        while time.perf_counter() - c0 < args.cpu_seconds and n < span:
            _, tok, _ = ref.step(tok, positions(n))
            n += 1
        cs = time.perf_counter() - c0
        cpu = {"value": round(n / cs, 3), "unit": "tok/s", "cores": oracle.num_threads(), "kind": "oracle",
               "sample": "%d greedy steps at positions %d..%d after the %s setup, fp64-accumulating C oracle" % (
                   n, g0, g0 + n - 1, "prefill" if wl.kv_prefill else "64-token prompt"),
               "cpu_model": cpu_model(), "nproc": os.cpu_count()}
        del ref

    # HBM bytes per launch from the committed counter summary, while it matches these kernel sources
    from persistent_megakernel_decode_wg_amd import profile_traffic
    rec = profile_traffic.read(os.path.join(ROOT, "profiles", "traffic_k_persistent_%s%s.md"
                                            % (wl.name, "-fp8" if fp8 else "")))
    traffic = round(rec["traffic_bytes"]) if rec else None
    if rec:
        extra["traffic_fetch_bytes"] = round(rec["fetch_bytes"])
        extra["traffic_write_bytes"] = round(rec["write_bytes"])
    dec.close()
    del dec, W, logits, am
    torch.cuda.empty_cache()
    if not args.no_configs:
        # every workload, measured the same way (the headline one again, so the table is self-consistent)
        extra["configs"] = {}
        for name in synth.WORKLOAD_ORDER:
            extra["configs"][name] = config_summary(synth.get(name))
            print("config %s: %s" % (name, json.dumps(extra["configs"][name])), file=sys.stderr, flush=True)
        # multi-token prefill: the 64-token prompt of the SmolLM-135M shape, a 512-token prompt on its
        # 4096-slot cache and a 1024-token prompt of the SmolLM-1.7B shape, against as many decode steps
        extra["prefill"] = {}
        for name, n in (("smollm135m-kv128", 64), ("smollm135m-kv4096", 512), ("smollm1.7b-kv4096", 1024)):
            dus = extra["configs"][name]["us_per_token_p50"]
            extra["prefill"]["%s/%d" % (name, n)] = prefill_summary(synth.get(name), n, dus)
            print("prefill %s/%d: %s" % (name, n, json.dumps(extra["prefill"]["%s/%d" % (name, n)])),
                  file=sys.stderr, flush=True)
        # the same decode step streaming FP8 (OCP E4M3) weights, on the two headline shapes
        extra["fp8_weights"] = {}
        for name in ("smollm135m-kv128", "smollm1.7b-kv4096"):
            extra["fp8_weights"][name] = fp8_summary(synth.get(name))
            print("fp8 %s: %s" % (name, json.dumps(extra["fp8_weights"][name])), file=sys.stderr, flush=True)
    timed = "%d-%d" % (g0, g0 + K - 1) if K <= span else "%d-%d cycled over %d steps" % (g0, g1 - 1, K)
    out = {
        "metric": "batch-1 decode tok/s (us/token) + achieved HBM GB/s vs 8 TB/s peak, 1 GPU",
        "value": round(K / elapsed, 2), "unit": "tok/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": round(elapsed / K * 1e3, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp8-e4m3 weights, f32 products" if fp8 else "bf16",
        "data": "synthetic (seeded random-init weights)",
        "config": {"workload": wl.name, "layers": wl.n_layers, "hidden": wl.hidden, "heads": wl.n_heads,
                   "kv_heads": wl.n_kv_heads, "head_dim": wl.head_dim, "intermediate": wl.intermediate,
                   "vocab": wl.vocab, "kv_capacity": wl.kv_capacity, "batch": 1,
                   "positions": timed, "weights": args.weights, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic},
        "cpu_baseline": cpu,
        "us_per_token": round(mean_kern_us, 2),
        "extra": extra,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
