"""HBM traffic of the persistent decode kernel from rocprofv3 counter passes.

Two `rocprofv3 --pmc` passes over `bench.py --calib-copy-mib N` (FETCH_SIZE, then WRITE_SIZE, in KiB per dispatch)
see the decode kernel and a plain device-to-device copy of N MiB. The copy's counters give the scale of each counter
(bytes the copy must read or write / what the counter reports); the decode kernel's per-dispatch averages are
multiplied by those scales.  The result is written as one machine-readable line into a summary under profiles/,
tagged with a hash of the decode kernel's sources, so that bench.py reports it only while that kernel is unchanged.

  python -m persistent_megakernel_decode_wg_amd.profile_traffic --fetch FETCH_counter_collection.csv \\
      --write WRITE_counter_collection.csv --copy-mib 256 --workload smollm135m-kv128 --out profiles/....md
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import statistics

_HERE = os.path.dirname(os.path.abspath(__file__))
KERNEL = "k_persistent"
MARK = "traffic-json: "


# The sources the decode kernel is built from (its bodies, the layouts, the kernel entry and the host code that
# plans and launches it); the prefill kernels and their host code (prefill.h, prefill_host.h) do not enter it.
DECODE_SOURCES = ("bodies.h", "layout.h", "mbk.hip")


def source_hash() -> str:
    """Hash of the decode kernel's sources (the counters describe exactly this code)."""
    h = hashlib.sha256()
    d = os.path.join(_HERE, "csrc")
    for f in DECODE_SOURCES:
        with open(os.path.join(d, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def _per_dispatch(path: str, counter: str):
    """{kernel name: [values per dispatch]} for one counter of a rocprofv3 counter_collection.csv."""
    out = {}
    with open(path) as f:
        for row in csv.DictReader(f):
            if row.get("Counter_Name") != counter:
                continue
            out.setdefault(row["Kernel_Name"], []).append(float(row["Counter_Value"]))
    return out


def _copy_kernel(vals, copy_kib: float):
    """The calibration copy: the largest dispatch of the runtime's device-to-device copy kernel (a same-type,
    contiguous tensor copy goes through hipMemcpy), else the largest non-decode dispatch.  Other copies in the
    same program (weight uploads, a KV prefix converted on the device) run through other kernels."""
    best = None
    for prefer in (True, False):
        for name, v in vals.items():
            if KERNEL in name or (prefer and "copyBuffer" not in name):
                continue
            m = max(v)
            if best is None or m > best[1]:
                best = (name, m)
        if best is not None:
            return best
    return best


def summarize(fetch_csv: str, write_csv: str, copy_mib: float):
    f = _per_dispatch(fetch_csv, "FETCH_SIZE")
    w = _per_dispatch(write_csv, "WRITE_SIZE")
    copy_kib = copy_mib * 1024.0
    cf, cw = _copy_kernel(f, copy_kib), _copy_kernel(w, copy_kib)
    dec_f = [v for n, vs in f.items() if KERNEL in n for v in vs]
    dec_w = [v for n, vs in w.items() if KERNEL in n for v in vs]
    sf, sw = copy_kib / cf[1], copy_kib / cw[1]
    fetch_b = statistics.median(dec_f) * 1024.0 * sf
    write_b = statistics.median(dec_w) * 1024.0 * sw
    return {"fetch_bytes": fetch_b, "write_bytes": write_b, "traffic_bytes": fetch_b + write_b,
            "fetch_scale": sf, "write_scale": sw, "copy_kernel": cf[0], "copy_mib": copy_mib,
            "dispatches": len(dec_f), "source_hash": source_hash()}


def read(path: str):
    """The traffic record of a summary file if it matches the current kernel sources, else None."""
    if not os.path.exists(path):
        return None
    with open(path) as f:
        for line in f:
            if line.startswith(MARK):
                rec = json.loads(line[len(MARK):])
                return rec if rec.get("source_hash") == source_hash() else None
    return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--fetch", required=True)
    ap.add_argument("--write", required=True)
    ap.add_argument("--copy-mib", type=float, required=True)
    ap.add_argument("--workload", required=True)
    ap.add_argument("--out", required=True)
    ap.add_argument("--command", default="")
    a = ap.parse_args()
    rec = summarize(a.fetch, a.write, a.copy_mib)
    rec["workload"] = a.workload
    lines = [
        "# HBM traffic of %s, workload %s (rocprofv3 --pmc, two passes)" % (KERNEL, a.workload),
        "",
        "Commands:" if a.command else "",
        a.command,
        "",
        "| quantity | value |",
        "|---|---|",
        "| decode dispatches counted | %d |" % rec["dispatches"],
        "| FETCH_SIZE scale (copy of %.0f MiB) | %.4f |" % (a.copy_mib, rec["fetch_scale"]),
        "| WRITE_SIZE scale | %.4f |" % rec["write_scale"],
        "| fetched bytes per step (scaled) | %.0f |" % rec["fetch_bytes"],
        "| written bytes per step (scaled) | %.0f |" % rec["write_bytes"],
        "| traffic per step | %.0f |" % rec["traffic_bytes"],
        "",
        MARK + json.dumps(rec),
        "",
    ]
    with open(a.out, "w") as f:
        f.write("\n".join(lines))
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
