"""Host logic of the HBM-traffic summary (no GPU): counter scaling from the calibration copy."""
import csv
import json
import os

from persistent_megakernel_decode_wg_amd import profile_traffic


def _write(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, value in rows:
            w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_calibration_uses_the_runtime_copy_kernel_and_scales_the_decode_kernel(tmp_path):
    """A 256 MiB device-to-device copy reports FETCH 128 MiB and WRITE 256 MiB (KiB per dispatch); a larger
    elementwise tensor copy in the same program must not be taken for it.  The decode kernel's median
    counters times those scales are the bytes per step."""
    kib = 256 * 1024.0
    big_other = "void at::native::elementwise_kernel<copy>(int)"
    f, w = tmp_path / "f.csv", tmp_path / "w.csv"
    _write(f, "FETCH_SIZE", [("__amd_rocclr_copyBuffer", kib / 2), (big_other, 3 * kib),
                             ("void k_persistent<3>(mbk::Params)", 1000.0), ("void k_persistent<3>(mbk::Params)", 1002.0),
                             ("void k_persistent<3>(mbk::Params)", 1004.0)])
    _write(w, "WRITE_SIZE", [("__amd_rocclr_copyBuffer", kib), (big_other, 5 * kib),
                             ("void k_persistent<3>(mbk::Params)", 10.0), ("void k_persistent<3>(mbk::Params)", 12.0),
                             ("void k_persistent<3>(mbk::Params)", 14.0)])
    rec = profile_traffic.summarize(str(f), str(w), 256)
    assert rec["copy_kernel"] == "__amd_rocclr_copyBuffer"
    assert abs(rec["fetch_scale"] - 2.0) < 1e-12 and abs(rec["write_scale"] - 1.0) < 1e-12
    assert rec["dispatches"] == 3
    assert abs(rec["fetch_bytes"] - 1002.0 * 1024 * 2.0) < 1e-6
    assert abs(rec["write_bytes"] - 12.0 * 1024 * 1.0) < 1e-6
    assert abs(rec["traffic_bytes"] - (rec["fetch_bytes"] + rec["write_bytes"])) < 1e-6


def test_summary_is_read_back_only_for_the_current_sources(tmp_path):
    rec = {"fetch_bytes": 1.0, "write_bytes": 2.0, "traffic_bytes": 3.0, "source_hash": profile_traffic.source_hash()}
    p = tmp_path / "t.md"
    p.write_text("# x\n\n" + profile_traffic.MARK + json.dumps(rec) + "\n")
    assert profile_traffic.read(str(p))["traffic_bytes"] == 3.0
    rec["source_hash"] = "0" * 16
    p.write_text("# x\n\n" + profile_traffic.MARK + json.dumps(rec) + "\n")
    assert profile_traffic.read(str(p)) is None
    assert profile_traffic.read(os.path.join(str(tmp_path), "missing.md")) is None
