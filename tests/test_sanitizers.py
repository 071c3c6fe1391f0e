"""Host AddressSanitizer / UndefinedBehaviorSanitizer runs (CPU only, no device).

* the CPU oracle and the seeded input generator, built with gcc -fsanitize=address,undefined, stepping the
  tiny decoder through every KV slot and calling each building block on edge sizes;
* libmbk's host side (shape validation, the planner, size queries, argument checks of every entry point),
  the library built by hipcc with only its host pass instrumented, driven on every workload shape with the
  workgroup count fixed so that no call reaches a device.

Any sanitizer report fails the run (-fno-sanitize-recover=all; leak detection on)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANGXX = "/opt/rocm/llvm/bin/clang++"
SAN_ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, **kw)
    return r.returncode, r.stdout


def _clean(out: str) -> bool:
    return "ERROR: AddressSanitizer" not in out and "ERROR: LeakSanitizer" not in out and "runtime error" not in out


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_and_generator_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    rc, out = _run(["gcc", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-fno-omit-frame-pointer", "-fopenmp", "-I", os.path.join(ROOT, "oracle"),
                    os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"), os.path.join(ROOT, "oracle", "oracle.c"),
                    os.path.join(ROOT, "synth", "synth.c"), "-lm", "-o", exe])
    assert rc == 0, out
    rc, out = _run([exe], env=SAN_ENV)
    assert rc == 0 and _clean(out) and "oracle driver: ok" in out, out


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANGXX)), reason="ROCm compilers not available")
def test_library_host_side_under_asan_ubsan(tmp_path):
    obj, drv, exe = str(tmp_path / "mbk_san.o"), str(tmp_path / "planner_driver.o"), str(tmp_path / "planner_driver")
    # the library: device code as always, the host pass instrumented
    rc, out = _run([HIPCC, "--offload-arch=gfx950", "-g", "-std=c++17", "-Xarch_host", "-O1", "-Xarch_device", "-O1",
                    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                    "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
                    "-I", os.path.join(ROOT, "include"), "-c",
                    os.path.join(ROOT, "persistent_megakernel_decode_wg_amd", "csrc", "mbk.hip"), "-o", obj])
    assert rc == 0, out
    # the driver: plain host C++ against the C header
    rc, out = _run([CLANGXX, "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-I", os.path.join(ROOT, "include"), "-c",
                    os.path.join(ROOT, "tests", "sanitize", "planner_driver.cpp"), "-o", drv])
    assert rc == 0, out
    rc, out = _run([CLANGXX, "-fsanitize=address,undefined", drv, obj, "-L/opt/rocm/lib", "-Wl,-rpath,/opt/rocm/lib",
                    "-lamdhip64", "-o", exe])
    assert rc == 0, out
    rc, out = _run([exe], env=SAN_ENV)
    assert rc == 0 and _clean(out) and "planner driver: ok" in out, out
