"""The host side of the C ABI (validation, preparation, layer files, the GEMM
planner) built with the address and undefined-behaviour sanitizers and run
through tests/native/host_sanitize.cpp, with the device launchers replaced by
tests/native/device_stubs.cpp (no GPU, no HIP runtime).  Any out-of-bounds
access, use after free, leak or undefined behaviour aborts the driver."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "w4a4_rank_corrected_amd", "csrc")
NATIVE = os.path.join(ROOT, "tests", "native")
SOURCES = [os.path.join(CSRC, f) for f in ("api.cpp", "prep.cpp", "bundle.cpp", "plan.cpp")] + \
          [os.path.join(NATIVE, f) for f in ("device_stubs.cpp", "host_sanitize.cpp")]


def test_host_code_under_address_and_ub_sanitizers(tmp_path):
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path / "host_sanitize")
    flags = ["-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=undefined", "-ffp-contract=off",
             f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}"]
    res = subprocess.run(["g++", *flags, *SOURCES, "-o", exe, "-pthread"], capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1",
               TMPDIR=str(tmp_path))
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    out = run.stdout + run.stderr
    assert run.returncode == 0 and "host sanitize ok" in run.stdout, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
