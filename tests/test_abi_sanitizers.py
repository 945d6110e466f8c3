"""The C ABI's host-side argument validation, built with AddressSanitizer
and UndefinedBehaviorSanitizer (host code only) and run on the CPU.

tests/sanitize/abi_validation_driver.cpp links the ABI layer against stub
launchers and calls every entry point with invalid, empty, extreme and
valid arguments; the test builds it with hipcc (the sanitizer flags apply to
the host compilation only) and runs it.  Invalid calls must return their
documented status without reaching a launcher, and the sanitizers must
report nothing (any report aborts the run)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "ulysses_sequence_parallelism_head_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_abi_validation_under_host_sanitizers(tmp_path):
    exe = tmp_path / "abi_validation"
    san = []
    for check in ("address", "undefined"):
        san += ["-Xarch_host", f"-fsanitize={check}"]
    cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fno-omit-frame-pointer",
           "-Xarch_host", "-fno-sanitize-recover=all", *san,
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(ROOT, "tests", "sanitize", "abi_validation_driver.cpp"),
           os.path.join(CSRC, "abi.hip"), os.path.join(CSRC, "workspace.hip"), "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "abi validation under sanitizers: ok" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
