"""The C-ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only): the library's sources and abi_host_checks.cpp are built into one
program whose host code carries both sanitizers (-Xarch_host; the device code
is built as the library's is), then every entry point is called with invalid
arguments and must return its documented status with no sanitizer report.
No call reaches a launch, so no GPU is needed.  The build takes about a
minute."""
import os
import shutil
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
sys.path.insert(0, os.path.join(ROOT, "smc_resampling_amd"))


def _clang_asan_runtime():
    import glob

    found = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    return found[0] if found else None


def test_host_argument_checks_under_sanitizers(tmp_path):
    if shutil.which("hipcc") is None or _clang_asan_runtime() is None:
        pytest.skip("hipcc or clang's AddressSanitizer runtime is not installed")
    import build  # the library's own hipcc flags

    exe = str(tmp_path / "abi_host_checks")
    flags = [f for f in build.HIPCC_FLAGS if f not in ("-shared", "-fPIC")]
    san = ["-g"]
    for f in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all"):
        san += ["-Xarch_host", f]
    cmd = ["hipcc", *flags, *san, "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "smc_resampling_amd",
                                                                                        "csrc"),
           *build.sources(), os.path.join(HERE, "abi_host_checks.cpp"), "-o", exe]
    b = subprocess.run(cmd, capture_output=True, text=True, timeout=900)
    assert b.returncode == 0, b.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    out = r.stdout + r.stderr
    assert "Sanitizer" not in out and "runtime error" not in out, out[-3000:]
    assert r.returncode == 0 and "0 failed" in r.stdout, out[-3000:]
