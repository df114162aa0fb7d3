"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only):
built with gcc -fsanitize=address,undefined (aborting at the first report),
every deterministic pin and the statistical pins run in a child process with
the ASan runtime preloaded, and must pass with no report.  An out-of-bounds
read or write, a use after free or an undefined operation anywhere the pins
reach fails the test."""
import os
import subprocess
import sys

import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def _asan_runtime():
    path = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.fixture(scope="module")
def sanitized_oracle(tmp_path_factory):
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    so = str(tmp_path_factory.mktemp("asan") / "liboracle_asan.so")
    subprocess.check_call(["gcc", "-O1", "-g", "-std=c99", "-fPIC", "-shared", "-fsanitize=address,undefined",
                           "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-o", so, oracle.SRC, "-lm"])
    return so, rt


def test_pins_pass_under_address_and_undefined_sanitizers(sanitized_oracle):
    so, rt = sanitized_oracle
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, os.path.join(HERE, "mutant_runner.py"), so], capture_output=True, text=True,
                       timeout=600, env=env)
    out = r.stdout + r.stderr
    assert "Sanitizer" not in out, out[-3000:]
    assert r.returncode == 0 and "survived" in r.stdout, out[-3000:]
