"""Build libsmcsd.so (HIP kernels for gfx950 + the C-ABI) in-tree with hipcc."""
from __future__ import annotations

import glob
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libsmcsd.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # packed fp32 VALU forms stay off: ordinary float code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def sources():
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))


def build(out: str = LIB, extra_flags=()) -> str:
    cmd = ["hipcc", *HIPCC_FLAGS, *extra_flags, "-I", os.path.join(ROOT, "include"), "-I",
           os.path.join(HERE, "csrc"), *sources(), "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stderr}")
    return out


# A test build whose member workgroups never wait for each other's tile
# masses (tests/test_wait_expiry.py: calls still end, and raise
# SMCSD_FLAG_WAIT_EXPIRED or decide correctly).
NOWAIT_LIB = os.path.join(HERE, "libsmcsd_nowait.so")


def build_nowait(out: str = NOWAIT_LIB) -> str:
    return build(out, ["-DSMCSD_TAG_WAIT_TICKS=0"])


if __name__ == "__main__":
    print(build())
    print(build_nowait())
