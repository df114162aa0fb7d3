"""The bounded wait of member workgroups, forced from the host: a test build
of the library whose waits run out at once (-DSMCSD_TAG_WAIT_TICKS=0, built by
__graft_entry__.build()) runs SD, tree and SMC calls in a child process.  Every
call must end; shared decisions (and SMC prompts whose work runs in a particle's
workgroup) either raise SMCSD_FLAG_WAIT_EXPIRED or match the oracle, and the
others match the oracle."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
NOWAIT = os.path.join(os.path.dirname(HERE), "smc_resampling_amd", "libsmcsd_nowait.so")


def test_member_waits_that_run_out_end_the_call():
    from gpu_util import say

    assert os.path.exists(NOWAIT), f"{NOWAIT} is missing: run __graft_entry__.build() first"
    env = dict(os.environ, SMCSD_LIBRARY=NOWAIT)
    child = os.path.join(HERE, "wait_expiry_child.py")
    r = subprocess.run([sys.executable, "-u", child], capture_output=True, text=True, timeout=300, env=env)
    say(r.stdout.strip().replace("\n", "; "))
    assert r.returncode == 0 and r.stdout.strip().endswith("OK"), (r.stdout + r.stderr)[-3000:]
