"""Child process of test_wait_expiry.py, run with SMCSD_LIBRARY naming the
test build whose member workgroups never wait for each other's tile masses
(-DSMCSD_TAG_WAIT_TICKS=0).  Calls whose decisions are shared by member
workgroups, and SMC calls whose prompt work runs in a particle's workgroup
(log-weights collected as tagged words), must still end, and each must either
raise SMCSD_FLAG_WAIT_EXPIRED or decide as the oracle does; calls with no
waits (one workgroup per decision, a prompt kernel) must decide as the oracle
does and raise no such flag.  Prints one line per call, then OK."""
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path[:0] = [os.path.dirname(HERE), HERE]

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import smc_resampling_amd as s  # noqa: E402
from compare import compare_sd, compare_smc, compare_tree  # noqa: E402
from gpu_util import run_sd_gpu, run_smc_gpu, run_tree_gpu  # noqa: E402
from synth.small import sd_case, smc_case, tree_case, tree_parents  # noqa: E402

EXPIRED = s.FLAG_WAIT_EXPIRED


def main():
    assert os.environ.get("SMCSD_LIBRARY", "").endswith("libsmcsd_nowait.so"), "run by test_wait_expiry.py"
    expired = 0
    full = tree_parents("full", width=2, depth=3)
    for label, B, members in (("trees, 4 members", 8, True), ("trees, one workgroup each", 300, False)):
        trees = [full] * B if members else [full] * 8 + [tree_parents("root")] * (B - 8)
        c = tree_case(7000 + B, trees, 32768, T=0.8, delta=1.0, dtype="bf16")
        na, ln, ft, fl = run_tree_gpu(c)
        if fl & EXPIRED:
            assert members, (label, fl)
            expired += 1
            print(f"{label}: wait expired (flags {fl})", flush=True)
            continue
        ref = oracle.tree_verify(c["target"], c["draft"], c["node_off"], c["draft_off"], c["parent"], c["tokens"],
                                 c["uniforms"], c["T"])
        compare_tree(c, ref, na, ln, ft, label).assert_ok()
        print(f"{label}: equal to the oracle (flags {fl})", flush=True)
    for label, B in (("sd, 4 members", 16), ("sd, one workgroup each", 300)):
        c = sd_case(7100 + B, B, 32768, T=0.9, K=4, delta=1.0, dtype="bf16")
        na, ft, fl = run_sd_gpu(c)
        if fl & EXPIRED:
            assert B <= 64, (label, fl)
            expired += 1
            print(f"{label}: wait expired (flags {fl})", flush=True)
            continue
        ref = oracle.sd_verify(c["target"], c["draft"], c["tokens"], c["uniforms"], c["T"], K=c["K"])
        compare_sd(c, ref, na, ft, label).assert_ok()
        print(f"{label}: equal to the oracle (flags {fl})", flush=True)
    # at most 512 particles: the prompt's work in its last particle's workgroup
    for label, P, N, waits in (("smc, 1x16 particles", 1, 16, True), ("smc, 8x64 particles", 8, 64, True),
                               ("smc, 9x64 particles (prompt kernel)", 9, 64, False)):
        c = smc_case(7200 + P * N, P, N, 3, 4096, dtype="bf16", L=8, logw_scale=2.0)
        g = run_smc_gpu(c, c["logw"], c["pt"], ess_frac=0.9)
        if g["flags"] & EXPIRED:
            assert waits, (label, g["flags"])
            expired += 1
            print(f"{label}: wait expired (flags {g['flags']})", flush=True)
            continue
        ref = oracle.smc_step(c["target"], c["draft"], c["tokens"], c["bonus_u"], c["resample_u"], c["logw"], c["T"],
                              0.9, P, N, c["K"], pt_in=c["pt"])
        compare_smc(c, ref, g, c["logw"], c["pt"], label).assert_ok()
        print(f"{label}: equal to the oracle (flags {g['flags']})", flush=True)
    print(f"calls whose waits ran out: {expired}", flush=True)
    print("OK", flush=True)


if __name__ == "__main__":
    main()
