"""Helpers for the GPU parity tests: move numpy cases to the device, run the
library through its C ABI, run the oracle on the same inputs, compare."""
from __future__ import annotations

import os
import sys

import numpy as np
import torch

import oracle
from compare import compare_sd, compare_smc, compare_tree

DEV = torch.device("cuda:0")


def say(msg):
    """Progress line; also appended to $SMCSD_PARITY_LOG when set (exemption tallies)."""
    print(msg, flush=True)
    path = os.environ.get("SMCSD_PARITY_LOG")
    if path:
        with open(path, "a") as f:
            f.write(msg + "\n")


def lib():
    import smc_resampling_amd as s

    return s


def oracle_lengths(scores, block, max_blocks, t0, rho):
    """PACER draft lengths of a ragged workload, by the oracle (the lengths a
    parity test feeds both sides come from the oracle, never the library)."""
    return oracle.pacer_lengths(scores, block, max_blocks, t0, rho)[0]


def dev_logits(a: np.ndarray):
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(a).to(DEV)


def host_logits(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def run_sd_gpu(case):
    s = lib()
    off = case.get("offsets")
    na, ft, fl = s.sd_verify(dev_logits(case["target"]), dev_logits(case["draft"]),
                             torch.from_numpy(case["tokens"]).to(DEV), torch.from_numpy(case["uniforms"]).to(DEV),
                             case["T"], K=case["K"],
                             draft_offsets=None if off is None else torch.from_numpy(off).to(DEV))
    torch.cuda.synchronize()
    return na.cpu().numpy(), ft.cpu().numpy(), int(fl.item())


def run_sd_oracle(case):
    return oracle.sd_verify(case["target"], case["draft"], case["tokens"], case["uniforms"], case["T"], K=case["K"],
                            offsets=case.get("offsets"))


def check_sd(case, label="", ignore_flags=8):
    """GPU vs oracle; flag bits in ignore_flags may differ (CDF_CLAMP is a
    rounding-level fallback on either side)."""
    na, ft, fl = run_sd_gpu(case)
    ref = run_sd_oracle(case)
    t = compare_sd(case, ref, na, ft, label)
    say(f"[sd {label}] {t.summary()} flags gpu={fl} oracle={ref['flags']}")
    t.assert_ok()
    assert (fl & ~ignore_flags) == (ref["flags"] & ~ignore_flags), (fl, ref["flags"])
    return t


def oracle_threads():
    """Host threads for oracle calls that run side by side (the oracle's C
    calls release the GIL): one per available core, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def check_sd_many(cases, labels, ignore_flags=8):
    """check_sd over many cases: every GPU call first, then the oracle on a
    pool of host threads, then the comparisons in order.  Returns the merged
    tally."""
    import concurrent.futures as cf

    from compare import Tally

    gpu = [run_sd_gpu(c) for c in cases]
    total = Tally()
    with cf.ThreadPoolExecutor(max_workers=oracle_threads()) as ex:
        refs = ex.map(run_sd_oracle, cases)
        for c, lab, (na, ft, fl), ref in zip(cases, labels, gpu, refs):
            t = compare_sd(c, ref, na, ft, lab)
            say(f"[sd {lab}] {t.summary()} flags gpu={fl} oracle={ref['flags']}")
            t.assert_ok()
            assert (fl & ~ignore_flags) == (ref["flags"] & ~ignore_flags), (fl, ref["flags"])
            total.merge(t)
    return total


def run_smc_gpu(case, logw, pt, ess_frac=0.5):
    s = lib()
    lw = torch.from_numpy(np.array(logw, np.float32)).to(DEV)
    ptd = None if pt is None else torch.from_numpy(pt).to(DEV)
    out = s.smc_reweight_resample(dev_logits(case["target"]), dev_logits(case["draft"]),
                                  torch.from_numpy(case["tokens"]).to(DEV), torch.from_numpy(case["bonus_u"]).to(DEV),
                                  torch.from_numpy(case["resample_u"]).to(DEV), lw, case["T"], ess_frac, case["P"],
                                  case["N"], case["K"], page_table_in=ptd, beta=case.get("beta"))
    torch.cuda.synchronize()
    return dict(bonus=out["bonus_token"].cpu().numpy(), ancestors=out["ancestors"].cpu().numpy(),
                ess=out["ess"].cpu().numpy(), resampled=out["resampled"].cpu().numpy(), logw=lw.cpu().numpy(),
                pt_out=None if pt is None else out["page_table_out"].cpu().numpy(),
                flags=int(out["status_flags"].item()))


def check_smc_steps(case, steps=1, ess_frac=0.5, label="", new_inputs=None):
    """Lockstep: each step starts the oracle from the GPU's previous state."""
    logw, pt = case["logw"], case.get("pt")
    total = None
    for s in range(steps):
        if s and new_inputs is not None:
            case = new_inputs(s, case)
        g = run_smc_gpu(case, logw, pt, ess_frac)
        ref = oracle.smc_step(case["target"], case["draft"], case["tokens"], case["bonus_u"], case["resample_u"],
                              logw, case["T"], ess_frac, case["P"], case["N"], case["K"], pt_in=pt,
                              beta=case.get("beta"))
        t = compare_smc(case, ref, g, logw, pt, f"{label} step {s}")
        say(f"[smc {label} step {s}] {t.summary()} resampled={int(g['resampled'].sum())}/{case['P']} "
            f"flags gpu={g['flags']} oracle={ref['flags']}")
        t.assert_ok()
        assert (g["flags"] & ~8) == (ref["flags"] & ~8), (g["flags"], ref["flags"])
        total = t if total is None else (total.merge(t) or total)
        logw, pt = g["logw"], g["pt_out"]
    return total


def run_tree_gpu(case):
    s = lib()
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)  # noqa: E731
    out = s.tree_verify(dev_logits(case["target"]), dev_logits(case["draft"]), t(case["node_off"]),
                        t(case["draft_off"]), t(case["parent"]), t(case["tokens"]), t(case["uniforms"]), case["T"])
    torch.cuda.synchronize()
    return (out["num_accepted"].cpu().numpy(), out["last_node"].cpu().numpy(), out["final_token"].cpu().numpy(),
            int(out["status_flags"].item()))


def run_tree_oracle(case):
    return oracle.tree_verify(case["target"], case["draft"], case["node_off"], case["draft_off"], case["parent"],
                              case["tokens"], case["uniforms"], case["T"])


def check_tree(case, label="", ignore_flags=8):
    na, ln, ft, fl = run_tree_gpu(case)
    ref = run_tree_oracle(case)
    assert ref["status"] == 0
    t = compare_tree(case, ref, na, ln, ft, label)
    say(f"[tree {label}] {t.summary()} accepted={int(na.sum())} flags gpu={fl} oracle={ref['flags']}")
    t.assert_ok()
    assert (fl & ~ignore_flags) == (ref["flags"] & ~ignore_flags), (fl, ref["flags"])
    return t
