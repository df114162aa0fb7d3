"""GPU-vs-oracle comparison with the decision band of the verify step.

Integer outputs must match the oracle exactly, except decisions whose uniform
lies within BAND of a ratio or CDF boundary (the oracle reports its margins).
When such a decision differs, the rest of that sequence's (or prompt's) step
is excused.  Counts are kept at BAND and, for information, at BAND_TIGHT.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

import oracle

BAND = 1e-5
BAND_TIGHT = 1e-6
LOGW_TOL = 1e-5  # |g - o| <= LOGW_TOL * max(1, |o|)
ESS_TOL = 1e-5   # relative


@dataclass
class Tally:
    equal: int = 0
    exempt_equal: int = 0
    exempt_diff: int = 0
    nonexempt_diff: int = 0
    tight_exempt_diff: int = 0
    tight_nonexempt_diff: int = 0
    failures: list = field(default_factory=list)

    def merge(self, o: "Tally"):
        for k in ("equal", "exempt_equal", "exempt_diff", "nonexempt_diff", "tight_exempt_diff",
                  "tight_nonexempt_diff"):
            setattr(self, k, getattr(self, k) + getattr(o, k))
        self.failures += o.failures

    def summary(self):
        return (f"equal={self.equal} exempt_equal={self.exempt_equal} exempt_diff={self.exempt_diff} "
                f"nonexempt_diff={self.nonexempt_diff} | band 1e-6: exempt_diff={self.tight_exempt_diff} "
                f"nonexempt_diff={self.tight_nonexempt_diff}")

    def assert_ok(self):
        assert self.nonexempt_diff == 0, self.summary() + "\n" + "\n".join(self.failures[:20])


def _interval(cdf, y):
    lo = cdf[y - 1] if y > 0 else 0.0
    return lo, cdf[y]


def _token_diff(t: Tally, u, cdf, y_gpu, what):
    lo, hi = _interval(cdf, y_gpu)
    dist = max(lo - u, u - hi, 0.0)
    if dist <= BAND:
        t.exempt_diff += 1
    else:
        t.nonexempt_diff += 1
        t.failures.append(f"{what}: gpu token {y_gpu} interval [{lo:.9f},{hi:.9f}) u={u:.9f}")
    if dist <= BAND_TIGHT:
        t.tight_exempt_diff += 1
    else:
        t.tight_nonexempt_diff += 1


def compare_sd(inp, ref, na_g, ft_g, label="") -> Tally:
    """inp: dict(target, draft, tokens, uniforms, offsets, K, T) numpy; ref: oracle.sd_verify output."""
    t = Tally()
    offs = inp.get("offsets")
    K = inp["K"]
    B = len(na_g)
    for b in range(B):
        d0 = int(offs[b]) if offs is not None else b * K
        Kb = int(offs[b + 1] - offs[b]) if offs is not None else K
        t0 = d0 + b
        n_o, y_o = int(ref["num_accepted"][b]), int(ref["final_token"][b])
        n_g, y_g = int(na_g[b]), int(ft_g[b])
        am = ref["accept_margin"][d0:d0 + min(n_o + 1, Kb)]
        near = (len(am) and am.min() < BAND) or ref["sample_margin"][b] < BAND
        if n_g == n_o and y_g == y_o:
            t.equal += 1
            t.exempt_equal += int(bool(near))
            continue
        if n_g != n_o:
            j = min(n_g, n_o)
            m = ref["accept_margin"][d0 + j]
            if 0 <= m <= BAND:
                t.exempt_diff += 1
            else:
                t.nonexempt_diff += 1
                t.failures.append(f"{label} seq {b}: accept at j={j} differs (gpu n={n_g}, oracle n={n_o}, margin={m})")
            if 0 <= m <= BAND_TIGHT:
                t.tight_exempt_diff += 1
            else:
                t.tight_nonexempt_diff += 1
            continue
        cdf, _ = oracle.sd_final_cdf(inp["target"], inp["draft"], b, n_o, inp["T"], K=K, offsets=offs)
        _token_diff(t, float(inp["uniforms"][t0 + Kb]), cdf, y_g, f"{label} seq {b} final")
    return t


def bonus_cdf(target, p_row, T):
    row = np.ascontiguousarray(target[p_row:p_row + 1])
    cdf, _ = oracle.sd_final_cdf(row, row[:0], 0, 0, T, K=0)
    return cdf


def compare_draft(logits, uniforms, T, ref, tokens_g, label="") -> Tally:
    """Draft draws: tokens_g (GPU) against ref = oracle.draft_sample(logits,
    uniforms, T), row by row, with the CDF band."""
    t = Tally()
    for r in range(len(tokens_g)):
        yg, yo = int(tokens_g[r]), int(ref["tokens"][r])
        if yg == yo:
            t.equal += 1
            t.exempt_equal += int(ref["margin"][r] < BAND)
        else:
            _token_diff(t, float(uniforms[r]), bonus_cdf(logits, r, T), yg, f"{label} row {r}")
    return t


def compare_smc(inp, ref, out_g, logw_in, pt_in, label="") -> Tally:
    """Lockstep check of one SMC step.  inp: numpy inputs (target, draft, tokens,
    bonus_u, resample_u, P, N, K, T, optional beta); ref: oracle.smc_step(...) run from the same
    logw_in / pt_in as the GPU; out_g: numpy GPU outputs (bonus, ancestors, ess,
    resampled, logw, pt_out)."""
    t = Tally()
    P, N, K, T = inp["P"], inp["N"], inp["K"], inp["T"]
    Tb = T / inp["beta"] if inp.get("beta") is not None else T  # the bonus row's temperature
    for i in range(P * N):
        yg, yo = int(out_g["bonus"][i]), int(ref["bonus"][i])
        if yg == yo:
            t.equal += 1
            t.exempt_equal += int(ref["bonus_margin"][i] < BAND)
        else:
            _token_diff(t, float(inp["bonus_u"][i]), bonus_cdf(inp["target"], i * (K + 1) + K, Tb), yg,
                        f"{label} particle {i} bonus")
    for p in range(P):
        sl = slice(p * N, (p + 1) * N)
        eo, eg = float(ref["ess"][p]), float(out_g["ess"][p])
        flag_near = ref["ess_margin"][p] < BAND
        if abs(eg - eo) > ESS_TOL * max(eo, 1e-30):
            t.nonexempt_diff += 1
            t.failures.append(f"{label} prompt {p}: ess gpu {eg} oracle {eo}")
        rg, ro = int(out_g["resampled"][p]), int(ref["resampled"][p])
        if rg != ro:
            if flag_near:
                t.exempt_diff += 1
            else:
                t.nonexempt_diff += 1
                t.failures.append(f"{label} prompt {p}: resampled gpu {rg} oracle {ro} (ess {eo})")
            continue
        ag, ao = out_g["ancestors"][sl], ref["ancestors"][sl]
        lwg, lwo = out_g["logw"][sl], ref["logw"][sl]
        if ro:
            C = ref["cum_weight"][sl]
            for k in range(N):
                if ag[k] == ao[k]:
                    t.equal += 1
                    continue
                U = (float(inp["resample_u"][p]) + k) / N
                lo = C[ag[k] - 1] if ag[k] > 0 else 0.0
                dist = max(lo - U, U - C[ag[k]], 0.0)
                if dist <= BAND:
                    t.exempt_diff += 1
                else:
                    t.nonexempt_diff += 1
                    t.failures.append(f"{label} prompt {p} slot {k}: ancestor gpu {ag[k]} oracle {ao[k]}")
                if dist <= BAND_TIGHT:
                    t.tight_exempt_diff += 1
                else:
                    t.tight_nonexempt_diff += 1
            if not (lwg == 0).all():
                t.nonexempt_diff += 1
                t.failures.append(f"{label} prompt {p}: log-weights not reset")
        else:
            t.equal += int((ag == np.arange(N)).all())
            if not (ag == np.arange(N)).all():
                t.nonexempt_diff += 1
                t.failures.append(f"{label} prompt {p}: ancestors not identity without resampling")
            bad = np.abs(lwg.astype(np.float64) - lwo) > LOGW_TOL * np.maximum(1.0, np.abs(lwo.astype(np.float64)))
            if bad.any():
                t.nonexempt_diff += int(bad.sum())
                t.failures.append(f"{label} prompt {p}: logw gpu {lwg[bad][:4]} oracle {lwo[bad][:4]}")
        if pt_in is not None:
            want = pt_in[p * N + ag]
            if not (out_g["pt_out"][sl] == want).all():
                t.nonexempt_diff += 1
                t.failures.append(f"{label} prompt {p}: page table is not the ancestor gather")
    return t


def _depth_path(parent, n0, node):
    """Nodes root .. node (local indices) of a tree whose parents start at n0."""
    path = [node]
    while path[-1] > 0:
        path.append(int(parent[n0 + path[-1]]))
    return path[::-1]


def compare_tree(inp, ref, na_g, ln_g, ft_g, label="") -> Tally:
    """Tree verification: the GPU's stopping node, depth and final token against
    the oracle's.  When the walks part, the first child tested differently at
    the deepest common node must have its uniform within BAND of its ratio."""
    t = Tally()
    noff, par = inp["node_off"], inp["parent"]
    for b in range(len(na_g)):
        n0, M = int(noff[b]), int(noff[b + 1] - noff[b])
        lo, yo = int(ref["last_node"][b]), int(ref["final_token"][b])
        lg, yg, ng = int(ln_g[b]), int(ft_g[b]), int(na_g[b])
        if not (0 <= lg < M) or ng != len(_depth_path(par, n0, lg)) - 1:
            t.nonexempt_diff += 1
            t.failures.append(f"{label} tree {b}: gpu stop node {lg} / depth {ng} is not a node and its depth")
            continue
        po, pg = _depth_path(par, n0, lo), _depth_path(par, n0, lg)
        am = ref["accept_margin"][n0:n0 + M]
        tested = am[am >= 0]
        near = (len(tested) and tested.min() < BAND) or ref["sample_margin"][b] < BAND
        if lg == lo and yg == yo:
            t.equal += 1
            t.exempt_equal += int(bool(near))
            continue
        if lg != lo:
            k = 0
            while k + 1 < min(len(po), len(pg)) and po[k + 1] == pg[k + 1]:
                k += 1
            co = po[k + 1] if k + 1 < len(po) else None
            cg = pg[k + 1] if k + 1 < len(pg) else None
            first = cg if co is None else co if cg is None else min(co, cg)
            m = float(am[first])
            if 0 <= m <= BAND:
                t.exempt_diff += 1
            else:
                t.nonexempt_diff += 1
                t.failures.append(f"{label} tree {b}: walks part at node {po[k]} (gpu stop {lg}, oracle {lo}); "
                                  f"test of node {first} margin {m}")
            if 0 <= m <= BAND_TIGHT:
                t.tight_exempt_diff += 1
            else:
                t.tight_nonexempt_diff += 1
            continue
        cdf, _ = oracle.tree_final_cdf(inp["target"], inp["draft"], noff, inp["draft_off"], par, b, lo, inp["T"])
        _token_diff(t, float(inp["uniforms"][n0]), cdf, yg, f"{label} tree {b} final")
    return t
