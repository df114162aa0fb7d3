"""Checks that pin the oracle to facts fixed outside itself.

Each ``check_*`` takes a loaded oracle library (``oracle.load()`` or a mutant
built by the mutation test) and raises ``AssertionError`` on a violation.  The
pins are hand-derived worked examples (``tests/golden``), closed forms,
textbook invariants, library routines (scipy ``log_softmax``, numpy
``searchsorted``), exact rational brute force and exact output laws obtained by
integrating the oracle's piecewise-constant decisions over the uniforms.
"""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np
from scipy.special import log_softmax, softmax

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _logits(probs):
    with np.errstate(divide="ignore"):  # probability 0 is logit -inf
        return np.log(np.asarray(probs, dtype=np.float64)).astype(np.float32)


def rand_sd_problem(rng, B, K, V, T, delta, scale=3.0, dtype=np.float32):
    """Random SD inputs with x_j ~ q_j (drawn here with numpy)."""
    zt = (scale * rng.standard_normal((B * (K + 1), V))).astype(np.float32)
    rows_t = zt.reshape(B, K + 1, V)
    zd = (rows_t[:, :K, :] + delta * rng.standard_normal((B, K, V))).astype(np.float32).reshape(B * K, V)
    q = softmax(zd.astype(np.float64) / T, axis=-1)
    cq = np.cumsum(q, axis=-1)
    r = rng.random((B * K, 1))
    tok = np.minimum((cq < r * cq[:, -1:]).sum(axis=-1), V - 1).astype(np.int32)
    u = rng.random(B * (K + 1)).astype(np.float32)
    return zt, zd, tok, u


# --------------------------------------------------------------------------
# golden worked examples
# --------------------------------------------------------------------------


def check_golden_sd_fixed(lib):
    g = _load_golden("sd_fixed_k2.json")
    r = oracle.sd_verify(_logits(g["target_probs"]), _logits(g["draft_probs"]), g["tokens"], g["uniforms"],
                         g["T"], K=g["K"], lib=lib)
    assert r["num_accepted"].tolist() == g["expect"]["num_accepted"], r
    assert r["final_token"].tolist() == g["expect"]["final_token"], r


def check_golden_sd_csr(lib):
    g = _load_golden("sd_csr_ragged.json")
    r = oracle.sd_verify(_logits(g["target_probs"]), _logits(g["draft_probs"]), g["tokens"], g["uniforms"],
                         g["T"], offsets=g["offsets"], lib=lib)
    assert r["num_accepted"].tolist() == g["expect"]["num_accepted"], r
    assert r["final_token"].tolist() == g["expect"]["final_token"], r


def check_golden_smc(lib):
    g = _load_golden("smc_step_n4.json")
    lw = (np.array(g["logw_in_ln4_multiples"], np.float64) * math.log(4.0)).astype(np.float32)
    r = oracle.smc_step(_logits(g["target_probs"]), _logits(g["draft_probs"]), g["tokens"], g["bonus_u"],
                        g["resample_u"], lw, g["T"], g["ess_frac"], g["P"], g["N"], g["K"],
                        pt_in=np.array(g["page_table_in"], np.int32), lib=lib)
    e = g["expect"]
    assert r["resampled"].tolist() == e["resampled"], r
    assert r["ancestors"].tolist() == e["ancestors"], r
    assert r["bonus"].tolist() == e["bonus"], r
    assert r["logw"].tolist() == e["logw_out"], r
    assert r["pt_out"].tolist() == e["page_table_out"], r
    assert abs(float(r["ess"][0]) - e["ess"]) < 1e-6, r


# --------------------------------------------------------------------------
# row statistics (temperature softmax)
# --------------------------------------------------------------------------


def check_constant_row(lib):
    for V in (1, 7, 32000):
        for T in (1.0, 0.7):
            row = np.full(V, 1.25, np.float32)
            lp = oracle.logprob(row, T, V // 2, lib=lib)
            assert lp == -math.log(V), (V, T, lp)


def check_two_valued_row(lib):
    V, k, a, b = 1000, 7, 2.5, -1.0
    for T in (1.0, 0.7, 2.0):
        row = np.full(V, b, np.float32)
        row[[3, 50, 51, 400, 777, 998, 999]] = a
        expect_a = -math.log(k + (V - k) * math.exp((b - a) / T))
        expect_b = (b - a) / T + expect_a
        assert abs(oracle.logprob(row, T, 50, lib=lib) - expect_a) < 1e-13
        assert abs(oracle.logprob(row, T, 0, lib=lib) - expect_b) < 1e-13


def _bf16_bits(x32):
    """Round float32 to bf16 (round to nearest even); returns uint16 bits."""
    b = np.asarray(x32, np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return b.astype(np.uint16)


def _bf16_to_f64(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def check_rows_vs_scipy(lib):
    rng = np.random.default_rng(11)
    for V, T in ((33, 1.0), (4096, 0.7), (151936, 1.0)):
        z = (3 * rng.standard_normal(V)).astype(np.float32)
        ref = log_softmax(z.astype(np.float64) / T)
        for i in (0, V // 3, V - 1):
            assert abs(oracle.logprob(z, T, i, lib=lib) - ref[i]) < 1e-11
        zb = _bf16_bits(z)
        refb = log_softmax(_bf16_to_f64(zb) / T)
        for i in (1, V // 2, V - 2):
            assert abs(oracle.logprob(zb, T, i, lib=lib) - refb[i]) < 1e-11


# --------------------------------------------------------------------------
# SD verify
# --------------------------------------------------------------------------


def check_accept_tie_rejects(lib):
    """rho = p/q = 0.5 exactly and u = 0.5: the strict test rejects."""
    target = np.array([[0.0, 0.0], [0.0, 0.0]], np.float32)  # p = (1/2, 1/2)
    draft = np.array([[0.0, -np.inf]], np.float32)  # q = (1, 0)
    rho = math.exp(oracle.logprob(target[0], 1.0, 0, lib=lib) - oracle.logprob(draft[0], 1.0, 0, lib=lib))
    assert rho == 0.5, rho
    r = oracle.sd_verify(target, draft, [0], [0.5, 0.1], 1.0, K=1, lib=lib)
    assert r["num_accepted"].tolist() == [0], r
    r = oracle.sd_verify(target, draft, [0], [np.nextafter(np.float32(0.5), np.float32(0)), 0.1], 1.0, K=1, lib=lib)
    assert r["num_accepted"].tolist() == [1], r


def check_cdf_tie(lib):
    """Uniform p over 4 tokens has CDF (1/4, 1/2, 3/4, 1); u = 1/4 exactly picks index 1."""
    target = np.zeros((1, 4), np.float32)
    draft = np.zeros((0, 4), np.float32)
    for u, want in ((0.0, 0), (0.25, 1), (0.5, 2), (0.7499, 2), (0.75, 3), (0.99999994, 3)):
        r = oracle.sd_verify(target, draft, np.zeros(0, np.int32), [u], 1.0, K=0, lib=lib)
        assert r["final_token"].tolist() == [want], (u, r)
        assert r["num_accepted"].tolist() == [0]


def _midpoints(cdf):
    """Midpoints and lengths of the intervals [C_{i-1}, C_i) with positive length."""
    edges = np.concatenate([[0.0], cdf])
    lo, hi = edges[:-1], edges[1:]
    keep = hi - lo > 1e-9
    return (0.5 * (lo + hi))[keep], (hi - lo)[keep]


def check_sd_exact_law(lib):
    """K=1: integrate the oracle's decisions over (x_0 ~ q, u_0, u_1) exactly.

    The first emitted token must follow p_0 and, given acceptance, the second
    must follow p_1 (standard SD is exact).
    """
    rng = np.random.default_rng(5)
    for V, T, delta in ((3, 1.0, 1.0), (5, 0.7, 2.0), (6, 1.3, 0.4)):
        zt = (2 * rng.standard_normal((2, V))).astype(np.float32)
        zd = (zt[:1] + delta * rng.standard_normal((1, V))).astype(np.float32)
        p0 = softmax(zt[0].astype(np.float64) / T)
        p1 = softmax(zt[1].astype(np.float64) / T)
        q0 = softmax(zd[0].astype(np.float64) / T)
        a = np.minimum(1.0, p0 / q0)
        res = np.maximum(0.0, p0 - q0)
        res_mid, res_len = _midpoints(np.cumsum(res / res.sum()))
        bon_mid, bon_len = _midpoints(np.cumsum(p1))
        law0 = np.zeros(V)
        law1 = np.zeros(V)
        for x in range(V):
            # accept region u_0 in [0, a): followed by the bonus draw from p_1
            B = len(bon_mid)
            u = np.stack([np.full(B, a[x] / 2), bon_mid], axis=1).astype(np.float32).ravel()
            r = oracle.sd_verify(np.tile(zt, (B, 1)), np.tile(zd, (B, 1)), np.full(B, x, np.int32), u, T, K=1, lib=lib)
            assert (r["num_accepted"] == 1).all(), (x, r)
            law0[x] += q0[x] * a[x]
            for t, w in zip(r["final_token"], bon_len):
                law1[t] += q0[x] * a[x] * w
            if a[x] < 1.0:
                B = len(res_mid)
                u = np.stack([np.full(B, (1 + a[x]) / 2), res_mid], axis=1).astype(np.float32).ravel()
                r = oracle.sd_verify(np.tile(zt, (B, 1)), np.tile(zd, (B, 1)), np.full(B, x, np.int32), u, T, K=1,
                                     lib=lib)
                assert (r["num_accepted"] == 0).all(), (x, r)
                for t, w in zip(r["final_token"], res_len):
                    law0[t] += q0[x] * (1 - a[x]) * w
        acc = float(np.sum(np.minimum(p0, q0)))
        assert np.abs(law0 - p0).max() < 1e-9, (law0, p0)
        assert np.abs(law1 / acc - p1).max() < 1e-9, (law1 / acc, p1)


def check_zero_residual_fallback(lib):
    """Reading: a rejection whose residual max(0, p_n - q_n) has no mass
    (p_n equal to q_n) draws the final token from p_n with the same final
    uniform, and raises ZERO_RESIDUAL.  Identical target and draft rows make
    rho = 1 exactly, and an accept uniform of 1.0 (outside the documented
    [0, 1), but defined) then rejects.  The residual is exactly 0, and the
    final token must be numpy's searchsorted on cumsum(p_n)."""
    rng = np.random.default_rng(57)
    V, K, T = 9, 2, 0.8
    zt = (2 * rng.standard_normal((K + 1, V))).astype(np.float32)
    zd = zt[:K].copy()
    tok = rng.integers(0, V, K).astype(np.int32)
    for n in range(K):
        p = softmax(zt[n].astype(np.float64) / T)
        c = np.cumsum(p)
        for uf in (0.05, 0.3, 0.61, 0.93):
            u = np.full(K + 1, 0.5, np.float32)
            u[n], u[K] = 1.0, uf
            r = oracle.sd_verify(zt, zd, tok, u, T, K=K, lib=lib)
            assert r["num_accepted"].tolist() == [n], (n, r)
            assert r["flags"] & oracle.FLAG_ZERO_RESIDUAL, r
            want = int(np.searchsorted(c, np.float64(np.float32(uf)) * c[-1], side="right"))
            if np.min(np.abs(c / c[-1] - np.float32(uf))) > 1e-9:
                assert r["final_token"].tolist() == [want], (n, uf, r["final_token"], want)


def check_cdf_clamp_last_positive(lib):
    """Reading: when no inclusive prefix exceeds u * Z (u = 1.0 here, where the
    last prefix equals Z), the draw takes the last index with positive weight
    and raises CDF_CLAMP, its margin 0 (no interval holds u).  Rows whose
    trailing (and some inner) logits are -inf: the answer is the last finite
    logit, neither index 0 nor V - 1.  Checked on the bonus draw (draft =
    target, all accepted) and on the residual draw (a rejection)."""
    ninf = -np.inf
    for row, last in (([1.0, 2.0, ninf, 0.5, ninf, ninf], 3), ([ninf, 0.25, 3.0, ninf], 2),
                      ([0.0, 0.0, 0.0, 0.0, 0.0, ninf, ninf, ninf], 4)):
        z = np.asarray([row], np.float32)
        r = oracle.sd_verify(z, np.zeros((0, z.shape[1]), np.float32), np.zeros(0, np.int32), [1.0], 1.0, K=0,
                             lib=lib)
        assert r["final_token"].tolist() == [last], (row, r)
        assert r["flags"] & oracle.FLAG_CDF_CLAMP and r["sample_margin"][0] == 0.0, r
    # residual: p puts mass on tokens 0..3, q on token 0 only; max(0, p - q)
    # is positive on 1..3 (trailing tokens -inf in both rows); token 0 rejects
    zt = np.asarray([[0.0, 0.0, 0.0, 0.0, ninf, ninf], [0.0] * 6], np.float32)
    zd = np.asarray([[0.0, ninf, ninf, ninf, ninf, ninf]], np.float32)
    r = oracle.sd_verify(zt, zd, np.zeros(1, np.int32), [0.5, 1.0], 1.0, K=1, lib=lib)
    assert r["num_accepted"].tolist() == [0] and r["final_token"].tolist() == [3], r
    assert r["flags"] & oracle.FLAG_CDF_CLAMP and r["sample_margin"][0] == 0.0, r


def check_bonus_vs_numpy(lib):
    """draft == target (delta = 0): every token accepted, final token is a plain
    categorical inverse-CDF draw from p_K, i.e. numpy searchsorted."""
    rng = np.random.default_rng(7)
    B, K, V, T = 64, 3, 777, 0.8
    zt, zd, tok, u = rand_sd_problem(rng, B, K, V, T, delta=0.0)
    zd = zt.reshape(B, K + 1, V)[:, :K].reshape(B * K, V).copy()
    r = oracle.sd_verify(zt, zd, tok, u, T, K=K, lib=lib)
    assert (r["num_accepted"] == K).all()
    for b in range(B):
        p = softmax(zt[b * (K + 1) + K].astype(np.float64) / T)
        c = np.cumsum(p)
        uf = float(u[b * (K + 1) + K])
        want = int(np.searchsorted(c, uf * c[-1], side="right"))
        if np.min(np.abs(c / c[-1] - uf)) > 1e-12:
            assert r["final_token"][b] == want, (b, r["final_token"][b], want)


def check_residual_vs_numpy(lib):
    rng = np.random.default_rng(8)
    B, K, V, T = 96, 2, 500, 1.0
    zt, zd, tok, u = rand_sd_problem(rng, B, K, V, T, delta=2.0)
    r = oracle.sd_verify(zt, zd, tok, u, T, K=K, lib=lib)
    seen = 0
    for b in range(B):
        n = int(r["num_accepted"][b])
        if n == K:
            continue
        seen += 1
        p = softmax(zt[b * (K + 1) + n].astype(np.float64) / T)
        q = softmax(zd[b * K + n].astype(np.float64) / T)
        c = np.cumsum(np.maximum(0.0, p - q))
        uf = float(u[b * (K + 1) + K])
        want = int(np.searchsorted(c, uf * c[-1], side="right"))
        if np.min(np.abs(c / c[-1] - uf)) > 1e-12:
            assert r["final_token"][b] == want, (b, r["final_token"][b], want)
    assert seen > B // 2


def check_final_cdf_vs_numpy(lib):
    """The normalised CDF the comparison judges differing tokens against: the
    residual cumsum(max(0, p_n - q_n)) / Z for n < K_b, cumsum(p_K) for n = K_b."""
    rng = np.random.default_rng(10)
    B, K, V, T = 3, 2, 611, 0.8
    zt, zd, tok, u = rand_sd_problem(rng, B, K, V, T, delta=1.5)
    for b in range(B):
        for n in range(K + 1):
            cdf, fl = oracle.sd_final_cdf(zt, zd, b, n, T, K=K, lib=lib)
            p = softmax(zt[b * (K + 1) + n].astype(np.float64) / T)
            w = np.maximum(0.0, p - softmax(zd[b * K + n].astype(np.float64) / T)) if n < K else p
            want = np.cumsum(w) / w.sum()
            assert fl == 0 and np.abs(cdf - want).max() < 1e-12, (b, n, np.abs(cdf - want).max())


def check_accept_decisions_vs_scipy(lib):
    """n = index of the first j with u_j >= p_j(x_j)/q_j(x_j) (scipy softmax)."""
    rng = np.random.default_rng(9)
    B, K, V, T = 128, 4, 300, 0.9
    zt, zd, tok, u = rand_sd_problem(rng, B, K, V, T, delta=1.0)
    r = oracle.sd_verify(zt, zd, tok, u, T, K=K, lib=lib)
    lp = log_softmax(zt.astype(np.float64) / T, axis=-1).reshape(B, K + 1, V)
    lq = log_softmax(zd.astype(np.float64) / T, axis=-1).reshape(B, K, V)
    for b in range(B):
        n = K
        for j in range(K):
            x = tok[b * K + j]
            rho = math.exp(lp[b, j, x] - lq[b, j, x])
            if abs(u[b * (K + 1) + j] - min(1.0, rho)) < 1e-12:
                n = None
                break
            if not u[b * (K + 1) + j] < rho:
                n = j
                break
        if n is not None:
            assert r["num_accepted"][b] == n, (b, r["num_accepted"][b], n)


def check_sd_statistics(lib, trials=200_000, configs=((5, 2), (3, 1), (8, 4))):
    """Chi-square: the token emitted at position j, given it is reached, follows
    p_j; the acceptance rate at position 0 is sum(min(p, q))."""
    from scipy.stats import chisquare

    rng = np.random.default_rng(123)
    for V, K in configs:
        T = 1.0
        zt1 = (1.5 * rng.standard_normal((K + 1, V))).astype(np.float32)
        zd1 = (zt1[:K] + 1.0 * rng.standard_normal((K, V))).astype(np.float32)
        q = softmax(zd1.astype(np.float64) / T, axis=-1)
        p = softmax(zt1.astype(np.float64) / T, axis=-1)
        B = trials
        tok = np.stack([rng.choice(V, size=B, p=q[j]) for j in range(K)], axis=1).astype(np.int32).ravel()
        u = rng.random(B * (K + 1)).astype(np.float32)
        r = oracle.sd_verify(np.tile(zt1, (B, 1)), np.tile(zd1, (B, 1)), tok, u, T, K=K, lib=lib)
        n = r["num_accepted"]
        y = r["final_token"]
        toks = tok.reshape(B, K)
        alpha0 = float(np.minimum(p[0], q[0]).sum())
        rate = float(np.mean(n >= 1)) if K >= 1 else None
        if rate is not None:
            sd = math.sqrt(alpha0 * (1 - alpha0) / B)
            assert abs(rate - alpha0) < 5 * sd, (rate, alpha0)
        for j in range(K + 1):
            reach = n >= j
            emitted = np.where(n[reach] > j, toks[reach][:, min(j, K - 1)] if K > 0 else 0, y[reach])
            cnt = np.bincount(emitted, minlength=V)
            exp = p[j] * reach.sum()
            keep = exp > 5
            stat = chisquare(cnt[keep], exp[keep] * cnt[keep].sum() / exp[keep].sum())
            assert stat.pvalue > 1e-4, (V, K, j, stat)


def check_particle_l1_trend(lib, reps=300, Ns=(32, 128, 512, 2048)):
    """The weighted particles' error shrinks like 1/sqrt(N) ("Faster LLM
    Inference via Sequential Monte Carlo", sec. 3: the L1 bias falls as
    O(1/sqrt(N)); the constants, set by the draft/target chi-square divergence,
    are not given, so only the trend is checked).  One SMC step with K = 1 and
    no resampling: particle i drafts x_i ~ q and carries log p(x_i) - log q(x_i);
    the weighted histogram of the x_i against p, mean L1 distance over `reps`
    independent prompts, must halve (within [1.6, 2.5]) each time N
    quadruples.  A weight that is not log p - log q (a flipped sign, a dropped
    term) leaves a bias that does not shrink."""
    rng = np.random.default_rng(2604)
    V, K, T = 6, 1, 1.0
    zt = (1.5 * rng.standard_normal((K + 1, V))).astype(np.float32)
    zd = (zt[:K] + 1.0 * rng.standard_normal((K, V))).astype(np.float32)
    p = softmax(zt[0].astype(np.float64) / T)
    q = softmax(zd[0].astype(np.float64) / T)
    means = []
    for N in Ns:
        P = reps
        x = rng.choice(V, size=P * N, p=q).astype(np.int32)
        r = oracle.smc_step(np.tile(zt, (P * N, 1)), np.tile(zd, (P * N, 1)), x,
                            rng.random(P * N).astype(np.float32), rng.random(P).astype(np.float32),
                            np.zeros(P * N, np.float32), T, 0.0, P, N, K, lib=lib)
        assert r["resampled"].sum() == 0 and r["flags"] == 0
        lw = r["logw"].astype(np.float64).reshape(P, N)
        w = np.exp(lw - lw.max(axis=1, keepdims=True))
        l1 = [np.abs(np.bincount(x.reshape(P, N)[i], weights=w[i], minlength=V) / w[i].sum() - p).sum()
              for i in range(P)]
        means.append(float(np.mean(l1)))
    ratios = [a / b for a, b in zip(means, means[1:])]
    assert all(1.6 < t < 2.5 for t in ratios), (means, ratios)


def check_expected_length(lib, trials=200_000):
    """Identical (p, q) at every position make the acceptance events iid with
    alpha = sum(min(p, q)); then E[n + 1] = (1 - alpha^(K+1)) / (1 - alpha)."""
    rng = np.random.default_rng(77)
    V, K, T = 6, 4, 1.0
    zt1 = (1.5 * rng.standard_normal(V)).astype(np.float32)
    zd1 = (zt1 + 1.2 * rng.standard_normal(V)).astype(np.float32)
    p = softmax(zt1.astype(np.float64))
    q = softmax(zd1.astype(np.float64))
    alpha = float(np.minimum(p, q).sum())
    B = trials
    tok = rng.choice(V, size=B * K, p=q).astype(np.int32)
    u = rng.random(B * (K + 1)).astype(np.float32)
    r = oracle.sd_verify(np.tile(zt1, (B * (K + 1), 1)), np.tile(zd1, (B * K, 1)), tok, u, T, K=K, lib=lib)
    L = r["num_accepted"].astype(np.float64) + 1
    want = (1 - alpha ** (K + 1)) / (1 - alpha)
    assert abs(L.mean() - want) < 5 * L.std() / math.sqrt(B), (L.mean(), want)


# --------------------------------------------------------------------------
# SMC step
# --------------------------------------------------------------------------


def _smc_from_logw(lib, logw, u_r, ess_frac=0.5, L=3):
    """Run the SMC step with K=0 (no draft rows), so logw' = logw exactly."""
    N = len(logw)
    V = 4
    target = np.zeros((N, V), np.float32)
    draft = np.zeros((0, V), np.float32)
    pt = np.arange(N * L, dtype=np.int32).reshape(N, L)
    return oracle.smc_step(target, draft, np.zeros(0, np.int32), np.full(N, 0.5, np.float32), [u_r],
                           np.asarray(logw, np.float32), 1.0, ess_frac, 1, N, 0, pt_in=pt, lib=lib)


def check_ess_closed_forms(lib):
    for N in (1, 4, 16, 64):
        r = _smc_from_logw(lib, np.full(N, -3.25), 0.3)
        assert r["ess"][0] == N, r["ess"]
        assert r["resampled"][0] == 0
    lw = np.full(16, -np.inf)
    lw[5] = 1.0
    r = _smc_from_logw(lib, lw, 0.3)
    assert r["ess"][0] == 1.0 and r["resampled"][0] == 1
    assert r["ancestors"].tolist() == [5] * 16
    # two-valued: k particles at weight 1, N-k at weight e^-2
    N, k = 10, 3
    lw = np.full(N, -2.0)
    lw[:k] = 0.0
    a, b = 1.0, math.exp(-2.0)
    want = (k * a + (N - k) * b) ** 2 / (k * a * a + (N - k) * b * b)
    r = _smc_from_logw(lib, lw, 0.3)
    assert abs(float(r["ess"][0]) - want) < 1e-5, (r["ess"], want)
    rng = np.random.default_rng(3)
    for _ in range(20):
        N = int(rng.integers(1, 80))
        r = _smc_from_logw(lib, 4 * rng.standard_normal(N), float(rng.random()))
        assert 1.0 - 1e-6 <= r["ess"][0] <= N + 1e-4


def check_threshold_strict(lib):
    """N=2, weights (1, 0): ESS = 1 = 0.5 * N exactly, which is not below it."""
    r = _smc_from_logw(lib, [0.0, -np.inf], 0.3)
    assert r["ess"][0] == 1.0 and r["resampled"][0] == 0, r
    r = _smc_from_logw(lib, [0.0, -np.inf], 0.3, ess_frac=0.51)
    assert r["resampled"][0] == 1 and r["ancestors"].tolist() == [0, 0], r


def check_systematic_invariants(lib):
    rng = np.random.default_rng(21)
    for trial in range(60):
        N = int(rng.integers(2, 65))
        lw = 2.5 * rng.standard_normal(N)
        u = float(rng.random())
        r = _smc_from_logw(lib, lw, u, ess_frac=1.01)  # always resample
        assert r["resampled"][0] == 1
        a = r["ancestors"]
        assert (np.diff(a) >= 0).all(), a
        w = np.exp(lw.astype(np.float32).astype(np.float64) - lw.max())
        w /= w.sum()
        cnt = np.bincount(a, minlength=N)
        assert cnt.sum() == N
        lo, hi = np.floor(N * w - 1e-9), np.ceil(N * w + 1e-9)
        assert ((cnt >= lo) & (cnt <= hi)).all(), (N * w, cnt)
        assert (r["logw"] == 0).all()
        pt = np.arange(N * 3).reshape(N, 3)
        assert (r["pt_out"] == pt[a]).all()
    for N in (1, 2, 7, 64):
        for u in (0.0, 0.3, 0.9999999):
            r = _smc_from_logw(lib, np.zeros(N), u, ess_frac=1.01)
            assert r["ancestors"].tolist() == list(range(N)), (N, u, r["ancestors"])


def check_systematic_clamp_last_positive(lib):
    """Reading: a systematic point U_k that no normalised prefix C_i exceeds
    (resample uniform 1.0 puts U_{N-1} = 1.0, and the last prefix equals 1)
    goes to the last particle with positive weight, CDF_CLAMP is raised and
    the resampling margin is 0.
    Particles with weight 0 (log-weight -inf) at the end: the last slot's
    ancestor is the last live particle, not particle 0 or N - 1; the other
    slots follow the exact rational rule."""
    ninf = -np.inf
    for lw, last in (([0.3, -1.0, 0.5, ninf, ninf], 2), ([ninf, 0.0, ninf, 1.5, -0.5, ninf], 4),
                     ([0.0, 0.0, 0.0, ninf], 2)):
        N = len(lw)
        r = _smc_from_logw(lib, lw, 1.0, ess_frac=1.01)
        a = r["ancestors"].tolist()
        assert r["resampled"][0] == 1 and a[-1] == last, (lw, a)
        assert r["flags"] & oracle.FLAG_CDF_CLAMP and r["resample_margin"][0] == 0.0, r
        M = max(x for x in lw if x > ninf)
        w = [Fraction(math.exp(float(np.float32(x)) - M)) if x > ninf else Fraction(0) for x in lw]
        C, acc = [], Fraction(0)
        for x in w:
            acc += x
            C.append(acc / sum(w))
        for k in range(N - 1):
            U = Fraction(1 + k, N)
            assert a[k] == next(i for i in range(N) if C[i] > U), (lw, k, a)


def check_systematic_fraction_bruteforce(lib):
    """Exact rational systematic resampling on the oracle's own float weights."""
    rng = np.random.default_rng(31)
    for trial in range(40):
        N = int(rng.integers(1, 9))
        lw = (1.5 * rng.standard_normal(N)).astype(np.float32)
        u = np.float32(rng.random())
        r = _smc_from_logw(lib, lw, float(u), ess_frac=1.01)
        M = float(lw.max())
        w = [Fraction(math.exp(float(x) - M)) for x in lw]
        S = sum(w)
        C = []
        acc = Fraction(0)
        for x in w:
            acc += x
            C.append(acc / S)
        want = []
        for k in range(N):
            U = (Fraction(float(u)) + k) / N
            want.append(next(i for i in range(N) if C[i] > U))
        near = min(abs(float(C[i] - (Fraction(float(u)) + k) / N)) for i in range(N) for k in range(N))
        if near > 1e-12:
            assert r["ancestors"].tolist() == want, (lw, u, r["ancestors"], want)


def check_smc_reweight_vs_scipy(lib):
    rng = np.random.default_rng(41)
    P, N, K, V, T = 2, 5, 3, 257, 0.9
    zt = (3 * rng.standard_normal((P * N * (K + 1), V))).astype(np.float32)
    zd = (zt.reshape(P * N, K + 1, V)[:, :K] + rng.standard_normal((P * N, K, V))).astype(np.float32)
    zd = zd.reshape(P * N * K, V)
    tok = rng.integers(0, V, P * N * K).astype(np.int32)
    lw0 = rng.standard_normal(P * N).astype(np.float32)
    r = oracle.smc_step(zt, zd, tok, rng.random(P * N), rng.random(P), lw0, T, 0.0, P, N, K, lib=lib)
    lp = log_softmax(zt.astype(np.float64) / T, axis=-1).reshape(P * N, K + 1, V)
    lq = log_softmax(zd.astype(np.float64) / T, axis=-1).reshape(P * N, K, V)
    for i in range(P * N):
        d = sum(lp[i, j, tok[i * K + j]] - lq[i, j, tok[i * K + j]] for j in range(K))
        assert abs(float(r["logw"][i]) - (float(lw0[i]) + d)) <= 1e-6 * max(1.0, abs(float(lw0[i]) + d)), i
    assert (r["resampled"] == 0).all()


def check_smc_delta_zero(lib):
    """draft == target: every increment is exactly 0, so the log-weights carry over."""
    rng = np.random.default_rng(43)
    P, N, K, V = 1, 6, 2, 100
    zt = (3 * rng.standard_normal((P * N * (K + 1), V))).astype(np.float32)
    zd = zt.reshape(P * N, K + 1, V)[:, :K].reshape(P * N * K, V).copy()
    tok = rng.integers(0, V, P * N * K).astype(np.int32)
    lw0 = (0.01 * rng.standard_normal(P * N)).astype(np.float32)
    r = oracle.smc_step(zt, zd, tok, rng.random(P * N), [0.5], lw0, 1.0, 0.5, P, N, K, lib=lib)
    assert (r["logw"] == lw0).all(), (r["logw"], lw0)


def check_smc_bonus_law(lib):
    """The (K+1)-th token's law over its uniform is exactly p_K."""
    rng = np.random.default_rng(45)
    V, K, T = 7, 2, 1.1
    zt = (2 * rng.standard_normal((K + 1, V))).astype(np.float32)
    zd = (zt[:K] + rng.standard_normal((K, V))).astype(np.float32)
    pK = softmax(zt[K].astype(np.float64) / T)
    mid, ln = _midpoints(np.cumsum(pK))
    N = len(mid)
    tok = np.tile(rng.integers(0, V, K).astype(np.int32), N)
    r = oracle.smc_step(np.tile(zt, (N, 1)), np.tile(zd, (N, 1)), tok, mid.astype(np.float32), [0.5],
                        np.zeros(N, np.float32), T, 0.0, 1, N, K, lib=lib)
    law = np.zeros(V)
    for t, w in zip(r["bonus"], ln):
        law[t] += w
    assert np.abs(law - pK).max() < 1e-9, (law, pK)


def check_smc_page_table_identity(lib):
    rng = np.random.default_rng(47)
    N, L = 8, 5
    r = _smc_from_logw(lib, 0.01 * rng.standard_normal(N), 0.4, L=L)
    assert r["resampled"][0] == 0
    assert r["ancestors"].tolist() == list(range(N))
    assert (r["pt_out"] == np.arange(N * L).reshape(N, L)).all()


def check_power_bonus_law(lib):
    """Power target: the (K+1)-th token's law over its uniform is exactly
    softmax(beta z_K / T) (scipy), for a sharpening and a flattening beta."""
    rng = np.random.default_rng(49)
    V, K, T = 6, 1, 0.9
    zt = (2 * rng.standard_normal((K + 1, V))).astype(np.float32)
    zd = (zt[:K] + rng.standard_normal((K, V))).astype(np.float32)
    for beta in (2.5, 0.4):
        law_ref = softmax(beta * zt[K].astype(np.float64) / T)
        mid, ln = _midpoints(np.cumsum(law_ref))
        N = len(mid)
        tok = np.tile(rng.integers(0, V, K).astype(np.int32), N)
        r = oracle.smc_step(np.tile(zt, (N, 1)), np.tile(zd, (N, 1)), tok, mid.astype(np.float32), [0.5],
                            np.zeros(N, np.float32), T, 0.0, 1, N, K, lib=lib, beta=beta)
        law = np.zeros(V)
        for t, w in zip(r["bonus"], ln):
            law[t] += w
        assert np.abs(law - law_ref).max() < 1e-9, (beta, law, law_ref)


def _power_paths(rng, V, K, T, spread=2.5):
    """Rows of a K-token draft whose later rows depend on the tokens drafted
    before them: target row j and draft row j of path (x_0 .. x_{j-1}), and
    the bonus row K of each full path (indexed by the path's base-V number)."""
    tgt = [(spread * rng.standard_normal((V ** j, V))).astype(np.float32) for j in range(K + 1)]
    drf = [(tgt[j] + 1.0 * rng.standard_normal((V ** j, V))).astype(np.float32) for j in range(K)]
    return tgt, drf


def _path_index(path, V):
    h = 0
    for x in path:
        h = h * V + int(x)
    return h


def check_power_weighted_law(lib):
    """Power target p^beta: the weights make the proposal exact.

    The target of one step's K+1 tokens is gamma(x) = prod_j p_j(x_j)^beta
    (unnormalised), p_j the target's conditional at row j, which depends on
    the tokens before it.  For importance weights of a proposal r, r(x) w(x) =
    gamma(x) up to one constant per step; with log-weights starting at 0 that
    constant is 1.  The oracle's decisions are integrated exactly: every draft
    path x_0..x_{K-1} (probability prod_j q_j(x_j), scipy), and for the
    (K+1)-th token every interval of its uniform (midpoints; the token is the
    one the oracle draws, the interval length its probability).  Summed per
    cell (path, drawn token), r * exp(logw) must equal gamma (scipy softmax)
    to the fp32 rounding of the log-weight.  A dropped or misscaled weight of
    the (K+1)-th token, beta on the wrong side, or a bonus drawn at the wrong
    temperature all break it."""
    rng = np.random.default_rng(55)
    for V, K, T, beta in ((4, 1, 0.9, 2.0), (4, 1, 1.1, 0.5), (3, 2, 1.0, 3.0), (3, 0, 0.8, 2.5)):
        tgt, drf = _power_paths(rng, V, K, T, spread=1.2)
        sm = lambda z, b=1.0: softmax(b * z.astype(np.float64) / T)  # noqa: E731
        cells_zt, cells_zd, cells_tok, cells_u, cells_r, cells_key = [], [], [], [], [], []
        for path in np.ndindex(*([V] * K)):
            r_path = 1.0
            rows_t, rows_d = [], []
            for j in range(K):
                h = _path_index(path[:j], V)
                rows_t.append(tgt[j][h])
                rows_d.append(drf[j][h])
                r_path *= sm(drf[j][h])[path[j]]
            hb = _path_index(path, V)
            rows_t.append(tgt[K][hb])
            mid, ln = _midpoints(np.cumsum(sm(tgt[K][hb], beta)))
            assert len(mid) == V and ln.min() > 1e-5  # every interval holds fp32 uniforms
            for m, w in zip(mid, ln):
                cells_zt.append(np.stack(rows_t))
                cells_zd.append(np.stack(rows_d) if K else np.zeros((0, V), np.float32))
                cells_tok.append(np.asarray(path, np.int32))
                cells_u.append(m)
                cells_r.append(r_path * w)
                cells_key.append(path)
        N = len(cells_u)
        r = oracle.smc_step(np.concatenate(cells_zt), np.concatenate(cells_zd), np.concatenate(cells_tok),
                            np.asarray(cells_u, np.float32), [0.5], np.zeros(N, np.float32), T, 0.0, 1, N, K,
                            lib=lib, beta=beta)
        assert r["resampled"][0] == 0 and r["flags"] == 0, r["flags"]
        got = {}
        for key, y, rr, lw in zip(cells_key, r["bonus"], cells_r, r["logw"]):
            got[key + (int(y),)] = got.get(key + (int(y),), 0.0) + rr * math.exp(float(lw))
        for path in np.ndindex(*([V] * (K + 1))):
            g = 1.0
            for j in range(K + 1):
                g *= sm(tgt[j][_path_index(path[:j], V)])[path[j]] ** beta
            have = got.get(tuple(int(x) for x in path), 0.0)
            assert abs(have - g) <= 1e-6 * g, (V, K, beta, path, have, g)


def check_power_particle_trend(lib, reps=300, Ns=(32, 128, 512, 2048)):
    """Power target: weighted particles approach the normalised target at the
    1/sqrt(N) rate ("Faster LLM Inference via Sequential Monte Carlo", sec. 3:
    the L1 bias falls as O(1/sqrt(N))).  K = 1, V = 4, beta = 2: particle i
    drafts x_0 ~ q_0 (numpy), its bonus row depends on x_0, and the oracle
    draws x_1 and weighs the particle.  The mean L1 distance of the weighted
    (x_0, x_1) histogram to gamma / sum(gamma), gamma = p_0^beta p_1(.|x_0)^beta,
    over `reps` prompts must halve (ratio in [1.6, 2.5]) each time N
    quadruples.  A weight that leaves out the bonus token's Z_beta has a bias
    that does not shrink, and ratios near 1."""
    rng = np.random.default_rng(2605)
    V, K, T, beta = 4, 1, 1.0, 2.0
    tgt, drf = _power_paths(rng, V, K, T, spread=1.0)
    # bonus rows from nearly flat to sharply peaked, so Z_beta(x_0) spans a factor of about 3
    tgt[1] = (tgt[1] * np.array([[0.1], [0.8], [2.5], [4.0]])).astype(np.float32)
    sm = lambda z, b=1.0: softmax(b * z.astype(np.float64) / T)  # noqa: E731
    q0, p0 = sm(drf[0][0]), sm(tgt[0][0])
    gamma = np.array([[p0[a] ** beta * sm(tgt[1][a])[b] ** beta for b in range(V)] for a in range(V)])
    gamma /= gamma.sum()
    means = []
    for N in Ns:
        P = reps
        x0 = rng.choice(V, size=P * N, p=q0).astype(np.int32)
        zt = np.empty((P * N * 2, V), np.float32)
        zt[0::2] = tgt[0][0]
        zt[1::2] = tgt[1][x0]
        r = oracle.smc_step(zt, np.tile(drf[0][0], (P * N, 1)), x0, rng.random(P * N).astype(np.float32),
                            rng.random(P).astype(np.float32), np.zeros(P * N, np.float32), T, 0.0, P, N, K,
                            lib=lib, beta=beta)
        assert r["resampled"].sum() == 0 and r["flags"] == 0
        lw = r["logw"].astype(np.float64).reshape(P, N)
        w = np.exp(lw - lw.max(axis=1, keepdims=True))
        cell = (x0 * V + r["bonus"]).reshape(P, N)
        l1 = [np.abs(np.bincount(cell[i], weights=w[i], minlength=V * V) / w[i].sum() - gamma.ravel()).sum()
              for i in range(P)]
        means.append(float(np.mean(l1)))
    ratios = [a / b for a, b in zip(means, means[1:])]
    assert all(1.6 < t < 2.5 for t in ratios), (means, ratios)


def check_power_one_is_plain(lib):
    """beta = 1 is the plain step, output for output."""
    rng = np.random.default_rng(53)
    P, N, K, V = 2, 8, 2, 300
    zt = (3 * rng.standard_normal((P * N * (K + 1), V))).astype(np.float32)
    zd = (zt.reshape(P * N, K + 1, V)[:, :K] + rng.standard_normal((P * N, K, V))).astype(np.float32)
    zd = zd.reshape(P * N * K, V)
    tok = rng.integers(0, V, P * N * K).astype(np.int32)
    args = (zt, zd, tok, rng.random(P * N).astype(np.float32), rng.random(P).astype(np.float32),
            rng.standard_normal(P * N).astype(np.float32), 0.8, 0.7, P, N, K)
    a = oracle.smc_step(*args, pt_in=np.arange(P * N * 3, dtype=np.int32).reshape(P * N, 3), lib=lib)
    b = oracle.smc_step(*args, pt_in=np.arange(P * N * 3, dtype=np.int32).reshape(P * N, 3), lib=lib, beta=1.0)
    for k in ("logw", "bonus", "ancestors", "ess", "resampled", "pt_out"):
        assert (a[k] == b[k]).all(), k


def _pages_invariants(table, lens, ref, free, fc, S, M):
    """Reference counts equal the entries naming each page; the free stack holds
    exactly the pages nobody names, once each."""
    count = np.zeros(M, np.int64)
    for r in range(table.shape[0]):
        u = (int(lens[r]) + S - 1) // S
        assert u <= table.shape[1]
        assert (table[r, :u] >= 0).all() and (table[r, :u] < M).all(), r
        np.add.at(count, table[r, :u], 1)
    assert (count == ref).all(), np.nonzero(count != ref)[0][:8]
    stack = free[:fc]
    assert len(set(stack.tolist())) == fc, "a page is on the free stack twice"
    assert set(stack.tolist()) == set(np.nonzero(count == 0)[0].tolist()), "leaked or live page on the free stack"


def _read_kv(phys, table, lens, S):
    return [[int(phys[table[r, t // S], t % S]) for t in range(int(lens[r]))] for r in range(table.shape[0])]


def check_pages_content_model(lib):
    """The bookkeeping against what it is for: a physical page pool that the
    copy list and the new-token slots are applied to must read back, through
    each particle's row, exactly the particle's logical token sequence, over
    appends and resamplings (with heavy duplication); reference counts and
    the free stack stay exact."""
    from synth.small import pages_state, sorted_ancestors

    P, N, L, S, M, A = 2, 6, 14, 4, 160, 3
    st = pages_state(61, P, N, L, S, M, max_len=9)
    rng = np.random.default_rng(62)
    R = P * N
    table, lens, ref, free, fc = st["table"], st["len"], st["ref"], st["free_pages"], st["free_count"]
    phys = np.full((M, S), -1, np.int64)
    logical = []
    for r in range(R):
        seq = rng.integers(0, 1000, int(lens[r])).tolist()
        for t, v in enumerate(seq):
            phys[table[r, t // S], t % S] = v
        logical.append(seq)
    n_cow = 0
    for step in range(6):
        out = oracle.pages_append(table, lens, ref, free, fc, S, A, lib=lib)
        assert out["status"] == 0, out["status"]
        for src, dst, n in out["cow"]:
            phys[dst, :n] = phys[src, :n]
        n_cow += len(out["cow"])
        new = rng.integers(1000, 2000, (R, A))
        for r in range(R):
            for t in range(A):
                sl = int(out["slots"][r, t])
                phys[sl // S, sl % S] = new[r, t]
            logical[r] = logical[r] + new[r].tolist()
        table, lens, ref, free, fc = out["table"], out["len"], out["ref"], out["free_pages"], out["free_count"]
        _pages_invariants(table, lens, ref, free, fc, S, M)
        assert _read_kv(phys, table, lens, S) == logical, f"append {step}"
        anc = sorted_ancestors(70 + step, P, N, concentrate=0.5)
        src = (np.arange(R) // N) * N + anc
        table_new = table[src].copy()
        res = oracle.pages_resample(P, N, anc, table, table_new, lens, ref, free, fc, S, lib=lib)
        assert res["status"] == 0
        logical = [list(logical[k]) for k in src]
        table, lens, ref, free, fc = table_new, res["len"], res["ref"], res["free_pages"], res["free_count"]
        _pages_invariants(table, lens, ref, free, fc, S, M)
        assert _read_kv(phys, table, lens, S) == logical, f"resample {step}"
    assert n_cow > 0, "the scenario never shared a partially filled page"


def check_pages_errors(lib):
    """Capacity, an exhausted pool and a broken sharing rule leave the state
    unchanged with their status."""
    from synth.small import pages_state

    st = pages_state(63, 1, 4, 4, 4, 40, max_len=10)
    args = (st["table"], st["len"], st["ref"], st["free_pages"], st["free_count"])
    full = oracle.pages_append(*args, 4, 7, lib=lib)   # 10 + 7 tokens > 4 pages of 4
    assert full["status"] == 1 and (full["table"] == st["table"]).all() and (full["len"] == st["len"]).all()
    dry = oracle.pages_append(st["table"], st["len"], st["ref"], st["free_pages"], 1, 4, 5, lib=lib)
    assert dry["status"] == 2 and (dry["ref"] == st["ref"]).all() and dry["free_count"] == 1
    bad_ref = st["ref"].copy()
    r0 = int(np.argmax(st["len"] % 4 != 0))
    tail = st["table"][r0, (int(st["len"][r0]) + 3) // 4 - 1]
    bad_ref[tail] = 2  # a partially filled page counted twice, named once
    bad = oracle.pages_append(st["table"], st["len"], bad_ref, st["free_pages"], st["free_count"], 4, 2, lib=lib)
    assert bad["status"] == 3 and (bad["table"] == st["table"]).all()
    anc = np.array([0, 1, 4, 3], np.int32)  # 4 is outside the prompt's 0..3
    res = oracle.pages_resample(1, 4, anc, st["table"], st["table"], st["len"], st["ref"], st["free_pages"],
                                st["free_count"], 4, lib=lib)
    assert res["status"] == 3 and (res["ref"] == st["ref"]).all() and res["free_count"] == st["free_count"]


def _interval_margin(cdf, y, u):
    """Distance from u to the nearer edge of [cdf[y-1], cdf[y]) (normalised cdf)."""
    lo = cdf[y - 1] if y > 0 else 0.0
    return min(u - lo, cdf[y] - u)


def check_margins_vs_numpy(lib):
    """The decision margins the GPU comparison uses to excuse boundary cases,
    recomputed here from scipy / numpy: SD accept margins |u_j - min(1, rho_j)|
    for the tested positions and -1 after the first rejection, the final
    draw's distance to its CDF interval edges; SMC bonus margins, the ESS
    margin |ESS - ess_frac N| / N, the systematic margins and the cumulative
    weights the draw used (-1 when a prompt keeps its particles)."""
    rng = np.random.default_rng(59)
    B, K, V, T = 24, 3, 40, 0.9
    zt, zd, tok, u = rand_sd_problem(rng, B, K, V, T, delta=1.5)
    r = oracle.sd_verify(zt, zd, tok, u, T, K=K, lib=lib)
    lp = log_softmax(zt.astype(np.float64) / T, axis=-1)
    lq = log_softmax(zd.astype(np.float64) / T, axis=-1)
    for b in range(B):
        n = int(r["num_accepted"][b])
        for j in range(K):
            got = r["accept_margin"][b * K + j]
            if j <= n and j < K:
                rho = math.exp(lp[b * (K + 1) + j, tok[b * K + j]] - lq[b * K + j, tok[b * K + j]])
                assert abs(got - abs(float(u[b * (K + 1) + j]) - min(1.0, rho))) < 1e-9, (b, j, got)
            else:
                assert got == -1.0, (b, j, got)
        p = np.exp(lp[b * (K + 1) + n])
        w = np.maximum(0.0, p - np.exp(lq[b * K + n])) if n < K else p
        cdf = np.cumsum(w) / w.sum()
        uf = float(u[b * (K + 1) + K])
        assert abs(r["sample_margin"][b] - _interval_margin(cdf, int(r["final_token"][b]), uf)) < 1e-9, b
    P, N, K, V, T = 3, 8, 2, 30, 1.1
    zt = (2 * rng.standard_normal((P * N * (K + 1), V))).astype(np.float32)
    zd = (zt.reshape(P * N, K + 1, V)[:, :K] + rng.standard_normal((P * N, K, V))).astype(np.float32)
    zd = zd.reshape(P * N * K, V)
    tok = rng.integers(0, V, P * N * K).astype(np.int32)
    ub, ur = rng.random(P * N).astype(np.float32), rng.random(P).astype(np.float32)
    lw0 = (1.5 * rng.standard_normal(P * N)).astype(np.float32)
    for ess_frac in (2.0, 0.0):
        r = oracle.smc_step(zt, zd, tok, ub, ur, lw0, T, ess_frac, P, N, K, lib=lib)
        for i in range(P * N):
            cdf = np.cumsum(softmax(zt[i * (K + 1) + K].astype(np.float64) / T))
            assert abs(r["bonus_margin"][i] - _interval_margin(cdf, int(r["bonus"][i]), float(ub[i]))) < 1e-9, i
        lp = log_softmax(zt.astype(np.float64) / T, axis=-1).reshape(P * N, K + 1, V)
        lq = log_softmax(zd.astype(np.float64) / T, axis=-1).reshape(P * N, K, V)
        for p in range(P):
            lw = np.array([np.float32(float(lw0[p * N + n]) + sum(
                lp[p * N + n, j, tok[(p * N + n) * K + j]] - lq[p * N + n, j, tok[(p * N + n) * K + j]]
                for j in range(K))) for n in range(N)], np.float64)
            w = np.exp(lw - lw.max())
            E = w.sum() ** 2 / (w * w).sum()
            assert abs(r["ess_margin"][p] - abs(E - ess_frac * N) / N) < 1e-9, p
            C = np.cumsum(w) / w.sum()
            cw = r["cum_weight"][p * N:(p + 1) * N]
            if ess_frac == 2.0:
                assert np.abs(cw - C).max() < 1e-12, p
                a = r["ancestors"][p * N:(p + 1) * N]
                m = min(min((float(ur[p]) + k) / N - (C[a[k] - 1] if a[k] > 0 else 0.0), C[a[k]] - (float(ur[p]) + k) / N)
                        for k in range(N))
                assert abs(r["resample_margin"][p] - m) < 1e-12, p
            else:
                assert (cw == -1.0).all() and r["resample_margin"][p] == np.inf, p


def check_nonfinite_and_zero_weight_flags(lib):
    """NONFINITE for a NaN or +inf logit and for a row of -inf logits (SD and
    SMC rows), and for a NaN or +inf log-weight; a row with some -inf logits
    (masked tokens) is no error.  Every log-weight -inf: ZERO_WEIGHTS, ESS 0,
    no resampling, identity ancestors, log-weights carried over."""
    ninf = -np.inf
    t = np.array([[0.5, 1.0, -0.5], [0.1, 0.2, 0.3]], np.float32)
    d = np.array([[0.4, 1.1, -0.2]], np.float32)
    assert oracle.sd_verify(t, d, [1], [0.3, 0.6], 1.0, K=1, lib=lib)["flags"] == 0
    for bad in (np.nan, np.inf):
        for which in ("t", "d"):
            tt, dd = t.copy(), d.copy()
            (tt if which == "t" else dd)[0, 2] = bad
            assert oracle.sd_verify(tt, dd, [1], [0.3, 0.6], 1.0, K=1, lib=lib)["flags"] & oracle.FLAG_NONFINITE, (bad,
                                                                                                                     which)
    masked = t.copy()
    masked[0, 2] = ninf
    assert oracle.sd_verify(masked, d, [1], [0.3, 0.6], 1.0, K=1, lib=lib)["flags"] == 0
    dead = d.copy()
    dead[0, :] = ninf
    assert oracle.sd_verify(t, dead, [1], [0.3, 0.6], 1.0, K=1, lib=lib)["flags"] & oracle.FLAG_NONFINITE
    N, V = 4, 3
    zt = np.tile(t[:1], (N * 2, 1))
    zd = np.tile(d, (N, 1))
    args = (zt, zd, np.ones(N, np.int32), np.full(N, 0.5, np.float32), [0.3])
    assert oracle.smc_step(*args, np.zeros(N, np.float32), 1.0, 0.5, 1, N, 1, lib=lib)["flags"] == 0
    for bad in (np.nan, np.inf):
        lw = np.zeros(N, np.float32)
        lw[2] = bad
        assert oracle.smc_step(*args, lw, 1.0, 0.5, 1, N, 1, lib=lib)["flags"] & oracle.FLAG_NONFINITE, bad
    zb = zt.copy()
    zb[1, 0] = np.nan  # a bonus row (row K = 1 of particle 0)
    assert oracle.smc_step(zb, *args[1:], np.zeros(N, np.float32), 1.0, 0.5, 1, N, 1, lib=lib)["flags"] & 1
    r = _smc_from_logw(lib, np.full(5, ninf), 0.4, ess_frac=2.0)
    assert r["flags"] & oracle.FLAG_ZERO_WEIGHTS and r["ess"][0] == 0.0 and r["resampled"][0] == 0, r
    assert r["ancestors"].tolist() == list(range(5)) and np.isneginf(r["logw"]).all(), r


def _pages_used_entries(table, lens, S):
    return [int(table[r, j]) for r in range(table.shape[0]) for j in range((int(lens[r]) + S - 1) // S)]


def check_pages_exact_capacity(lib):
    """An append that needs exactly the free pages succeeds and empties the
    stack; one page short it fails (status 2) and changes nothing.  A shared
    partially filled tail costs a copy (the highest-index sharer keeps the
    page); a tail named by one row costs none."""
    S, L, M = 4, 4, 8
    # rows 0 and 1 share page 5 as their tail (2 tokens), pages 0, 1, 3 free
    table = np.full((2, L), -1, np.int32)
    table[:, 0] = 5
    lens = np.array([2, 2], np.int32)
    ref = np.zeros(M, np.int32)
    ref[5] = 2
    free = np.array([0, 1, 3, 0, 0, 0, 0, 0], np.int32)
    # 6 more tokens: each row reaches a second page, row 0 also copies its tail
    ok = oracle.pages_append(table, lens, ref, free, 3, S, 6, lib=lib)
    assert ok["status"] == 0 and ok["free_count"] == 0, ok
    assert ok["cow"].tolist() == [[5, 3, 2]] and ok["table"][1, 0] == 5 and ok["table"][0, 0] == 3, ok
    assert ok["ref"][5] == 1 and sorted(_pages_used_entries(ok["table"], ok["len"], S)) == [0, 1, 3, 5]
    short = oracle.pages_append(table, lens, ref, free, 2, S, 6, lib=lib)
    assert short["status"] == 2 and (short["table"] == table).all() and (short["ref"] == ref).all(), short
    assert short["free_count"] == 2 and (short["len"] == lens).all()
    # a tail named once (page 2, 2 tokens) and a full page (page 4): one token
    # each needs one new page (row 1's), no copy
    table = np.array([[2, -1, -1, -1], [4, -1, -1, -1]], np.int32)
    lens = np.array([2, 4], np.int32)
    ref = np.zeros(M, np.int32)
    ref[2] = ref[4] = 1
    one = oracle.pages_append(table, lens, ref, np.array([6] + [0] * 7, np.int32), 1, S, 1, lib=lib)
    assert one["status"] == 0 and one["free_count"] == 0 and one["cow"].size == 0, one
    assert one["table"].tolist() == [[2, -1, -1, -1], [4, 6, -1, -1]] and one["slots"].tolist() == [[10], [24]], one


def check_pages_invalid_states(lib):
    """States the bookkeeping cannot take change nothing and return status 3:
    for an append, a negative length, a length past L pages, a tail page id
    outside the pool (-1 or M); for a resampling, an ancestor outside 0..N-1,
    a length outside 0..L*S, a page id outside the pool in a used entry of an
    old or a gathered row."""
    S, L, M = 4, 2, 6
    table = np.array([[1, -1], [2, 3]], np.int32)
    lens = np.array([3, 6], np.int32)
    ref = np.array([0, 1, 1, 1, 0, 0], np.int32)
    free = np.array([0, 4, 5, 0, 0, 0], np.int32)
    assert oracle.pages_append(table, lens, ref, free, 3, S, 1, lib=lib)["status"] == 0
    cases = []
    for r, v in ((0, -1), (1, 9)):
        ll = lens.copy()
        ll[r] = v
        cases.append((table, ll, ref))
    for pg in (-1, M):
        tt = table.copy()
        tt[0, 0] = pg
        cases.append((tt, lens, ref))
    for tt, ll, rr in cases:
        res = oracle.pages_append(tt, ll, rr, free, 3, S, 1, lib=lib)
        assert res["status"] == 3 and (res["table"] == tt).all() and (res["len"] == ll).all(), (tt, ll, res)
        assert (res["ref"] == rr).all() and res["free_count"] == 3
    N = 2
    good = oracle.pages_resample(1, N, [1, 1], table, table[[1, 1]], lens, ref, free, 3, S, lib=lib)
    assert good["status"] == 0 and good["len"].tolist() == [6, 6], good
    bad = [([-1, 1], table, table[[1, 1]], lens), ([1, 2], table, table[[1, 1]], lens),
           ([1, 1], table, table[[1, 1]], np.array([-2, 6], np.int32)),
           ([1, 1], table, table[[1, 1]], np.array([3, 9], np.int32))]
    for pg in (-1, M):
        tn = table[[1, 1]].copy()
        tn[0, 1] = pg
        bad.append(([1, 1], table, tn, lens))
        to = table.copy()
        to[1, 1] = pg
        bad.append(([0, 0], to, to[[0, 0]], lens))
    for anc, told, tnew, ll in bad:
        res = oracle.pages_resample(1, N, np.array(anc, np.int32), told, tnew, ll, ref, free, 3, S, lib=lib)
        assert res["status"] == 3 and (res["ref"] == ref).all() and res["free_count"] == 3, (anc, told, tnew, ll)


def check_pages_empty_rows_and_page_zero(lib):
    """Length 0 is a valid row (no used entry, no tail) for an append and for
    a resampling; page 0 is a page of the pool like any other, also as a
    shared tail."""
    S, L, M = 4, 2, 6
    table = np.array([[0, -1], [-1, -1], [0, -1]], np.int32)
    lens = np.array([1, 0, 1], np.int32)
    ref = np.array([2, 0, 0, 0, 0, 0], np.int32)
    free = np.array([5, 4, 3, 2, 1, 0], np.int32)
    r = oracle.pages_append(table, lens, ref, free, 5, S, 2, lib=lib)
    # rows in order pop the stack's top: row 0 copies its shared tail (page 0,
    # 1 token) into page 1; row 1 takes page 2; row 2, the highest-index
    # sharer, keeps page 0
    assert r["status"] == 0 and r["len"].tolist() == [3, 2, 3], r
    assert r["table"][:, 0].tolist() == [1, 2, 0] and r["cow"].tolist() == [[0, 1, 1]], r
    assert r["slots"].tolist() == [[5, 6], [8, 9], [1, 2]] and r["free_count"] == 3, r
    assert r["ref"].tolist() == [1, 1, 1, 0, 0, 0], r
    rs = oracle.pages_resample(1, 3, np.array([1, 1, 0], np.int32), table, table[[1, 1, 0]], lens, ref, free, 5, S,
                               lib=lib)
    # rows 0 and 2 named page 0; only the new row 2 does: count 1, no page freed
    assert rs["status"] == 0 and rs["len"].tolist() == [0, 0, 1] and rs["ref"].tolist() == [1, 0, 0, 0, 0, 0], rs
    assert rs["free_count"] == 5


def check_pages_full_rows(lib):
    """A resampling over rows filled to their last page: every page's count
    equals the used entries naming it in the gathered rows, and the free stack
    gains exactly the pages no gathered row names."""
    S, L, M = 4, 2, 12
    table = np.array([[0, 1], [2, 3], [4, -1], [5, 6]], np.int32)
    lens = np.array([8, 8, 3, 8], np.int32)  # rows 0, 1 and 3 full
    ref = np.zeros(M, np.int32)
    for pg in (0, 1, 2, 3, 4, 5, 6):
        ref[pg] = 1
    free = np.array(list(range(7, 12)) + [0] * 7, np.int32)
    anc = np.array([0, 0, 3, 3], np.int32)
    r = oracle.pages_resample(1, 4, anc, table, table[anc], lens, ref, free, 5, S, lib=lib)
    assert r["status"] == 0 and r["len"].tolist() == [8, 8, 8, 8], r
    want = np.zeros(M, np.int32)
    for pg in _pages_used_entries(table[anc], r["len"], S):
        want[pg] += 1
    assert (r["ref"] == want).all(), (r["ref"], want)
    assert sorted(r["free_pages"][5:r["free_count"]].tolist()) == [2, 3, 4], r


# --------------------------------------------------------------------------
# draft side: token draws from q, PACER lengths
# --------------------------------------------------------------------------


def check_golden_draft_sample(lib):
    g = _load_golden("draft_sample.json")
    z = _logits(np.array(g["weights"])[None, :])
    for case in g["cases"]:
        u = np.array(case["uniforms"], np.float32)
        r = oracle.draft_sample(np.repeat(z, len(u), axis=0), u, case["T"], lib=lib)
        assert r["tokens"].tolist() == case["tokens"], (case, r["tokens"])


def check_draft_sample_vs_numpy(lib):
    """A categorical inverse-CDF draw per row: numpy searchsorted on the
    cumulative softmax (scipy), away from interval edges."""
    rng = np.random.default_rng(71)
    R, V, T = 48, 777, 0.8
    z = (3 * rng.standard_normal((R, V))).astype(np.float32)
    u = rng.random(R).astype(np.float32)
    r = oracle.draft_sample(z, u, T, lib=lib)
    for i in range(R):
        c = np.cumsum(softmax(z[i].astype(np.float64) / T))
        want = int(np.searchsorted(c, float(u[i]) * c[-1], side="right"))
        if np.min(np.abs(c / c[-1] - float(u[i]))) > 1e-12:
            assert r["tokens"][i] == want, (i, r["tokens"][i], want)


def check_draft_sample_law(lib):
    """The draw's law over its uniform is exactly softmax(z / T): each CDF
    interval's midpoint yields that interval's token, masked (-inf) tokens
    never appear, and the rows are drawn independently of one another."""
    rng = np.random.default_rng(73)
    for V, T in ((3, 1.0), (6, 0.6), (9, 2.5)):
        z = (2 * rng.standard_normal(V)).astype(np.float32)
        z[rng.integers(0, V)] = -np.inf
        p = softmax(z.astype(np.float64) / T)
        mid, length = _midpoints(np.cumsum(p))
        r = oracle.draft_sample(np.tile(z, (len(mid), 1)), mid.astype(np.float32), T, lib=lib)
        law = np.zeros(V)
        for t, w in zip(r["tokens"], length):
            law[t] += w
        assert np.abs(law - p).max() < 1e-7, (law, p)
    # rows are independent: row i's token depends on row i and uniform i only
    z = (2 * rng.standard_normal((5, 40))).astype(np.float32)
    u = rng.random(5).astype(np.float32)
    both = oracle.draft_sample(z, u, 1.0, lib=lib)["tokens"]
    alone = [int(oracle.draft_sample(z[i:i + 1], u[i:i + 1], 1.0, lib=lib)["tokens"][0]) for i in range(5)]
    assert both.tolist() == alone, (both, alone)


def check_golden_pacer(lib):
    g = _load_golden("pacer_lengths.json")
    scores = np.array([[float(x) for x in row] for row in g["scores"]], np.float32)
    lengths, offsets = oracle.pacer_lengths(scores, g["block"], g["max_blocks"], g["t0"], g["rho"], lib=lib)
    assert lengths.tolist() == g["expect"]["lengths"], lengths
    assert offsets.tolist() == g["expect"]["offsets"], offsets


def check_pacer_special_cases(lib):
    """A threshold no mean can fall below drafts every block; one no mean can
    reach stops after the first; one block is always the last; offsets are the
    exclusive prefix sums of the lengths."""
    rng = np.random.default_rng(79)
    B, blk, mb = 200, 3, 5
    s = rng.random((B, blk * mb)).astype(np.float32)
    lens, offs = oracle.pacer_lengths(s, blk, mb, 0.0, 1.3, lib=lib)
    assert (lens == blk * mb).all()
    lens, offs = oracle.pacer_lengths(s, blk, mb, 1.0, 1.3, lib=lib)  # scores < 1
    assert (lens == blk).all()
    lens, _ = oracle.pacer_lengths(s[:, :blk], blk, 1, 0.9, 1.3, lib=lib)
    assert (lens == blk).all()
    lens, offs = oracle.pacer_lengths(s, blk, mb, 0.5, 1.1, lib=lib)
    assert offs[0] == 0 and (np.diff(offs) == lens).all() and set(np.unique(lens)) <= {blk * m for m in range(1, 6)}
    # a constant threshold (rho = 1): the number of blocks is the first block
    # whose mean falls below t0, counted directly
    lens, _ = oracle.pacer_lengths(s, blk, mb, 0.45, 1.0, lib=lib)
    means = s.astype(np.float64).reshape(B, mb, blk).sum(axis=2) / blk
    below = means < 0.45
    first = np.where(below.any(axis=1), below.argmax(axis=1) + 1, mb)
    assert (lens == blk * np.minimum(first, mb)).all()


def _irwin_hall_cdf(x, n):
    return sum((-1) ** k * math.comb(n, k) * (x - k) ** n for k in range(int(math.floor(x)) + 1)) / math.factorial(n)


def check_pacer_law(lib):
    """With scores ~ U(0,1) the chance of stopping after block m is the
    Irwin-Hall CDF of n = block scores at n * t0 * rho^(m-1): the length law of
    the rule, against 100k sequences (5-sigma bands; numpy's seeded stream)."""
    rng = np.random.default_rng(83)
    B, blk, mb, t0, rho = 102400, 4, 4, 0.5, 1.1
    s = rng.random((B, blk * mb)).astype(np.float32)
    lens, _ = oracle.pacer_lengths(s, blk, mb, t0, rho, lib=lib)
    stop = [_irwin_hall_cdf(blk * t0 * rho ** m, blk) for m in range(mb - 1)]
    p, go = [], 1.0
    for m in range(mb - 1):
        p.append(go * stop[m])
        go *= 1 - stop[m]
    p.append(go)
    for m in range(mb):
        f = float(np.mean(lens == blk * (m + 1)))
        assert abs(f - p[m]) < 5 * math.sqrt(p[m] * (1 - p[m]) / B), (m, f, p[m])


# --------------------------------------------------------------------------
# tree verification (multi-draft speculative sampling over a token tree)
# --------------------------------------------------------------------------


def _pack_trees(trees):
    """Concatenate per-tree dicts (parent, tokens, target [M, V], draft [D, V],
    uniforms [M]) into the CSR layout of oracle.tree_verify."""
    node_off, draft_off = [0], [0]
    for t in trees:
        node_off.append(node_off[-1] + len(t["parent"]))
        draft_off.append(draft_off[-1] + len(t["draft"]))
    V = trees[0]["target"].shape[-1]
    dt = trees[0]["target"].dtype
    cat = lambda k, w: np.concatenate([np.asarray(t[k]) for t in trees]) if trees else np.zeros((0,) * w)
    draft = np.concatenate([t["draft"] for t in trees]) if draft_off[-1] else np.zeros((0, V), dt)
    return dict(node_off=np.array(node_off, np.int32), draft_off=np.array(draft_off, np.int32),
                parent=cat("parent", 1).astype(np.int32), tokens=cat("tokens", 1).astype(np.int32),
                target=np.concatenate([t["target"] for t in trees]), draft=draft,
                uniforms=cat("uniforms", 1).astype(np.float32))


def _tree_run(lib, packed, T):
    return oracle.tree_verify(packed["target"], packed["draft"], packed["node_off"], packed["draft_off"],
                              packed["parent"], packed["tokens"], packed["uniforms"], T, lib=lib)


def check_golden_tree(lib):
    g = _load_golden("tree_verify.json")
    trees = []
    for case in g["cases"]:
        t = g["trees"][case["tree"]]
        trees.append(dict(parent=t["parent"], tokens=t["tokens"], target=_logits(t["target_probs"]),
                          draft=_logits(t["draft_probs"]), uniforms=case["uniforms"]))
    r = _tree_run(lib, _pack_trees(trees), g["T"])
    got = np.stack([r["num_accepted"], r["last_node"], r["final_token"]], axis=1).tolist()
    assert r["status"] == 0 and got == [c["expect"] for c in g["cases"]], got


def check_tree_chain_is_sd(lib):
    """A chain (every node one child) is plain SD with K_b = M_b - 1: same
    accepted counts and final tokens, bit for bit, for every chain length."""
    rng = np.random.default_rng(41)
    for K, V, T, delta in ((1, 50, 1.0, 1.0), (3, 300, 0.8, 1.5), (6, 97, 1.2, 0.7), (0, 40, 1.0, 1.0)):
        B = 64
        zt, zd, tok, u = rand_sd_problem(rng, B, K, V, T, delta)
        ref = oracle.sd_verify(zt, zd, tok, u, T, K=K, lib=lib)
        trees = []
        for b in range(B):
            ub = u[b * (K + 1):(b + 1) * (K + 1)]
            trees.append(dict(parent=np.arange(-1, K), tokens=np.concatenate([[0], tok[b * K:(b + 1) * K]]),
                              target=zt[b * (K + 1):(b + 1) * (K + 1)], draft=zd[b * K:(b + 1) * K],
                              uniforms=np.concatenate([[ub[K]], ub[:K]])))
        r = _tree_run(lib, _pack_trees(trees), T)
        assert r["status"] == 0
        assert (r["num_accepted"] == ref["num_accepted"]).all(), (K, r["num_accepted"], ref["num_accepted"])
        assert (r["last_node"] == ref["num_accepted"]).all()
        assert (r["final_token"] == ref["final_token"]).all(), (K, r["final_token"], ref["final_token"])


def check_tree_star_exact_law(lib):
    """A root with k children drawn iid from q (k = 2, 3), each child a leaf
    whose row depends only on its token.  Integrating the oracle's decisions
    exactly over the child tokens and all uniforms: the first emitted token
    follows p_root, and after an accepted child with token x the next token
    follows that child's row -- multi-draft speculative sampling is exact
    only with the residual renormalised after every rejection."""
    import itertools

    rng = np.random.default_rng(43)
    for V, k, T, delta in ((3, 2, 1.0, 1.5), (4, 3, 0.8, 1.0), (4, 2, 1.0, 0.3)):
        zt0 = (2 * rng.standard_normal(V)).astype(np.float32)
        zd0 = (zt0 + delta * rng.standard_normal(V)).astype(np.float32)
        child_rows = (2 * rng.standard_normal((V, V))).astype(np.float32)  # row of a child with token x
        p0 = softmax(zt0.astype(np.float64) / T)
        q0 = softmax(zd0.astype(np.float64) / T)
        pc = softmax(child_rows.astype(np.float64) / T, axis=-1)
        # Breakpoints of the uniforms: for child tokens xs, the acceptance
        # thresholds of the children and every CDF edge of every final
        # distribution; between consecutive breakpoints the oracle's decisions
        # are constant, so one midpoint per interval, weighted by its length,
        # integrates them exactly.  (The thresholds are computed here only to
        # place the midpoints; the assertions are the laws below.)
        def chains(xs):
            rr = p0.copy()
            out = []
            for x in xs:
                out.append(min(1.0, rr[x] / q0[x]))
                w = np.maximum(0.0, rr - q0)
                rr = w / w.sum() if w.sum() > 0 else rr
            return out, np.cumsum(rr)
        law0 = np.zeros(V)
        law1 = np.zeros((V, V))
        acc_mass = np.zeros(V)
        for xs in itertools.product(range(V), repeat=k):
            wx = float(np.prod([q0[x] for x in xs]))
            thr, cres = chains(xs)
            grids = []
            for j in range(k):
                e = sorted({0.0, 1.0, thr[j]})
                grids.append([(0.5 * (a + b), b - a) for a, b in zip(e[:-1], e[1:]) if b - a > 1e-12])
            fe = sorted(set(np.concatenate([[0.0], cres, np.cumsum(pc, axis=-1).ravel(), [1.0]]).tolist()))
            fgrid = [(0.5 * (a + b), b - a) for a, b in zip(fe[:-1], fe[1:]) if b - a > 1e-9]
            trees, weights = [], []
            for combo in itertools.product(*grids):
                for uf, lf in fgrid:
                    trees.append(dict(parent=[-1] + [0] * k, tokens=[0] + list(xs),
                                      target=np.concatenate([zt0[None], child_rows[list(xs)]]), draft=zd0[None],
                                      uniforms=[uf] + [c[0] for c in combo]))
                    weights.append(wx * lf * float(np.prod([c[1] for c in combo])))
            res = _tree_run(lib, _pack_trees(trees), T)
            assert res["status"] == 0
            for t, w_, (na, ln, ft) in zip(trees, weights, zip(res["num_accepted"], res["last_node"],
                                                              res["final_token"])):
                if na == 0:
                    law0[ft] += w_
                else:
                    x = t["tokens"][ln]
                    law0[x] += w_
                    law1[x, ft] += w_
                    acc_mass[x] += w_
        assert abs(law0.sum() - 1.0) < 1e-9, law0.sum()
        assert np.abs(law0 - p0).max() < 1e-7, (V, k, law0, p0)
        for x in range(V):
            if acc_mass[x] > 1e-6:
                assert np.abs(law1[x] / acc_mass[x] - pc[x]).max() < 1e-7, (V, k, x, law1[x] / acc_mass[x], pc[x])


def check_tree_accept_tie(lib):
    """r(x)/q(x) = 0.5 exactly for the first child (p = (1/2, 1/2), q = (1, 0))
    and u = 0.5: the strict test rejects it, the residual (0, 1) then accepts
    the second child; just below 0.5 the first child is accepted."""
    target = np.zeros((3, 2), np.float32)
    draft = np.array([[0.0, -np.inf]], np.float32)
    for u1, want in ((0.5, 2), (float(np.nextafter(np.float32(0.5), np.float32(0))), 1)):
        r = _tree_run(lib, _pack_trees([dict(parent=[-1, 0, 0], tokens=[0, 0, 1], target=target, draft=draft,
                                             uniforms=[0.3, u1, 0.9])]), 1.0)
        assert r["last_node"].tolist() == [want], (u1, r)


def check_tree_identical_rows(lib):
    """Draft rows equal to the target rows make every ratio 1: the first child
    is always accepted, so the walk follows first children to a leaf and the
    final token is the inverse-CDF draw from that leaf's row (numpy)."""
    rng = np.random.default_rng(47)
    V, T = 211, 0.9
    trees = []
    for b in range(40):
        M = int(rng.integers(1, 12))
        par = [-1] + [int(rng.integers(0, n)) for n in range(1, M)]
        zt = (3 * rng.standard_normal((M, V))).astype(np.float32)
        internal = sorted({p for p in par[1:]})
        trees.append(dict(parent=par, tokens=[0] + rng.integers(0, V, M - 1).tolist(), target=zt,
                          draft=zt[internal] if internal else np.zeros((0, V), np.float32),
                          uniforms=rng.random(M).astype(np.float32)))
    r = _tree_run(lib, _pack_trees(trees), T)
    assert r["status"] == 0
    for b, t in enumerate(trees):
        u, depth = 0, 0
        while True:
            kids = [c for c in range(len(t["parent"])) if t["parent"][c] == u]
            if not kids:
                break
            u, depth = kids[0], depth + 1
        assert r["last_node"][b] == u and r["num_accepted"][b] == depth, (b, r["last_node"][b], u)
        p = softmax(t["target"][u].astype(np.float64) / T)
        c = np.cumsum(p)
        uf = float(t["uniforms"][0])
        if np.min(np.abs(c / c[-1] - uf)) > 1e-12:
            assert r["final_token"][b] == int(np.searchsorted(c, uf * c[-1], side="right"))


def check_tree_root_only(lib):
    """Trees of one node: the final token is the inverse-CDF draw from the root's
    row (numpy searchsorted), nothing is accepted."""
    rng = np.random.default_rng(53)
    V, T = 333, 1.1
    zt = (3 * rng.standard_normal((30, V))).astype(np.float32)
    u = rng.random(30).astype(np.float32)
    trees = [dict(parent=[-1], tokens=[0], target=zt[i:i + 1], draft=np.zeros((0, V), np.float32), uniforms=[u[i]])
             for i in range(30)]
    r = _tree_run(lib, _pack_trees(trees), T)
    assert (r["num_accepted"] == 0).all() and (r["last_node"] == 0).all()
    for i in range(30):
        c = np.cumsum(softmax(zt[i].astype(np.float64) / T))
        if np.min(np.abs(c / c[-1] - u[i])) > 1e-12:
            assert r["final_token"][i] == int(np.searchsorted(c, u[i] * c[-1], side="right"))


def check_tree_malformed(lib):
    """Parents out of tree order, or a draft-row count that disagrees with the
    nodes that have children, are refused."""
    V = 8
    z = np.zeros((3, V), np.float32)
    for par, nd in (([-1, 1, 0], 1), ([0, 0, 0], 1), ([-1, 0, 0], 2), ([-1, 0, 1], 1)):
        r = _tree_run(lib, _pack_trees([dict(parent=par, tokens=[0, 1, 2], target=z, draft=z[:nd],
                                             uniforms=[0.5, 0.5, 0.5])]), 1.0)
        assert r["status"] == -1, (par, nd)


def _residual_chain(p, q, rejections):
    """numpy: r = p, then `rejections` times r <- max(0, r - q) / Z (r kept when
    Z is 0); returns (r, weights of the final draw after them)."""
    r, w = p.copy(), p.copy()
    for _ in range(rejections):
        w = np.maximum(0.0, r - q)
        if w.sum() > 0:
            r = w / w.sum()
        else:
            w = r.copy()
    return r, w


def check_tree_zero_residual_and_bad_tokens(lib):
    """A rejection whose residual has no mass (the node's draft row equal to
    its target row, accept uniform 1.0) keeps r and raises ZERO_RESIDUAL: the
    next child's ratio is still 1, so it is accepted with u < 1, and when it
    is rejected too the final token is drawn from r = p_root (numpy
    searchsorted).  A child whose token lies outside the vocabulary has ratio
    0 and is rejected even with u = 0; the final token then follows the
    numpy residual chain."""
    rng = np.random.default_rng(61)
    V, T, uf = 9, 1.0, 0.4321
    zr = (2 * rng.standard_normal(V)).astype(np.float32)
    z1, z2 = (2 * rng.standard_normal((2, V))).astype(np.float32)
    zq = (zr + rng.standard_normal(V)).astype(np.float32)
    mk = lambda d, toks, us: dict(parent=[-1, 0, 0], tokens=toks, target=np.stack([zr, z1, z2]),  # noqa: E731
                                  draft=d[None, :], uniforms=[uf] + us)
    trees = [mk(zr, [0, 3, 5], [1.0, 0.3]), mk(zr, [0, 3, 5], [1.0, 1.0]), mk(zq, [0, V, -1], [0.0, 0.0])]
    r = _tree_run(lib, _pack_trees(trees), T)
    assert r["status"] == 0 and r["flags"] & oracle.FLAG_ZERO_RESIDUAL, r
    assert r["num_accepted"].tolist() == [1, 0, 0] and r["last_node"].tolist() == [2, 0, 0], r
    sm = lambda z: softmax(z.astype(np.float64) / T)  # noqa: E731
    p_root, q_root = sm(zr), sm(zq)
    _, w = _residual_chain(p_root, q_root, 2)
    for b, wt in ((0, sm(z2)), (1, p_root), (2, w)):
        c = np.cumsum(wt)
        assert np.min(np.abs(c / c[-1] - uf)) > 1e-9
        assert r["final_token"][b] == int(np.searchsorted(c, uf * c[-1], side="right")), (b, r["final_token"])


def check_tree_margins_vs_numpy(lib):
    """Tree margins against numpy: each tested child's |u - min(1, r(x)/q(x))|
    with r the residual chain at its parent, -1 for untested nodes and the
    root, and the final draw's distance to its CDF interval edges."""
    rng = np.random.default_rng(67)
    V, T = 12, 0.8
    trees = []
    for b in range(30):
        zt = (2 * rng.standard_normal((4, V))).astype(np.float32)
        zd = (zt[:1] + 1.5 * rng.standard_normal((1, V))).astype(np.float32)
        trees.append(dict(parent=[-1, 0, 0, 0], tokens=[0] + rng.integers(0, V, 3).tolist(), target=zt, draft=zd,
                          uniforms=rng.random(4).astype(np.float32)))
    r = _tree_run(lib, _pack_trees(trees), T)
    assert r["status"] == 0
    sm = lambda z: softmax(z.astype(np.float64) / T)  # noqa: E731
    for b, t in enumerate(trees):
        am = r["accept_margin"][4 * b:4 * b + 4]
        p, q = sm(t["target"][0]), sm(t["draft"][0])
        rr, w = p.copy(), p.copy()
        assert am[0] == -1.0
        stop = None
        for c in (1, 2, 3):
            if stop is not None:
                assert am[c] == -1.0, (b, c, am)
                continue
            x, uc = t["tokens"][c], float(t["uniforms"][c])
            ratio = rr[x] / q[x]
            assert abs(am[c] - abs(uc - min(1.0, ratio))) < 1e-9, (b, c, am[c])
            if uc < ratio:
                stop = c
            else:
                rr, w = _residual_chain(rr, q, 1)
        wt = sm(t["target"][stop]) if stop is not None else w
        cdf = np.cumsum(wt) / wt.sum()
        assert r["last_node"][b] == (stop or 0)
        assert abs(r["sample_margin"][b] - _interval_margin(cdf, int(r["final_token"][b]), float(t["uniforms"][0]))) \
            < 1e-9, b


def check_tree_malformed_orders(lib):
    """A node that is its own parent, or whose parent comes after it, is
    refused even when the count of nodes with children matches the draft
    rows; and the final-draw CDF refuses a node outside the tree (a tree of
    one node, the root alone, has the root's softmax as its CDF)."""
    V = 8
    z = np.zeros((3, V), np.float32)
    for par, nd in (([-1, 1], 1), ([-1, 2, 0], 2), ([-1, 0, 2], 1)):
        r = _tree_run(lib, _pack_trees([dict(parent=par, tokens=[0] * len(par), target=z[:len(par)], draft=z[:nd],
                                             uniforms=[0.5] * len(par))]), 1.0)
        assert r["status"] == -1, (par, nd)
    one = np.asarray([[0.5, -1.0, 2.0, 0.0, 0.0, 1.0, -2.0, 0.25]], np.float32)
    pk = _pack_trees([dict(parent=[-1], tokens=[0], target=one, draft=z[:0], uniforms=[0.5])])
    cdf, fl = oracle.tree_final_cdf(pk["target"], pk["draft"], pk["node_off"], pk["draft_off"], pk["parent"], 0, 0,
                                    1.0, lib=lib)
    assert fl == 0 and np.allclose(cdf, np.cumsum(softmax(one[0].astype(np.float64))), rtol=0, atol=1e-12), cdf
    pk = _pack_trees([dict(parent=[-1, 0], tokens=[0, 1], target=z[:2], draft=z[:1], uniforms=[0.5, 0.5])])
    for u in (-1, 2):
        _, fl = oracle.tree_final_cdf(pk["target"], pk["draft"], pk["node_off"], pk["draft_off"], pk["parent"], 0, u,
                                      1.0, lib=lib)
        assert fl == -1, u


def check_tree_final_cdf(lib):
    """The CDF the comparison judges a differing final token against: p_u at a
    leaf; after every child of u is rejected, the last max(0, r - q) of the
    chain r <- max(0, r - q) / Z (numpy)."""
    rng = np.random.default_rng(59)
    V, T = 97, 0.8
    par = [-1, 0, 0, 0, 1, 1]
    zt = (2 * rng.standard_normal((6, V))).astype(np.float32)
    zd = (zt[[0, 1]] + rng.standard_normal((2, V))).astype(np.float32)
    pk = _pack_trees([dict(parent=par, tokens=[0, 1, 2, 3, 4, 5], target=zt, draft=zd, uniforms=np.zeros(6))])
    for u, drow, k in ((0, 0, 3), (1, 1, 2), (2, None, 0), (5, None, 0)):
        cdf, fl = oracle.tree_final_cdf(pk["target"], pk["draft"], pk["node_off"], pk["draft_off"], pk["parent"],
                                        0, u, T, lib=lib)
        r = softmax(zt[u].astype(np.float64) / T)
        w = r
        if drow is not None:
            q = softmax(zd[drow].astype(np.float64) / T)
            for _ in range(k):
                w = np.maximum(0.0, r - q)
                r = w / w.sum()
        want = np.cumsum(w) / w.sum()
        assert fl == 0 and np.abs(cdf - want).max() < 1e-12, (u, np.abs(cdf - want).max())


def check_tree_statistics(lib, trials=100_000):
    """Chi-square on a depth-2 tree (root with 2 children, each with 2
    children), children drawn iid from their parent's draft row and every
    row a function of its token path: the first emitted token follows p_root,
    and after an accepted first-level child with token x the second emitted
    token follows that child's row."""
    from scipy.stats import chisquare

    rng = np.random.default_rng(61)
    V, T = 5, 1.0
    root = (1.5 * rng.standard_normal(V)).astype(np.float32)
    lvl1 = (1.5 * rng.standard_normal((V, V))).astype(np.float32)     # row after token x
    lvl2 = (1.5 * rng.standard_normal((V, V, V))).astype(np.float32)  # row after tokens x, y
    droot = (root + rng.standard_normal(V)).astype(np.float32)
    dl1 = (lvl1 + rng.standard_normal((V, V))).astype(np.float32)
    B = trials
    qr = softmax(droot.astype(np.float64) / T)
    x = rng.choice(V, size=(B, 2), p=qr)
    ql1 = softmax(dl1.astype(np.float64) / T, axis=-1)
    u2 = rng.random((B, 2, 2))  # second-level children: inverse CDF of q at their parent
    y = np.empty((B, 2, 2), np.int64)
    for a in range(2):
        c = np.cumsum(ql1[x[:, a]], axis=-1)
        for s2 in range(2):
            y[:, a, s2] = np.minimum((c < u2[:, a, s2:s2 + 1] * c[:, -1:]).sum(-1), V - 1)
    par = np.array([-1, 0, 0, 1, 1, 2, 2], np.int32)
    tok = np.stack([np.zeros(B, np.int64), x[:, 0], x[:, 1], y[:, 0, 0], y[:, 0, 1], y[:, 1, 0], y[:, 1, 1]], 1)
    target = np.stack([np.broadcast_to(root, (B, V)), lvl1[x[:, 0]], lvl1[x[:, 1]], lvl2[x[:, 0], y[:, 0, 0]],
                       lvl2[x[:, 0], y[:, 0, 1]], lvl2[x[:, 1], y[:, 1, 0]], lvl2[x[:, 1], y[:, 1, 1]]], 1)
    draft = np.stack([np.broadcast_to(droot, (B, V)), dl1[x[:, 0]], dl1[x[:, 1]]], 1)
    pk = dict(node_off=np.arange(0, 7 * B + 1, 7, dtype=np.int32), draft_off=np.arange(0, 3 * B + 1, 3, dtype=np.int32),
              parent=np.tile(par, B), tokens=tok.astype(np.int32).ravel(), target=target.reshape(7 * B, V),
              draft=draft.reshape(3 * B, V), uniforms=rng.random(7 * B).astype(np.float32))
    r = _tree_run(lib, pk, T)
    assert r["status"] == 0
    ln, na, ft = r["last_node"], r["num_accepted"], r["final_token"]
    first = np.where(na >= 1, tok[np.arange(B), np.where(ln >= 3, par[ln], ln)], ft)
    pr = softmax(root.astype(np.float64) / T)
    stat = chisquare(np.bincount(first, minlength=V), pr * B)
    assert stat.pvalue > 1e-4, stat
    # the second emitted token after an accepted first-level child with token x0
    reach = na >= 1
    x0 = tok[np.arange(B), np.where(ln >= 3, par[ln], ln)]
    second = np.where(na >= 2, tok[np.arange(B), ln], ft)
    for xv in range(V):
        sel = reach & (x0 == xv)
        if sel.sum() < 2000:
            continue
        pxv = softmax(lvl1[xv].astype(np.float64) / T)
        cnt = np.bincount(second[sel], minlength=V)
        keep = pxv * sel.sum() > 5
        st = chisquare(cnt[keep], pxv[keep] * cnt[keep].sum() / pxv[keep].sum())
        assert st.pvalue > 1e-4, (xv, st)


DETERMINISTIC_CHECKS = [
    check_golden_tree,
    check_tree_chain_is_sd,
    check_tree_star_exact_law,
    check_tree_accept_tie,
    check_tree_identical_rows,
    check_tree_root_only,
    check_tree_malformed,
    check_tree_malformed_orders,
    check_tree_zero_residual_and_bad_tokens,
    check_tree_margins_vs_numpy,
    check_tree_final_cdf,
    check_golden_sd_fixed,
    check_golden_sd_csr,
    check_golden_smc,
    check_constant_row,
    check_two_valued_row,
    check_rows_vs_scipy,
    check_accept_tie_rejects,
    check_cdf_tie,
    check_sd_exact_law,
    check_zero_residual_fallback,
    check_cdf_clamp_last_positive,
    check_bonus_vs_numpy,
    check_residual_vs_numpy,
    check_accept_decisions_vs_scipy,
    check_final_cdf_vs_numpy,
    check_margins_vs_numpy,
    check_nonfinite_and_zero_weight_flags,
    check_ess_closed_forms,
    check_threshold_strict,
    check_systematic_invariants,
    check_systematic_clamp_last_positive,
    check_systematic_fraction_bruteforce,
    check_smc_reweight_vs_scipy,
    check_smc_delta_zero,
    check_smc_bonus_law,
    check_smc_page_table_identity,
    check_power_bonus_law,
    check_power_weighted_law,
    check_power_one_is_plain,
    check_pages_content_model,
    check_pages_errors,
    check_pages_exact_capacity,
    check_pages_invalid_states,
    check_pages_full_rows,
    check_pages_empty_rows_and_page_zero,
    check_golden_draft_sample,
    check_draft_sample_vs_numpy,
    check_draft_sample_law,
    check_golden_pacer,
    check_pacer_special_cases,
    check_pacer_law,
]
