"""The draft-side step on the GPU against the oracle: token draws from the
draft distribution (bit for bit outside the CDF decision band) and PACER draft
lengths with their CSR offsets (bit for bit)."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu


def _bf16_bits(x):
    """Round float32 to bfloat16 (nearest even) and return the 16-bit patterns."""
    b = np.ascontiguousarray(x, np.float32).view(np.uint32).astype(np.uint64)
    r = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)
    return r


def _sample(z, u, T, label, rows=None):
    """GPU draws for every row; the oracle's for `rows` (all by default)."""
    import torch

    import oracle
    import smc_resampling_amd as s
    from compare import compare_draft
    from gpu_util import DEV, dev_logits, say

    zd = z if isinstance(z, torch.Tensor) else dev_logits(z)
    out = s.draft_sample(zd, torch.from_numpy(np.ascontiguousarray(u, np.float32)).to(DEV), T)
    torch.cuda.synchronize()
    tok, fl = out["tokens"].cpu().numpy(), int(out["status_flags"].item())
    idx = np.arange(len(u)) if rows is None else np.asarray(rows)
    zh = z[idx] if not isinstance(z, torch.Tensor) else _host(z, idx)
    ref = oracle.draft_sample(zh, np.asarray(u, np.float32)[idx], T)
    t = compare_draft(zh, np.asarray(u, np.float32)[idx], T, ref, tok[idx], label)
    say(f"[draft {label}] {t.summary()} flags gpu={fl} oracle={ref['flags']}")
    t.assert_ok()
    if rows is None:
        assert (fl & ~8) == (ref["flags"] & ~8), (fl, ref["flags"])
    return tok, fl


def _host(t, idx):
    from gpu_util import host_logits

    return np.ascontiguousarray(np.stack([host_logits(t[int(i)]) for i in idx]))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_draft_sample_shapes(dtype):
    """Rows from one logit up to several tiles with ragged tails, three temperatures."""
    rng = np.random.default_rng(101)
    for R, V, T in ((1, 1, 1.0), (5, 7, 0.7), (33, 2047, 1.3), (64, 2048, 1.0), (17, 2049, 0.7), (40, 6000, 1.0),
                    (300, 4096, 0.9), (8, 32768 + 8, 1.1)):
        z = (3 * rng.standard_normal((R, V))).astype(np.float32)
        if dtype == "bf16":
            z = _bf16_bits(z)
        u = rng.random(R).astype(np.float32)
        _sample(z, u, T, f"{dtype} R={R} V={V} T={T}")


def test_draft_sample_masks_and_flags():
    rng = np.random.default_rng(103)
    R, V = 12, 3000
    z = (2 * rng.standard_normal((R, V))).astype(np.float32)
    z[0, :] = -np.inf
    z[0, 1234] = 0.5           # one finite token: always drawn
    z[1, ::2] = -np.inf        # half the vocabulary masked
    z[2, :] = 7.0              # constant row: token floor(u V)
    u = rng.random(R).astype(np.float32)
    tok, _ = _sample(z, u, 1.0, "masked rows")
    assert tok[0] == 1234 and tok[1] % 2 == 1
    z[3, 17] = np.nan          # a row that is not a distribution
    import torch

    import smc_resampling_amd as s
    from gpu_util import DEV, dev_logits

    out = s.draft_sample(dev_logits(z), torch.from_numpy(u).to(DEV), 1.0)
    torch.cuda.synchronize()
    assert int(out["status_flags"].item()) & s.FLAG_NONFINITE


def test_draft_sample_is_the_verify_draw():
    """A draw is sd_verify's final draw with no draft tokens, bit for bit."""
    import torch

    import smc_resampling_amd as s
    from gpu_util import DEV, dev_logits

    rng = np.random.default_rng(107)
    R, V = 96, 12345
    z = dev_logits(_bf16_bits((3 * rng.standard_normal((R, V))).astype(np.float32)))
    u = torch.from_numpy(rng.random(R).astype(np.float32)).to(DEV)
    a = s.draft_sample(z, u, 0.8)["tokens"]
    _, ft, _ = s.sd_verify(z, None, None, u, 0.8, K=0)
    torch.cuda.synchronize()
    assert torch.equal(a, ft)


def test_draft_sample_workload_shapes():
    """One draft position of the batched SD workload (64 sequences, V=32768,
    T=0.7), every row; and of the 32x64-particle SMC workload (2048 rows,
    V=151936), on 64 sampled rows."""
    import torch

    import synth
    from gpu_util import DEV, host_logits

    cfg = synth.CONFIGS[1]
    bt = synth.Generator(cfg).sd_step(0)
    z = bt["draft"][:cfg.B].contiguous()
    u = np.random.default_rng(109).random(cfg.B).astype(np.float32)
    _sample(host_logits(z), u, cfg.T, "64 x 32768 bf16")
    cfg = synth.CONFIGS[3]
    gen = synth.Generator(cfg)
    bt = gen.smc_step(0)
    R = cfg.P * cfg.N
    z = bt["draft"][:R].contiguous()
    del bt
    torch.cuda.empty_cache()
    u = np.random.default_rng(113).random(R).astype(np.float32)
    rows = np.sort(np.random.default_rng(127).choice(R, 64, replace=False))
    _sample(z, u, cfg.T, "2048 x 151936 bf16 (sampled rows)", rows=rows)


def _pacer(scores, block, max_blocks, t0, rho, label):
    import torch

    import oracle
    import smc_resampling_amd as s
    from gpu_util import DEV, say

    g = s.pacer_lengths(torch.from_numpy(np.ascontiguousarray(scores, np.float32)).to(DEV), block, max_blocks, t0,
                        rho)
    torch.cuda.synchronize()
    lo, oo = oracle.pacer_lengths(scores, block, max_blocks, t0, rho)
    assert np.array_equal(g["lengths"].cpu().numpy(), lo), label
    assert np.array_equal(g["offsets"].cpu().numpy(), oo), label
    say(f"[pacer {label}] B={len(lo)} lengths equal, total {int(oo[-1])}")
    return lo


def test_pacer_lengths_cases():
    rng = np.random.default_rng(131)
    _pacer(np.zeros((0, 16), np.float32), 4, 4, 0.5, 1.1, "no sequences")
    for B, blk, mb, t0, rho in ((1, 4, 4, 0.5, 1.1), (256, 4, 4, 0.5, 1.1), (3000, 3, 6, 0.45, 1.05),
                                (1500, 1, 9, 0.5, 0.9), (700, 8, 1, 0.5, 1.1), (2049, 5, 3, 0.0, 2.0),
                                (64, 2, 2, 2.0, 1.0)):
        _pacer(rng.random((B, blk * mb)).astype(np.float32), blk, mb, t0, rho, f"B={B} b={blk} m={mb} t0={t0} rho={rho}")
    # exact ties with the threshold (means of multiples of 1/8), and NaN scores
    s = (rng.integers(0, 9, (512, 16)) / 8).astype(np.float32)
    _pacer(s, 4, 4, 0.5, 1.25, "ties at the threshold")
    s = rng.random((512, 16)).astype(np.float32)
    s[rng.random((512, 16)) < 0.05] = np.nan
    _pacer(s, 4, 4, 0.5, 1.1, "NaN scores")


def test_pacer_lengths_ragged_workload():
    """The ragged SD workload's 128 steps of pre-verifier scores: the library's
    lengths and offsets equal the oracle's at every step."""
    import synth

    cfg = synth.CONFIGS[4]
    pc = cfg.pacer
    total = 0
    for step in range(cfg.steps):
        sc = synth.pacer_scores(cfg.B, cfg.seed, step, pc["block"], pc["max_blocks"])
        total += int(_pacer(sc, pc["block"], pc["max_blocks"], pc["t0"], pc["rho"], f"step {step}").sum())
    assert total > 0
