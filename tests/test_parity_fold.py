"""Rows that leave the streaming fold's common path, against the oracle.

The streaming kernel folds a tile at the lane's current offset and keeps the
fold while every term stays below 2^64; a value far above the offset, a NaN
or +inf, or a first chunk of -inf sends the tile to a second fold at the
running maximum.  These rows are built to take each branch, in one-tile
segments (a small call) and in multi-tile segments (the same sequences
replicated into a large call), and the decisions and log-weights must match
the oracle as everywhere else."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

from synth.small import gumbel_tokens, sd_case, smc_case, stored  # noqa: E402

PATTERNS = ("spike", "ramp", "steps", "masked_prefix", "deep_prefix", "high_level", "plain")


def _shape(z, pattern, rng):
    """Apply `pattern` to a float32 logit row in place (a view of the case's rows)."""
    V = z.shape[-1]
    if pattern == "spike":  # one logit 55 above the rest in a middle tile: 79 in the log2 domain at T = 1
        z[..., min(V - 1, 9 * 2048 + 777)] += 55.0
    elif pattern == "ramp":  # rising by 40 per 2048-logit tile: terms up to about 2^50 inside a
        # tile, and past the 2^64 ceiling one tile into a longer segment
        z += (np.arange(V, dtype=np.float32) * np.float32(40.0 / 2048))
    elif pattern == "steps":  # +70 from logit 1024 on (past a lane's first chunk, inside the
        # first tile) and +70 more from tile 5 on (inside a segment of 2 to 4 tiles)
        z[..., 1024:] += 70.0
        z[..., 5 * 2048:] += 70.0
    elif pattern == "masked_prefix":  # the first 3000 logits masked
        z[..., :min(V, 3000)] = -np.inf
    elif pattern == "deep_prefix":  # the first 600 logits far below the rest
        z[..., :min(V, 600)] = -1.0e4
    elif pattern == "high_level":  # every logit near 1e4
        z += 1.0e4
    return z


def _sd_patterned(seed, B, V, K, T, dtype):
    """An SD case whose sequence b carries PATTERNS[b % len] on its target rows
    and (with its own noise) on its draft rows; tokens redrawn from the
    patterned drafts."""
    c = sd_case(seed, B, V, T=T, K=K, delta=0.7, dtype="f32")
    rng = np.random.default_rng(seed + 1)
    zt = c["target"].reshape(B, K + 1, V).copy()
    zd = c["draft"].reshape(B, K, V).copy()
    for b in range(B):
        p = PATTERNS[b % len(PATTERNS)]
        _shape(zt[b], p, rng)
        _shape(zd[b], p, rng)
    zt, zd = zt.reshape(B * (K + 1), V), zd.reshape(B * K, V)
    c["target"], _ = stored(zt, dtype)
    c["draft"], d64 = stored(zd, dtype)
    c["tokens"] = gumbel_tokens(rng, d64, T)
    c["dtype"] = dtype
    return c


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_fold_branches_one_tile_segments(dtype):
    from gpu_util import check_sd

    for T in (1.0, 0.6):
        c = _sd_patterned(7100 + int(T * 10), 2 * len(PATTERNS), 32768, 3, T, dtype)
        check_sd(c, f"fold branches {dtype} T={T}")


def test_fold_branches_multi_tile_segments():
    """The patterned sequences replicated into a call of 148 x 14 sequences
    (K=8, V=32768 bf16: 563584 tiles; at most 8192 wavefronts take 32 units
    each, so every segment spans two tiles or more), fresh uniforms per
    replica; a sample of them against the oracle."""
    import torch

    import smc_resampling_amd as s
    from compare import compare_sd
    from gpu_util import DEV, dev_logits, run_sd_oracle, say

    B0, R, K, V, T = 2 * len(PATTERNS), 148, 8, 32768, 1.0
    c = _sd_patterned(7200, B0, V, K, T, "bf16")
    B = B0 * R
    rng = np.random.default_rng(7201)
    u = rng.random(B * (K + 1)).astype(np.float32)
    tgt = dev_logits(c["target"]).repeat(R, 1)
    drf = dev_logits(c["draft"]).repeat(R, 1)
    tok = torch.from_numpy(np.tile(c["tokens"], R)).to(DEV)
    assert (tgt.shape[0] + drf.shape[0]) * (V // 2048) >= 64 * 8192
    na, ft, fl = s.sd_verify(tgt, drf, tok, torch.from_numpy(u).to(DEV), T, K=K)
    torch.cuda.synchronize()
    na, ft = na.cpu().numpy(), ft.cpu().numpy()
    del tgt, drf
    pick = np.array(sorted(set(range(B0)) | set(range(B - B0, B)) | set(rng.choice(B, 36, replace=False).tolist())))
    src = pick % B0
    sub = dict(target=np.concatenate([c["target"][b * (K + 1):(b + 1) * (K + 1)] for b in src]),
               draft=np.concatenate([c["draft"][b * K:(b + 1) * K] for b in src]),
               tokens=np.concatenate([c["tokens"][b * K:(b + 1) * K] for b in src]),
               uniforms=np.concatenate([u[b * (K + 1):(b + 1) * (K + 1)] for b in pick]),
               offsets=None, K=K, Kb=np.full(len(pick), K, np.int32), T=T, dtype="bf16")
    ref = run_sd_oracle(sub)
    t = compare_sd(sub, ref, na[pick], ft[pick], "fold branches, multi-tile segments")
    say(f"[sd fold branches multi-tile B={B}] {t.summary()} flags gpu={int(fl.item())} oracle={ref['flags']}")
    t.assert_ok()
    assert (int(fl.item()) & ~8) == (ref["flags"] & ~8)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_fold_branches_smc(dtype):
    """SMC steps (log-weights and ESS in lockstep) on particles whose rows
    carry the patterns, one pattern per particle."""
    from gpu_util import check_smc_steps

    P, N, K, V = 2, len(PATTERNS), 3, 20000
    c = smc_case(7300, P, N, K, V, dtype="f32", L=3, logw_scale=1.0)  # f32 rows, patterned below
    rng = np.random.default_rng(7301)
    zt = c["target"].reshape(P * N, K + 1, V).copy()
    zd = c["draft"].reshape(P * N, K, V).copy()
    for i in range(P * N):
        p = PATTERNS[i % N]
        _shape(zt[i], p, rng)
        _shape(zd[i], p, rng)
    c["target"], _ = stored(zt.reshape(-1, V), dtype)
    c["draft"], d64 = stored(zd.reshape(-1, V), dtype)
    c["tokens"] = gumbel_tokens(rng, d64, c["T"])
    c["dtype"] = dtype
    check_smc_steps(c, steps=1, label=f"fold branches {dtype}")
    check_smc_steps(c, steps=1, ess_frac=2.0, label=f"fold branches {dtype}, always resample")
