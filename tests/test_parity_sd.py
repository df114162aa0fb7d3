"""sd_verify on the GPU against the oracle (element by element, decision band)."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

from synth.small import sd_case  # noqa: E402


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("V,K,B,T", [
    (1, 2, 3, 1.0), (2, 1, 5, 1.0), (7, 3, 4, 0.7), (9, 2, 6, 1.3), (1000, 4, 8, 1.0), (2048, 1, 3, 0.7),
    (2049, 3, 5, 1.0), (4097, 0, 4, 1.0), (6000, 8, 3, 0.9), (32768, 4, 2, 0.7)])
def test_sd_shapes(dtype, V, K, B, T):
    from gpu_util import check_sd

    for delta in (0.5, 2.0):
        check_sd(sd_case(V * 31 + K * 7 + B, B, V, T=T, K=K, delta=delta, dtype=dtype), f"V={V} K={K} B={B} d={delta}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_sd_ragged(dtype):
    from gpu_util import check_sd

    lengths = [0, 4, 1, 16, 0, 7, 3, 12, 8, 0, 2, 5]
    check_sd(sd_case(5, len(lengths), 3000, T=0.8, lengths=lengths, delta=1.5, dtype=dtype), "ragged")
    check_sd(sd_case(6, 3, 40, T=1.0, lengths=[0, 0, 0], dtype=dtype), "all-zero lengths")


def test_sd_max_vocab_and_max_k():
    """Rows of the largest vocabulary (524288 logits: 256 tiles, so the
    statistics merge takes more than one batch of partials) and the largest
    draft length (K = 128: 257 rows per sequence, several merge passes)."""
    from gpu_util import check_sd

    for dtype in ("bf16", "f32"):
        check_sd(sd_case(4100, 2, 524288, T=1.0, K=2, delta=1.0, dtype=dtype), f"V=524288 {dtype}")
        check_sd(sd_case(4101, 3, 524288, T=0.8, K=1, delta=0.0, dtype=dtype), f"V=524288 accept-all {dtype}")
    check_sd(sd_case(4102, 2, 3000, T=1.0, K=128, delta=0.3, dtype="bf16"), "K=128")
    check_sd(sd_case(4103, 1, 2048, T=1.0, K=128, delta=0.0, dtype="f32"), "K=128 accept-all")


def test_sd_identical_rows_accept_all():
    """draft == target: every draft accepted, final token is the bonus draw."""
    from gpu_util import check_sd, run_sd_gpu

    c = sd_case(9, 16, 5000, T=1.0, K=4, delta=0.0, dtype="bf16")
    na, _, _ = run_sd_gpu(c)
    assert (na == 4).all()
    check_sd(c, "delta=0")


def test_sd_uniform_and_masked_rows():
    from gpu_util import check_sd

    c = sd_case(10, 4, 4096, K=3, delta=1.0, dtype="f32", scale=0.0, prior=False)  # constant rows
    check_sd(c, "constant rows")
    c = sd_case(11, 4, 4096, K=3, delta=1.0, dtype="f32")
    c["target"][:, ::3] = -np.inf  # masked tokens in the target only
    check_sd(c, "masked")


def test_sd_empty_batch():
    import torch

    import smc_resampling_amd as s

    t = torch.empty((0, 100), dtype=torch.float32, device="cuda")
    na, ft, fl = s.sd_verify(t, t, torch.empty(0, dtype=torch.int32, device="cuda"),
                             torch.empty(0, dtype=torch.float32, device="cuda"), 1.0, K=2)
    assert na.numel() == 0 and ft.numel() == 0 and int(fl.item()) == 0


def test_sd_flags_nonfinite_and_bad_input():
    from gpu_util import run_sd_gpu

    c = sd_case(12, 3, 500, K=2, dtype="f32")
    c["target"][1, 7] = np.nan
    _, _, fl = run_sd_gpu(c)
    assert fl & 1
    c = sd_case(13, 3, 500, K=2, dtype="f32")
    c["tokens"][2] = 500
    _, _, fl = run_sd_gpu(c)
    assert fl & 16
    c = sd_case(14, 3, 500, lengths=[1, 2, 1], dtype="f32")
    c["offsets"] = np.array([0, 2, 1, 4], np.int32)  # not monotone
    na, _, fl = run_sd_gpu(c)
    assert fl & 16


def test_sd_deterministic():
    from gpu_util import run_sd_gpu

    c = sd_case(15, 32, 32768, K=4, T=0.7, delta=1.0, dtype="bf16")
    a = run_sd_gpu(c)
    b = run_sd_gpu(c)
    assert (a[0] == b[0]).all() and (a[1] == b[1]).all()


def _config_steps(idx, steps, chunk=16):
    """Full-size steps of a workload, element by element against the oracle
    (the oracle's calls side by side on host threads, `chunk` steps at a time)."""
    from gpu_util import check_sd_many, host_logits, oracle_lengths, say

    import synth
    from compare import Tally

    cfg = synth.CONFIGS[idx]
    gen = synth.Generator(cfg, lengths=oracle_lengths)
    total = Tally()
    steps = list(steps)
    for c0 in range(0, len(steps), chunk):
        cases, labels = [], []
        for s in steps[c0:c0 + chunk]:
            st = gen.sd_step(s)
            cases.append(dict(target=host_logits(st["target"]), draft=host_logits(st["draft"]),
                              tokens=st["tokens"].cpu().numpy(), uniforms=st["uniforms"].cpu().numpy(),
                              offsets=None if st["offsets"] is None else st["offsets"].cpu().numpy(), K=st["K"],
                              T=cfg.T))
            labels.append(f"{cfg.name} step {s}")
        total.merge(check_sd_many(cases, labels))
    say(f"[{cfg.name}] {len(steps)} steps, total {total.summary()}")
    total.assert_ok()


def test_cfg0_all_steps():
    _config_steps(0, range(64))


def test_cfg1_full_size():
    """32 of the 256 steps of the 64-sequence workload."""
    _config_steps(1, range(32))


def test_cfg4_ragged_full_size():
    """16 of the 128 steps of the ragged 256-sequence workload."""
    _config_steps(4, range(16), chunk=8)


def test_sd_side_stream_without_workspace():
    """A call on a stream other than the current one, with no workspace or
    outputs given: the binding allocates and zero-fills them on that stream,
    so the kernels see zeroed counters and flags (the current stream is kept
    busy meanwhile, so an unordered fill would land late)."""
    import torch

    import smc_resampling_amd as s
    from compare import compare_sd
    from gpu_util import DEV, dev_logits, run_sd_oracle

    side = torch.cuda.Stream(device=DEV)
    for i in range(3):
        c = sd_case(300 + i, 48, 20000, T=0.9, K=4, delta=1.0, dtype="bf16")
        args = [dev_logits(c["target"]), dev_logits(c["draft"]), torch.from_numpy(c["tokens"]).to(DEV),
                torch.from_numpy(c["uniforms"]).to(DEV)]
        torch.cuda.synchronize()
        torch.cuda._sleep(20_000_000)  # the current stream is busy
        na, ft, fl = s.sd_verify(*args, c["T"], K=c["K"], stream=side.cuda_stream)
        side.synchronize()
        torch.cuda.synchronize()
        compare_sd(c, run_sd_oracle(c), na.cpu().numpy(), ft.cpu().numpy(), f"side stream {i}").assert_ok()
        assert int(fl.item()) & ~8 == 0


def test_sd_workspace_reuse():
    """One zero-filled workspace across many calls of different shapes: the
    kernel returns its counters to zero after every call."""
    import torch

    import smc_resampling_amd as s
    from compare import compare_sd
    from gpu_util import DEV, dev_logits, run_sd_oracle

    ws = s.new_workspace(s.sd_verify_workspace_bytes(1, 40, 16, 40000, 40 * 16), DEV)
    for i, (B, V, K, lengths) in enumerate([(40, 40000, 4, None), (7, 333, 2, None), (12, 5000, None, [3, 0, 16, 1, 2,
                                            5, 8, 9, 0, 4, 4, 12]), (40, 40000, 16, None), (1, 10, 0, None)]):
        c = sd_case(100 + i, B, V, T=0.9, K=K, lengths=lengths, delta=1.0, dtype="bf16")
        off = None if c["offsets"] is None else torch.from_numpy(c["offsets"]).to(DEV)
        na, ft, fl = s.sd_verify(dev_logits(c["target"]), dev_logits(c["draft"]), torch.from_numpy(c["tokens"]).to(DEV),
                                 torch.from_numpy(c["uniforms"]).to(DEV), c["T"], K=c["K"], draft_offsets=off,
                                 workspace=ws)
        torch.cuda.synchronize()
        t = compare_sd(c, run_sd_oracle(c), na.cpu().numpy(), ft.cpu().numpy(), f"reuse {i}")
        t.assert_ok()
        assert int(fl.item()) & ~8 == 0


def test_sd_zero_residual_fallback():
    """Identical rows and an accept uniform of exactly 1.0 (outside the
    documented range, but defined on both sides): the test rejects, the residual
    mass is exactly 0 (the kernel's row statistics depend on the row's logits
    alone, so identical rows give identical probabilities) and the final token
    is drawn from p_n instead."""
    from gpu_util import check_sd, run_sd_gpu

    c = sd_case(21, 6, 9000, T=1.0, K=3, delta=0.0, dtype="bf16")
    for b in (0, 2, 5):
        c["uniforms"][b * 4 + (b % 3)] = 1.0
    na, _, fl = run_sd_gpu(c)
    assert fl & 2
    assert [int(na[b]) for b in (0, 2, 5)] == [0, 2, 2]
    check_sd(c, "zero residual")


def test_sd_multi_tile_segments_sampled():
    """A batch large enough (2048 sequences, K=8, V=32768: 557056 tiles) that
    every streamed segment spans at least two tiles whatever the occupancy
    (at most 8192 wavefronts, 32 tiles each per segment step), so a bonus draw
    locates its tile through the bonus row's own tile partials.  The batch is
    32 replicas of a 64-sequence case (every other sequence with draft ==
    target, so all of its drafts are accepted) with fresh uniforms; a sample
    of the sequences is checked against the oracle."""
    import torch

    import smc_resampling_amd as s
    from compare import compare_sd
    from gpu_util import DEV, dev_logits, run_sd_oracle, say

    B0, R, K, V, T = 64, 32, 8, 32768, 0.7
    c = sd_case(4242, B0, V, T=T, K=K, delta=np.where(np.arange(B0) % 2 == 0, 0.0, 1.0), dtype="bf16")
    B = B0 * R
    rng = np.random.default_rng(4243)
    u = rng.random(B * (K + 1)).astype(np.float32)
    tgt = dev_logits(c["target"]).repeat(R, 1)
    drf = dev_logits(c["draft"]).repeat(R, 1)
    tok = torch.from_numpy(np.tile(c["tokens"], R)).to(DEV)
    na, ft, fl = s.sd_verify(tgt, drf, tok, torch.from_numpy(u).to(DEV), T, K=K)
    torch.cuda.synchronize()
    na, ft = na.cpu().numpy(), ft.cpu().numpy()
    del tgt, drf
    pick = np.array(sorted(set([0, 1, 62, 63, 64, 1001, B - 2, B - 1]) | set(rng.choice(B, 24, replace=False).tolist())))
    src = pick % B0
    sub = dict(target=np.concatenate([c["target"][b * (K + 1):(b + 1) * (K + 1)] for b in src]),
               draft=np.concatenate([c["draft"][b * K:(b + 1) * K] for b in src]),
               tokens=np.concatenate([c["tokens"][b * K:(b + 1) * K] for b in src]),
               uniforms=np.concatenate([u[b * (K + 1):(b + 1) * (K + 1)] for b in pick]),
               offsets=None, K=K, Kb=np.full(len(pick), K, np.int32), T=T, dtype="bf16")
    ref = run_sd_oracle(sub)
    t = compare_sd(sub, ref, na[pick], ft[pick], "multi-tile segments")
    say(f"[sd multi-tile segments B={B}] {t.summary()} all-accepted={int((na[pick] == K).sum())}/{len(pick)} "
        f"flags gpu={int(fl.item())}")
    t.assert_ok()
    assert (na[pick] == K).sum() >= 4  # the picked even sequences (draft == target) take the bonus draw
    assert int(fl.item()) & ~8 == 0


def test_sd_decisions_do_not_depend_on_segmentation():
    """The same 64 sequences decided in a small call (one-tile segments) and
    as 40 identical replicas in one large call (multi-tile segments, where the
    bonus rows keep tile partials): every replica decides alike, and the two
    calls agree on every decision whose uniform is not within the band of a
    boundary (the row statistics then differ only in rounding)."""
    import torch

    import smc_resampling_amd as s
    from compare import BAND
    from gpu_util import DEV, dev_logits, run_sd_oracle

    B0, R, K, V, T = 64, 40, 4, 32768, 0.7
    c = sd_case(4300, B0, V, T=T, K=K, delta=np.array([(0.5, 1.0, 2.0)[b % 3] for b in range(B0)]), dtype="bf16")
    tok = torch.from_numpy(c["tokens"]).to(DEV)
    u = torch.from_numpy(c["uniforms"]).to(DEV)
    na1, ft1, _ = s.sd_verify(dev_logits(c["target"]), dev_logits(c["draft"]), tok, u, T, K=K)
    naR, ftR, flR = s.sd_verify(dev_logits(c["target"]).repeat(R, 1), dev_logits(c["draft"]).repeat(R, 1),
                                tok.repeat(R), u.repeat(R), T, K=K)
    torch.cuda.synchronize()
    na1, ft1 = na1.cpu().numpy(), ft1.cpu().numpy()
    naR, ftR = naR.cpu().numpy().reshape(R, B0), ftR.cpu().numpy().reshape(R, B0)
    assert (naR == naR[0]).all() and (ftR == ftR[0]).all()  # replicas alike
    ref = run_sd_oracle(c)
    am = ref["accept_margin"].reshape(B0, K)
    near = (np.where(am >= 0, am, np.inf).min(axis=1) < BAND) | (ref["sample_margin"] < BAND)
    differ = (naR[0] != na1) | (ftR[0] != ft1)
    assert not (differ & ~near).any(), np.nonzero(differ & ~near)
    assert int(flR.item()) & ~8 == 0


def _concat_sd_cases(a, b):
    """One call's inputs holding the sequences of case a, then those of b
    (fixed K in both, or CSR offsets in both)."""
    out = dict(T=a["T"], dtype=a["dtype"], K=max(a["K"], b["K"]))
    for k in ("target", "draft", "tokens", "uniforms"):
        out[k] = np.concatenate([a[k], b[k]])
    if a.get("offsets") is not None:
        out["offsets"] = np.concatenate([a["offsets"], b["offsets"][1:] + a["offsets"][-1]]).astype(np.int32)
    return out


@pytest.mark.parametrize("B,V,K,dtype,ragged", [(64, 32768, 4, "bf16", False), (1, 32000, 2, "f32", False),
                                                (13, 2049, 3, "bf16", False), (100, 6000, 5, "f32", False),
                                                (40, 20000, 6, "bf16", True), (8, 151936, 8, "bf16", True)])
def test_sd_split_members_match_one_workgroup(B, V, K, dtype, ragged):
    """Calls of few sequences share each sequence's residual pass among
    several workgroups (4 up to 64 sequences, 2 up to 128, fewer when a row
    has fewer tiles); the same sequences in a call of 300 run on one
    workgroup each.  Both must decide bit for bit alike, and match the
    oracle."""
    from gpu_util import check_sd, run_sd_gpu
    from synth.small import sd_case

    rng = np.random.default_rng(B * 11 + V)
    delta = np.array([(0.5, 1.0, 2.0)[b % 3] for b in range(B)])
    if ragged:
        lens = rng.integers(0, K + 1, B)
        small = sd_case(B * 17 + 1, B, V, T=0.9, lengths=lens, delta=delta, dtype=dtype)
        pad = sd_case(B * 17 + 2, 300 - B, V, T=0.9, lengths=np.zeros(300 - B, np.int32), dtype=dtype)
    else:
        small = sd_case(B * 17 + 1, B, V, T=0.9, K=K, delta=delta, dtype=dtype)
        pad = sd_case(B * 17 + 2, 300 - B, V, T=0.9, K=K, dtype=dtype)
    check_sd(small, f"split call B={B} V={V} K={K} {dtype} ragged={ragged}")
    big = _concat_sd_cases(small, pad)
    na_s, ft_s, fl_s = run_sd_gpu(small)
    na_b, ft_b, fl_b = run_sd_gpu(big)
    assert np.array_equal(na_s, na_b[:B]) and np.array_equal(ft_s, ft_b[:B])
    assert (fl_s & 128) == 0 and (fl_b & 128) == 0
