"""smc_reweight_resample on the GPU against the oracle, in lockstep."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

from synth.small import smc_case  # noqa: E402


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("P,N,K,V,T,L", [
    (1, 1, 2, 50, 1.0, 3), (2, 4, 1, 7, 1.0, 2), (1, 16, 4, 4096, 1.0, 8), (3, 64, 2, 2049, 0.8, 5),
    (2, 5, 0, 1000, 1.0, 4), (1, 100, 3, 300, 1.2, 0)])
def test_smc_shapes(dtype, P, N, K, V, T, L):
    from gpu_util import check_smc_steps

    c = smc_case(P * 1000 + N * 10 + K, P, N, K, V, T=T, dtype=dtype, L=L, logw_scale=2.0)
    if L == 0:
        c["pt"] = None
    check_smc_steps(c, steps=1, label=f"P={P} N={N} K={K} V={V}")
    check_smc_steps(c, steps=1, ess_frac=2.0, label="always resample")
    check_smc_steps(c, steps=1, ess_frac=0.0, label="never resample")


def test_smc_max_particles():
    from gpu_util import check_smc_steps

    c = smc_case(77, 1, 1024, 1, 64, dtype="bf16", L=2, logw_scale=3.0)
    check_smc_steps(c, steps=1, ess_frac=2.0, label="N=1024")


def test_smc_max_vocab_and_max_k():
    """SMC rows of 524288 logits (256 tiles: four batches of partials in the
    256-thread merge) and K = 128 draft rows per particle."""
    from gpu_util import check_smc_steps

    for dtype in ("bf16", "f32"):
        c = smc_case(4200, 1, 3, 2, 524288, dtype=dtype, L=2, logw_scale=1.0)
        check_smc_steps(c, steps=1, ess_frac=2.0, label=f"V=524288 {dtype}")
    c = smc_case(4201, 1, 2, 128, 1500, dtype="bf16", L=2, logw_scale=1.0)
    check_smc_steps(c, steps=1, ess_frac=2.0, label="K=128")


def test_smc_dominant_particle():
    """One particle holds all the weight (first, middle or last of its prompt):
    every slot descends from it, the other particles' slot ranges are empty."""
    from gpu_util import check_smc_steps, run_smc_gpu

    c = smc_case(90, 3, 64, 2, 500, dtype="bf16", L=3)
    lw = np.zeros(3 * 64, np.float32)
    lw[0], lw[64 + 37], lw[2 * 64 + 63] = 90.0, 90.0, 90.0
    c["logw"] = lw
    g = run_smc_gpu(c, lw, c["pt"])
    assert (g["resampled"] == 1).all()
    anc = g["ancestors"].reshape(3, 64)
    assert (anc[0] == 0).all() and (anc[1] == 37).all() and (anc[2] == 63).all()
    check_smc_steps(c, steps=1, label="dominant particle")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("beta", [0.5, 2.0, 4.0])
def test_smc_power_target(dtype, beta):
    """Power-sampling target p^beta against the oracle: increments
    beta log p - log q, bonus from softmax(beta z / T)."""
    from gpu_util import check_smc_steps

    for P, N, K, V, T, L in ((2, 16, 3, 3000, 1.0, 4), (1, 64, 2, 2049, 0.8, 3), (3, 5, 0, 700, 1.1, 2)):
        c = smc_case(int(beta * 10) + P * 100 + K, P, N, K, V, T=T, dtype=dtype, L=L, logw_scale=1.0)
        c["beta"] = beta
        check_smc_steps(c, steps=1, label=f"power beta={beta} P={P} N={N} K={K} V={V}")
        check_smc_steps(c, steps=1, ess_frac=2.0, label=f"power beta={beta} always resample")


def test_smc_power_one_is_plain():
    """beta = 1 through the power entry point gives the plain step's outputs bit for bit."""
    from gpu_util import run_smc_gpu

    for dtype in ("f32", "bf16"):
        c = smc_case(91, 2, 32, 3, 5000, dtype=dtype, L=3, logw_scale=2.0)
        a = run_smc_gpu(c, c["logw"], c["pt"])
        b = run_smc_gpu(dict(c, beta=1.0), c["logw"], c["pt"])
        for k in ("bonus", "ancestors", "ess", "resampled", "logw", "pt_out", "flags"):
            assert np.array_equal(np.asarray(a[k]), np.asarray(b[k])), k


def test_smc_zero_weights_flag():
    from gpu_util import run_smc_gpu

    c = smc_case(78, 2, 8, 1, 100, dtype="f32", L=2)
    logw = np.full(16, -np.inf, np.float32)
    g = run_smc_gpu(c, logw, c["pt"])
    assert g["flags"] & 4
    assert (g["resampled"] == 0).all() and (g["ess"] == 0).all()
    assert (g["ancestors"] == np.tile(np.arange(8), 2)).all()


def test_smc_multi_step_lockstep():
    from gpu_util import check_smc_steps

    def fresh(s, case):
        n = smc_case(500 + s, case["P"], case["N"], case["K"], 3000, dtype="bf16", L=4)
        return n

    c = smc_case(500, 2, 16, 4, 3000, dtype="bf16", L=4)
    check_smc_steps(c, steps=6, label="6 steps", new_inputs=fresh)


def _cfg_smc(idx, steps, prompts=None, beta=None):
    """Full-size workload in lockstep: every step runs on the GPU for all
    prompts; the oracle checks `prompts` (all when None) from the GPU's state
    before the step (with ``beta``, the power-sampling target).  The oracle's
    per-prompt calls run side by side on host threads."""
    import concurrent.futures as cf

    import torch

    import oracle
    import smc_resampling_amd as s
    import synth
    from compare import Tally, compare_smc
    from gpu_util import host_logits, oracle_threads, say

    cfg = synth.CONFIGS[idx]
    gen = synth.Generator(cfg)
    P, N, K = cfg.P, cfg.N, cfg.K
    prompts = list(range(P)) if prompts is None else prompts
    logw = torch.zeros(P * N, dtype=torch.float32, device="cuda")
    pt = torch.from_numpy(synth.initial_page_table(P, N, cfg.L)).cuda()
    total = Tally()
    with cf.ThreadPoolExecutor(max_workers=oracle_threads()) as ex:
        for step in steps:
            st = gen.smc_step(step)
            lw_in = logw.cpu().numpy()
            pt_in = pt.cpu().numpy()
            out = s.smc_reweight_resample(st["target"], st["draft"], st["tokens"], st["bonus_u"], st["resample_u"],
                                          logw, cfg.T, cfg.ess_frac, P, N, K, page_table_in=pt, beta=beta)
            torch.cuda.synchronize()
            g = {k: v.cpu().numpy() for k, v in out.items() if k != "log_weights"}
            g["logw"] = logw.cpu().numpy()
            assert int(out["status_flags"].item()) & ~8 == 0
            # invariants on every prompt
            anc = g["ancestors"].reshape(P, N)
            assert (np.diff(anc, axis=1) >= 0).all()
            assert (g["page_table_out"] == pt_in[(np.arange(P)[:, None] * N + anc).ravel()]).all()
            cases = []
            for p in prompts:
                rows_t = slice(p * N * (K + 1), (p + 1) * N * (K + 1))
                rows_d = slice(p * N * K, (p + 1) * N * K)
                cases.append(dict(target=host_logits(st["target"][rows_t]), draft=host_logits(st["draft"][rows_d]),
                                  tokens=st["tokens"][rows_d].cpu().numpy(),
                                  bonus_u=st["bonus_u"][p * N:(p + 1) * N].cpu().numpy(),
                                  resample_u=st["resample_u"][p:p + 1].cpu().numpy(), P=1, N=N, K=K, T=cfg.T,
                                  beta=beta))

            def ref_of(pc):
                p, c = pc
                sl = slice(p * N, (p + 1) * N)
                return oracle.smc_step(c["target"], c["draft"], c["tokens"], c["bonus_u"], c["resample_u"], lw_in[sl],
                                       cfg.T, cfg.ess_frac, 1, N, K, pt_in=pt_in[sl], beta=beta)

            for (p, case), ref in zip(zip(prompts, cases), ex.map(ref_of, zip(prompts, cases))):
                sl = slice(p * N, (p + 1) * N)
                gp = dict(bonus=g["bonus_token"][sl], ancestors=g["ancestors"][sl], ess=g["ess"][p:p + 1],
                          resampled=g["resampled"][p:p + 1], logw=g["logw"][sl], pt_out=g["page_table_out"][sl])
                t = compare_smc(case, ref, gp, lw_in[sl], pt_in[sl], f"{cfg.name} step {step} prompt {p}")
                total.merge(t)
                t.assert_ok()
            say(f"[{cfg.name} step {step}] {len(prompts)} prompts checked, resampled {int(g['resampled'].sum())}/{P} "
                f"ess[0]={g['ess'][0]:.3f} {total.summary()}")
            pt = out["page_table_out"]
    total.assert_ok()


def test_cfg2_full_size():
    _cfg_smc(2, range(8))


def test_cfg3_full_size_all_prompts():
    """Steps 0-3 of the 32-prompt x 64-particle workload, every prompt."""
    _cfg_smc(3, range(4))


def test_cfg3_full_size_two_prompts_16_steps():
    """Steps 0-15 in lockstep, prompts 0 (delta 0.5) and 31 (delta 2) checked."""
    _cfg_smc(3, range(16), prompts=[0, 31])


def test_cfg2_power_full_size():
    _cfg_smc(2, range(2), beta=2.0)


def test_cfg3_power_sampled_prompts():
    """cfg3 shape (multi-tile segments: bonus rows with their own tile partials,
    at their own scale) with the power target."""
    _cfg_smc(3, range(1), prompts=[0, 17], beta=3.0)


def test_smc_side_stream_without_workspace():
    """An SMC call on a stream other than the current one, with no workspace
    or outputs given: the binding zero-fills the workspace (whose counters
    decide which particle runs its prompt's resampling) on the call's own
    stream, while the current stream is kept busy."""
    import torch

    import oracle
    import smc_resampling_amd as s
    from compare import compare_smc
    from gpu_util import DEV, dev_logits

    side = torch.cuda.Stream(device=DEV)
    for i in range(3):
        c = smc_case(700 + i, 6, 32, 3, 9000, dtype="bf16", L=4, logw_scale=2.0)
        lw = torch.from_numpy(c["logw"]).to(DEV)
        pt = torch.from_numpy(c["pt"]).to(DEV)
        args = [dev_logits(c["target"]), dev_logits(c["draft"]), torch.from_numpy(c["tokens"]).to(DEV),
                torch.from_numpy(c["bonus_u"]).to(DEV), torch.from_numpy(c["resample_u"]).to(DEV), lw]
        torch.cuda.synchronize()
        torch.cuda._sleep(20_000_000)  # the current stream is busy
        out = s.smc_reweight_resample(*args, 1.0, 0.9, 6, 32, 3, page_table_in=pt, stream=side.cuda_stream)
        side.synchronize()
        torch.cuda.synchronize()
        ref = oracle.smc_step(c["target"], c["draft"], c["tokens"], c["bonus_u"], c["resample_u"], c["logw"], 1.0, 0.9,
                              6, 32, 3, pt_in=c["pt"])
        g = dict(bonus=out["bonus_token"].cpu().numpy(), ancestors=out["ancestors"].cpu().numpy(),
                 ess=out["ess"].cpu().numpy(), resampled=out["resampled"].cpu().numpy(), logw=lw.cpu().numpy(),
                 pt_out=out["page_table_out"].cpu().numpy())
        compare_smc(c, ref, g, c["logw"], c["pt"], f"side stream {i}").assert_ok()
        assert int(out["status_flags"].item()) & ~8 == 0


def test_smc_workspace_reuse():
    import torch

    import oracle
    import smc_resampling_amd as s
    from compare import compare_smc
    from gpu_util import DEV, dev_logits

    ws = s.new_workspace(s.smc_workspace_bytes(1, 4, 64, 8, 20000), DEV)
    for i, (P, N, K, V) in enumerate([(4, 64, 8, 20000), (1, 3, 1, 50), (2, 17, 0, 2049), (4, 64, 8, 20000)]):
        c = smc_case(200 + i, P, N, K, V, dtype="bf16", L=3, logw_scale=2.0)
        lw = torch.from_numpy(c["logw"]).to(DEV)
        pt = torch.from_numpy(c["pt"]).to(DEV)
        out = s.smc_reweight_resample(dev_logits(c["target"]), dev_logits(c["draft"]),
                                      torch.from_numpy(c["tokens"]).to(DEV), torch.from_numpy(c["bonus_u"]).to(DEV),
                                      torch.from_numpy(c["resample_u"]).to(DEV), lw, 1.0, 0.9, P, N, K,
                                      page_table_in=pt, workspace=ws)
        torch.cuda.synchronize()
        ref = oracle.smc_step(c["target"], c["draft"], c["tokens"], c["bonus_u"], c["resample_u"], c["logw"], 1.0, 0.9,
                              P, N, K, pt_in=c["pt"])
        g = dict(bonus=out["bonus_token"].cpu().numpy(), ancestors=out["ancestors"].cpu().numpy(),
                 ess=out["ess"].cpu().numpy(), resampled=out["resampled"].cpu().numpy(), logw=lw.cpu().numpy(),
                 pt_out=out["page_table_out"].cpu().numpy())
        compare_smc(c, ref, g, c["logw"], c["pt"], f"reuse {i}").assert_ok()
        assert int(out["status_flags"].item()) & ~8 == 0


def test_smc_deterministic():
    """Two runs of the same SMC step give bitwise-equal outputs."""
    from gpu_util import run_smc_gpu

    c = smc_case(4400, 4, 64, 4, 20000, dtype="bf16", L=8, logw_scale=2.0)
    a = run_smc_gpu(c, c["logw"], c["pt"], 0.9)
    b = run_smc_gpu(c, c["logw"], c["pt"], 0.9)
    for k in ("bonus", "ancestors", "ess", "resampled", "logw", "pt_out"):
        assert (a[k] == b[k]).all(), k


def test_smc_many_small_prompts():
    """Thousands of workgroups handing their prompts' log-weights to the last
    particle to count: 1024 prompts of 2 particles, and 300 prompts of 7 with
    resampling at almost every prompt, over two lockstep steps."""
    from gpu_util import check_smc_steps

    c = smc_case(4600, 1024, 2, 2, 3000, dtype="bf16", L=3, logw_scale=2.0)
    check_smc_steps(c, steps=2, ess_frac=0.9, label="1024x2")
    c = smc_case(4601, 300, 7, 3, 1500, T=0.8, dtype="f32", L=5, logw_scale=3.0)
    check_smc_steps(c, steps=2, ess_frac=1.0, label="300x7")


def _concat_smc_cases(a, b):
    """One call's inputs holding the prompts of case a, then those of b (same N, K, V)."""
    out = dict(a)
    for k in ("target", "draft", "tokens", "bonus_u", "resample_u", "logw", "pt"):
        out[k] = np.concatenate([a[k], b[k]])
    out["P"] = a["P"] + b["P"]
    return out


@pytest.mark.parametrize("P,N,K,V,dtype", [(1, 16, 4, 20000, "bf16"), (4, 64, 3, 4096, "bf16"),
                                           (3, 7, 2, 3001, "f32"), (1, 512, 1, 2048, "bf16")])
def test_smc_prompt_work_in_particle_kernel_matches_prompt_kernel(P, N, K, V, dtype):
    """Calls of at most 512 particles (whose workgroups all fit on the
    device) do each prompt's ESS, resampling and page gather in the prompt's
    last particle's workgroup (log-weights through tagged words); larger calls
    use a prompt kernel.  The same prompts decided both ways (alone, then
    padded to more than 2048 particles) must agree bit for bit, and the small
    call must match the oracle."""
    from gpu_util import check_smc_steps, run_smc_gpu
    from synth.small import smc_case

    small = smc_case(P * 100 + N, P, N, K, V, dtype=dtype, L=8, logw_scale=2.0)
    check_smc_steps(small, steps=1, ess_frac=0.9, label=f"prompt work in the particle kernel P={P} N={N}")
    pad_p = (2100 + N - 1) // N
    pad = smc_case(P * 100 + N + 1, pad_p, N, K, V, dtype=dtype, L=8, logw_scale=2.0)
    pad["pt"] = pad["pt"] + small["pt"].size  # page ids of their own
    big = _concat_smc_cases(small, pad)
    a = run_smc_gpu(small, small["logw"], small["pt"], ess_frac=0.9)
    b = run_smc_gpu(big, big["logw"], big["pt"], ess_frac=0.9)
    PN = P * N
    for k in ("bonus", "ancestors", "logw"):
        assert np.array_equal(a[k], b[k][:PN]), k
    for k in ("ess", "resampled"):
        assert np.array_equal(a[k], b[k][:P]), k
    assert np.array_equal(a["pt_out"], b["pt_out"][:PN])
    assert (a["flags"] & 128) == 0 and (b["flags"] & 128) == 0


@pytest.mark.parametrize("P,N,L", [(40, 13, 1000), (40, 13, 999), (9, 64, 300), (33, 16, 2048)])
def test_smc_prompt_shared_by_workgroups(P, N, L):
    """More than 512 particles with large page tables: each prompt's work is
    shared by up to eight workgroups, each gathering its share of the rows
    (3 parts of 13 rows, 4 of 64, 8 of 16; 16-byte and element copies).  Every
    output, the page table included, must match the oracle, with resampling
    forced (ess_frac 2) and left to the threshold."""
    from gpu_util import check_smc_steps

    c = smc_case(P * 1000 + N + L, P, N, 2, 2048, dtype="bf16", L=L, logw_scale=2.0)
    check_smc_steps(c, steps=1, ess_frac=2.0, label=f"shared prompt P={P} N={N} L={L} forced")
    check_smc_steps(c, steps=1, ess_frac=0.9, label=f"shared prompt P={P} N={N} L={L}")
