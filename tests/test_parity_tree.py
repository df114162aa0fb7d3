"""tree_verify on the GPU against the oracle (element by element, decision band)."""
import re

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

from synth.small import tree_case, tree_parents  # noqa: E402


def _mixed_trees(rng, n):
    shapes = [tree_parents("root"), tree_parents("chain", M=5), tree_parents("star", M=4),
              tree_parents("full", width=2, depth=3), tree_parents("random", rng, M=30),
              tree_parents("full", width=3, depth=2), tree_parents("star", M=9)]
    return [shapes[i % len(shapes)] for i in range(n)]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("V,T", [(1, 1.0), (7, 0.7), (2047, 1.0), (2048, 1.3), (2049, 0.8), (6000, 1.0),
                                 (32768 + 8, 0.7)])
def test_tree_shapes(dtype, V, T):
    from gpu_util import check_tree

    rng = np.random.default_rng(V)
    for delta in (0.5, 2.0):
        c = tree_case(V * 13 + int(delta * 10), _mixed_trees(rng, 14), V, T=T, delta=delta, dtype=dtype)
        check_tree(c, f"V={V} T={T} d={delta} {dtype}")


def test_tree_largest_and_random_trees():
    """Trees of SMCSD_TREE_MAX_NODES nodes, random shapes of every size, and a
    wide star (many rejections in a row at one node, each renormalising the
    residual)."""
    from gpu_util import check_tree

    rng = np.random.default_rng(7)
    trees = [tree_parents("random", rng, M=256), tree_parents("star", M=256), tree_parents("chain", M=256)]
    trees += [tree_parents("random", rng, M=int(m)) for m in rng.integers(1, 120, 20)]
    for dtype in ("bf16", "f32"):
        check_tree(tree_case(8, trees, 3000, T=1.0, delta=2.5, dtype=dtype), f"large trees {dtype}")


def test_tree_chain_is_sd_verify_bit_for_bit():
    """A chain of K+1 nodes decides exactly as sd_verify with K draft tokens
    (same accepted counts and final tokens), on the GPU, for both dtypes."""
    import torch

    import smc_resampling_amd as s
    from gpu_util import DEV, dev_logits
    from synth.small import sd_case

    for dtype, V, K, B in (("bf16", 32768, 4, 64), ("f32", 5000, 3, 40), ("bf16", 151936, 8, 4)):
        c = sd_case(K * 100 + B, B, V, T=0.8, K=K, delta=1.0, dtype=dtype)
        na, ft, _ = s.sd_verify(dev_logits(c["target"]), dev_logits(c["draft"]), torch.from_numpy(c["tokens"]).to(DEV),
                                torch.from_numpy(c["uniforms"]).to(DEV), c["T"], K=K)
        # the same rows as chains: node j of tree b is target row b*(K+1)+j, its
        # draft row b*K+j; node j+1 carries token x_j; the root's uniform is the final one
        u = c["uniforms"].reshape(B, K + 1)
        par = np.tile(np.arange(-1, K, dtype=np.int32), B)
        tok = np.concatenate([np.zeros((B, 1), np.int32), c["tokens"].reshape(B, K)], 1).ravel()
        uu = np.concatenate([u[:, K:], u[:, :K]], 1).ravel().astype(np.float32)
        t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)  # noqa: E731
        out = s.tree_verify(dev_logits(c["target"]), dev_logits(c["draft"]),
                            t(np.arange(0, B * (K + 1) + 1, K + 1, dtype=np.int32)),
                            t(np.arange(0, B * K + 1, K, dtype=np.int32)), t(par), t(tok), t(uu), c["T"])
        torch.cuda.synchronize()
        assert (out["num_accepted"].cpu() == na.cpu()).all()
        assert (out["last_node"].cpu() == na.cpu()).all()
        assert (out["final_token"].cpu() == ft.cpu()).all(), (dtype, V)


def test_tree_identical_rows_follow_first_children():
    """Draft rows equal to their target rows: every ratio is 1, so the walk
    takes the first child down to a leaf."""
    from gpu_util import check_tree, run_tree_gpu

    rng = np.random.default_rng(11)
    trees = _mixed_trees(rng, 21)
    c = tree_case(12, trees, 4096, T=1.0, delta=0.0, dtype="bf16")
    na, ln, _, _ = run_tree_gpu(c)
    for b, par in enumerate(trees):
        u, d = 0, 0
        while any(p == u for p in par[1:]):
            u, d = par.index(u), d + 1
        assert ln[b] == u and na[b] == d, (b, ln[b], u)
    check_tree(c, "delta=0")


def test_tree_masked_tokens_and_bad_tokens():
    from gpu_util import check_tree, run_tree_gpu

    rng = np.random.default_rng(13)
    trees = _mixed_trees(rng, 14)
    c = tree_case(14, trees, 3000, T=0.9, delta=1.0, dtype="f32")
    c["target"][:, ::4] = -np.inf  # masked tokens in the target rows
    check_tree(c, "masked target tokens")
    # tokens outside [0, V): rejected on both sides; the library also flags them
    c = tree_case(15, trees, 3000, T=0.9, delta=0.3, dtype="bf16")
    bad = np.arange(1, len(c["tokens"]), 5)
    c["tokens"][bad] = np.where(bad % 2 == 0, -1, 3000)
    check_tree(c, "bad tokens", ignore_flags=8 | 16)
    _, _, _, fl = run_tree_gpu(c)
    assert fl & 16


def test_tree_zero_residual():
    """Identical rows and a rejected first child (a token outside the
    vocabulary): max(0, p - q) has no mass, r stays p (ZERO_RESIDUAL); the
    next child is then accepted (ratio 1), or, with no next child, the final
    token is drawn from p."""
    from gpu_util import check_tree, run_tree_gpu

    for shape in (tree_parents("star", M=3), tree_parents("chain", M=3)):
        c = tree_case(16, [shape] * 8, 5000, T=1.0, delta=0.0, dtype="bf16")
        c["tokens"][c["node_off"][:-1] + 1] = 5000  # every tree's node 1: outside the vocabulary
        na, ln, _, fl = run_tree_gpu(c)
        assert fl & 2 and fl & 16, fl
        check_tree(c, f"zero residual {shape}", ignore_flags=8 | 16)


def test_tree_malformed_trees_raise_bad_input():
    """Parents out of tree order, or parents whose nodes with children disagree
    with the draft offsets: BAD_INPUT, and the well-formed trees of the same
    call still match the oracle."""
    from compare import compare_tree
    from gpu_util import run_tree_gpu, run_tree_oracle, say

    good = tree_case(17, [tree_parents("full", width=2, depth=2)] * 4, 1000, T=1.0, dtype="f32")
    ref = run_tree_oracle(good)
    for bad_par in ([0, 0, 0, 1, 1, 2, 2], [-1, 2, 0, 1, 1, 2, 2], [-1, 0, 0, 3, 1, 2, 2], [-1, 0, 0, 1, 1, 1, 1]):
        c = dict(good, parent=good["parent"].copy())
        c["parent"][7:14] = bad_par  # tree 1 of 4
        na, ln, ft, fl = run_tree_gpu(c)
        assert fl & 16, (bad_par, fl)
        keep = [0, 2, 3]
        sub = dict(good, node_off=good["node_off"])
        t = compare_tree(sub, ref, na, ln, ft, f"malformed {bad_par}")
        bad_trees = {re.search(r"tree (\d+)", f).group(1) for f in t.failures}
        say(f"[tree malformed {bad_par}] {t.summary()}")
        assert bad_trees <= {"1"}, t.failures
        assert t.equal + t.exempt_diff >= len(keep)


def test_tree_workloads_full_size():
    """64 binary trees of depth 3 (15 nodes, 7 draft rows each) at V=32768
    bf16, T=0.7, draft noise 0.5 / 1 / 2 by tree; and 16 random 64-node trees
    at V=151936 bf16."""
    from gpu_util import check_tree

    full = tree_parents("full", width=2, depth=3)
    c = tree_case(18, [full] * 64, 32768, T=0.7, delta=np.array([(0.5, 1.0, 2.0)[b % 3] for b in range(64)]),
                  dtype="bf16")
    check_tree(c, "64 x binary depth 3, V=32768")
    rng = np.random.default_rng(19)
    c = tree_case(20, [tree_parents("random", rng, M=64) for _ in range(16)], 151936, T=1.0, delta=1.0,
                  dtype="bf16")
    check_tree(c, "16 x random 64 nodes, V=151936")


def test_tree_generated_workload_steps():
    """Two steps of the benchmark's tree workload as the GPU generator makes
    them (64 binary trees of depth 3, V=32768 bf16): the library against the
    oracle on host copies of the same bytes."""
    import synth
    from gpu_util import DEV, check_tree, host_logits

    cfg = synth.CONFIGS[5]
    gen = synth.Generator(cfg, DEV)
    for step in (0, 1):
        bt = gen.tree_step(step)
        case = dict(target=host_logits(bt["target"]), draft=host_logits(bt["draft"]), T=cfg.T,
                    **{k: bt[k].cpu().numpy() for k in ("node_off", "draft_off", "parent", "tokens", "uniforms")})
        check_tree(case, f"{cfg.name} step {step}")


def test_tree_workspace_shared_with_sd_verify():
    """One workspace serves tree calls of different shapes interleaved with
    sd_verify calls: the tree call uses no counters, and the partials each
    call reads are the ones it wrote."""
    import torch

    import oracle
    import smc_resampling_amd as s
    from compare import compare_sd, compare_tree
    from gpu_util import DEV, dev_logits
    from synth.small import sd_case

    rng = np.random.default_rng(23)
    nbytes = max(s.tree_verify_workspace_bytes(1, 40, 20000, 40 * 64, 40 * 63),
                 s.sd_verify_workspace_bytes(1, 40, 8, 20000, 40 * 8))
    ws = s.new_workspace(nbytes, DEV)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)  # noqa: E731
    for i, (B, V) in enumerate([(40, 20000), (3, 50), (17, 2049), (40, 20000)]):
        trees = [tree_parents("random", rng, M=int(m)) for m in rng.integers(1, 65, B)]
        c = tree_case(300 + i, trees, V, T=0.8, delta=1.0, dtype="bf16")
        out = s.tree_verify(dev_logits(c["target"]), dev_logits(c["draft"]), t(c["node_off"]), t(c["draft_off"]),
                            t(c["parent"]), t(c["tokens"]), t(c["uniforms"]), c["T"], workspace=ws)
        torch.cuda.synchronize()
        ref = oracle.tree_verify(c["target"], c["draft"], c["node_off"], c["draft_off"], c["parent"], c["tokens"],
                                 c["uniforms"], c["T"])
        compare_tree(c, ref, out["num_accepted"].cpu().numpy(), out["last_node"].cpu().numpy(),
                     out["final_token"].cpu().numpy(), f"shared workspace tree {i}").assert_ok()
        assert int(out["status_flags"].item()) & ~8 == 0
        sc = sd_case(310 + i, min(B, 40), V, T=1.0, K=int(rng.integers(0, 9)), delta=1.0, dtype="bf16")
        na, ft, fl = s.sd_verify(dev_logits(sc["target"]), dev_logits(sc["draft"]), t(sc["tokens"]),
                                 t(sc["uniforms"]), sc["T"], K=sc["K"], workspace=ws)
        torch.cuda.synchronize()
        ref = oracle.sd_verify(sc["target"], sc["draft"], sc["tokens"], sc["uniforms"], sc["T"], K=sc["K"])
        compare_sd(sc, ref, na.cpu().numpy(), ft.cpu().numpy(), f"shared workspace sd {i}").assert_ok()


def test_tree_deterministic():
    """Two runs of the same tree call give bitwise-equal outputs."""
    from gpu_util import run_tree_gpu

    rng = np.random.default_rng(29)
    c = tree_case(4500, [tree_parents("random", rng, M=int(m)) for m in rng.integers(1, 80, 32)], 20000, T=0.8,
                  delta=1.5, dtype="bf16")
    a = run_tree_gpu(c)
    b = run_tree_gpu(c)
    for x, y in zip(a, b):
        assert np.array_equal(np.asarray(x), np.asarray(y))


def _concat_tree_cases(a, b):
    """One call's inputs holding the trees of case a, then those of case b."""
    na, da = int(a["node_off"][-1]), int(a["draft_off"][-1])
    out = dict(T=a["T"], dtype=a["dtype"])
    out["target"] = np.concatenate([a["target"], b["target"]])
    out["draft"] = np.concatenate([a["draft"], b["draft"]])
    out["node_off"] = np.concatenate([a["node_off"], b["node_off"][1:] + na]).astype(np.int32)
    out["draft_off"] = np.concatenate([a["draft_off"], b["draft_off"][1:] + da]).astype(np.int32)
    for k in ("parent", "tokens", "uniforms"):
        out[k] = np.concatenate([a[k], b[k]])
    return out


@pytest.mark.parametrize("B,V,dtype", [(1, 32768, "bf16"), (13, 32768, "bf16"), (64, 32768, "bf16"),
                                       (65, 6000, "f32"), (128, 2049, "bf16"), (8, 151936, "bf16"),
                                       (40, 20000, "f32")])
def test_tree_split_members_match_one_workgroup(B, V, dtype):
    """Calls of few trees run each tree on several workgroups that share its
    rejection passes (4 members up to 64 trees, 2 up to 128, fewer when a
    row has fewer tiles); the same trees in a call of 300 trees run on one
    workgroup each.  Both must decide bit for bit alike, and match the
    oracle."""
    from gpu_util import check_tree, run_tree_gpu

    rng = np.random.default_rng(B * 7 + V)
    shapes = [tree_parents("full", width=2, depth=3), tree_parents("star", M=6), tree_parents("chain", M=5),
              tree_parents("random", rng, M=40), tree_parents("full", width=3, depth=2)]
    trees = [shapes[i % len(shapes)] for i in range(B)]
    small = tree_case(B * 31 + 5, trees, V, T=0.8, delta=np.array([(0.5, 1.0, 2.0)[b % 3] for b in range(B)]),
                      dtype=dtype)
    check_tree(small, f"split call B={B} V={V} {dtype}")
    pad = tree_case(B * 31 + 6, [tree_parents("root")] * (300 - B), V, T=0.8, delta=1.0, dtype=dtype)
    big = _concat_tree_cases(small, pad)
    na_s, ln_s, ft_s, fl_s = run_tree_gpu(small)
    na_b, ln_b, ft_b, fl_b = run_tree_gpu(big)
    assert np.array_equal(na_s, na_b[:B]) and np.array_equal(ln_s, ln_b[:B]) and np.array_equal(ft_s, ft_b[:B])
    assert (fl_s & 128) == 0 and (fl_b & 128) == 0
