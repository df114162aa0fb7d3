"""Paged-KV bookkeeping on the GPU against the oracle, step by step, bit for bit."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

from synth.small import pages_state, sorted_ancestors  # noqa: E402


def _dev(x):
    import torch

    return torch.from_numpy(np.ascontiguousarray(x, np.int32)).cuda()


def _host(t):
    return t.cpu().numpy()


def _scratch_bytes(P, N, L, M):
    """Bytes at the start of the workspace that every call leaves at zero: two
    per-page arrays, then a row of entry marks per particle."""
    al = lambda x: (x + 255) // 256 * 256  # noqa: E731
    return 2 * al(4 * M) + al(4 * P * N * ((L + 31) // 32))


def _lockstep(P, N, L, S, M, A, steps, seed, max_len=None, concentrate=0.5, shuffle=False, identity_every=0):
    import torch

    import oracle
    import smc_resampling_amd as s
    from gpu_util import say

    st = pages_state(seed, P, N, L, S, M, max_len=max_len)
    R = P * N
    table, lens, ref, free, fc = st["table"], st["len"], st["ref"], st["free_pages"], st["free_count"]
    g_table, g_len, g_ref, g_free, g_fc = _dev(table), _dev(lens), _dev(ref), _dev(free), _dev([fc])
    ws = s.new_workspace(s.smc_pages_workspace_bytes(P, N, L, M), "cuda")
    n_cow = 0
    for step in range(steps):
        o = oracle.pages_append(table, lens, ref, free, fc, S, A)
        g = s.smc_pages_append(g_table, g_len, g_ref, g_free, g_fc, P, N, S, A, workspace=ws)
        torch.cuda.synchronize()
        assert o["status"] == 0 and int(g["status_flags"].item()) == 0, (step, o["status"], int(g["status_flags"].item()))
        nc = int(g["cow_count"].item())
        assert nc == len(o["cow"]), (nc, len(o["cow"]))
        assert (_host(g["cow_list"])[:nc] == o["cow"]).all(), "copy list"
        assert (_host(g["slots"]) == o["slots"]).all(), "slots"
        assert (_host(g_table) == o["table"]).all(), "page table after append"
        assert (_host(g_len) == o["len"]).all() and (_host(g_ref) == o["ref"]).all(), "lengths / counts"
        fc = o["free_count"]
        assert int(g_fc.item()) == fc
        table, lens, ref = o["table"], o["len"], o["ref"]
        n_cow += nc
        anc = sorted_ancestors(seed * 100 + step, P, N, concentrate=concentrate)
        if shuffle:  # copies no longer neighbours: runs of a shared page split
            rng = np.random.default_rng(seed * 100 + step)
            anc = np.concatenate([rng.permutation(anc[p * N:(p + 1) * N]) for p in range(P)]).astype(np.int32)
        if identity_every and step % identity_every == 0:  # a step that did not resample
            anc = np.tile(np.arange(N, dtype=np.int32), P)
        src = (np.arange(R) // N) * N + anc
        table_new = table[src].copy()
        o = oracle.pages_resample(P, N, anc, table, table_new, lens, ref, free, fc, S)
        g_new = _dev(table_new)
        g_out = torch.empty_like(g_len)
        r = s.smc_pages_resample(_dev(anc), g_table, g_len, g_ref, g_free, g_fc, P, N, S, seq_len_out=g_out,
                                 workspace=ws)
        torch.cuda.synchronize()
        assert o["status"] == 0 and int(r["status_flags"].item()) == 0, (step, o["status"], int(r["status_flags"].item()))
        fc = o["free_count"]
        assert int(g_fc.item()) == fc, (int(g_fc.item()), fc)
        assert (_host(g_out) == o["len"]).all(), "lengths after resampling"
        assert (_host(g_ref) == o["ref"]).all(), "counts after resampling"
        assert (_host(g_free)[:fc] == o["free_pages"][:fc]).all(), "free stack"
        table, lens, ref, free = table_new, o["len"], o["ref"], o["free_pages"]
        g_table, g_len = g_new, g_out
    # the calls leave the scratch as they found it (the staging area aside)
    assert int(ws[:_scratch_bytes(P, N, L, M)].count_nonzero().item()) == 0, "page scratch not cleared"
    say(f"[pages P={P} N={N} L={L} S={S} M={M} A={A}] {steps} steps, {n_cow} copies, free {fc}")
    return n_cow


def test_pages_small_lockstep():
    assert _lockstep(2, 6, 14, 4, 160, 3, steps=6, seed=11, max_len=9) > 0


def test_pages_odd_sizes():
    _lockstep(3, 5, 9, 3, 200, 2, steps=5, seed=12, max_len=7, concentrate=0.8)
    _lockstep(1, 1, 4, 16, 8, 5, steps=3, seed=13, max_len=10)      # one particle, no sharing
    _lockstep(2, 7, 30, 1, 800, 1, steps=4, seed=14, max_len=5)     # one-token pages


def test_pages_single_workgroup_bounds():
    """Calls of at most 16 rows of at most 256 entries resample in one
    workgroup; the sizes at and just past those bounds, and the 1 x 16-particle
    SMC workload's shape (16-token pages, K+1 = 5 tokens a step, 256-entry rows)."""
    _lockstep(1, 16, 256, 16, 16 * 300, 5, steps=4, seed=21, max_len=3000, concentrate=0.4)
    _lockstep(16, 1, 256, 4, 16 * 300, 7, steps=3, seed=22, max_len=1000)    # every particle a prompt
    _lockstep(2, 8, 256, 2, 16 * 300, 3, steps=4, seed=23, max_len=500, concentrate=0.3, shuffle=True)
    _lockstep(4, 4, 256, 1, 16 * 300, 2, steps=6, seed=26, max_len=250, concentrate=0.2, identity_every=3)
    _lockstep(1, 17, 64, 4, 17 * 80, 5, steps=3, seed=24, max_len=200, concentrate=0.4)    # one row too many
    _lockstep(1, 16, 257, 2, 16 * 300, 3, steps=3, seed=25, max_len=500, concentrate=0.4)  # rows too long


def test_pages_chunked_particles():
    """More particles than the append workgroup's threads (several particles
    per thread), and more than it holds in registers at once (chunks)."""
    _lockstep(5, 300, 12, 8, 30000, 9, steps=3, seed=15, max_len=40, concentrate=0.3)
    _lockstep(3, 3000, 6, 4, 3 * 3000 * 8, 3, steps=3, seed=18, max_len=10, concentrate=0.3)


def test_pages_unsorted_ancestors():
    """Ancestors in any order (copies of a row not adjacent) and steps that did
    not resample (every row its own ancestor)."""
    _lockstep(2, 6, 14, 4, 160, 3, steps=6, seed=19, max_len=9, shuffle=True)
    _lockstep(4, 70, 20, 4, 4 * 70 * 25, 5, steps=6, seed=20, max_len=40, concentrate=0.6, shuffle=True,
              identity_every=2)


def test_pages_batched_smc_shape():
    """The batched SMC workload's shape: 32 prompts x 64 particles, 16-token pages,
    K+1 = 9 tokens per step, 512-page rows."""
    P, N, L, S, A = 32, 64, 512, 16, 9
    _lockstep(P, N, L, S, P * N * 300, A, steps=3, seed=16, max_len=4000, concentrate=0.4)


def test_pages_rejections_change_nothing():
    import torch

    import oracle
    import smc_resampling_amd as s

    st = pages_state(17, 1, 4, 4, 4, 40, max_len=10)
    full_a = 16 - int(st["len"].max()) + 1  # the longest row needs a fifth page
    cases = [("full", st["ref"], st["free_count"], full_a, s.FLAG_PAGES_FULL, 1),
             ("exhausted", st["ref"], 1, 5, s.FLAG_PAGES_EXHAUSTED, 2)]
    bad_ref = st["ref"].copy()
    assert (st["len"] % 4 != 0).any()
    r0 = int(np.argmax(st["len"] % 4 != 0))
    bad_ref[st["table"][r0, (int(st["len"][r0]) + 3) // 4 - 1]] = 2
    cases.append(("sharing", bad_ref, st["free_count"], 2, s.FLAG_BAD_INPUT, 3))
    for name, ref, fc, A, flag, status in cases:
        o = oracle.pages_append(st["table"], st["len"], ref, st["free_pages"], fc, 4, A)
        assert o["status"] == status, name
        g_table, g_len, g_ref, g_fc = _dev(st["table"]), _dev(st["len"]), _dev(ref), _dev([fc])
        ws = s.new_workspace(s.smc_pages_workspace_bytes(1, 4, 4, 40), "cuda")
        g = s.smc_pages_append(g_table, g_len, g_ref, _dev(st["free_pages"]), g_fc, 1, 4, 4, A, workspace=ws)
        torch.cuda.synchronize()
        assert int(g["status_flags"].item()) & flag, name
        assert (_host(g_table) == st["table"]).all() and (_host(g_len) == st["len"]).all(), name
        assert (_host(g_ref) == ref).all() and int(g_fc.item()) == fc, name
        assert int(ws.count_nonzero().item()) == 0, f"{name}: scratch not cleared"
