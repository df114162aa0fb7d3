"""The library's calls captured in a HIP graph and replayed, the way the
benchmark times them, against the same calls run eagerly.

Each case prepares its calls twice, each set with its own outputs and state:
one set runs eagerly, the other is captured into a graph.  The graph is then
replayed three times; before every replay (and before the eager run) the
outputs are filled with the same poison and the state (log-weights, page
tables, paged-KV metadata) is restored, and between replays the eager set
runs again.  Every replay must leave outputs and state equal to the eager
run's, bit for bit.  The eager results are themselves held to the oracle at
these sizes by the parity tests."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

REPLAYS = 3
POISON = -7


class Case:
    """Calls prepared on one stream, the tensors they write (`outs`), and the
    state they update in place, as (tensor, initial value) pairs."""

    def __init__(self, calls, outs, state=()):
        self.calls, self.outs, self.state = calls, outs, list(state)

    def reset(self):
        for k, t in self.outs.items():
            if k.endswith("flags"):  # OR-ed into by the calls
                t.zero_()
            else:
                t.fill_(float("nan") if t.is_floating_point() else POISON)
        for t, init in self.state:
            t.copy_(init)

    def host(self):
        return {k: t.detach().cpu().clone() for k, t in self.outs.items()}


def _same(want, got, label):
    for k, a in want.items():
        b = got[k]
        if a.is_floating_point():
            a, b = a.view(torch.int32), b.view(torch.int32)  # bitwise, NaN included
        bad = int((a != b).sum())
        assert bad == 0, f"{label}: {k} differs at {bad} of {a.numel()} elements"


def _graph_vs_eager(make, label):
    from gpu_util import DEV, say

    side = torch.cuda.Stream(device=DEV)
    eager, captured = make(side.cuda_stream), make(side.cuda_stream)

    def run_eager():
        eager.reset()
        with torch.cuda.stream(side):
            for c in eager.calls:
                c()
        torch.cuda.synchronize()
        return eager.host()

    want = run_eager()
    for k, a in want.items():  # every output but a copy list (empty while no page is shared) is written
        if not k.startswith("cow") and not k.endswith("flags"):
            w = ~torch.isnan(a) if a.is_floating_point() else a != POISON
            assert bool(w.any()), f"{label}: the eager run wrote nothing to {k}"
    for k in ("status_flags", "page_flags"):  # nothing but the informational CDF-clamp bit
        assert k not in want or int(want[k][0]) & ~8 == 0, f"{label}: {k} {int(want[k][0])}"
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        for c in captured.calls:
            c()
    torch.cuda.synchronize()
    for r in range(REPLAYS):
        captured.reset()
        torch.cuda.synchronize()
        with torch.cuda.stream(side):
            graph.replay()
        torch.cuda.synchronize()
        _same(want, captured.host(), f"{label} replay {r}")
        _same(want, run_eager(), f"{label} eager run after replay {r}")
    say(f"[graph {label}] {len(captured.calls)} calls, {REPLAYS} replays equal to the eager run")


def _sd_maker(idx, steps):
    import smc_resampling_amd as s
    import synth
    from gpu_util import DEV, oracle_lengths

    cfg = synth.CONFIGS[idx]
    gen = synth.Generator(cfg, DEV, lengths=oracle_lengths)
    batches = [gen.sd_step(i) for i in range(steps)]
    rows_d = max(b["total_draft_rows"] for b in batches)

    def make(stream):
        ws = s.new_workspace(s.sd_verify_workspace_bytes(int(cfg.dtype == "bf16"), cfg.B, cfg.K, cfg.V, rows_d), DEV)
        outs = {"status_flags": torch.zeros(1, dtype=torch.int32, device=DEV)}
        calls = []
        for i, bt in enumerate(batches):
            call, o = s.prepare_sd_verify(bt["target"], bt["draft"], bt["tokens"], bt["uniforms"], cfg.T, K=cfg.K,
                                          draft_offsets=bt["offsets"], workspace=ws,
                                          status_flags=outs["status_flags"], stream=stream)
            calls.append(call)
            outs[f"num_accepted{i}"], outs[f"final_token{i}"] = o["num_accepted"], o["final_token"]
        return Case(calls, outs)

    return make


def _smc_maker(idx, steps, noalloc=False):
    import smc_resampling_amd as s
    import synth
    from gpu_util import DEV

    cfg = synth.CONFIGS[idx]
    P, N, K = cfg.P, cfg.N, cfg.K
    gen = synth.Generator(cfg, DEV)
    batches = [gen.smc_step(i) for i in range(steps)]
    rng = np.random.default_rng(idx)
    logw0 = torch.from_numpy(rng.normal(0.0, 2.0, P * N).astype(np.float32)).to(DEV)
    pt0 = torch.from_numpy(synth.initial_page_table(P, N, cfg.L)).to(DEV)

    def make(stream):
        logw = torch.empty_like(logw0)
        pts = [torch.empty_like(pt0), torch.empty_like(pt0)]
        ws = None if noalloc else s.new_workspace(s.smc_workspace_bytes(1, P, N, K, cfg.V), DEV)
        outs = {"status_flags": torch.zeros(1, dtype=torch.int32, device=DEV)}
        calls = []
        for i, bt in enumerate(batches):
            call, o = s.prepare_smc_reweight_resample(
                bt["target"], bt["draft"], bt["tokens"], bt["bonus_u"], bt["resample_u"], logw, cfg.T, cfg.ess_frac,
                P, N, K, page_table_in=pts[i % 2], page_table_out=pts[(i + 1) % 2], workspace=ws,
                status_flags=outs["status_flags"], stream=stream, noalloc=noalloc)
            calls.append(call)
            for k in ("bonus_token", "ancestors", "ess", "resampled"):
                outs[f"{k}{i}"] = o[k]
        outs["log_weights"], outs["page_table"] = logw, pts[steps % 2]
        return Case(calls, outs, [(logw, logw0), (pts[0], pt0)])

    return make


def _smc_pages_maker(idx, steps):
    """SMC steps with the paged-KV bookkeeping around each (append K+1 tokens
    before, resample after), as the benchmark's paged-KV option runs them."""
    import smc_resampling_amd as s
    import synth
    from gpu_util import DEV
    from synth.small import pages_state

    cfg = synth.CONFIGS[idx]
    P, N, K, L = cfg.P, cfg.N, cfg.K, cfg.L
    S, A, R = 16, K + 1, P * N
    M = R * L + R
    gen = synth.Generator(cfg, DEV)
    batches = [gen.smc_step(i) for i in range(steps)]
    st0 = pages_state(idx, P, N, L, S, M, fixed_len=max(0, L * S - (steps + 1) * A - S))
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(DEV)  # noqa: E731
    init = dict(table=i32(st0["table"]), len=i32(st0["len"]), ref=i32(st0["ref"]), free=i32(st0["free_pages"]),
                fc=i32([st0["free_count"]]), logw=torch.zeros(R, dtype=torch.float32, device=DEV))

    def make(stream):
        pts = [torch.empty_like(init["table"]), torch.empty_like(init["table"])]
        lens = [torch.empty_like(init["len"]), torch.empty_like(init["len"])]
        ref, free, fc = (torch.empty_like(init[k]) for k in ("ref", "free", "fc"))
        logw = torch.empty_like(init["logw"])
        pws = s.new_workspace(s.smc_pages_workspace_bytes(P, N, L, M), DEV)
        ws = s.new_workspace(s.smc_workspace_bytes(1, P, N, K, cfg.V), DEV)
        outs = {"status_flags": torch.zeros(1, dtype=torch.int32, device=DEV),
                "page_flags": torch.zeros(1, dtype=torch.int32, device=DEV)}
        calls = []
        for i, bt in enumerate(batches):
            cur, nxt = i % 2, (i + 1) % 2
            slots = torch.empty((R, A), dtype=torch.int32, device=DEV)
            cow = torch.empty((R, 3), dtype=torch.int32, device=DEV)
            ncow = torch.empty(1, dtype=torch.int32, device=DEV)
            call, o = s.prepare_smc_reweight_resample(
                bt["target"], bt["draft"], bt["tokens"], bt["bonus_u"], bt["resample_u"], logw, cfg.T, cfg.ess_frac,
                P, N, K, page_table_in=pts[cur], page_table_out=pts[nxt], workspace=ws,
                status_flags=outs["status_flags"], stream=stream)

            def step(call=call, o=o, cur=cur, nxt=nxt, slots=slots, cow=cow, ncow=ncow):
                s.smc_pages_append(pts[cur], lens[cur], ref, free, fc, P, N, S, A, workspace=pws,
                                   status_flags=outs["page_flags"], stream=stream, slots=slots, cow_list=cow,
                                   cow_count=ncow)
                call()
                s.smc_pages_resample(o["ancestors"], pts[cur], lens[cur], ref, free, fc, P, N, S,
                                     seq_len_out=lens[nxt], workspace=pws, status_flags=outs["page_flags"],
                                     stream=stream)

            calls.append(step)
            outs.update({f"slots{i}": slots, f"cow{i}": cow, f"cow_count{i}": ncow, f"ancestors{i}": o["ancestors"],
                         f"bonus_token{i}": o["bonus_token"]})
        outs.update(page_table=pts[steps % 2], seq_len=lens[steps % 2], ref_count=ref, free_pages=free,
                    free_count=fc, log_weights=logw)
        state = [(pts[0], init["table"]), (lens[0], init["len"]), (ref, init["ref"]), (free, init["free"]),
                 (fc, init["fc"]), (logw, init["logw"]), (pws, torch.zeros_like(pws))]
        return Case(calls, outs, state)

    return make


@pytest.mark.parametrize("idx,steps", [(0, 4), (1, 4), (4, 3)])
def test_graph_sd(idx, steps):
    import synth

    _graph_vs_eager(_sd_maker(idx, steps), synth.CONFIGS[idx].name)


def test_graph_smc_cfg2():
    import synth

    _graph_vs_eager(_smc_maker(2, 3), synth.CONFIGS[2].name)


def test_graph_smc_cfg3_full_size():
    """Two steps of the 32-prompt x 64-particle workload (10.58 GB of logits per
    step), as the benchmark's headline graph runs them."""
    import synth

    _graph_vs_eager(_smc_maker(3, 2), synth.CONFIGS[3].name)


def test_graph_smc_noalloc():
    """The entry point that allocates nothing, captured: its static scratch is
    shared by every call in the graph, as it is eagerly."""
    import synth

    _graph_vs_eager(_smc_maker(2, 3, noalloc=True), synth.CONFIGS[2].name + " noalloc")


def test_graph_smc_with_pages():
    import synth

    _graph_vs_eager(_smc_pages_maker(2, 3), synth.CONFIGS[2].name + " with paged-KV bookkeeping")


def test_graph_tree():
    import smc_resampling_amd as s
    import synth
    from gpu_util import DEV

    cfg = next(c for c in synth.CONFIGS if c.kind == "tree")
    gen = synth.Generator(cfg, DEV)
    batches = [gen.tree_step(i) for i in range(3)]

    def make(stream):
        b0 = batches[0]
        ws = s.new_workspace(s.tree_verify_workspace_bytes(1, cfg.B, cfg.V, b0["target"].shape[0],
                                                           b0["draft"].shape[0]), DEV)
        outs = {"status_flags": torch.zeros(1, dtype=torch.int32, device=DEV)}
        calls = []
        for i, bt in enumerate(batches):
            call, o = s.prepare_tree_verify(bt["target"], bt["draft"], bt["node_off"], bt["draft_off"], bt["parent"],
                                            bt["tokens"], bt["uniforms"], cfg.T, workspace=ws,
                                            status_flags=outs["status_flags"], stream=stream)
            calls.append(call)
            for k in ("num_accepted", "last_node", "final_token"):
                outs[f"{k}{i}"] = o[k]
        return Case(calls, outs)

    _graph_vs_eager(make, cfg.name)
