"""Seeded synthetic inputs for the verify-and-sample step (test / bench infrastructure).

Both the GPU library (through its tests and benchmark) and the CPU oracle
consume what this module produces; it contains none of the verify, resample or
drafting arithmetic.  Logits, draft tokens and uniforms are generated on the
GPU by ``libsmcsd_synth.so`` (Philox4x32-10 streams); the rank prior, the PACER
pre-verifier scores and the page tables are built on the host.  Draft tokens are
drawn by the Gumbel-max method, not by the inverse CDF that the library and the
oracle use for their own draws.

The five workloads stand in for the pages' model families and draft lengths:
vocabulary widths 32000 / 32768 (Mistral-family ~32k tokenizer), 128256 and
151936 (Llama / Qwen families); draft lengths K in {2, 4, 8} and PACER blocks of
4.  The logits are synthetic: z_t = 3 N(0,1) - 0.5 ln(1 + rank), z_d = z_t +
delta N(0,1).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "synth.hip")
LIB = os.path.join(HERE, "libsmcsd_synth.so")

STREAM_RANK, STREAM_TARGET, STREAM_DRAFT, STREAM_TOKENS, STREAM_UNIFORM, STREAM_RESAMPLE, STREAM_PACER = range(7)


def build() -> str:
    subprocess.check_call(["hipcc", "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
                           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-o", LIB, SRC],
                          stderr=subprocess.DEVNULL if os.environ.get("SMCSD_QUIET_BUILD") else None)
    return LIB


_lib = None


def lib():
    """Load the generator library (build first with ``build()``)."""
    global _lib
    if _lib is None:
        try:  # the HIP runtime torch loaded must be the one this library binds to
            import torch  # noqa: F401
        except ImportError:
            pass
        if not os.path.exists(LIB):
            raise FileNotFoundError(f"{LIB} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(LIB)
        P, I32, I64, U32, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_float
        L.synth_philox4x32_10.argtypes = [P, P, P]
        L.synth_rank_base.argtypes = [I64, U32, P, P]
        L.synth_pacer_scores.argtypes = [I32, I32, I32, U32, U32, P]
        L.synth_logits.argtypes = [I32, I64, I64, P, P, P, U32, U32, P, P, P]
        L.synth_logits.restype = I32
        L.synth_draft_tokens.argtypes = [I32, I64, I64, F, P, U32, U32, P, P]
        L.synth_draft_tokens.restype = I32
        L.synth_draft_tokens_rows.argtypes = [I32, I64, I64, F, P, P, U32, U32, P, P]
        L.synth_draft_tokens_rows.restype = I32
        L.synth_uniforms.argtypes = [I64, U32, U32, U32, P, P]
        L.synth_uniforms.restype = I32
        _lib = L
    return _lib


def _np_ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def philox4x32_10(ctr, key):
    c = np.asarray(ctr, np.uint32)
    k = np.asarray(key, np.uint32)
    out = np.zeros(4, np.uint32)
    lib().synth_philox4x32_10(_np_ptr(c), _np_ptr(k), _np_ptr(out))
    return out


def rank_base(V: int, seed: int):
    rank = np.zeros(V, np.int32)
    base = np.zeros(V, np.float32)
    lib().synth_rank_base(V, seed, _np_ptr(rank), _np_ptr(base))
    return rank, base


def pacer_scores(B, seed, step, block=4, max_blocks=4):
    """Pre-verifier stand-in scores [B, max_blocks * block] ~ U(0,1) of one step."""
    out = np.zeros((B, max_blocks * block), np.float32)
    lib().synth_pacer_scores(B, block, max_blocks, seed, step, _np_ptr(out))
    return out


@dataclass
class Config:
    name: str
    kind: str  # "sd" | "sd_ragged" | "smc" | "tree"
    V: int
    dtype: str  # "f32" | "bf16"
    T: float
    steps: int
    seed: int
    B: int = 0
    K: int = 0
    P: int = 0
    N: int = 0
    deltas: tuple = (1.0,)  # cycled over sequences (SD) or prompts (SMC)
    ess_frac: float = 0.5
    page_tokens: int = 16
    context: int = 0
    pacer: dict = field(default_factory=dict)
    tree: dict = field(default_factory=dict)  # complete tree shape: width, depth

    @property
    def L(self):
        return self.context // self.page_tokens if self.context else 0


CONFIGS = [
    Config("cfg0_sd_b1_k2_v32000_f32", "sd", V=32000, dtype="f32", T=1.0, steps=64, seed=0, B=1, K=2),
    Config("cfg1_sd_b64_k4_v32768_bf16", "sd", V=32768, dtype="bf16", T=0.7, steps=256, seed=1, B=64, K=4,
           deltas=(0.5, 1.0, 2.0)),
    Config("cfg2_smc_p1_n16_k4_v128256_bf16", "smc", V=128256, dtype="bf16", T=1.0, steps=64, seed=2, P=1, N=16,
           K=4, context=4096),
    Config("cfg3_smc_p32_n64_k8_v151936_bf16", "smc", V=151936, dtype="bf16", T=1.0, steps=128, seed=3, P=32,
           N=64, K=8, deltas=(0.5, 2.0), context=8192),
    Config("cfg4_sd_ragged_b256_v32000_bf16", "sd_ragged", V=32000, dtype="bf16", T=1.0, steps=128, seed=4, B=256,
           K=16, pacer=dict(block=4, max_blocks=4, t0=0.5, rho=1.1)),
    # token trees in the shape of the batched SD workload: 64 complete binary
    # trees of depth 3 (15 nodes, 14 draft tokens, 7 draft rows each)
    Config("tree_b64_binary_d3_v32768_bf16", "tree", V=32768, dtype="bf16", T=0.7, steps=256, seed=5, B=64,
           deltas=(0.5, 1.0, 2.0), tree=dict(width=2, depth=3)),
]


def full_tree_parents(width, depth):
    """Parents of a complete width-ary tree with depth levels below the root,
    numbered level by level (-1 at the root)."""
    par, level = [-1], [0]
    for _ in range(depth):
        nxt = []
        for p in level:
            for _ in range(width):
                par.append(p)
                nxt.append(len(par) - 1)
        level = nxt
    return par


def _torch():
    import torch

    return torch


class Generator:
    """Builds one step of inputs for a config on a torch device.

    ``lengths(scores, block, max_blocks, t0, rho) -> int32 [B]`` turns a ragged
    workload's PACER scores into draft lengths; the caller supplies it (the
    oracle in tests, the library in the benchmark), so this module holds no
    part of the rule."""

    def __init__(self, cfg: Config, device="cuda", lengths=None):
        torch = _torch()
        self.cfg = cfg
        self.lengths = lengths
        self.device = torch.device(device)
        _, base = rank_base(cfg.V, cfg.seed)
        self.base = torch.from_numpy(base).to(self.device)
        self.tdtype = torch.float32 if cfg.dtype == "f32" else torch.bfloat16
        self.bf16 = int(cfg.dtype == "bf16")

    def _stream(self):
        return ctypes.c_void_p(_torch().cuda.current_stream(self.device).cuda_stream)

    def layout(self, step):
        """(group draft-row starts d0, draft lengths Kb, per-group delta) as numpy."""
        c = self.cfg
        if c.kind == "sd":
            G, Kb = c.B, np.full(c.B, c.K, np.int32)
            delta = np.array([c.deltas[b % len(c.deltas)] for b in range(G)], np.float32)
        elif c.kind == "sd_ragged":
            G = c.B
            if self.lengths is None:
                raise ValueError("a ragged workload needs a lengths function (PACER rule)")
            pc = c.pacer
            scores = pacer_scores(c.B, c.seed, step, pc["block"], pc["max_blocks"])
            Kb = np.asarray(self.lengths(scores, pc["block"], pc["max_blocks"], pc["t0"], pc["rho"]), np.int32)
            delta = np.array([c.deltas[b % len(c.deltas)] for b in range(G)], np.float32)
        else:
            G, Kb = c.P * c.N, np.full(c.P * c.N, c.K, np.int32)
            delta = np.array([c.deltas[(i // c.N) % len(c.deltas)] for i in range(G)], np.float32)
        d0 = np.concatenate([[0], np.cumsum(Kb)]).astype(np.int64)
        return d0, Kb, delta

    def logits(self, step, d0, Kb, delta):
        torch = _torch()
        c = self.cfg
        G = len(Kb)
        rows_d = int(d0[-1])
        rows_t = rows_d + G
        draft_row = np.full(rows_t, -1, np.int32)
        delta_row = np.zeros(rows_t, np.float32)
        for g in range(G):
            t0 = int(d0[g]) + g
            delta_row[t0:t0 + Kb[g] + 1] = delta[g]
            draft_row[t0:t0 + Kb[g]] = np.arange(d0[g], d0[g] + Kb[g])
        target = torch.empty((rows_t, c.V), dtype=self.tdtype, device=self.device)
        draft = torch.empty((max(rows_d, 0), c.V), dtype=self.tdtype, device=self.device)
        dr = torch.from_numpy(draft_row).to(self.device)
        dl = torch.from_numpy(delta_row).to(self.device)
        rc = lib().synth_logits(self.bf16, rows_t, c.V, self.base.data_ptr(), dr.data_ptr(), dl.data_ptr(), c.seed,
                                step, target.data_ptr(), draft.data_ptr(), self._stream())
        assert rc == 0, rc
        tokens = torch.empty(rows_d, dtype=torch.int32, device=self.device)
        rc = lib().synth_draft_tokens(self.bf16, rows_d, c.V, c.T, draft.data_ptr(), c.seed, step, tokens.data_ptr(),
                                      self._stream())
        assert rc == 0, rc
        return target, draft, tokens

    def uniforms(self, n, stream_id, step):
        torch = _torch()
        out = torch.empty(n, dtype=torch.float32, device=self.device)
        rc = lib().synth_uniforms(n, self.cfg.seed, stream_id, step, out.data_ptr(), self._stream())
        assert rc == 0, rc
        return out

    def tree_step(self, step):
        """dict(target, draft, node_off, draft_off, parent, tokens, uniforms, M): B
        trees of the config's shape; each node with children has a draft row
        made from its own target row, and every child's token is drawn from
        its parent's draft row."""
        torch = _torch()
        c = self.cfg
        par = full_tree_parents(c.tree["width"], c.tree["depth"])
        M = len(par)
        internal = sorted({p for p in par[1:]})
        rank = {n: i for i, n in enumerate(internal)}
        D = len(internal)
        B = c.B
        draft_row = np.full(B * M, -1, np.int32)
        delta_row = np.zeros(B * M, np.float32)
        rowmap = np.zeros(B * M, np.int32)  # the draft row each node's token is drawn from
        for b in range(B):
            delta_row[b * M:(b + 1) * M] = c.deltas[b % len(c.deltas)]
            for n in internal:
                draft_row[b * M + n] = b * D + rank[n]
            for n in range(1, M):
                rowmap[b * M + n] = b * D + rank[par[n]]
            rowmap[b * M] = b * D  # the root's token is not read
        target = torch.empty((B * M, c.V), dtype=self.tdtype, device=self.device)
        draft = torch.empty((B * D, c.V), dtype=self.tdtype, device=self.device)
        dr, dl, rm = (torch.from_numpy(a).to(self.device) for a in (draft_row, delta_row, rowmap))
        rc = lib().synth_logits(self.bf16, B * M, c.V, self.base.data_ptr(), dr.data_ptr(), dl.data_ptr(), c.seed,
                                step, target.data_ptr(), draft.data_ptr(), self._stream())
        assert rc == 0, rc
        tokens = torch.empty(B * M, dtype=torch.int32, device=self.device)
        rc = lib().synth_draft_tokens_rows(self.bf16, B * M, c.V, c.T, draft.data_ptr(), rm.data_ptr(), c.seed, step,
                                           tokens.data_ptr(), self._stream())
        assert rc == 0, rc
        i32 = lambda a: torch.from_numpy(np.asarray(a, np.int32)).to(self.device)  # noqa: E731
        return dict(target=target, draft=draft, node_off=i32(np.arange(0, B * M + 1, M)),
                    draft_off=i32(np.arange(0, B * D + 1, D)), parent=i32(np.tile(par, B)), tokens=tokens,
                    uniforms=self.uniforms(B * M, STREAM_UNIFORM, step), M=M, D=D, _keep=(dr, dl, rm))

    def sd_step(self, step):
        """dict(target, draft, tokens, uniforms, offsets or None, total_draft_rows, K, Kb)."""
        torch = _torch()
        d0, Kb, delta = self.layout(step)
        target, draft, tokens = self.logits(step, d0, Kb, delta)
        u = self.uniforms(target.shape[0], STREAM_UNIFORM, step)
        offsets = None
        if self.cfg.kind == "sd_ragged":
            offsets = torch.from_numpy(d0.astype(np.int32)).to(self.device)
        return dict(target=target, draft=draft, tokens=tokens, uniforms=u, offsets=offsets,
                    total_draft_rows=int(d0[-1]), K=int(self.cfg.K), Kb=Kb)

    def smc_step(self, step):
        """dict(target, draft, tokens, bonus_u, resample_u)."""
        c = self.cfg
        d0, Kb, delta = self.layout(step)
        target, draft, tokens = self.logits(step, d0, Kb, delta)
        return dict(target=target, draft=draft, tokens=tokens,
                    bonus_u=self.uniforms(c.P * c.N, STREAM_UNIFORM, step),
                    resample_u=self.uniforms(c.P, STREAM_RESAMPLE, step))


def initial_page_table(P, N, L):
    """pt[p, n, j] = (p*N + n)*L + j: every page id distinct, so a permutation is visible."""
    return np.arange(P * N * L, dtype=np.int32).reshape(P * N, L)


def step_bytes(cfg: Config, Kb=None) -> int:
    """Algorithmic logit bytes of one step: every target and draft row read once."""
    e = 4 if cfg.dtype == "f32" else 2
    if cfg.kind == "tree":
        par = full_tree_parents(cfg.tree["width"], cfg.tree["depth"])
        return cfg.B * (len(par) + len(set(par[1:]))) * cfg.V * e
    if cfg.kind == "smc":
        rows = cfg.P * cfg.N * (2 * cfg.K + 1)
    elif Kb is not None:
        rows = int(np.sum(2 * np.asarray(Kb) + 1))
    else:
        rows = cfg.B * (2 * cfg.K + 1)
    return rows * cfg.V * e


def verified_positions(cfg: Config, Kb=None) -> int:
    """Draft positions submitted for verification in one step."""
    if cfg.kind == "smc":
        return cfg.P * cfg.N * cfg.K
    if cfg.kind == "tree":
        return cfg.B * (len(full_tree_parents(cfg.tree["width"], cfg.tree["depth"])) - 1)
    if Kb is not None:
        return int(np.sum(Kb))
    return cfg.B * cfg.K
