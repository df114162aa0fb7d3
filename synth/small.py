"""Small seeded synthetic cases built on the host with numpy (edge-case shapes).

Same recipe as the GPU generator: z_t = scale * N(0,1) (+ optional rank prior),
z_d = z_t + delta * N(0,1), rounded once to the stored dtype; draft tokens are
Gumbel-max draws from softmax(z_d / T); uniforms are U[0,1) in fp32.
"""
from __future__ import annotations

import numpy as np


def to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest even (NaN kept NaN)."""
    b = np.asarray(x32, np.float32).view(np.uint32).astype(np.uint64)
    nan = np.isnan(np.asarray(x32, np.float32))
    r = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)
    r[nan] = 0x7FC0
    return r


def gumbel_tokens(rng, z_draft_f64: np.ndarray, T: float) -> np.ndarray:
    g = -np.log(-np.log(rng.random(z_draft_f64.shape).clip(1e-300, 1.0 - 1e-16)))
    return np.argmax(z_draft_f64 / T + g, axis=-1).astype(np.int32)


def stored(z32: np.ndarray, dtype: str):
    """(array passed to the library/oracle, float64 view of the stored values)."""
    if dtype == "bf16":
        bits = to_bf16_bits(z32)
        return bits, (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    z = np.asarray(z32, np.float32)
    return z, z.astype(np.float64)


def sd_case(seed, B, V, T=1.0, K=None, lengths=None, delta=1.0, dtype="f32", scale=3.0, prior=True):
    """Fixed-K (``K``) or ragged (``lengths``) SD inputs as numpy arrays."""
    rng = np.random.default_rng(seed)
    Kb = np.full(B, K, np.int32) if lengths is None else np.asarray(lengths, np.int32)
    d0 = np.concatenate([[0], np.cumsum(Kb)]).astype(np.int64)
    rows_d = int(d0[-1])
    rows_t = rows_d + B
    base = -0.5 * np.log1p(rng.permutation(V)) if prior else np.zeros(V)
    zt = (scale * rng.standard_normal((rows_t, V)) + base).astype(np.float32)
    zd = np.zeros((rows_d, V), np.float32)
    dl = np.broadcast_to(np.asarray(delta, np.float64), (B,))
    for b in range(B):
        t0 = int(d0[b]) + b
        for j in range(int(Kb[b])):
            zd[d0[b] + j] = (zt[t0 + j] + dl[b] * rng.standard_normal(V)).astype(np.float32)
    tgt, _ = stored(zt, dtype)
    drf, drf64 = stored(zd, dtype)
    tok = gumbel_tokens(rng, drf64, T) if rows_d else np.zeros(0, np.int32)
    u = rng.random(rows_t).astype(np.float32)
    offsets = None if lengths is None else d0.astype(np.int32)
    return dict(target=tgt, draft=drf, tokens=tok, uniforms=u, offsets=offsets, K=int(Kb.max()) if B else 0,
                Kb=Kb, T=T, dtype=dtype)


def smc_case(seed, P, N, K, V, T=1.0, delta=1.0, dtype="f32", scale=3.0, L=4, logw_scale=1.0):
    rng = np.random.default_rng(seed)
    PN = P * N
    base = -0.5 * np.log1p(rng.permutation(V))
    zt = (scale * rng.standard_normal((PN * (K + 1), V)) + base).astype(np.float32)
    zd = (zt.reshape(PN, K + 1, V)[:, :K] + delta * rng.standard_normal((PN, K, V))).astype(np.float32)
    zd = zd.reshape(PN * K, V)
    tgt, _ = stored(zt, dtype)
    drf, drf64 = stored(zd, dtype)
    tok = gumbel_tokens(rng, drf64, T) if PN * K else np.zeros(0, np.int32)
    return dict(target=tgt, draft=drf, tokens=tok, bonus_u=rng.random(PN).astype(np.float32),
                resample_u=rng.random(P).astype(np.float32),
                logw=(logw_scale * rng.standard_normal(PN)).astype(np.float32),
                pt=np.arange(PN * L, dtype=np.int32).reshape(PN, L), P=P, N=N, K=K, T=T, dtype=dtype)


def pages_state(seed, P, N, L, S, M, max_len=None, fixed_len=None):
    """A paged-KV state to start from: every particle owns distinct pages for a
    random length (at most max_len tokens, default half the row; or
    fixed_len for all), reference
    count 1 on them, every other page on the free stack (shuffled).  Returns
    dict(table [P*N, L] with -1 past the used entries, len, ref [M],
    free_pages [M], free_count)."""
    rng = np.random.default_rng(seed)
    R = P * N
    max_len = L * S // 2 if max_len is None else max_len
    lens = rng.integers(0, max_len + 1, R).astype(np.int32) if fixed_len is None else np.full(R, fixed_len, np.int32)
    perm = rng.permutation(M).astype(np.int32)
    table = np.full((R, L), -1, np.int32)
    ref = np.zeros(M, np.int32)
    nxt = 0
    for r in range(R):
        u = (int(lens[r]) + S - 1) // S
        table[r, :u] = perm[nxt:nxt + u]
        ref[perm[nxt:nxt + u]] = 1
        nxt += u
    assert nxt <= M, "pool too small for the lengths drawn"
    free = np.zeros(M, np.int32)
    free[:M - nxt] = perm[nxt:]
    return dict(table=table, len=lens, ref=ref, free_pages=free, free_count=M - nxt)


def sorted_ancestors(seed, P, N, concentrate=0.0):
    """Ancestor indices per prompt, ascending (as systematic resampling gives),
    drawn with replacement; concentrate in [0, 1) favours low indices."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(P):
        w = (1.0 - concentrate) ** np.arange(N) if concentrate else np.ones(N)
        out.append(np.sort(rng.choice(N, N, p=w / w.sum())))
    return np.concatenate(out).astype(np.int32)


def tree_parents(kind, rng=None, M=None, width=2, depth=3):
    """Parent lists (local indices, -1 at the root) of token-tree shapes:
    "root" (one node), "chain" (M nodes), "star" (a root with M-1 children),
    "full" (complete `width`-ary tree of `depth` levels below the root, nodes
    numbered level by level) and "random" (M nodes, each parent drawn
    uniformly from the earlier nodes)."""
    if kind == "root":
        return [-1]
    if kind == "chain":
        return list(range(-1, M - 1))
    if kind == "star":
        return [-1] + [0] * (M - 1)
    if kind == "full":
        par, level = [-1], [0]
        for _ in range(depth):
            nxt = []
            for p in level:
                for _ in range(width):
                    par.append(p)
                    nxt.append(len(par) - 1)
            level = nxt
        return par
    if kind == "random":
        return [-1] + [int(rng.integers(0, n)) for n in range(1, M)]
    raise ValueError(kind)


def tree_case(seed, parents_list, V, T=1.0, delta=1.0, dtype="f32", scale=3.0, prior=True):
    """Token trees as numpy arrays in the layout of tree_verify.

    Each node has a target row z_t = scale * N(0,1) (+ rank prior); each node
    with children has a draft row z_d = z_t + delta * N(0,1) of its own target
    row; every child's token is a Gumbel-max draw from its parent's draft
    distribution (iid across siblings); uniforms U[0,1) per node.  ``delta``
    may be one value or one per tree."""
    rng = np.random.default_rng(seed)
    B = len(parents_list)
    base = -0.5 * np.log1p(rng.permutation(V)) if prior else np.zeros(V)
    dl = np.broadcast_to(np.asarray(delta, np.float64), (B,))
    node_off, draft_off = [0], [0]
    zt_rows, zd_rows, par_all, internal_of = [], [], [], []
    for b, par in enumerate(parents_list):
        M = len(par)
        zt = (scale * rng.standard_normal((M, V)) + base).astype(np.float32)
        internal = sorted({p for p in par[1:]})
        zd = (zt[internal] + dl[b] * rng.standard_normal((len(internal), V))).astype(np.float32)
        zt_rows.append(zt)
        zd_rows.append(zd)
        par_all.extend(par)
        internal_of.append(internal)
        node_off.append(node_off[-1] + M)
        draft_off.append(draft_off[-1] + len(internal))
    tgt, _ = stored(np.concatenate(zt_rows) if zt_rows else np.zeros((0, V), np.float32), dtype)
    zd_all = np.concatenate(zd_rows) if draft_off[-1] else np.zeros((0, V), np.float32)
    drf, drf64 = stored(zd_all, dtype)
    tokens = np.zeros(node_off[-1], np.int32)
    for b, par in enumerate(parents_list):
        rank = {p: i for i, p in enumerate(internal_of[b])}
        kids = list(range(1, len(par)))
        if kids:
            rows = np.stack([drf64[draft_off[b] + rank[par[n]]] for n in kids])
            tokens[node_off[b] + 1:node_off[b + 1]] = gumbel_tokens(rng, rows, T)
    u = rng.random(node_off[-1]).astype(np.float32)
    return dict(target=tgt, draft=drf, node_off=np.array(node_off, np.int32), draft_off=np.array(draft_off, np.int32),
                parent=np.array(par_all, np.int32), tokens=tokens, uniforms=u, T=T, dtype=dtype)
