"""Plain fp64 CPU oracle of the verify-and-sample step (test infrastructure).

Only the test suite, the package smoke check and the CPU-baseline leg of the
benchmark may import this module.  The product library never does; it shares no
code with this C file.  See ``oracle.c`` for the definitions and the passages of
the pages each one follows.

The wrappers take numpy arrays (bf16 logits as ``uint16`` bit patterns) and
return numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

FLAG_NONFINITE = 1
FLAG_ZERO_RESIDUAL = 2
FLAG_ZERO_WEIGHTS = 4
FLAG_CDF_CLAMP = 8

DTYPE_F32 = 0
DTYPE_BF16 = 1

# value the wrappers fill output buffers with before a call
UNWRITTEN = -7


def build(src: str = SRC, out: str = LIB, strict: bool = True) -> str:
    """Compile the oracle with plain gcc (-O2, IEEE semantics, no fast-math)."""
    warn = ["-Wall", "-Werror"] if strict else ["-w"]
    subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", *warn, "-o", out, src, "-lm"])
    return out


_P = ctypes.c_void_p
_I = ctypes.c_int
_I64 = ctypes.c_int64
_D = ctypes.c_double


def _declare(lib):
    lib.oracle_row_stats.argtypes = [_I, _P, _I64, _D, _P, _P]
    lib.oracle_row_stats.restype = _I
    lib.oracle_logprob.argtypes = [_I, _P, _I64, _D, _I64]
    lib.oracle_logprob.restype = _D
    lib.oracle_sd_verify.argtypes = [_I, _I, _I, _I64, _D, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]
    lib.oracle_sd_verify.restype = _I
    lib.oracle_sd_final_cdf.argtypes = [_I, _I, _I, _I64, _D, _P, _P, _P, _I, _P]
    lib.oracle_sd_final_cdf.restype = _I
    lib.oracle_smc_step.argtypes = [_I, _I, _I, _I, _I64, _D, _D] + [_P] * 8 + [_I] + [_P] * 9
    lib.oracle_smc_step.restype = _I
    lib.oracle_smc_step_power.argtypes = [_I, _I, _I, _I, _I64, _D, _D, _D] + [_P] * 8 + [_I] + [_P] * 9
    lib.oracle_smc_step_power.restype = _I
    lib.oracle_pages_append.argtypes = [_I, _I, _I, _I, _I64] + [_P] * 8
    lib.oracle_pages_append.restype = _I
    lib.oracle_pages_resample.argtypes = [_I, _I, _I, _I, _I64] + [_P] * 8
    lib.oracle_pages_resample.restype = _I
    lib.oracle_draft_sample.argtypes = [_I, _I64, _I64, _D, _P, _P, _P, _P]
    lib.oracle_draft_sample.restype = _I
    lib.oracle_pacer_lengths.argtypes = [_I, _I, _I, _D, _D, _P, _P, _P]
    lib.oracle_pacer_lengths.restype = None
    lib.oracle_tree_verify.argtypes = [_I, _I, _I64, _D] + [_P] * 13
    lib.oracle_tree_verify.restype = _I
    lib.oracle_tree_final_cdf.argtypes = [_I, _I, _I64, _D] + [_P] * 5 + [_I, _P]
    lib.oracle_tree_final_cdf.restype = _I
    return lib


_lib_cache: dict = {}


def load(path: str = LIB):
    """Load (building first if absent) an oracle shared object."""
    if path not in _lib_cache:
        if not os.path.exists(path):
            if path != LIB:
                raise FileNotFoundError(path)
            build()
        _lib_cache[path] = _declare(ctypes.CDLL(path))
    return _lib_cache[path]


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _dtype_code(logits: np.ndarray) -> int:
    if logits.dtype == np.float32:
        return DTYPE_F32
    if logits.dtype == np.uint16:
        return DTYPE_BF16
    raise TypeError(f"logits must be float32 or uint16 (bf16 bits), got {logits.dtype}")


def row_stats(row: np.ndarray, T: float, lib=None):
    """(M, log S, bad) of one row: M = max z/T, S = sum exp(z/T - M)."""
    lib = lib or load()
    row = np.ascontiguousarray(row)
    M = ctypes.c_double()
    lS = ctypes.c_double()
    bad = lib.oracle_row_stats(_dtype_code(row), _ptr(row), row.shape[-1], T, ctypes.byref(M), ctypes.byref(lS))
    return M.value, lS.value, bad


def logprob(row: np.ndarray, T: float, i: int, lib=None) -> float:
    lib = lib or load()
    row = np.ascontiguousarray(row)
    return lib.oracle_logprob(_dtype_code(row), _ptr(row), row.shape[-1], T, int(i))


def sd_verify(target, draft, tokens, uniforms, T, K=None, offsets=None, lib=None):
    """Standard SD verify of B sequences.

    Fixed K: target [B*(K+1), V], draft [B*K, V], tokens [B*K],
    uniforms [B*(K+1)].  CSR: ``offsets`` [B+1] over draft rows; target rows
    and uniforms of sequence b start at offsets[b] + b.

    Returns dict(num_accepted, final_token, flags, accept_margin, sample_margin).
    """
    lib = lib or load()
    target = np.ascontiguousarray(target)
    draft = np.ascontiguousarray(draft)
    V = target.shape[-1]
    tokens = np.ascontiguousarray(tokens, dtype=np.int32)
    uniforms = np.ascontiguousarray(uniforms, dtype=np.float32)
    if offsets is not None:
        offsets = np.ascontiguousarray(offsets, dtype=np.int32)
        B = offsets.shape[0] - 1
        K = int(np.max(np.diff(offsets))) if B > 0 else 0
    else:
        B = target.shape[0] // (K + 1)
    nd = tokens.shape[0]
    # outputs start at a sentinel (not 0), so an output left unwritten shows
    na = np.full(B, UNWRITTEN, np.int32)
    ft = np.full(B, UNWRITTEN, np.int32)
    fl = np.zeros(1, np.uint32)
    am = np.full(max(nd, 1), float(UNWRITTEN))
    sm = np.full(max(B, 1), float(UNWRITTEN))
    lib.oracle_sd_verify(_dtype_code(target), B, K, V, T, _ptr(target), _ptr(draft), _ptr(tokens),
                         _ptr(uniforms), _ptr(offsets), _ptr(na), _ptr(ft), _ptr(fl), _ptr(am), _ptr(sm))
    return dict(num_accepted=na, final_token=ft, flags=int(fl[0]), accept_margin=am[:nd], sample_margin=sm[:B])


def sd_final_cdf(target, draft, b, n, T, K=None, offsets=None, lib=None):
    """Normalised CDF of the distribution sequence b's final token is drawn from."""
    lib = lib or load()
    target = np.ascontiguousarray(target)
    draft = np.ascontiguousarray(draft)
    V = target.shape[-1]
    if offsets is not None:
        offsets = np.ascontiguousarray(offsets, dtype=np.int32)
    cdf = np.zeros(V)
    fl = lib.oracle_sd_final_cdf(_dtype_code(target), int(b), int(K or 0), V, T, _ptr(target), _ptr(draft),
                                 _ptr(offsets), int(n), _ptr(cdf))
    return cdf, fl


def smc_step(target, draft, tokens, bonus_u, resample_u, logw, T, ess_frac, P, N, K, pt_in=None, lib=None,
             beta=None):
    """One SMC-SD reweight / ESS / systematic-resample step (with ``beta``, the
    power target: increments beta log p - log q, bonus from softmax(beta z/T)).

    ``logw`` (float32 [P*N]) is not modified; the updated log-weights are
    returned.  Returns dict(logw, bonus, ancestors, ess, resampled, pt_out,
    flags, cum_weight, bonus_margin, ess_margin, resample_margin).
    """
    lib = lib or load()
    target = np.ascontiguousarray(target)
    draft = np.ascontiguousarray(draft)
    V = target.shape[-1]
    tokens = np.ascontiguousarray(tokens, dtype=np.int32)
    bonus_u = np.ascontiguousarray(bonus_u, dtype=np.float32)
    resample_u = np.ascontiguousarray(resample_u, dtype=np.float32)
    lw = np.array(logw, dtype=np.float32, copy=True)
    PN = P * N
    L = 0
    pt_out = None
    if pt_in is not None:
        pt_in = np.ascontiguousarray(pt_in, dtype=np.int32)
        L = pt_in.size // max(PN, 1)
        pt_out = np.full_like(pt_in, UNWRITTEN)
    bonus = np.full(PN, UNWRITTEN, np.int32)
    anc = np.full(PN, UNWRITTEN, np.int32)
    ess = np.full(P, UNWRITTEN, np.float32)
    res = np.full(P, UNWRITTEN, np.int32)
    fl = np.zeros(1, np.uint32)
    cw = np.full(max(PN, 1), float(UNWRITTEN))
    bm = np.full(max(PN, 1), float(UNWRITTEN))
    em = np.full(max(P, 1), float(UNWRITTEN))
    rm = np.full(max(P, 1), float(UNWRITTEN))
    tail = (_ptr(target), _ptr(draft), _ptr(tokens), _ptr(bonus_u), _ptr(resample_u), _ptr(lw), _ptr(pt_in),
            _ptr(pt_out), L, _ptr(bonus), _ptr(anc), _ptr(ess), _ptr(res), _ptr(fl), _ptr(cw), _ptr(bm), _ptr(em),
            _ptr(rm))
    if beta is None:
        lib.oracle_smc_step(_dtype_code(target), P, N, K, V, T, ess_frac, *tail)
    else:
        lib.oracle_smc_step_power(_dtype_code(target), P, N, K, V, T, float(beta), ess_frac, *tail)
    return dict(logw=lw, bonus=bonus, ancestors=anc, ess=ess, resampled=res, pt_out=pt_out, flags=int(fl[0]),
                cum_weight=cw[:PN], bonus_margin=bm[:PN], ess_margin=em[:P], resample_margin=rm[:P])


def pages_append(table, lens, ref, free_pages, free_count, S, A, lib=None):
    """Paged-KV append of A tokens per particle (copy-on-write of shared tail
    pages, new pages from the free stack).  Inputs are not modified; returns
    dict(status, table, len, ref, free_pages, free_count, slots, cow)."""
    lib = lib or load()
    table = np.array(table, np.int32, copy=True)
    R, L = table.shape
    lens = np.array(lens, np.int32, copy=True)
    ref = np.array(ref, np.int32, copy=True)
    free_pages = np.array(free_pages, np.int32, copy=True)
    fc = np.array([free_count], np.int32)
    slots = np.full(max(R * A, 1), UNWRITTEN, np.int32)
    cow = np.full(max(3 * R, 3), UNWRITTEN, np.int32)
    nc = np.zeros(1, np.int32)
    st = lib.oracle_pages_append(R, L, S, A, ref.size, _ptr(table), _ptr(lens), _ptr(ref), _ptr(free_pages),
                                 _ptr(fc), _ptr(slots), _ptr(cow), _ptr(nc))
    return dict(status=int(st), table=table, len=lens, ref=ref, free_pages=free_pages, free_count=int(fc[0]),
                slots=slots[:R * A].reshape(R, A), cow=cow[:3 * int(nc[0])].reshape(-1, 3))


def pages_resample(P, N, ancestors, table_old, table_new, lens, ref, free_pages, free_count, S, lib=None):
    """Paged-KV bookkeeping of a resampling: lengths by ancestor, reference
    counts, freed pages pushed.  Returns dict(status, len, ref, free_pages, free_count)."""
    lib = lib or load()
    table_old = np.ascontiguousarray(table_old, np.int32)
    table_new = np.ascontiguousarray(table_new, np.int32)
    L = table_old.shape[1]
    anc = np.ascontiguousarray(ancestors, np.int32)
    lens = np.ascontiguousarray(lens, np.int32)
    len_out = np.full_like(lens, UNWRITTEN)
    ref = np.array(ref, np.int32, copy=True)
    free_pages = np.array(free_pages, np.int32, copy=True)
    fc = np.array([free_count], np.int32)
    st = lib.oracle_pages_resample(P, N, L, S, ref.size, _ptr(anc), _ptr(table_old), _ptr(table_new), _ptr(lens),
                                   _ptr(len_out), _ptr(ref), _ptr(free_pages), _ptr(fc))
    return dict(status=int(st), len=len_out, ref=ref, free_pages=free_pages, free_count=int(fc[0]))


def draft_sample(logits, uniforms, T, lib=None):
    """One token per row from softmax(z / T) by inverse CDF with the row's
    uniform.  Returns dict(tokens, margin, flags)."""
    lib = lib or load()
    logits = np.ascontiguousarray(logits)
    R, V = logits.shape
    u = np.ascontiguousarray(uniforms, np.float32)
    assert u.size == R
    tokens = np.full(R, UNWRITTEN, np.int32)
    margin = np.full(R, float(UNWRITTEN), np.float64)
    fl = lib.oracle_draft_sample(_dtype_code(logits), R, V, T, _ptr(logits), _ptr(u), _ptr(tokens), _ptr(margin))
    return dict(tokens=tokens, margin=margin, flags=int(fl))


def pacer_lengths(scores, block, max_blocks, t0, rho, lib=None):
    """PACER draft lengths from scores [B, max_blocks * block].  Returns
    (lengths [B], offsets [B + 1])."""
    lib = lib or load()
    scores = np.ascontiguousarray(scores, np.float32)
    B = scores.shape[0]
    assert scores.shape == (B, max_blocks * block)
    lengths = np.full(B, UNWRITTEN, np.int32)
    offsets = np.full(B + 1, UNWRITTEN, np.int32)
    lib.oracle_pacer_lengths(B, block, max_blocks, t0, rho, _ptr(scores), _ptr(lengths), _ptr(offsets))
    return lengths, offsets


def tree_verify(target, draft, node_off, draft_off, parent, tokens, uniforms, T, lib=None):
    """Multi-draft speculative sampling over B token trees.

    node_off [B+1] CSR over nodes (one target row, one uniform, one parent and
    one token per node); draft_off [B+1] CSR over the draft rows (one per node
    with children, in node order); parent: local parent index (-1 at the root);
    uniforms[node_off[b] + n]: acceptance uniform of node n >= 1, the root's
    slot holding the final draw's uniform.

    Returns dict(num_accepted, last_node, final_token, flags, accept_margin,
    sample_margin, status) -- status -1 when a tree is malformed.
    """
    lib = lib or load()
    target = np.ascontiguousarray(target)
    draft = np.ascontiguousarray(draft)
    V = target.shape[-1]
    node_off = np.ascontiguousarray(node_off, dtype=np.int32)
    draft_off = np.ascontiguousarray(draft_off, dtype=np.int32)
    parent = np.ascontiguousarray(parent, dtype=np.int32)
    tokens = np.ascontiguousarray(tokens, dtype=np.int32)
    uniforms = np.ascontiguousarray(uniforms, dtype=np.float32)
    B = node_off.shape[0] - 1
    nn = int(node_off[-1]) if B >= 0 else 0
    na = np.full(max(B, 1), UNWRITTEN, np.int32)
    ln = np.full(max(B, 1), UNWRITTEN, np.int32)
    ft = np.full(max(B, 1), UNWRITTEN, np.int32)
    fl = np.zeros(1, np.uint32)
    am = np.full(max(nn, 1), float(UNWRITTEN))
    sm = np.full(max(B, 1), float(UNWRITTEN))
    st = lib.oracle_tree_verify(_dtype_code(target), B, V, T, _ptr(node_off), _ptr(draft_off), _ptr(parent),
                                _ptr(tokens), _ptr(target), _ptr(draft), _ptr(uniforms), _ptr(na), _ptr(ln),
                                _ptr(ft), _ptr(fl), _ptr(am), _ptr(sm))
    return dict(num_accepted=na[:B], last_node=ln[:B], final_token=ft[:B], flags=int(fl[0]), accept_margin=am[:nn],
                sample_margin=sm[:B], status=st)


def tree_final_cdf(target, draft, node_off, draft_off, parent, b, u, T, lib=None):
    """Normalised CDF of tree b's final draw when the walk stops at node u."""
    lib = lib or load()
    target = np.ascontiguousarray(target)
    draft = np.ascontiguousarray(draft)
    V = target.shape[-1]
    node_off = np.ascontiguousarray(node_off, dtype=np.int32)
    draft_off = np.ascontiguousarray(draft_off, dtype=np.int32)
    parent = np.ascontiguousarray(parent, dtype=np.int32)
    cdf = np.zeros(V)
    fl = lib.oracle_tree_final_cdf(_dtype_code(target), int(b), V, T, _ptr(node_off), _ptr(draft_off),
                                   _ptr(parent), _ptr(target), _ptr(draft), int(u), _ptr(cdf))
    return cdf, fl
