"""smc_resampling_amd -- MI355X (gfx950) verify-and-sample step of speculative
decoding and SMC speculative decoding.

Thin binding over the C ABI in ``include/smcsd.h`` (``libsmcsd.so``): it only
marshals arguments.  torch tensors provide device memory and the current HIP
stream; every step of the computation runs in the library's HIP kernels.
There is no CPU fallback: importing fails loudly when the library is missing.
"""
from __future__ import annotations

import contextlib
import ctypes
import os

import torch

__all__ = [
    "sd_verify", "smc_reweight_resample", "sd_verify_workspace_bytes", "smc_workspace_bytes",
    "prepare_sd_verify", "prepare_smc_reweight_resample", "status_string", "abi_version", "lib", "SmcsdError",
    "FLAG_NONFINITE", "FLAG_ZERO_RESIDUAL", "FLAG_ZERO_WEIGHTS", "FLAG_CDF_CLAMP", "FLAG_BAD_INPUT",
    "FLAG_PAGES_FULL", "FLAG_PAGES_EXHAUSTED", "FLAG_WAIT_EXPIRED",
    "new_workspace", "time_next_call", "smc_pages_workspace_bytes", "smc_pages_append", "smc_pages_resample",
    "draft_sample_workspace_bytes", "prepare_draft_sample", "draft_sample", "pacer_lengths",
    "tree_verify_workspace_bytes", "prepare_tree_verify", "tree_verify", "TREE_MAX_NODES", "read_ceiling",
    "NOALLOC_SCRATCH_BYTES", "phase_stamps", "STAMP_WGS", "STAMP_EVENTS",
]

HERE = os.path.dirname(os.path.abspath(__file__))
# SMCSD_LIBRARY names another build of the same library (a measurement build
# with different compile options); by default the one built here
LIB_PATH = os.environ.get("SMCSD_LIBRARY") or os.path.join(HERE, "libsmcsd.so")

SMCSD_OK, SMCSD_ERR_INVALID_ARG, SMCSD_ERR_UNSUPPORTED, SMCSD_ERR_WORKSPACE, SMCSD_ERR_HIP = range(5)
SMCSD_F32, SMCSD_BF16 = 0, 1
FLAG_NONFINITE, FLAG_ZERO_RESIDUAL, FLAG_ZERO_WEIGHTS, FLAG_CDF_CLAMP, FLAG_BAD_INPUT = 1, 2, 4, 8, 16
FLAG_PAGES_FULL, FLAG_PAGES_EXHAUSTED, FLAG_WAIT_EXPIRED = 32, 64, 128
WORKSPACE_ALIGN = 256
TREE_MAX_NODES = 256
NOALLOC_SCRATCH_BYTES = 32 << 20
STAMP_WGS, STAMP_EVENTS = 4096, 16

_P, _I32, _I64, _F, _SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t

_SIGNATURES = {
    "smcsd_abi_version": ([], _I32),
    "smcsd_status_string": ([_I32], ctypes.c_char_p),
    "smcsd_time_next_call": ([_P, _P, _P, _P], None),
    "smcsd_read_ceiling": ([_P, _SZ, _P, _SZ, _P, _P, _P, _P], _I32),
    "smcsd_phase_stamps": ([_P, _SZ, _I32], _I32),
    "sd_verify_workspace_bytes": ([_I32, _I32, _I32, _I32, _I64], _SZ),
    "sd_verify": ([_I32, _I32, _I32, _I32, _F, _P, _P, _P, _P, _P, _I64, _P, _P, _P, _P, _SZ, _P], _I32),
    "smc_workspace_bytes": ([_I32, _I32, _I32, _I32, _I32], _SZ),
    "smc_reweight_resample": ([_I32, _I32, _I32, _I32, _I32, _F, _F, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _P, _P,
                               _P, _P, _P, _P, _SZ, _P], _I32),
    "smc_reweight_resample_power": ([_I32, _I32, _I32, _I32, _I32, _F, _F, _F, _P, _P, _P, _P, _P, _P, _P, _P, _I32,
                                     _P, _P, _P, _P, _P, _P, _SZ, _P], _I32),
    "smc_reweight_resample_noalloc": ([_I32, _I32, _I32, _I32, _I32, _F, _F, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _P,
                                       _P, _P, _P, _P, _P], _I32),
    "draft_sample_workspace_bytes": ([_I32, _I32, _I32], _SZ),
    "draft_sample": ([_I32, _I32, _I32, _F, _P, _P, _P, _P, _P, _SZ, _P], _I32),
    "pacer_lengths": ([_I32, _I32, _I32, ctypes.c_double, ctypes.c_double, _P, _P, _P, _P], _I32),
    "tree_verify_workspace_bytes": ([_I32, _I32, _I32, _I64, _I64], _SZ),
    "tree_verify": ([_I32, _I32, _I32, _F, _P, _P, _P, _I64, _P, _P, _I64, _P, _P, _P, _P, _P, _P, _P, _SZ, _P],
                    _I32),
    "smc_pages_workspace_bytes": ([_I32, _I32, _I32, _I64], _SZ),
    "smc_pages_append": ([_I32, _I32, _I32, _I32, _I32, _I64] + [_P] * 10 + [_SZ, _P], _I32),
    "smc_pages_resample": ([_I32, _I32, _I32, _I32, _I64] + [_P] * 9 + [_SZ, _P], _I32),
}


class SmcsdError(RuntimeError):
    pass


def _load(path: str = LIB_PATH):
    if not os.path.exists(path):
        raise ImportError(f"smc_resampling_amd: {path} is not built (run __graft_entry__.build()); "
                          "there is no CPU fallback")
    L = ctypes.CDLL(path)
    for name, (args, res) in _SIGNATURES.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = res
    return L


_lib = _load()


def lib():
    """The raw ctypes handle of libsmcsd.so."""
    return _lib


def abi_version() -> int:
    return _lib.smcsd_abi_version()


def time_next_call(stream_start=None, stream_stop=None, tail_start=None, tail_stop=None) -> None:
    """Have this thread's next library call attach the given events (timing
    torch.cuda.Event objects whose handles exist, i.e. recorded once, or None)
    to the start and stop of its streaming kernel and its decision kernel
    (benchmark aid)."""
    h = [None if e is None else e.cuda_event for e in (stream_start, stream_stop, tail_start, tail_stop)]
    _lib.smcsd_time_next_call(*h)


def read_ceiling(a, b=None, *, sink=None, start=None, stop=None, stream=None):
    """Launch the plain-read ceiling kernel over the bytes of tensors ``a``
    and ``b`` (``smcsd_read_ceiling``): the streaming kernel's loads with no
    arithmetic.  ``start`` / ``stop``: torch.cuda.Event objects whose handles
    exist (recorded once), attached to the kernel itself (measurement aid)."""
    dev = a.device
    ctx, st = _on_stream(stream, dev)
    with ctx:
        sink = sink if sink is not None else torch.empty(64, dtype=torch.int32, device=dev)
    nb = lambda t: 0 if t is None else t.numel() * t.element_size()  # noqa: E731
    _check(_lib.smcsd_read_ceiling(_ptr(a), nb(a), _ptr(b), nb(b), _ptr(sink),
                                   None if start is None else start.cuda_event,
                                   None if stop is None else stop.cuda_event, st))
    return sink


def phase_stamps(clear: bool = False):
    """The decision kernels' phase timestamps of a measurement build
    (``smcsd_phase_stamps``): uint64 numpy array [STAMP_WGS, STAMP_EVENTS, 2]
    of (100 MHz clock, phase code), 0 where nothing was recorded; ``clear``
    zeroes them after the copy.  Raises SmcsdError on the library's own build,
    which records none."""
    import numpy as np

    out = np.zeros((STAMP_WGS, STAMP_EVENTS, 2), dtype=np.uint64)
    _check(_lib.smcsd_phase_stamps(out.ctypes.data, out.nbytes, 1 if clear else 0))
    return out


def status_string(code: int) -> str:
    return _lib.smcsd_status_string(code).decode()


def _check(code: int):
    if code != SMCSD_OK:
        raise SmcsdError(status_string(code))


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return SMCSD_F32
    if t.dtype == torch.bfloat16:
        return SMCSD_BF16
    raise TypeError(f"logits must be float32 or bfloat16, got {t.dtype}")


def _ptr(t):
    return None if t is None else t.data_ptr()


def _need(t, dtype, name):
    if t is None:
        return
    if not t.is_cuda or t.dtype != dtype or not t.is_contiguous():
        raise TypeError(f"{name} must be a contiguous {dtype} tensor on a HIP device")


def _stream(device):
    return torch.cuda.current_stream(device).cuda_stream


def _on_stream(stream, device):
    """(context, handle) for one call on ``stream`` (a HIP stream handle, or
    None for the current stream).  The binding makes its own tensors (outputs,
    zeroed status flags, a temporary workspace) inside the context, so their
    allocation and zero-fill are ordered on the stream the kernels run on, and
    the caching allocator hands a temporary freed after the call only to later
    work on that same stream."""
    if stream is None:
        return contextlib.nullcontext(), _stream(device)
    return torch.cuda.stream(torch.cuda.ExternalStream(stream, device=device)), stream


def _workspace(nbytes, device, workspace):
    if nbytes == 0:
        return None, 0
    if workspace is None:  # zero-filled: the paged-KV calls need zeros on first use (the others any contents)
        workspace = torch.zeros(nbytes + WORKSPACE_ALIGN, dtype=torch.uint8, device=device)
    off = (-workspace.data_ptr()) % WORKSPACE_ALIGN
    view = workspace[off:]
    return view, view.numel()


def sd_verify_workspace_bytes(dtype_code, B, K, V, total_draft_rows) -> int:
    return _lib.sd_verify_workspace_bytes(dtype_code, B, K, V, total_draft_rows)


def smc_workspace_bytes(dtype_code, P, N, K, V) -> int:
    return _lib.smc_workspace_bytes(dtype_code, P, N, K, V)


def new_workspace(nbytes, device):
    """A zero-filled workspace of at least ``nbytes`` (plus alignment slack).

    Reuse it across calls of the same or smaller size; calls on one workspace
    must not overlap.  The verify, SMC, draft and tree calls write every
    workspace byte they read; the paged-KV calls need zeros on first use and
    leave them."""
    return torch.zeros(nbytes + WORKSPACE_ALIGN, dtype=torch.uint8, device=device)


def prepare_sd_verify(target_logits, draft_logits, draft_tokens, uniforms, temperature, *, K=None,
                      draft_offsets=None, num_accepted=None, final_token=None, status_flags=None, workspace=None,
                      stream=None):
    """Validate and marshal one sd_verify call; returns (call, outputs).

    ``call()`` enqueues the step on the stream (current stream by default) and
    raises on a non-OK status; ``outputs`` holds num_accepted, final_token and
    status_flags.  Fixed K: target [B*(K+1), V], draft [B*K, V].  Ragged:
    ``draft_offsets`` int32 [B+1] and ``K`` = largest draft length (required:
    the binding reads nothing back from the device).
    """
    dev = target_logits.device
    dt = _dtype_code(target_logits)
    V = target_logits.shape[-1]
    rows_t = target_logits.shape[0]
    rows_d = draft_logits.shape[0] if draft_logits is not None else 0
    B = rows_t - rows_d
    if draft_offsets is None:
        K = rows_d // B if B > 0 else (K or 0)
    elif K is None:
        raise ValueError("draft_offsets needs K, the largest draft length")
    for t, d, n in ((target_logits, target_logits.dtype, "target_logits"), (draft_logits, target_logits.dtype,
                    "draft_logits"), (draft_tokens, torch.int32, "draft_tokens"), (uniforms, torch.float32,
                    "uniforms"), (draft_offsets, torch.int32, "draft_offsets")):
        _need(t, d, n)
    ctx, st = _on_stream(stream, dev)
    with ctx:
        num_accepted = num_accepted if num_accepted is not None else torch.empty(B, dtype=torch.int32, device=dev)
        final_token = final_token if final_token is not None else torch.empty(B, dtype=torch.int32, device=dev)
        status_flags = status_flags if status_flags is not None else torch.zeros(1, dtype=torch.int32, device=dev)
        nbytes = sd_verify_workspace_bytes(dt, B, K, V, rows_d)
        ws, wsb = _workspace(nbytes, dev, workspace)
    args = (dt, B, K, V, float(temperature), _ptr(target_logits), _ptr(draft_logits), _ptr(draft_tokens),
            _ptr(uniforms), _ptr(draft_offsets), rows_d, _ptr(num_accepted), _ptr(final_token), _ptr(status_flags),
            _ptr(ws), wsb, st)
    fn = _lib.sd_verify
    keep = (target_logits, draft_logits, draft_tokens, uniforms, draft_offsets, ws)

    def call():
        _check(fn(*args))
        return keep

    return call, dict(num_accepted=num_accepted, final_token=final_token, status_flags=status_flags)


def sd_verify(target_logits, draft_logits, draft_tokens, uniforms, temperature, **kw):
    """Standard SD verify; returns (num_accepted, final_token, status_flags)."""
    call, out = prepare_sd_verify(target_logits, draft_logits, draft_tokens, uniforms, temperature, **kw)
    call()
    return out["num_accepted"], out["final_token"], out["status_flags"]


def prepare_smc_reweight_resample(target_logits, draft_logits, draft_tokens, bonus_uniforms, resample_uniforms,
                                  log_weights, temperature, ess_frac, P, N, K, *, page_table_in=None,
                                  page_table_out=None, bonus_token=None, ancestors=None, ess=None, resampled=None,
                                  status_flags=None, workspace=None, stream=None, beta=None, noalloc=False):
    """Validate and marshal one SMC step; returns (call, outputs).  ``log_weights``
    is updated in place when the call runs.  With ``beta``, the power-sampling
    target (``smc_reweight_resample_power``).  With ``noalloc``, the entry point
    that allocates nothing (``smc_reweight_resample_noalloc``: its scratch is a
    static device array; no workspace is made or passed)."""
    if noalloc and (beta is not None or workspace is not None):
        raise ValueError("noalloc takes neither beta nor a workspace")
    dev = target_logits.device
    dt = _dtype_code(target_logits)
    V = target_logits.shape[-1]
    PN = P * N
    for t, d, n in ((target_logits, target_logits.dtype, "target_logits"), (draft_logits, target_logits.dtype,
                    "draft_logits"), (draft_tokens, torch.int32, "draft_tokens"), (bonus_uniforms, torch.float32,
                    "bonus_uniforms"), (resample_uniforms, torch.float32, "resample_uniforms"),
                    (log_weights, torch.float32, "log_weights"), (page_table_in, torch.int32, "page_table_in"),
                    (page_table_out, torch.int32, "page_table_out")):
        _need(t, d, n)
    L = 0
    ctx, st = _on_stream(stream, dev)
    with ctx:
        if page_table_in is not None:
            L = page_table_in.numel() // max(PN, 1)
            if page_table_out is None:
                page_table_out = torch.empty_like(page_table_in)
        mk = lambda n, d: torch.empty(n, dtype=d, device=dev)  # noqa: E731
        bonus_token = bonus_token if bonus_token is not None else mk(PN, torch.int32)
        ancestors = ancestors if ancestors is not None else mk(PN, torch.int32)
        ess = ess if ess is not None else mk(P, torch.float32)
        resampled = resampled if resampled is not None else mk(P, torch.int32)
        status_flags = status_flags if status_flags is not None else torch.zeros(1, dtype=torch.int32, device=dev)
        ws, wsb = (None, 0) if noalloc else _workspace(smc_workspace_bytes(dt, P, N, K, V), dev, workspace)
    scal = (float(temperature), float(ess_frac)) if beta is None else (float(temperature), float(beta), float(ess_frac))
    args = (dt, P, N, K, V, *scal, _ptr(target_logits), _ptr(draft_logits),
            _ptr(draft_tokens), _ptr(bonus_uniforms), _ptr(resample_uniforms), _ptr(log_weights), _ptr(page_table_in),
            _ptr(page_table_out), L, _ptr(bonus_token), _ptr(ancestors), _ptr(ess), _ptr(resampled),
            _ptr(status_flags), *(() if noalloc else (_ptr(ws), wsb)), st)
    fn = (_lib.smc_reweight_resample_noalloc if noalloc else
          _lib.smc_reweight_resample if beta is None else _lib.smc_reweight_resample_power)
    keep = (target_logits, draft_logits, draft_tokens, bonus_uniforms, resample_uniforms, log_weights,
            page_table_in, ws)

    def call():
        _check(fn(*args))
        return keep

    return call, dict(bonus_token=bonus_token, ancestors=ancestors, ess=ess, resampled=resampled,
                      page_table_out=page_table_out, status_flags=status_flags, log_weights=log_weights)


def smc_reweight_resample(target_logits, draft_logits, draft_tokens, bonus_uniforms, resample_uniforms, log_weights,
                          temperature, ess_frac, P, N, K, **kw):
    """One SMC-SD step (``beta=...``: power-sampling target); ``log_weights`` is
    updated in place.  Returns a dict of outputs."""
    call, out = prepare_smc_reweight_resample(target_logits, draft_logits, draft_tokens, bonus_uniforms,
                                              resample_uniforms, log_weights, temperature, ess_frac, P, N, K, **kw)
    call()
    return out


def smc_pages_workspace_bytes(P, N, L, num_pages) -> int:
    return _lib.smc_pages_workspace_bytes(P, N, L, num_pages)


def smc_pages_append(page_table, seq_len, ref_count, free_pages, free_count, P, N, page_size, new_tokens, *,
                     workspace=None, status_flags=None, stream=None, slots=None, cow_list=None, cow_count=None):
    """Paged-KV append of ``new_tokens`` slots per particle (see
    ``smc_pages_append`` in include/smcsd.h); page_table, seq_len, ref_count
    and free_count (int32 [1]) are updated in place.  Returns dict(slots,
    cow_list, cow_count, status_flags)."""
    for t, n in ((page_table, "page_table"), (seq_len, "seq_len"), (ref_count, "ref_count"),
                 (free_pages, "free_pages"), (free_count, "free_count")):
        _need(t, torch.int32, n)
    dev = page_table.device
    R, L = P * N, page_table.shape[-1]
    M = ref_count.numel()
    ctx, st = _on_stream(stream, dev)
    with ctx:
        slots = slots if slots is not None else torch.empty((R, new_tokens), dtype=torch.int32, device=dev)
        cow = cow_list if cow_list is not None else torch.empty((max(R, 1), 3), dtype=torch.int32, device=dev)
        cow_count = cow_count if cow_count is not None else torch.zeros(1, dtype=torch.int32, device=dev)
        for t, n in ((slots, "slots"), (cow, "cow_list"), (cow_count, "cow_count")):
            _need(t, torch.int32, n)
        status_flags = status_flags if status_flags is not None else torch.zeros(1, dtype=torch.int32, device=dev)
        ws, wsb = _workspace(smc_pages_workspace_bytes(P, N, L, M), dev, workspace)
    _check(_lib.smc_pages_append(P, N, L, page_size, new_tokens, M, _ptr(page_table), _ptr(seq_len),
                                 _ptr(ref_count), _ptr(free_pages), _ptr(free_count), _ptr(slots), _ptr(cow),
                                 _ptr(cow_count), _ptr(status_flags), _ptr(ws), wsb, st))
    return dict(slots=slots, cow_list=cow, cow_count=cow_count, status_flags=status_flags)


def smc_pages_resample(ancestors, page_table_old, seq_len_in, ref_count, free_pages, free_count, P, N, page_size, *,
                       seq_len_out=None, workspace=None, status_flags=None, stream=None):
    """Paged-KV bookkeeping of a resampling (see ``smc_pages_resample`` in
    include/smcsd.h); ref_count, free_pages and free_count are updated in
    place.  Returns dict(seq_len_out, status_flags)."""
    for t, n in ((ancestors, "ancestors"), (page_table_old, "page_table_old"), (seq_len_in, "seq_len_in"),
                 (ref_count, "ref_count"), (free_pages, "free_pages"), (free_count, "free_count"),
                 (seq_len_out, "seq_len_out")):
        _need(t, torch.int32, n)
    dev = page_table_old.device
    L = page_table_old.shape[-1]
    M = ref_count.numel()
    ctx, st = _on_stream(stream, dev)
    with ctx:
        seq_len_out = seq_len_out if seq_len_out is not None else torch.empty_like(seq_len_in)
        status_flags = status_flags if status_flags is not None else torch.zeros(1, dtype=torch.int32, device=dev)
        ws, wsb = _workspace(smc_pages_workspace_bytes(P, N, L, M), dev, workspace)
    _check(_lib.smc_pages_resample(P, N, L, page_size, M, _ptr(ancestors), _ptr(page_table_old), _ptr(seq_len_in),
                                   _ptr(seq_len_out), _ptr(ref_count), _ptr(free_pages), _ptr(free_count),
                                   _ptr(status_flags), _ptr(ws), wsb, st))
    return dict(seq_len_out=seq_len_out, status_flags=status_flags)


def draft_sample_workspace_bytes(dtype_code, R, V) -> int:
    return int(_lib.draft_sample_workspace_bytes(dtype_code, R, V))


def prepare_draft_sample(logits, uniforms, temperature, *, tokens=None, status_flags=None, workspace=None,
                         stream=None):
    """Validate and marshal one draft_sample call (one token per row of
    ``logits`` [R, V] from softmax(z / T) by inverse CDF with ``uniforms``
    [R]); returns (call, outputs) with outputs tokens and status_flags."""
    dev = logits.device
    dt = _dtype_code(logits)
    R, V = logits.shape
    _need(logits, logits.dtype, "logits")
    _need(uniforms, torch.float32, "uniforms")
    if uniforms.numel() != R:
        raise ValueError(f"uniforms: {uniforms.numel()} values for {R} rows")
    ctx, st = _on_stream(stream, dev)
    with ctx:
        tokens = tokens if tokens is not None else torch.empty(R, dtype=torch.int32, device=dev)
        _need(tokens, torch.int32, "tokens")
        status_flags = status_flags if status_flags is not None else torch.zeros(1, dtype=torch.int32, device=dev)
        ws, wsb = _workspace(draft_sample_workspace_bytes(dt, R, V), dev, workspace)
    args = (dt, R, V, float(temperature), _ptr(logits), _ptr(uniforms), _ptr(tokens), _ptr(status_flags), _ptr(ws),
            wsb, st)
    fn = _lib.draft_sample
    keep = (logits, uniforms, ws)

    def call():
        _check(fn(*args))
        return keep

    return call, dict(tokens=tokens, status_flags=status_flags)


def draft_sample(logits, uniforms, temperature, **kw):
    call, out = prepare_draft_sample(logits, uniforms, temperature, **kw)
    call()
    return out


def pacer_lengths(scores, block, max_blocks, t0, rho, *, lengths=None, offsets=None, stream=None):
    """PACER draft lengths from ``scores`` [B, max_blocks * block] (see
    ``pacer_lengths`` in include/smcsd.h).  Returns dict(lengths, offsets)."""
    _need(scores, torch.float32, "scores")
    dev = scores.device
    B = scores.shape[0]
    if scores.dim() != 2 or scores.shape[1] != max_blocks * block:
        raise ValueError(f"scores must be [B, {max_blocks * block}], got {tuple(scores.shape)}")
    ctx, st = _on_stream(stream, dev)
    with ctx:
        lengths = lengths if lengths is not None else torch.empty(B, dtype=torch.int32, device=dev)
        offsets = offsets if offsets is not None else torch.empty(B + 1, dtype=torch.int32, device=dev)
    _need(lengths, torch.int32, "lengths")
    _need(offsets, torch.int32, "offsets")
    _check(_lib.pacer_lengths(B, block, max_blocks, float(t0), float(rho), _ptr(scores), _ptr(lengths),
                              _ptr(offsets), st))
    return dict(lengths=lengths, offsets=offsets)


def tree_verify_workspace_bytes(dtype_code, B, V, num_nodes, num_draft_rows) -> int:
    return _lib.tree_verify_workspace_bytes(dtype_code, B, V, num_nodes, num_draft_rows)


def prepare_tree_verify(target_logits, draft_logits, node_offsets, draft_offsets, parent, tokens, uniforms,
                        temperature, *, num_accepted=None, last_node=None, final_token=None, status_flags=None,
                        workspace=None, stream=None):
    """Validate and marshal one tree_verify call; returns (call, outputs).

    target [num_nodes, V] (one row per tree node), draft [num_draft_rows, V]
    (one row per node with children, node order), node_offsets / draft_offsets
    int32 [B+1], parent / tokens int32 [num_nodes] (local parent, -1 at the
    root), uniforms float32 [num_nodes] (the root's slot: the final draw)."""
    dev = target_logits.device
    dt = _dtype_code(target_logits)
    V = target_logits.shape[-1]
    nodes = target_logits.shape[0]
    rows_d = draft_logits.shape[0] if draft_logits is not None else 0
    B = node_offsets.numel() - 1
    for t, d, n in ((target_logits, target_logits.dtype, "target_logits"), (draft_logits, target_logits.dtype,
                    "draft_logits"), (node_offsets, torch.int32, "node_offsets"), (draft_offsets, torch.int32,
                    "draft_offsets"), (parent, torch.int32, "parent"), (tokens, torch.int32, "tokens"),
                    (uniforms, torch.float32, "uniforms")):
        _need(t, d, n)
    ctx, st = _on_stream(stream, dev)
    with ctx:
        mk = lambda n, d: torch.empty(n, dtype=d, device=dev)  # noqa: E731
        num_accepted = num_accepted if num_accepted is not None else mk(B, torch.int32)
        last_node = last_node if last_node is not None else mk(B, torch.int32)
        final_token = final_token if final_token is not None else mk(B, torch.int32)
        status_flags = status_flags if status_flags is not None else torch.zeros(1, dtype=torch.int32, device=dev)
        nbytes = tree_verify_workspace_bytes(dt, B, V, nodes, rows_d)
        ws, wsb = _workspace(nbytes, dev, workspace)
    args = (dt, B, V, float(temperature), _ptr(node_offsets), _ptr(parent), _ptr(tokens), nodes, _ptr(target_logits),
            _ptr(draft_offsets), rows_d, _ptr(draft_logits), _ptr(uniforms), _ptr(num_accepted), _ptr(last_node),
            _ptr(final_token), _ptr(status_flags), _ptr(ws), wsb, st)
    fn = _lib.tree_verify
    keep = (target_logits, draft_logits, node_offsets, draft_offsets, parent, tokens, uniforms, ws)

    def call():
        _check(fn(*args))
        return keep

    return call, dict(num_accepted=num_accepted, last_node=last_node, final_token=final_token,
                      status_flags=status_flags)


def tree_verify(target_logits, draft_logits, node_offsets, draft_offsets, parent, tokens, uniforms, temperature,
                **kw):
    """Tree verification; returns dict(num_accepted, last_node, final_token, status_flags)."""
    call, out = prepare_tree_verify(target_logits, draft_logits, node_offsets, draft_offsets, parent, tokens,
                                    uniforms, temperature, **kw)
    call()
    return out
