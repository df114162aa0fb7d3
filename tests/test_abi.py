"""The C-ABI library loads, exports every function include/smcsd.h declares,
and rejects bad arguments on the host before anything is launched (CPU only:
no call here reaches a kernel launch)."""
import ctypes
import math
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "smcsd.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "defined")))


@pytest.fixture(scope="module")
def s():
    import smc_resampling_amd

    return smc_resampling_amd


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("sd_verify", "smc_reweight_resample", "sd_verify_workspace_bytes", "smc_workspace_bytes",
              "smcsd_status_string", "smcsd_abi_version"):
        assert n in names, names


def test_every_declared_symbol_is_exported(s):
    L = ctypes.CDLL(s.LIB_PATH)
    for n in declared_functions():
        assert hasattr(L, n), f"{n} declared in smcsd.h but not exported"


def test_abi_version_and_status_strings(s):
    ver = int(re.search(r"#define SMCSD_ABI_VERSION (\d+)", open(HEADER).read()).group(1))
    assert s.abi_version() == ver
    assert s.status_string(0) == "SMCSD_OK"
    for code in range(1, 5):
        assert s.status_string(code).startswith("SMCSD_ERR_")
    assert s.status_string(99) == "SMCSD_UNKNOWN_STATUS"


def test_workspace_sizes(s):
    assert s.sd_verify_workspace_bytes(1, 0, 4, 32768, 0) == 0
    a = s.sd_verify_workspace_bytes(1, 64, 4, 32768, 256)
    b = s.sd_verify_workspace_bytes(1, 64, 4, 151936, 256)
    assert a > 0 and b > a and a % 256 == 0
    assert s.smc_workspace_bytes(1, 0, 16, 4, 100) == 0
    c = s.smc_workspace_bytes(1, 32, 64, 8, 151936)
    assert c % 256 == 0 and c >= 32 * 64 * 18 * 75 * 8


FAKE = 0x10000  # never dereferenced: every call below fails validation first


def _sd(s, **kw):
    a = dict(dtype=1, B=4, K=2, V=1000, T=1.0, tgt=FAKE, drf=FAKE, tok=FAKE, u=FAKE, off=None, rows_d=8, na=FAKE,
             ft=FAKE, fl=None, ws=FAKE, wsb=1 << 30, stream=None)
    a.update(kw)
    return s.lib().sd_verify(a["dtype"], a["B"], a["K"], a["V"], a["T"], a["tgt"], a["drf"], a["tok"], a["u"],
                             a["off"], a["rows_d"], a["na"], a["ft"], a["fl"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=2), 1), (dict(V=1 << 20), 2), (dict(T=0.0), 1), (dict(T=-1.0), 1), (dict(T=math.nan), 1), (dict(T=math.inf), 1),
    (dict(V=0), 1), (dict(B=-1), 1), (dict(K=-1), 1), (dict(K=300, rows_d=1200), 2), (dict(rows_d=7), 1),
    (dict(rows_d=9), 1), (dict(tgt=None), 1), (dict(u=None), 1), (dict(drf=None), 1), (dict(na=None), 1),
    (dict(ws=None), 3), (dict(wsb=16), 3), (dict(ws=FAKE + 8), 3), (dict(off=FAKE, rows_d=9), 1),
    (dict(B=0, rows_d=0, tgt=None, drf=None), 0),
    # more than INT32_MAX tiles of 2048 logits
    (dict(B=70000, K=128, V=1 << 19, rows_d=70000 * 128, wsb=1 << 62), 2)])
def test_sd_verify_host_validation(s, kw, code):
    assert _sd(s, **kw) == code


def _smc(s, **kw):
    a = dict(dtype=1, P=2, N=8, K=2, V=1000, T=1.0, ess=0.5, tgt=FAKE, drf=FAKE, tok=FAKE, ub=FAKE, ur=FAKE,
             lw=FAKE, pti=None, pto=None, L=0, bt=FAKE, anc=FAKE, es=FAKE, rs=FAKE, fl=None, ws=FAKE,
             wsb=1 << 30, stream=None)
    a.update(kw)
    return s.lib().smc_reweight_resample(a["dtype"], a["P"], a["N"], a["K"], a["V"], a["T"], a["ess"], a["tgt"],
                                         a["drf"], a["tok"], a["ub"], a["ur"], a["lw"], a["pti"], a["pto"], a["L"],
                                         a["bt"], a["anc"], a["es"], a["rs"], a["fl"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=5), 1), (dict(N=0), 1), (dict(P=-1), 1), (dict(T=0.0), 1), (dict(ess=-0.1), 1),
    (dict(ess=math.nan), 1), (dict(N=2000), 2), (dict(K=257), 2), (dict(lw=None), 1), (dict(ur=None), 1),
    (dict(pti=FAKE, pto=FAKE + 64, L=4), 1), (dict(pti=FAKE, pto=None, L=4), 1), (dict(ws=None), 3),
    (dict(wsb=100), 3), (dict(P=0, tgt=None), 0), (dict(L=-1), 1),
    (dict(P=300, N=1024, K=128, V=1 << 19, wsb=1 << 62), 2)])
def test_smc_host_validation(s, kw, code):
    assert _smc(s, **kw) == code


def _tree(s, **kw):
    a = dict(dtype=1, B=4, V=1000, T=1.0, noff=FAKE, par=FAKE, tok=FAKE, nodes=28, tgt=FAKE, doff=FAKE, rows_d=12,
             drf=FAKE, u=FAKE, na=FAKE, ln=FAKE, ft=FAKE, fl=None, ws=FAKE, wsb=1 << 30, stream=None)
    a.update(kw)
    return s.lib().tree_verify(a["dtype"], a["B"], a["V"], a["T"], a["noff"], a["par"], a["tok"], a["nodes"],
                               a["tgt"], a["doff"], a["rows_d"], a["drf"], a["u"], a["na"], a["ln"], a["ft"],
                               a["fl"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=3), 1), (dict(V=1 << 20), 2), (dict(V=0), 1), (dict(T=0.0), 1), (dict(T=math.nan), 1),
    (dict(B=-1), 1), (dict(nodes=3), 1), (dict(nodes=4 * 256 + 1), 1), (dict(rows_d=-1), 1), (dict(rows_d=25), 1),
    (dict(noff=None), 1), (dict(par=None), 1), (dict(tok=None), 1), (dict(doff=None), 1), (dict(u=None), 1),
    (dict(ln=None), 1), (dict(drf=None), 1), (dict(ws=None), 3), (dict(wsb=1000), 3), (dict(ws=FAKE + 4), 3),
    (dict(B=0, nodes=0, rows_d=0, tgt=None, drf=None), 0)])
def test_tree_verify_host_validation(s, kw, code):
    assert _tree(s, **kw) == code


def test_tree_workspace_sizes(s):
    assert s.tree_verify_workspace_bytes(1, 0, 100, 0, 0) == 0
    a = s.tree_verify_workspace_bytes(1, 64, 32768, 64 * 15, 64 * 7)
    assert a % 256 == 0 and a >= 2 * (64 * 22) * 16 * 8


def test_csr_call_needs_k(s):
    """A ragged (CSR) sd_verify call must name K, its largest draft length: the
    binding never reads a device value back to find it (checked before any
    tensor reaches the device, so host tensors do here)."""
    import torch

    t = torch.zeros((5, 16), dtype=torch.float32)
    d = torch.zeros((3, 16), dtype=torch.float32)
    off = torch.tensor([0, 1, 3], dtype=torch.int32)
    with pytest.raises(ValueError, match="needs K"):
        s.prepare_sd_verify(t, d, torch.zeros(3, dtype=torch.int32), torch.zeros(5), 1.0, draft_offsets=off)


def test_phase_stamps_are_absent_from_the_library_build(s):
    """The library's own build records no phase timestamps: the measurement
    aid answers SMCSD_ERR_UNSUPPORTED and touches nothing."""
    L = s.lib()
    assert L.smcsd_phase_stamps(None, 0, 1) == s.SMCSD_ERR_UNSUPPORTED
    buf = (ctypes.c_uint64 * 4)(7, 7, 7, 7)
    assert L.smcsd_phase_stamps(ctypes.addressof(buf), ctypes.sizeof(buf), 0) == s.SMCSD_ERR_UNSUPPORTED
    assert list(buf) == [7, 7, 7, 7]
    with pytest.raises(s.SmcsdError):
        s.phase_stamps()


def test_read_ceiling_rejects_bad_buffers(s):
    L = s.lib()
    sink = ctypes.c_void_p(1 << 40)
    assert L.smcsd_read_ceiling(None, 64, None, 0, sink, None, None, None) == 1  # NULL with a size
    assert L.smcsd_read_ceiling(ctypes.c_void_p(1 << 40), 63, None, 0, sink, None, None, None) == 1  # odd size
    assert L.smcsd_read_ceiling(ctypes.c_void_p((1 << 40) + 8), 64, None, 0, sink, None, None, None) == 1  # align
    assert L.smcsd_read_ceiling(ctypes.c_void_p(1 << 40), 64, None, 0, None, None, None, None) == 1  # no sink


def test_noalloc_validates_on_the_host(s):
    """The allocation-free SMC entry point checks its arguments before it looks
    up its scratch or plans a launch (so no device is touched here)."""
    L = s.lib()
    F = ctypes.c_void_p(1 << 40)
    args = lambda **kw: [kw.get("dtype", 1), kw.get("P", 2), 4, 2, 1000, kw.get("T", 1.0), 0.5, F, F, F, F, F, F,  # noqa
                         None, None, 0, F, F, F, F, None, None]
    assert L.smc_reweight_resample_noalloc(*args(dtype=5)) == 1
    assert L.smc_reweight_resample_noalloc(*args(T=0.0)) == 1
    assert L.smc_reweight_resample_noalloc(*args(P=0)) == 0
