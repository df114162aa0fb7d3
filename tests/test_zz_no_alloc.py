"""smc_reweight_resample_noalloc (scratch in a static device array, nothing
allocated by the call) against smc_reweight_resample with a workspace: the
same kernels, so the same outputs bit for bit, on two calls in a row (the
second smaller, on the scratch the first left behind), and the size limit."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu


def _run(c, ess_frac, noalloc):
    import torch

    import smc_resampling_amd as s
    from gpu_util import DEV, dev_logits

    lw = torch.from_numpy(np.array(c["logw"], np.float32)).to(DEV)
    pt = torch.from_numpy(c["pt"]).to(DEV)
    out = s.smc_reweight_resample(dev_logits(c["target"]), dev_logits(c["draft"]),
                                  torch.from_numpy(c["tokens"]).to(DEV), torch.from_numpy(c["bonus_u"]).to(DEV),
                                  torch.from_numpy(c["resample_u"]).to(DEV), lw, c["T"], ess_frac, c["P"], c["N"],
                                  c["K"], page_table_in=pt, noalloc=noalloc)
    torch.cuda.synchronize()
    r = {k: v.cpu().numpy() for k, v in out.items() if k != "log_weights"}
    r["logw"] = lw.cpu().numpy()
    return r


def test_noalloc_matches_workspace_call_twice():
    from synth.small import smc_case

    from gpu_util import say

    # a large call, then a smaller one on the scratch the first left behind
    for i, (P, N, K, V, dtype) in enumerate([(8, 64, 8, 151936, "bf16"), (3, 17, 2, 5000, "f32")]):
        c = smc_case(800 + i, P, N, K, V, dtype=dtype, L=6, logw_scale=2.0)
        for ess_frac in (0.5, 2.0):
            a = _run(c, ess_frac, noalloc=False)
            b = _run(c, ess_frac, noalloc=True)
            for k in ("bonus_token", "ancestors", "ess", "resampled", "logw", "page_table_out", "status_flags"):
                assert np.array_equal(a[k], b[k]), (i, ess_frac, k)
            say(f"[noalloc call {i}] P={P} N={N} K={K} V={V} ess_frac={ess_frac}: equal, "
                f"resampled {int(b['resampled'].sum())}/{P}")


def test_noalloc_refuses_calls_beyond_its_scratch():
    import torch

    import smc_resampling_amd as s

    P, N, K, V = 64, 64, 8, 151936  # 47 MB of workspace
    assert s.smc_workspace_bytes(1, P, N, K, V) > s.NOALLOC_SCRATCH_BYTES
    d = torch.device("cuda:0")
    z = torch.empty((1, V), dtype=torch.bfloat16, device=d)  # never read: refused before any launch
    f = torch.zeros(P * N, dtype=torch.float32, device=d)
    i = torch.zeros(P * N, dtype=torch.int32, device=d)
    code = s.lib().smc_reweight_resample_noalloc(1, P, N, K, V, 1.0, 0.5, z.data_ptr(), z.data_ptr(), i.data_ptr(),
                                                 f.data_ptr(), f.data_ptr(), f.data_ptr(), None, None, 0,
                                                 i.data_ptr(), i.data_ptr(), f.data_ptr(), i.data_ptr(), None, None)
    assert code == 2  # SMCSD_ERR_UNSUPPORTED


def test_noalloc_first_call_under_graph_capture():
    """A caller that captures from the start: in a fresh process, the entry
    point's first call (which looks up the scratch's device address) is made
    under graph capture; two replays equal the workspace call."""
    import os
    import subprocess
    import sys

    from gpu_util import say

    child = os.path.join(os.path.dirname(os.path.abspath(__file__)), "noalloc_capture_child.py")
    r = subprocess.run([sys.executable, "-u", child], capture_output=True, text=True, timeout=300)
    say(r.stdout.strip().replace("\n", "; "))
    assert r.returncode == 0 and r.stdout.strip().endswith("OK"), (r.stdout + r.stderr)[-3000:]
