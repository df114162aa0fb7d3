"""Child process of test_zz_no_alloc.py: the first call of
smc_reweight_resample_noalloc in a fresh process is made under HIP graph
capture (where the entry point looks up its scratch array's device address),
after an eager call of smc_reweight_resample with a workspace; the graph is
replayed twice and each replay must equal that eager call bit for bit.
Prints OK on success."""
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path[:0] = [os.path.dirname(HERE), HERE]

import numpy as np  # noqa: E402
import torch  # noqa: E402

import smc_resampling_amd as s  # noqa: E402
from gpu_util import DEV, dev_logits  # noqa: E402
from synth.small import smc_case  # noqa: E402


def main():
    c = smc_case(900, 2, 16, 4, 4096, dtype="bf16", L=4, logw_scale=2.0)
    ins = [dev_logits(c["target"]), dev_logits(c["draft"])] + [torch.from_numpy(c[k]).to(DEV) for k in
                                                                 ("tokens", "bonus_u", "resample_u")]
    lw0 = torch.from_numpy(np.array(c["logw"], np.float32)).to(DEV)
    pt = torch.from_numpy(c["pt"]).to(DEV)
    lw = lw0.clone()
    ref = s.smc_reweight_resample(*ins, lw, c["T"], 0.5, c["P"], c["N"], c["K"], page_table_in=pt)
    torch.cuda.synchronize()
    want = {k: v.cpu().clone() for k, v in ref.items()}
    print("eager call with a workspace done", flush=True)

    side = torch.cuda.Stream(device=DEV)
    lw2 = lw0.clone()
    call, o = s.prepare_smc_reweight_resample(*ins, lw2, c["T"], 0.5, c["P"], c["N"], c["K"], page_table_in=pt,
                                              noalloc=True, stream=side.cuda_stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        call()
    torch.cuda.synchronize()
    print("first noalloc call captured", flush=True)
    for r in range(2):
        lw2.copy_(lw0)
        o["status_flags"].zero_()
        for k in ("bonus_token", "ancestors", "resampled", "page_table_out"):
            o[k].fill_(-7)
        o["ess"].fill_(float("nan"))
        torch.cuda.synchronize()
        with torch.cuda.stream(side):
            graph.replay()
        torch.cuda.synchronize()
        for k, a in want.items():
            b = o[k].cpu()
            if a.is_floating_point():
                a, b = a.view(torch.int32), b.view(torch.int32)
            assert torch.equal(a, b), f"replay {r}: {k} differs"
        print(f"replay {r} equal", flush=True)
    print("OK", flush=True)


if __name__ == "__main__":
    main()
