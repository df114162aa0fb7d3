"""Benchmark of the verify-and-sample step on one MI355X.

A step is one library call over one batch of seeded synthetic inputs: for the
SD workloads sd_verify (row statistics, accept test with first-reject
truncation, residual / bonus draw), for the SMC workloads
smc_reweight_resample (reweight, bonus draw, ESS, systematic resampling,
page-table gather).  Every step reads its own input batch, resident in HBM
before timing starts; the batches together exceed the 256 MB Infinity Cache,
so the timed steps stream from HBM.

Prints one JSON line: verified draft positions per second (whole job), the
roofline of the logit-streaming kernel against the 8 TB/s HBM peak and against
the plain-read ceiling measured here at the call's byte count, the decision
kernel's time and the whole call's bandwidth, and the CPU oracle timed on a
bounded sample of the same workload (one thread, and one thread per host core
up to 16).  The default workload is the largest, the 32-prompt x 64-particle
SMC step at V = 151936.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
OTHER_WORKLOADS = (0, 1, 2, 4, 5)
SLEEP_CYCLES = 100_000_000
MALL_BYTES = 256 << 20


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def _elf_sections(d: bytes) -> dict:
    """name -> (offset, size) of the sections of a 64-bit little-endian ELF image."""
    import struct

    if d[:4] != b"\x7fELF" or d[4] != 2 or d[5] != 1:
        raise ValueError("not a 64-bit little-endian ELF image")
    shoff, = struct.unpack_from("<Q", d, 0x28)
    shentsize, shnum, shstrndx = struct.unpack_from("<HHH", d, 0x3A)
    entry = lambda i: struct.unpack_from("<IIQQQQ", d, shoff + i * shentsize)  # noqa: E731
    strtab = entry(shstrndx)[4]
    out = {}
    for i in range(shnum):
        name, _, _, _, off, size = entry(i)
        end = d.index(b"\0", strtab + name)
        out[d[strtab + name:end].decode()] = (off, size)
    return out


def kernel_code_hash(lib_path: str = None) -> str:
    """sha256 of the device code a build of the library holds: for each
    amdgcn code object of its offload bundles (section .hip_fatbin, one bundle
    per translation unit), its target and its .text, .rodata (kernel
    descriptors) and .note (kernel metadata: registers, LDS, ...) sections.  A change to any kernel's instructions,
    descriptor or resources changes it; comments, host code and the names the
    compiler makes up per build do not."""
    import hashlib
    import struct

    if lib_path is None:
        lib_path = os.environ.get("SMCSD_LIBRARY") or os.path.join(ROOT, "smc_resampling_amd", "libsmcsd.so")
    with open(lib_path, "rb") as f:
        d = f.read()
    off, size = _elf_sections(d)[".hip_fatbin"]
    fat = d[off:off + size]
    magic = b"__CLANG_OFFLOAD_BUNDLE__"
    if not fat.startswith(magic):
        raise ValueError("unexpected offload bundle format")
    h, nobj = hashlib.sha256(), 0
    start = 0
    while start >= 0:  # one bundle per translation unit, one after another
        b = fat[start:]
        n, = struct.unpack_from("<Q", b, len(magic))
        pos, end = len(magic) + 8, 0
        for _ in range(n):
            eoff, esize, tlen = struct.unpack_from("<QQQ", b, pos)
            triple = b[pos + 24:pos + 24 + tlen]
            pos += 24 + tlen
            end = max(end, eoff + esize)
            if b"amdgcn" not in triple or esize == 0:
                continue
            elf = b[eoff:eoff + esize]
            secs = _elf_sections(elf)
            h.update(triple + b"\0")
            for name in (".text", ".rodata", ".note"):
                so, ss = secs.get(name, (0, 0))
                h.update(name.encode() + b"\0" + elf[so:so + ss])
            nobj += 1
        start = fat.find(magic, start + max(end, len(magic)))
    if nobj == 0:
        raise ValueError("no amdgcn code object in the offload bundles")
    return h.hexdigest()


def _csv_rows(path):
    import csv

    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _find(d, suffix):
    for root, _, files in os.walk(d):
        for f in files:
            if f.endswith(suffix):
                return os.path.join(root, f)
    return None


# kernels of a call: the logit stream, and the decision path (one kernel, or
# for SMC the particle kernel and the prompt kernel), by name part
CALL_KERNELS = {"k_stream": ("k_stream",), "decision": ("_tail", "k_smc_prompt")}


VALU_CUS, VALU_XCDS = 256, 8  # MI355X


def summarize(dirs, copy_bytes=None):
    """Text summary of rocprofv3 output directories: kernel statistics
    (--kernel-trace --stats) and per-dispatch averages of PMC counters
    (--pmc), with HBM traffic per call of the streaming kernel and of the
    decision path (CALL_KERNELS) when the directories hold FETCH_SIZE /
    WRITE_SIZE and a copy of `copy_bytes` calibrates them."""
    out = [f"kernel_code_sha256: {kernel_code_hash()}"]
    avg = {}  # (kernel, counter) -> KiB per dispatch
    peak = {}  # (kernel, counter) -> largest single dispatch
    for d in dirs:
        st = _find(d, "kernel_stats.csv")
        if st:
            out.append(f"kernel statistics ({os.path.relpath(st, ROOT)}):")
            out.append("  name | calls | average ns | min ns | max ns")
            for r in _csv_rows(st)[:8]:
                out.append(f"  {r['Name'][:90]} | {r['Calls']} | {float(r['AverageNs']):.0f} | {r['MinNs']} | "
                           f"{r['MaxNs']}")
        cc = _find(d, "counter_collection.csv")
        if cc:
            acc = {}
            for r in _csv_rows(cc):
                key = (r["Kernel_Name"], r["Counter_Name"])
                acc.setdefault(key, []).append(float(r["Counter_Value"]))
            out.append(f"counters, average per dispatch ({os.path.relpath(cc, ROOT)}):")
            for (k, c), v in sorted(acc.items(), key=lambda kv: -sum(kv[1])):
                a = sum(v) / len(v)
                avg[(k, c)] = a
                peak[(k, c)] = max(v)
                if len(out) < 60:
                    out.append(f"  {k[:90]} | {c} | dispatches {len(v)} | {a:.1f}")
    if copy_bytes:
        for role, parts in CALL_KERNELS.items():
            res = {}
            for counter in ("FETCH_SIZE", "WRITE_SIZE"):
                # the calibration copy is the largest copy dispatch of the run
                cv = max([v for (k, c), v in peak.items() if "copyBuffer" in k and c == counter] or [0.0]) or None
                names = sorted(k for (k, c) in avg if c == counter and any(p in k for p in parts) and "k_read" not in k)
                if not names or cv is None:
                    continue
                factor = cv * 1024.0 / copy_bytes  # counter KiB per byte the copy moves
                res[counter] = 0.0
                for k in names:  # one dispatch of each per call
                    kv = avg[(k, counter)]
                    res[counter] += kv * 1024.0 / factor
                    out.append(f"{counter}: {k[:60]} {kv:.1f} KiB/dispatch, copy of {copy_bytes} B reads {cv:.1f} "
                               f"KiB (factor {factor:.4f}) -> {kv * 1024.0 / factor:.0f} B per launch")
            if len(res) == 2:
                out.append(f"traffic_bytes_per_call {role}: {res['FETCH_SIZE'] + res['WRITE_SIZE']:.0f}")
    valu = sorted({k for (k, c) in avg if c == "SQ_ACTIVE_INST_VALU" and "smcsd" in k})
    if valu and all((k, c) in avg for k in valu for c in ("GRBM_GUI_ACTIVE", "SQ_BUSY_CU_CYCLES")):
        # SQ_ACTIVE_INST_VALU and SQ_BUSY_CU_CYCLES are quad-cycles summed over
        # SIMDs and CUs, GRBM_GUI_ACTIVE is summed over the XCDs: device-wide
        # VALU busy = VALU / CUs / (GUI active / XCDs) (the VALUBusy metric);
        # per busy CU = VALU / busy-CU cycles
        out.append(f"VALU activity ({VALU_CUS} CUs, {VALU_XCDS} XCDs):")
        for k in valu:
            v, g, b = avg[(k, "SQ_ACTIVE_INST_VALU")], avg[(k, "GRBM_GUI_ACTIVE")], avg[(k, "SQ_BUSY_CU_CYCLES")]
            extra = ""
            if (k, "SQ_INSTS_VALU_TRANS_F32") in avg and (k, "SQ_INSTS_VALU") in avg:
                extra = f" | transcendental share {avg[(k, 'SQ_INSTS_VALU_TRANS_F32')] / avg[(k, 'SQ_INSTS_VALU')]:.2f}"
            out.append(f"  {k[:70]} | VALU busy {100 * v / VALU_CUS / (g / VALU_XCDS):.1f} % of the device | "
                       f"{100 * v / b:.1f} % of its busy CUs' time{extra}")
    return "\n".join(out)


def traffic_from_profiles(workload):
    """HBM bytes per launch of the streaming kernel and of the decision kernel
    from the committed counter summary of this workload: (stream, decision), each
    None when there is no summary or the kernels changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"k_stream_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None, None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith(" "):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    if fields.get("kernel_code_sha256") != kernel_code_hash():
        return None, None
    get = lambda k: float(fields[k]) if k in fields else None  # noqa: E731
    return get("traffic_bytes_per_call k_stream"), get("traffic_bytes_per_call decision")


STAMP_CALLS = 8  # calls whose decision-kernel stamps a phase summary pools
STAMP_CLOCK_MHZ = 100.0  # s_memrealtime


def phase_name(code):
    """What ended at a stamp with this code (the codes of the library's launch.h)."""
    fixed = {1: "statistics merged, token logits gathered", 2: "accept tests", 3: "bonus draw (all accepted)",
             4: "residual pass over the rejected row pair", 5: "residual draw: tile located",
             6: "residual draw: search in the tile", 7: "zero-residual draw from p_n",
             10: "parents read, statistics merged", 11: "draft rows ranked, token logits gathered",
             12: "pass: child tested, up to the pass", 13: "pass: own tiles weighed (thread 0's wavefront)",
             14: "pass: other members' masses read",
             300: "step to a leaf", 400: "final draw"}
    if code in fixed:
        return fixed[code]
    if 100 <= code < 200:
        return f"level: child accepted after {code - 100} rejections"
    if 200 <= code < 300:
        return f"level: all {code - 200} children rejected"
    return f"code {code}"


def pool_stamps(stamp_sets, ncalls):
    """Pool the phase stamps of several calls (each a uint64 array [workgroups,
    events, 2] of (100 MHz clock, code), 0 where nothing was recorded): per
    phase, named by the code of the stamp that ends it, the count and the
    median and 90th percentile of its duration in us; each workgroup's span
    from its first stamp to its last; and each call's span from its first
    workgroup's start to its last stamp (median)."""
    import numpy as np

    phases, spans, kernel = {}, [], []
    for st in stamp_sets:
        st = np.asarray(st).astype(np.int64)
        t, code = st[:, :, 0], st[:, :, 1]
        live = np.nonzero(t[:, 0])[0]
        if not len(live):
            continue
        ends = []
        for g in live:
            n = int(np.count_nonzero(t[g]))
            for k in range(1, n):
                phases.setdefault(int(code[g, k]), []).append((t[g, k] - t[g, k - 1]) / STAMP_CLOCK_MHZ)
            spans.append((t[g, n - 1] - t[g, 0]) / STAMP_CLOCK_MHZ)
            ends.append(t[g, n - 1])
        kernel.append((max(ends) - t[live, 0].min()) / STAMP_CLOCK_MHZ)
    if not spans:
        return {"note": "no stamps: the workload's decision kernel records none, or the library was built without"}
    q = lambda x: [round(float(v), 3) for v in np.percentile(x, [50, 90])]  # noqa: E731
    return {"calls": ncalls, "workgroups": len(spans),
            "phases_us_count_p50_p90": {phase_name(k): [len(v)] + q(v) for k, v in sorted(phases.items())},
            "workgroup_span_us_p50_p90_max": q(spans) + [round(float(max(spans)), 3)],
            "first_start_to_last_stamp_us_p50": round(float(np.median(kernel)), 3)}


def phase_summary(calls, stream):
    """Replay `calls` one at a time on a measurement build and pool the
    decision kernel's phase stamps (pool_stamps)."""
    import torch

    import smc_resampling_amd as smcsd

    torch.cuda.synchronize()
    try:
        smcsd.phase_stamps(clear=True)
    except smcsd.SmcsdError:
        sys.exit("--phase-stamps needs a library built with -DSMCSD_PHASE_STAMPS=1, named by SMCSD_LIBRARY")
    sets = []
    for c in calls:
        with torch.cuda.stream(stream):
            c()
        torch.cuda.synchronize()
        sets.append(smcsd.phase_stamps(clear=True))
    return pool_stamps(sets, len(calls))


def decision_stats(cfg, calls, outs, batches, W, nb, stream, reps=16):
    """What the method decided on up to `reps` of the timed steps, replayed one
    at a time after the timing: for SD and trees, the mean accepted draft
    tokens and tokens emitted per sequence per step (accepted + the residual or
    bonus token), and for linear SD the accepted fraction of draft positions;
    for SMC, the fraction of prompts that resampled and the mean ESS over N."""
    import numpy as np
    import torch

    n = min(reps, len(calls) - W)
    acc, kb, ess, res = [], [], [], []
    for s in range(W, W + n):
        with torch.cuda.stream(stream):
            calls[s]()
        torch.cuda.synchronize()
        if cfg.kind == "smc":
            ess.append(outs["ess"].cpu().numpy())
            res.append(outs["resampled"].cpu().numpy())
        else:
            acc.append(outs["num_accepted"].cpu().numpy().astype(np.int64))
            kb.append(np.asarray(batches[s % nb].get("Kb", np.full(len(acc[-1]), cfg.K))))
    if cfg.kind == "smc":
        return {"steps": n, "resample_rate": float(np.mean(np.concatenate(res) != 0)),
                "mean_ess_over_n": float(np.mean(np.concatenate(ess)) / cfg.N)}
    a = np.concatenate(acc)
    d = {"steps": n, "mean_accepted": float(a.mean()), "tokens_per_step": float(a.mean() + 1)}
    if cfg.kind != "tree":
        d["accepted_fraction"] = float(a.sum() / np.concatenate(kb).sum())
    return d


def environment():
    """The GPU and software the line was measured on."""
    import torch

    p = torch.cuda.get_device_properties(0)
    env = {"device": p.name, "arch": getattr(p, "gcnArchName", None), "compute_units": p.multi_processor_count,
           "hip": torch.version.hip, "torch": torch.__version__, "kernel_code_sha256": kernel_code_hash()}
    try:  # the shader clock the runtime reports (kHz)
        lib = ctypes.CDLL("libamdhip64.so")
        for key, attr in (("clock_mhz", 5), ("memory_clock_mhz", 60)):  # hipDeviceAttribute{,Memory}ClockRate
            khz = ctypes.c_int(0)
            if lib.hipDeviceGetAttribute(ctypes.byref(khz), attr, 0) == 0:
                env[key] = khz.value / 1000.0
    except OSError:
        pass
    return env


def launch_floor(reps=64):
    """Event-timed duration of the library's read kernel over one 4 KiB tile
    (one workgroup, one load): what any kernel timed the way the bench times
    its kernels costs at the least, in us (median over reps)."""
    import numpy as np
    import torch

    import smc_resampling_amd as smcsd

    a = torch.zeros(4096, dtype=torch.uint8, device="cuda")
    sink = torch.empty(64, dtype=torch.int32, device="cuda")
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
    st = torch.cuda.current_stream()
    for pair in ev:
        for e_ in pair:
            e_.record(st)  # creates the event handles the library attaches
    torch.cuda.synchronize()
    for pair in ev:
        smcsd.read_ceiling(a, None, sink=sink, start=pair[0], stop=pair[1], stream=st.cuda_stream)
    torch.cuda.synchronize()
    return float(np.median([p[0].elapsed_time(p[1]) for p in ev])) * 1e3


def graph_launch(reps=256):
    """Per-kernel time of a replayed graph of `reps` launches of the library's
    read kernel over one 4 KiB tile: what each kernel of a call costs at the
    least when the calls are replayed as the bench times them, in us (median
    of three replays)."""
    import numpy as np
    import torch

    import smc_resampling_amd as smcsd

    a = torch.zeros(4096, dtype=torch.uint8, device="cuda")
    sink = torch.empty(64, dtype=torch.int32, device="cuda")
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        for _ in range(reps):
            smcsd.read_ceiling(a, None, sink=sink, stream=side.cuda_stream)
    torch.cuda.synchronize()
    times = []
    for _ in range(3):
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(side):
            ev0.record(side)
            graph.replay()
            ev1.record(side)
        torch.cuda.synchronize()
        times.append(ev0.elapsed_time(ev1) * 1e3 / reps)
    return float(np.median(times))


def host_description():
    """CPU model and the cores this process may use."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    return model, avail


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=None,
                    help="workload index; by default the largest (SMC 32 prompts x 64 particles, K=8, V=151936 "
                         "bf16) is the line's headline and the others follow in other_workloads")
    ap.add_argument("--launch", choices=["graph", "eager"], default="graph")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="bound on each leg (one thread, all threads) of the oracle's CPU sample")
    ap.add_argument("--cpu-threads", type=int, default=16, help="most host threads for the all-cores oracle leg")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-others", action="store_true",
                    help="without --config the run also measures the smaller workloads (0, 1, 2, 4 and the token "
                         "trees) into other_workloads; this skips them")
    ap.add_argument("--max-batch-gb", type=float, default=24.0)
    ap.add_argument("--with-pages", action="store_true",
                    help="SMC workloads: each step also does the paged-KV bookkeeping (append K+1 tokens "
                         "before, resample after), 16-token pages")
    ap.add_argument("--draft-sample", action="store_true",
                    help="time the draft-side draw instead: one token per row of one draft position "
                         "(B sequences or P*N particles) of the workload")
    ap.add_argument("--beta", type=float, default=None,
                    help="SMC workloads: power-sampling target p^beta (smc_reweight_resample_power)")
    ap.add_argument("--copy-calibration", type=int, default=0,
                    help="also run a plain device copy of this many bytes (scales rocprofv3 byte counters)")
    ap.add_argument("--summarize", nargs="+", default=None,
                    help="print a summary of these rocprofv3 output directories and exit")
    ap.add_argument("--phase-stamps", action="store_true",
                    help="SD and tree workloads, with a library built with -DSMCSD_PHASE_STAMPS=1 (named by "
                         "SMCSD_LIBRARY): add the decision kernel's phase durations to the line")
    return ap.parse_args()


def cpu_baseline(args, cfg, batches, nb, positions, R_draw):
    """The oracle as it stands on a bounded sample of the workload's own
    inputs: its unit of work (an SMC prompt, an SD or tree step, eight draft
    rows) on host copies made before timing.  Two legs of about
    --cpu-seconds each: one thread, then a pool of threads (one per host core
    up to --cpu-threads; the oracle's C calls release the GIL), each worker
    taking the next unit of the sample in turn.  Returns the baseline record."""
    import concurrent.futures as cf

    import numpy as np

    import oracle
    import synth

    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from gpu_util import host_logits

    model, avail = host_description()
    threads = max(1, min(args.cpu_threads, avail))
    units = []  # (callable, positions), at most `threads` of them (host memory bound)
    if args.draft_sample:
        for i in range(nb):
            bt = batches[i]
            u = (bt["bonus_u"] if cfg.kind == "smc" else bt["uniforms"])[:R_draw].cpu().numpy()
            for r0 in range(0, R_draw, 8):
                z = host_logits(bt["draft"][r0:min(r0 + 8, R_draw)])
                units.append((lambda z=z, uu=u[r0:r0 + len(z)]: oracle.draft_sample(z, uu, cfg.T), len(z)))
                if len(units) >= threads:
                    break
            if len(units) >= threads:
                break
        what = "blocks of 8 draft rows"
    elif cfg.kind == "smc":
        P, N, K = cfg.P, cfg.N, cfg.K
        for i in range(nb):
            bt = batches[i]
            for p in range(P):
                rt = slice(p * N * (K + 1), (p + 1) * N * (K + 1))
                rd = slice(p * N * K, (p + 1) * N * K)
                tg, dr = host_logits(bt["target"][rt]), host_logits(bt["draft"][rd])
                tk = bt["tokens"][rd].cpu().numpy()
                ub = bt["bonus_u"][p * N:(p + 1) * N].cpu().numpy()
                ur = bt["resample_u"][p:p + 1].cpu().numpy()
                units.append((lambda tg=tg, dr=dr, tk=tk, ub=ub, ur=ur: oracle.smc_step(
                    tg, dr, tk, ub, ur, np.zeros(N, np.float32), cfg.T, cfg.ess_frac, 1, N, K, beta=args.beta),
                    N * K))
                if len(units) >= threads:
                    break
            if len(units) >= threads:
                break
        what = "prompts"
    else:
        for i in range(min(nb, threads)):
            bt = batches[i]
            tg, dr = host_logits(bt["target"]), host_logits(bt["draft"])
            if cfg.kind == "tree":
                host = {k: bt[k].cpu().numpy() for k in ("node_off", "draft_off", "parent", "tokens", "uniforms")}
                units.append((lambda tg=tg, dr=dr, h=host: oracle.tree_verify(
                    tg, dr, h["node_off"], h["draft_off"], h["parent"], h["tokens"], h["uniforms"], cfg.T),
                    positions[i]))
            else:
                tk, u = bt["tokens"].cpu().numpy(), bt["uniforms"].cpu().numpy()
                off = None
                if bt["offsets"] is not None:
                    # the oracle's own lengths for this step's scores (they equal the
                    # library's, which laid out the batch)
                    pc = cfg.pacer
                    _, off = oracle.pacer_lengths(synth.pacer_scores(cfg.B, cfg.seed, i, pc["block"],
                                                                     pc["max_blocks"]),
                                                  pc["block"], pc["max_blocks"], pc["t0"], pc["rho"])
                    if not np.array_equal(off, bt["offsets"].cpu().numpy()):
                        sys.exit("PACER lengths of the library and the oracle differ")
                units.append((lambda tg=tg, dr=dr, tk=tk, u=u, off=off: oracle.sd_verify(
                    tg, dr, tk, u, cfg.T, K=cfg.K, offsets=off), positions[i]))
        what = "steps"

    def leg(workers):
        done, n_units = 0, 0
        t0 = time.perf_counter()
        if workers == 1:
            while time.perf_counter() - t0 < args.cpu_seconds:
                fn, pos = units[n_units % len(units)]
                fn()
                done += pos
                n_units += 1
        else:
            with cf.ThreadPoolExecutor(max_workers=workers) as ex:
                pending = set()
                k = 0
                while True:
                    while len(pending) < workers and time.perf_counter() - t0 < args.cpu_seconds:
                        fn, pos = units[k % len(units)]
                        pending.add(ex.submit(lambda fn=fn, pos=pos: (fn(), pos)[1]))
                        k += 1
                    if not pending:
                        break
                    fin, pending = cf.wait(pending, return_when=cf.FIRST_COMPLETED)
                    for f in fin:
                        done += f.result()
                        n_units += 1
        return done / (time.perf_counter() - t0), n_units

    v1, n1 = leg(1)
    log(f"[bench] cpu oracle, 1 thread: {v1:.1f} positions/s over {n1} {what}")
    vn, nn = leg(threads)
    log(f"[bench] cpu oracle, {threads} threads: {vn:.1f} positions/s over {nn} {what}")
    unit = "sampled draft tokens/s" if args.draft_sample else "verified draft positions/s"
    return {"value": vn, "unit": unit, "cores": threads, "kind": "oracle",
            "sample": f"{nn} {what} of {cfg.name} ({len(units)} distinct, host copies made before timing) in "
                      f"about {args.cpu_seconds:.0f} s wall on {threads} threads; fp64 C oracle, gcc -O2, one call "
                      f"per {what[:-1]}",
            "single_thread_value": v1, "single_thread_sample": f"{n1} {what} in about {args.cpu_seconds:.0f} s",
            "host_cpu": model, "host_cores_available": avail}


def run_workload(args, config, steps_arg, with_cpu):
    """Measure one workload (index into synth.CONFIGS) and return its JSON record."""
    import numpy as np
    import torch

    import smc_resampling_amd as smcsd
    import synth

    cfg = synth.CONFIGS[config]
    steps = steps_arg if steps_arg is not None else cfg.steps
    W = args.warmup
    if args.draft_sample and (args.with_pages or args.beta is not None):
        sys.exit("--draft-sample times the draft-side draw alone")
    if cfg.kind == "tree" and (args.draft_sample or args.with_pages or args.beta is not None):
        sys.exit("the tree workload runs tree_verify alone")
    if args.with_pages:
        if cfg.kind != "smc":
            sys.exit("--with-pages applies to the SMC workloads")
        # the page tables alternate between two buffers: even counts keep every
        # pass on the buffer the previous one ended on
        steps += steps % 2
        W += W % 2
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    def lib_lengths(scores, block, max_blocks, t0, rho):
        # the ragged workload's draft lengths by the library's PACER rule
        out = smcsd.pacer_lengths(torch.from_numpy(scores).to(dev), block, max_blocks, t0, rho)
        return out["lengths"].cpu().numpy()

    gen = synth.Generator(cfg, dev, lengths=lib_lengths)

    # ---------------- inputs: distinct batches, resident in HBM -------------
    per_batch = synth.step_bytes(cfg, None if cfg.kind != "sd_ragged" else np.full(cfg.B, 7))
    nb = min(steps + W, max(2, int(args.max_batch_gb * 1e9 // max(per_batch, 1))))
    nb = max(nb, min(steps + W, -(-2 * MALL_BYTES // max(per_batch, 1))))
    log(f"[bench] {cfg.name}: generating {nb} input batches of ~{per_batch / 1e6:.1f} MB")
    batches = []
    for b in range(nb):
        batches.append(gen.tree_step(b) if cfg.kind == "tree" else gen.sd_step(b) if cfg.kind != "smc"
                       else gen.smc_step(b))
    torch.cuda.synchronize()
    positions = [synth.verified_positions(cfg, bt.get("Kb")) for bt in batches]
    nbytes = [synth.step_bytes(cfg, bt.get("Kb")) for bt in batches]
    R_draw = cfg.B if cfg.kind != "smc" else cfg.P * cfg.N  # rows of one draft position
    if args.draft_sample:
        positions = [R_draw] * nb
        nbytes = [R_draw * cfg.V * (4 if cfg.dtype == "f32" else 2)] * nb

    # ---------------- prepared library calls ---------------------------------
    def prepare(stream_handle):
        calls = []
        if args.draft_sample:
            # one draft position: the first R_draw draft rows of each batch, one
            # uniform per row
            ws = smcsd.new_workspace(smcsd.draft_sample_workspace_bytes(int(cfg.dtype == "bf16"), R_draw, cfg.V), dev)
            outs = None
            for s in range(steps + W):
                bt = batches[s % nb]
                u = bt["bonus_u"] if cfg.kind == "smc" else bt["uniforms"]
                call, o = smcsd.prepare_draft_sample(
                    bt["draft"][:R_draw], u[:R_draw], cfg.T, workspace=ws, stream=stream_handle,
                    **({} if outs is None else {k: outs[k] for k in ("tokens", "status_flags")}))
                outs = o
                calls.append(call)
            return calls, outs
        if cfg.kind == "tree":
            bt0 = batches[0]
            ws = smcsd.new_workspace(smcsd.tree_verify_workspace_bytes(1, cfg.B, cfg.V, bt0["target"].shape[0],
                                                                       bt0["draft"].shape[0]), dev)
            outs = None
            for s in range(steps + W):
                bt = batches[s % nb]
                call, o = smcsd.prepare_tree_verify(
                    bt["target"], bt["draft"], bt["node_off"], bt["draft_off"], bt["parent"], bt["tokens"],
                    bt["uniforms"], cfg.T, workspace=ws, stream=stream_handle,
                    **({} if outs is None else {k: outs[k] for k in ("num_accepted", "last_node", "final_token",
                                                                    "status_flags")}))
                outs = o
                calls.append(call)
            return calls, outs
        if cfg.kind == "smc":
            P, N, K = cfg.P, cfg.N, cfg.K
            logw = torch.zeros(P * N, dtype=torch.float32, device=dev)
            pts = [torch.from_numpy(synth.initial_page_table(P, N, cfg.L)).to(dev), None]
            pts[1] = torch.empty_like(pts[0])
            ws = smcsd.new_workspace(smcsd.smc_workspace_bytes(1, P, N, K, cfg.V), dev)
            outs = None
            pg = None
            if args.with_pages:
                # every particle starts with the same length, on pages of its own, with room for all steps
                from synth.small import pages_state

                S, A, R = 16, K + 1, P * N
                M = R * cfg.L + R
                # room for the warm-up, the graph replay and the eager timing pass
                st0 = pages_state(0, P, N, cfg.L, S, M, fixed_len=max(0, cfg.L * S - (W + 2 * steps + 1) * A - S))
                i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(dev)  # noqa: E731
                pts = [i32(st0["table"]), torch.empty_like(i32(st0["table"]))]
                pg = dict(S=S, A=A, lens=[i32(st0["len"]), i32(st0["len"])], ref=i32(st0["ref"]),
                          free=i32(st0["free_pages"]), fc=i32([st0["free_count"]]),
                          ws=smcsd.new_workspace(smcsd.smc_pages_workspace_bytes(P, N, cfg.L, M), dev),
                          slots=torch.empty((R, A), dtype=torch.int32, device=dev),
                          cow=torch.empty((R, 3), dtype=torch.int32, device=dev),
                          ncow=torch.zeros(1, dtype=torch.int32, device=dev),
                          flags=torch.zeros(1, dtype=torch.int32, device=dev))
            for s in range(steps + W):
                bt = batches[s % nb]
                call, o = smcsd.prepare_smc_reweight_resample(
                    bt["target"], bt["draft"], bt["tokens"], bt["bonus_u"], bt["resample_u"], logw, cfg.T,
                    cfg.ess_frac, P, N, K, page_table_in=pts[s % 2], page_table_out=pts[(s + 1) % 2],
                    workspace=ws, stream=stream_handle, beta=args.beta,
                    **({} if outs is None else {k: outs[k] for k in ("bonus_token", "ancestors", "ess", "resampled",
                                                                    "status_flags")}))
                outs = o
                if pg is not None:
                    def step(call=call, o=o, cur=s % 2, nxt=(s + 1) % 2):
                        smcsd.smc_pages_append(pts[cur], pg["lens"][cur], pg["ref"], pg["free"], pg["fc"], P, N,
                                               pg["S"], pg["A"], workspace=pg["ws"], status_flags=pg["flags"],
                                               stream=stream_handle, slots=pg["slots"], cow_list=pg["cow"],
                                               cow_count=pg["ncow"])
                        call()
                        smcsd.smc_pages_resample(o["ancestors"], pts[cur], pg["lens"][cur], pg["ref"],
                                                 pg["free"], pg["fc"], P, N, pg["S"], seq_len_out=pg["lens"][nxt],
                                                 workspace=pg["ws"], status_flags=pg["flags"], stream=stream_handle)
                    calls.append(step)
                else:
                    calls.append(call)
            if pg is not None:
                outs = dict(outs, page_flags=pg["flags"])
        else:
            rows_d = max(int(bt["total_draft_rows"]) for bt in batches)
            ws = smcsd.new_workspace(smcsd.sd_verify_workspace_bytes(1, cfg.B, cfg.K, cfg.V, rows_d), dev)
            outs = None
            for s in range(steps + W):
                bt = batches[s % nb]
                call, o = smcsd.prepare_sd_verify(
                    bt["target"], bt["draft"], bt["tokens"], bt["uniforms"], cfg.T, K=cfg.K,
                    draft_offsets=bt["offsets"], workspace=ws, stream=stream_handle,
                    **({} if outs is None else {k: outs[k] for k in ("num_accepted", "final_token", "status_flags")}))
                outs = o
                calls.append(call)
        return calls, outs

    # ---------------- timing: whole calls --------------------------------------
    if args.launch == "graph":
        side = torch.cuda.Stream(device=dev)
        calls, outs = prepare(side.cuda_stream)
        with torch.cuda.stream(side):
            for c in calls[:W]:
                c()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=side):
            for c in calls[W:]:
                c()
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(side):
            ev0.record(side)
            graph.replay()
            ev1.record(side)
        torch.cuda.synchronize()
        run_stream = side
    else:
        run_stream = torch.cuda.current_stream(dev)
        calls, outs = prepare(run_stream.cuda_stream)
        for c in calls[:W]:
            c()
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(SLEEP_CYCLES)  # the host enqueues every call before the GPU reaches them
        ev0.record(run_stream)
        for c in calls[W:]:
            c()
        ev1.record(run_stream)
        torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1)
    flags = int(outs["status_flags"].item()) | (int(outs["page_flags"].item()) if "page_flags" in outs else 0)
    ms_per_step = ms / steps

    # ---------------- timing: each kernel ----------------------------------------
    # The same calls again, eagerly on the same stream, each call's two kernels
    # launched with HIP events attached to their own start and stop (the
    # library's timing aid), so an event pair times one kernel's execution, as
    # a kernel trace does.  A sleep kernel first lets the host enqueue every
    # call, so the GPU runs them back to back as in the graph.
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    with torch.cuda.stream(run_stream):
        for quad in ev:
            for e in quad:
                e.record(run_stream)  # creates the event handles the library attaches
        torch.cuda.synchronize()
        torch.cuda._sleep(SLEEP_CYCLES)
        for s_, c in enumerate(calls[W:]):
            smcsd.time_next_call(*ev[s_])
            c()
    torch.cuda.synchronize()
    stream_each = [ev[i][0].elapsed_time(ev[i][1]) for i in range(steps)]
    tail_each = [ev[i][2].elapsed_time(ev[i][3]) for i in range(steps)]
    call_each = [ev[i][0].elapsed_time(ev[i][3]) for i in range(steps)]  # first kernel's start to last one's stop
    stream_ms = float(np.mean(stream_each))
    tail_ms = float(np.mean(tail_each))
    spread = lambda x: [round(float(v) * 1e3, 3) for v in np.percentile(x, [10, 50, 90])]  # noqa: E731  us
    timed = [(W + s) % nb for s in range(steps)]
    pos_total = sum(positions[i] for i in timed)
    bytes_total = sum(nbytes[i] for i in timed)
    value = pos_total / (ms / 1e3)
    achieved = bytes_total / steps / (stream_ms / 1e3) / 1e9
    log(f"[bench] {steps} steps in {ms:.3f} ms: {ms_per_step * 1e3:.2f} us/step, {value / 1e6:.2f} M positions/s, "
        f"{bytes_total / steps / (ms_per_step / 1e3) / 1e9:.0f} GB/s per call; k_stream {stream_ms * 1e3:.2f} us "
        f"({achieved:.0f} GB/s), decision kernel {tail_ms * 1e3:.2f} us, flags={flags}")

    stamps = phase_summary(calls[W:W + STAMP_CALLS], run_stream) if args.phase_stamps else None
    decisions = (None if args.draft_sample or args.with_pages
                 else decision_stats(cfg, calls, outs, batches, W, nb, run_stream))

    # ---------------- the plain-read ceiling at the call's byte count -------------
    # The library's read-only kernel (the streaming kernel's loads, no
    # arithmetic) over the same batches, in the same order, with events on
    # its own dispatches: the time these bytes take to stream with nothing
    # else to do.
    rev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    sink = torch.empty(64, dtype=torch.int32, device=dev)
    read_bytes = []
    with torch.cuda.stream(run_stream):
        for pair in rev:
            for e_ in pair:
                e_.record(run_stream)
        torch.cuda.synchronize()
        torch.cuda._sleep(SLEEP_CYCLES)
        for s_ in range(steps):
            bt = batches[(W + s_) % nb]
            if args.draft_sample:
                a_, b_ = bt["draft"][:R_draw], None
            else:
                a_, b_ = bt["target"], bt["draft"]
            read_bytes.append(sum(0 if t is None else t.numel() * t.element_size() for t in (a_, b_)))
            smcsd.read_ceiling(a_, b_, sink=sink, start=rev[s_][0], stop=rev[s_][1], stream=run_stream.cuda_stream)
    torch.cuda.synchronize()
    read_ms = float(np.mean([rev[i][0].elapsed_time(rev[i][1]) for i in range(steps)]))
    read_gbs = float(np.mean(read_bytes)) / (read_ms / 1e3) / 1e9
    log(f"[bench] plain read of the same {np.mean(read_bytes) / 1e6:.1f} MB: {read_ms * 1e3:.2f} us "
        f"({read_gbs:.0f} GB/s)")

    if args.copy_calibration:
        src = torch.empty(args.copy_calibration, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # ---------------- CPU oracle on a bounded sample --------------------------
    cpu = None
    if with_cpu:
        cpu = cpu_baseline(args, cfg, batches, nb, positions, R_draw)

    e = 4 if cfg.dtype == "f32" else 2
    t_stream, t_tail = (traffic_from_profiles(cfg.name) if args.beta is None and not args.draft_sample
                        else (None, None))
    call_gbs = bytes_total / steps / (ms_per_step / 1e3) / 1e9
    line = {
        "metric": ("sampled draft tokens/sec and achieved HBM GB/s (% of MI355X peak)" if args.draft_sample else
                   "verified draft positions/sec and achieved HBM GB/s (% of MI355X peak)"),
        "value": value,
        "unit": "sampled draft tokens/s" if args.draft_sample else "verified draft positions/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": W,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": cfg.name, "kind": cfg.kind, "B": cfg.B, "P": cfg.P, "N": cfg.N, "K": cfg.K,
                   "V": cfg.V, "logits": cfg.dtype, "temperature": cfg.T, "launch": args.launch,
                   "input_batches": nb, "status_flags": flags,
                   **({} if args.beta is None else {"power_beta": args.beta}),
                   **({"paged_kv_bookkeeping": True, "page_size": 16} if args.with_pages else {}),
                   **({"draft_sample_rows": R_draw} if args.draft_sample else {}),
                   **({"tree": dict(cfg.tree, nodes=len(synth.full_tree_parents(**cfg.tree)))}
                      if cfg.kind == "tree" else {})},
        "roofline": {"bound": "hbm", "kernel": "logit streaming (k_stream, or k_stream_wide for one-tile segments)",
                     "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": t_stream,
                     "algorithmic_bytes_per_launch": bytes_total / steps, "bytes_per_element": e,
                     "kernel_us": stream_ms * 1e3,
                     "read_ceiling": read_gbs, "read_ceiling_frac": read_gbs / HBM_PEAK_GBS,
                     "frac_of_read_ceiling": achieved / read_gbs,
                     "decision_kernel_us": tail_ms * 1e3, "decision_kernel_traffic": t_tail,
                     "call_us": ms_per_step * 1e3, "call_achieved": call_gbs, "call_frac": call_gbs / HBM_PEAK_GBS,
                     "call_traffic": (t_stream + t_tail) if t_stream is not None and t_tail is not None else None,
                     # per-step spread of the event-timed eager pass (us: p10, median, p90); the
                     # eager call span runs from the streaming kernel's start to the last decision
                     # kernel's stop, without the graph
                     "kernel_us_p10_p50_p90": spread(stream_each),
                     "decision_kernel_us_p10_p50_p90": spread(tail_each),
                     "eager_call_us_p10_p50_p90": spread(call_each)},
        "cpu_baseline": cpu,
        "decisions": decisions,
    }
    if stamps is not None:
        line["phase_stamps"] = stamps
    return line


def main():
    args = parse()
    if args.summarize:
        print(summarize(args.summarize, args.copy_calibration or None))
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this library runs on one GPU: --gpus N > 1 is not supported"}))
        sys.exit(2)
    import torch

    default_run = args.config is None
    line = run_workload(args, 3 if default_run else args.config, args.steps, not args.no_cpu_baseline)
    if default_run and not args.no_others and not (args.draft_sample or args.with_pages or args.beta is not None):
        # the smaller workloads, each with its own inputs (those of the one
        # before freed first), at their default step counts, no CPU leg
        others = []
        for c in OTHER_WORKLOADS:
            torch.cuda.empty_cache()
            o = run_workload(args, c, None, False)
            r = o["roofline"]
            others.append({"workload": o["config"]["workload"], "value": o["value"], "unit": o["unit"],
                           "ms_per_step": o["ms_per_step"], "steps": o["steps"], "kernel_us": r["kernel_us"],
                           "frac": r["frac"], "read_ceiling": r["read_ceiling"],
                           "frac_of_read_ceiling": r["frac_of_read_ceiling"],
                           "decision_kernel_us": r["decision_kernel_us"], "call_frac": r["call_frac"],
                           "traffic": r["traffic"], "call_traffic": r["call_traffic"],
                           "status_flags": o["config"]["status_flags"], "decisions": o["decisions"]})
        line["other_workloads"] = others
    line["environment"] = environment()
    line["environment"]["launch_floor_us"] = launch_floor()
    line["environment"]["graph_kernel_floor_us"] = graph_launch()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
