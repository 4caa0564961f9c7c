"""Benchmark of the fused indexer launch (scoring + exact top-2048) on one MI355X.

Workload: one request's 4 verify rows over 524,288 paged E4M3 keys (bounds
n-3..n), 64 heads x 128, page 64, top-2048.  A step is one indexer_launch
call (through a LaunchPlan: the arguments checked and marshalled once).
Inputs sit in HBM before timing starts; the timed steps rotate over
several copies of the key pool and page table (together larger than the
256 MB MALL) so each step streams its keys from HBM.  Before the warmup
steps the launch runs back to back, untimed, for --settle seconds, so the
timed steps run at the GPU's sustained clocks rather than in the first tens
of milliseconds after idle (the count is reported as settle_launches).

Prints one JSON line.  Extra keys: "roofline" for the launch's scoring kernel
(timed inside launches with HIP events on the launch stream after each of
the launch's two stages, less the events' own overhead) and "cpu_baseline" (the CPU oracle on the
same workload, or a bounded sample of it, as processes on the host's cores
and on one core).
"""
import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "indexer keys scored/s and µs/launch at 512K keys, 4 rows; % of roofline"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
FLOP_PER_KEY_ROW = 2 * 64 * 128
BYTES_PER_KEY = 128 + 4       # E4M3 codes + fp32 scale


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--pools", type=int, default=4, help="key-pool copies rotated over")
    ap.add_argument("--config", type=int, default=3, help="workload 1..8 (3 = 512K keys x 4 rows)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU work of the oracle sample")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--settle", type=float, default=0.3,
                    help="seconds of back-to-back untimed launches before the warmup steps, so the "
                         "timed steps run at the GPU's sustained clocks (0: none)")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip measuring the device's HBM and MFMA peaks (profiled runs)")
    ap.add_argument("--shards", type=int, default=0,
                    help="time the key-sharded selection instead: one shard's launch, its "
                         "candidates and the merge of G shards (G GPUs emulated on one)")
    ap.add_argument("--new-keys", action="store_true",
                    help="time the launch with the new-key write instead: the write alone, the "
                         "launch without and with it")
    ap.add_argument("--attention", action="store_true",
                    help="time the sparse attention over the selected keys (the step after the launch) "
                         "on the workload's rows and page table")
    ap.add_argument("--copy-calib", action="store_true",
                    help="only run a plain device copy of known size (counter calibration)")
    return ap.parse_args()


def algorithmic_bytes(p):
    """Bytes one launch must move at least: each distinct key once (codes +
    scale), the page-table entries, q/w/bounds per row, the selected indices."""
    distinct = p.distinct_keys()
    pages = sum(-(-int(b) // 64) for b in _group_max(p).values())
    per_row = 64 * 128 * 2 + 64 * 4 + 8
    out = 4 * sum(min(p.topk, int(b)) for b in p.row_bound)
    return BYTES_PER_KEY * distinct + 4 * pages + per_row * p.rows + out


def _group_max(p):
    g = {}
    for r in range(p.rows):
        k = int(p.row_pt[r])
        g[k] = max(g.get(k, 0), int(p.row_bound[r]))
    return g


def source_sha256():
    """sha256 over the HIP sources of the scoring kernel (the kernel whose
    traffic and MFMA figures the counter summary holds): the committed
    summaries carry the value they were taken on."""
    import hashlib
    h = hashlib.sha256()
    for fn in ("fp8_key_scoring_amd/csrc/score.hip", "fp8_key_scoring_amd/csrc/common.h"):
        with open(os.path.join(ROOT, fn), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def profile_figures(workload):
    """Figures read from the committed counter summary of this workload
    (profiles/pmc_score_<workload>.md): HBM bytes per launch of the scoring
    kernel (FETCH_SIZE + WRITE_SIZE, calibrated against a plain copy) and the
    fraction of its time the MFMA pipes were busy.  Empty when there is no
    summary or the kernel sources have changed since the counters were
    taken."""
    path = os.path.join(ROOT, "profiles", f"pmc_score_{workload}.md")
    if not os.path.exists(path):
        return {}
    fields = {}
    for line in open(path):
        if ":" in line and line.split(":")[0] in ("traffic_bytes_per_launch", "source_sha256", "mfma_busy_frac"):
            k, v = line.split(":", 1)
            fields[k] = v.strip()
    if fields.get("source_sha256") != source_sha256():
        return {}
    out = {}
    if "traffic_bytes_per_launch" in fields:
        out["traffic"] = int(float(fields["traffic_bytes_per_launch"]))
    if "mfma_busy_frac" in fields:
        out["mfma_busy_frac"] = float(fields["mfma_busy_frac"])
    return out


def host_cpus():
    """CPUs this process may run on: its affinity mask, capped by a cgroup
    CPU quota when one is set."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    try:
        with open("/sys/fs/cgroup/cpu.max") as f:
            quota, period = f.read().split()[:2]
        if quota != "max":
            n = min(n, max(1, int(quota) // int(period)))
    except (OSError, ValueError):
        pass
    return n


def cpu_model():
    """The host CPU's model name (lscpu's, else /proc/cpuinfo's), with the
    x86 family / model / stepping numbers from /proc/cpuinfo (a virtualised
    host may report only a generic name such as "AMD EPYC")."""
    import subprocess
    name = ""
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                name = line.split(":", 1)[1].strip()
                break
    except (OSError, subprocess.SubprocessError):
        pass
    ids = {}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if not line.strip():
                    break   # the first processor's block
                k, _, v = line.partition(":")
                ids[k.strip()] = v.strip()
    except OSError:
        pass
    name = name or ids.get("model name", "")
    fms = [f"{k} {ids[k]}" for k in ("cpu family", "model", "stepping") if k in ids]
    return f"{name} ({', '.join(fms)})" if fms else name


_CPU_PROBLEM = None   # the workload, inherited by the forked oracle workers


def _oracle_scores(task):
    import oracle
    r, s0, s1 = task
    return oracle.score_range(_CPU_PROBLEM, r, s0, s1)[0]


def cpu_baseline(p, seconds, max_procs=16):
    """The oracle (fp64 scores + exact top-k) on the host: sharded over
    (row, key range) as separate processes, one per available CPU (at most
    `max_procs`, the CPU share one GPU's job gets), and on one core.  Runs
    before anything touches the GPU (the workers are forked).  Each leg covers
    every row of the workload, the whole of it when that is at most about
    `seconds` of CPU work, else each row's first keys."""
    import multiprocessing as mp
    import oracle
    global _CPU_PROBLEM
    oracle.build(force=False)
    _CPU_PROBLEM = p
    t0 = time.perf_counter()
    oracle.score_range(p, 0, 0, 2048)
    per_key = (time.perf_counter() - t0) / 2048
    procs = max(1, min(max_procs, host_cpus()))

    def sample(cpu_s):
        keys = int(min(p.row_bound.max(), max(4096, cpu_s / per_key / p.rows)))
        return keys - keys % 1024 if keys < p.row_bound.max() else keys

    def run(keys_per_row, pool):
        tasks = [(r, s0, min(int(p.row_bound[r]), keys_per_row, s0 + 16384)) for r in range(p.rows)
                 for s0 in range(0, min(int(p.row_bound[r]), keys_per_row), 16384)]
        t = time.perf_counter()
        parts = pool.map(_oracle_scores, tasks, chunksize=1) if pool else [_oracle_scores(x) for x in tasks]
        rows = {}
        for (r, s0, s1), sc in zip(tasks, parts):
            rows.setdefault(r, []).append(sc)
        for r in rows:   # the selection: single-threaded per row
            oracle.topk(np.concatenate(rows[r]), p.topk)
        return sum(x[2] - x[1] for x in tasks), time.perf_counter() - t

    k_all = sample(seconds)
    with mp.get_context("fork").Pool(procs) as pool:
        n_all, wall_all = run(k_all, pool)
    k_one = sample(seconds / 2)
    n_one, wall_one = run(k_one, None)
    whole = k_all >= p.row_bound.max()
    return {"value": n_all / wall_all, "unit": "keys/s", "cores": procs, "kind": "oracle",
            "sample": (f"{'all' if whole else 'first ' + str(k_all)} keys of each of the {p.rows} rows "
                       f"({n_all} key-rows): fp64 scores + exact top-{p.topk}, {procs} processes, "
                       f"{wall_all:.2f} s"),
            "one_core": {"value": n_one / wall_one, "unit": "keys/s",
                         "sample": f"first {min(k_one, int(p.row_bound.max()))} keys of each row "
                                   f"({n_one} key-rows), one process, {wall_one:.2f} s"},
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count(), "cpus_available": host_cpus()}


def copy_calib():
    import torch
    n = 256 << 20
    a = torch.empty(n, dtype=torch.uint8, device="cuda:0")
    b = torch.empty_like(a)
    a.fill_(1)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calib_bytes_read_per_copy": n, "copies": 5}))


def measured_peaks(torch, dev):
    """Sustained HBM read rate and dense bf16 MFMA rate of this device, from
    the two measurement kernels in libfp8idx_peaks.so (16-byte streaming
    loads over 4 GiB; v_mfma_f32_16x16x32_bf16 with eight independent
    accumulators and random operands), each the best over a few grid sizes."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "fp8_key_scoring_amd", "libfp8idx_peaks.so"))
    lib.peak_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    lib.peak_mfma.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.peak_mfma32.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    stream = torch.cuda.current_stream(dev)
    sp = ctypes.c_void_p(stream.cuda_stream)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / reps

    nbytes = 4 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    buf.fill_(3)
    sink = torch.zeros(16384, dtype=torch.int32, device=dev)

    def rd(blocks):
        if lib.peak_read(ctypes.c_void_p(buf.data_ptr()), nbytes, ctypes.c_void_p(sink.data_ptr()),
                         blocks, sp):
            raise RuntimeError("peak_read launch failed")
    # best over a few grid sizes (the rate a well-shaped kernel can reach)
    read_s = min(timed(lambda: rd(b), 10) for b in (2048, 4096, 8192, 16384))
    del buf
    g = torch.Generator().manual_seed(11)
    opnd = torch.randn(64 * 6 * 8, generator=g).to(torch.bfloat16).to(dev)
    iters = 2048
    outm = torch.zeros(1024, dtype=torch.float32, device=dev)

    def mm(fn, blocks):
        if fn(ctypes.c_void_p(opnd.data_ptr()), ctypes.c_void_p(outm.data_ptr()), iters, blocks, sp):
            raise RuntimeError("peak MFMA launch failed")
    # both forms do 16 x 16x16x32 worth of flops per wave and iteration
    rates = {name: max(b * 4 * iters * 16 * (2 * 16 * 16 * 32) / timed(lambda: mm(fn, b), 5) / 1e12
                       for b in (256, 512, 1024))
             for name, fn in (("16x16x32", lib.peak_mfma), ("32x32x16", lib.peak_mfma32))}
    return {"hbm_read_GBs": round(nbytes / read_s / 1e9, 1),
            "bf16_mfma_TFLOPs": round(max(rates.values()), 1),
            "bf16_mfma_TFLOPs_by_form": {k: round(v, 1) for k, v in rates.items()},
            "how": "best over grid sizes (1-4 waves/SIMD) of: streaming 16-byte loads over 4 GiB; "
                   "v_mfma_f32_16x16x32_bf16 and v_mfma_f32_32x32x16_bf16 loops with independent "
                   "accumulators and random operands (the better form is the measured peak)"}


def sharded_report(args):
    """Key-sharded selection with G = args.shards shards (pages interleaved):
    the time one shard's launch takes (what each of G GPUs would spend), the
    conversion of its selection to (score, global index) candidates, and the
    merge of all G shards' candidates (run once, after the exchange).  Each
    part is timed over back-to-back calls between events on the launch
    stream."""
    import torch
    import fp8_key_scoring_amd as fk
    import synthetic as syn
    fk.load_library()
    dev = "cuda:0"
    G = args.shards
    p = syn.make_config(args.config)
    k = p.topk
    stream = torch.cuda.current_stream(dev)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)

    def timed(fn, n):
        for i in range(min(5, n)):
            fn(i)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(n):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / n

    cand_s = torch.empty((p.rows, G * k), dtype=torch.float32, device=dev)
    cand_i = torch.empty((p.rows, G * k), dtype=torch.int32, device=dev)
    shard_us, cand_us = [], []
    for g in range(G):
        ps = syn.shard_problem(p, g, G)
        d = syn.device_arrays(ps, dev)
        mb = ps.max_bound
        scores = torch.empty((ps.rows, max(1, mb)), dtype=torch.float32, device=dev)
        out = torch.empty((ps.rows, k), dtype=torch.int32, device=dev)
        prob = fk._problem_from(d["q"], d["k_e4m3"], d["page_table"], mb, k, scores.stride(0))
        ws = fk.new_workspace(prob, False, dev)
        shard_us.append(timed(lambda i: fk.indexer_launch(**d, max_bound=mb, topk=k, scores=scores,
                                                          out_idx=out, workspace=ws), args.steps))
        cand_us.append(timed(lambda i: fk.indexer_shard_candidates(scores, out, shard=g, shards=G, max_bound=mb,
                                                                   cand_score=cand_s, cand_idx=cand_i),
                             args.steps))
    merged = torch.empty((p.rows, k), dtype=torch.int32, device=dev)
    merge_us = timed(lambda i: fk.indexer_merge_topk(cand_s, cand_i, shards=G, topk=k, out_idx=merged),
                     args.steps)
    print(json.dumps({"metric": "key-sharded selection: per-shard launch, candidates and merge µs",
                      "config": {"workload": p.name, "shards": G, "rows": p.rows, "topk": k},
                      "shard_launch_us": {"median": round(float(np.median(shard_us)), 2),
                                          "max": round(max(shard_us), 2)},
                      "candidates_us": round(float(np.median(cand_us)), 2),
                      "merge_us": round(merge_us, 2),
                      "merge_bytes": p.rows * G * k * 8 + p.rows * k * 4,
                      "steps": args.steps}))


def new_keys_report(args):
    """The new-key write: each row's own key quantized and written at its last
    position ahead of scoring.  Times, over back-to-back calls between events
    on the launch stream (key pools rotated): the write alone, the ordinary
    launch, and the combined call (write + launch)."""
    import torch
    import fp8_key_scoring_amd as fk
    import synthetic as syn
    fk.load_library()
    dev = "cuda:0"
    p = syn.make_config(args.config)
    d = syn.device_arrays(p, dev)
    pools = [d] + [{**d, "k_e4m3": d["k_e4m3"].clone(), "k_scale": d["k_scale"].clone(),
                    "page_table": d["page_table"].clone()} for _ in range(1, args.pools)]
    kn = torch.from_numpy(syn.new_keys(p, 0, special=False).view(np.int16)).to(dev).view(torch.bfloat16)
    mb, k = p.max_bound, p.topk
    prob = fk._problem_from(d["q"], d["k_e4m3"], d["page_table"], mb, k, 0)
    ws = fk.new_workspace(prob, True, dev)
    outs = torch.empty((p.rows, k), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)

    def timed(fn, n):
        for i in range(min(args.warmup, n)):
            fn(i)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(n):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / n

    P = lambda i: pools[i % len(pools)]
    # (the write alone is a four-wave kernel: back-to-back calls of it are
    # bound by the host's call rate, so its figure is the call interval)
    res = {"write_call_interval_us": [], "launch_us": [], "launch_new_keys_us": []}
    for trial in range(5):
        res["write_call_interval_us"].append(timed(lambda i: fk.indexer_write_keys(
            kn, P(i)["k_e4m3"], P(i)["k_scale"], P(i)["page_table"], P(i)["row_pt"], P(i)["row_bound"],
            max_bound=mb), args.steps))
        res["launch_us"].append(timed(lambda i: fk.indexer_launch(**P(i), max_bound=mb, topk=k, out_idx=outs,
                                                                  workspace=ws), args.steps))
        res["launch_new_keys_us"].append(timed(lambda i: fk.indexer_launch_new_keys(
            P(i)["q"], P(i)["w"], kn, P(i)["k_e4m3"], P(i)["k_scale"], P(i)["page_table"], P(i)["row_pt"],
            P(i)["row_bound"], max_bound=mb, topk=k, out_idx=outs, workspace=ws), args.steps))
    med = {key: round(float(np.median(v)), 2) for key, v in res.items()}
    print(json.dumps({"metric": "launch with the new-key write: write, launch and combined µs",
                      "config": {"workload": p.name, "rows": p.rows, "new_keys": p.rows, "topk": k},
                      **med, "added_us": round(med["launch_new_keys_us"] - med["launch_us"], 2),
                      "trials": 5, "steps": args.steps}))


def attention_report(args):
    """Sparse attention over each row's selected keys on the workload's rows:
    16 heads x 576 over a bf16 latent cache paged like the index keys.  Timed
    over back-to-back calls between HIP events on the call's stream, with the
    selection rotated over enough seeded random selections (each row's topk
    distinct positions below its bound, as the indexer's output is) that their
    cache rows exceed the 256 MB last-level cache; also the indexer's own
    selection repeated (its rows stay cache-resident: `us_hot`).  The roofline
    figure is that of the whole call (the attention kernel and, with more than
    one split per row, the combine); the rocprofv3 trace of the same command
    splits it by kernel."""
    import torch
    import fp8_key_scoring_amd as fk
    import synthetic as syn
    fk.load_library()
    dev = "cuda:0"
    p = syn.make_config(args.config)
    d = syn.device_arrays(p, dev)
    mb, k = p.max_bound, p.topk
    q_attn, kv = syn.attention_inputs_device(p, 2024, dev)
    sel_idx = fk.indexer_launch(**d, max_bound=mb, topk=k)
    row_bytes = syn.ATTN_DIM * 2
    per_sel = p.rows * k * row_bytes
    nsel = max(2, int(math.ceil(2 * 256e6 / per_sel)))
    nsel = min(nsel, 64)
    sels = syn.random_selections_device(p, 77, nsel, dev)
    out = torch.empty((p.rows, syn.ATTN_HEADS, 512), dtype=torch.float32, device=dev)
    lse = torch.empty((p.rows, syn.ATTN_HEADS), dtype=torch.float32, device=dev)
    ws = fk.attention_workspace(p.rows, k, dev)
    sm = 1.0 / math.sqrt(192.0)
    stream = torch.cuda.current_stream(dev)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)

    def call(s):
        fk.indexer_sparse_attention(q_attn, kv, d["page_table"], d["row_pt"], s, max_bound=mb, sm_scale=sm,
                                    out=out, lse=lse, workspace=ws)

    def timed(pick, n):
        for i in range(min(args.warmup, n)):
            call(pick(i))
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(n):
            call(pick(i))
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / n

    rot, hot = [], []
    for _ in range(5):
        rot.append(timed(lambda i: sels[i % nsel], args.steps))
        hot.append(timed(lambda i: sel_idx, args.steps))
    us = float(np.median(rot))
    valid = int(sum(min(int(b), k) for b in p.row_bound))
    alg = valid * row_bytes + p.rows * k * 4 + p.rows * syn.ATTN_HEADS * (syn.ATTN_DIM * 2 + 512 * 4 + 4)
    print(json.dumps({"metric": "sparse attention over the selected keys: µs per call",
                      "config": {"workload": p.name, "rows": p.rows, "topk": k, "heads": syn.ATTN_HEADS,
                                 "dim": syn.ATTN_DIM, "selections_rotated": nsel},
                      "us": round(us, 2), "us_trials": [round(x, 2) for x in rot],
                      "us_hot": round(float(np.median(hot)), 2),
                      "algorithmic_bytes": alg,
                      "call_roofline": {"bound": "hbm", "achieved": round(alg / us / 1e3, 1), "peak": 8000.0,
                                        "unit": "GB/s", "frac": round(alg / us / 1e3 / 8000.0, 4)},
                      "steps": args.steps}))


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: it times the indexer launch on a single GPU "
              "(use --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if args.copy_calib:
        copy_calib()
        return
    if args.shards > 0:
        sharded_report(args)
        return
    if args.new_keys:
        new_keys_report(args)
        return
    if args.attention:
        attention_report(args)
        return
    import synthetic as syn
    p = syn.make_config(args.config)
    # the CPU baseline first: its worker processes are forked before anything
    # here has touched the GPU
    cpu = None if args.no_cpu else cpu_baseline(p, args.cpu_seconds)
    import torch
    import fp8_key_scoring_amd as fk

    fk.load_library()
    dev = "cuda:0"
    d = syn.device_arrays(p, dev)
    pools = [d]
    for i in range(1, args.pools):
        pools.append({**d, "k_e4m3": d["k_e4m3"].clone(), "k_scale": d["k_scale"].clone(),
                      "page_table": d["page_table"].clone()})
    mb = p.max_bound
    prob = fk._problem_from(d["q"], d["k_e4m3"], d["page_table"], mb, p.topk, 0)
    ws = fk.new_workspace(prob, True, dev)
    outs = torch.empty((p.rows, p.topk), dtype=torch.int32, device=dev)
    scores = torch.empty((p.rows, mb), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    # the device's own peaks are measured first: seconds of full-load work
    # that also bring the GPU's clocks to their sustained level (from idle,
    # back-to-back launches take ~30 ms to settle: 52-56 us per launch in the
    # first blocks of 20, ~47 us after ~600 launches, on one box)
    peaks = None if args.no_peaks else measured_peaks(torch, dev)

    # one prepared launch per key pool: arguments checked and marshalled
    # once, each step one C call (indexer_launch) on the current stream
    plans = [fk.LaunchPlan(**pl, max_bound=mb, topk=p.topk, out_idx=outs, workspace=ws) for pl in pools]

    def step(i):
        plans[i % len(plans)]()

    # Clock settling (untimed, reported as settle_launches / settle_s): from
    # idle, back-to-back launches slow down the first tens of milliseconds
    # (4 rows x 524,288 keys on one box: 51-56 us per launch in the first blocks, ~47 us after
    # ~600 launches), so short timed blocks would measure the ramp
    n_settle, t_settle = 0, time.time()
    while time.time() - t_settle < args.settle:
        for i in range(100):
            step(i)
        n_settle += 100
        torch.cuda.synchronize()
    t_settle = time.time() - t_settle
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    # the K timed steps, split into up to 7 trials by events recorded between
    # them on the launch stream (an event adds no gap); the value is the whole
    # block, the trials give the spread
    n_trials = max(1, min(7, args.steps))
    bounds = [args.steps * t // n_trials for t in range(n_trials + 1)]
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(n_trials + 1)]
    e0.record(stream)
    marks[0].record(stream)
    for t in range(n_trials):
        for i in range(bounds[t], bounds[t + 1]):
            step(i)
        marks[t + 1].record(stream)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_total = e0.elapsed_time(e1)
    ms_step = ms_total / args.steps
    trial_us = sorted(marks[t].elapsed_time(marks[t + 1]) * 1e3 / (bounds[t + 1] - bounds[t])
                      for t in range(n_trials))

    def block_us(fn, n):
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(n):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / n

    def hot(i):   # one pool: its keys may stay in the MALL between launches
        plans[0]()

    for i in range(args.warmup):
        hot(i)
    ms_step_hot = block_us(hot, args.steps) * 1e-3
    # two more rounds alternating the rotated-pool and the one-pool launches
    n_r = max(10, args.steps // 2)
    rounds = [{"rotated_pools": round(block_us(step, n_r), 2), "one_pool": round(block_us(hot, n_r), 2)}
              for _ in range(2)]

    # the same launches replayed from a HIP graph: one graph holds a launch on
    # each key pool; replaying it back to back removes the host's per-call
    # work (the launch enqueues kernels only, so it can be captured)
    us_graph = None
    try:
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            for i in range(len(pools)):
                step(i)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(len(pools)):
                step(i)
        torch.cuda.synchronize()
        reps = max(1, args.steps // len(pools))
        for _ in range(2):
            graph.replay()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            graph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        us_graph = e0.elapsed_time(e1) * 1e3 / (reps * len(pools))
    except RuntimeError as exc:   # a runtime without stream capture: report none
        print(f"graph replay not measured: {exc}", file=sys.stderr)

    # the launch's scoring kernel as the timed launch runs it: n_k launches,
    # each as its two stages (indexer_launch_score then indexer_launch_select,
    # which together are indexer_launch), with an event recorded on the launch
    # stream after each stage.  An event between two kernels exposes the
    # second one's dispatch (~2 us), which back-to-back kernels of one launch
    # hide, so each interval carries one marker's overhead d: the mean launch
    # with the two markers is a plain launch (timed right before) + 2d, and the kernel's
    # duration is the mean scoring interval - d (both intervals and d are
    # reported).  Back to back, with no selection between them, the same
    # kernel runs slower (score_stage_back_to_back_us): the MFMA pipes are
    # power-limited, and in a launch the selection kernels let the chip
    # recover.
    n_k = max(20, min(args.steps, 200))
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * n_k + 1)]

    def staged(i, ev_mid=None, ev_end=None):
        pi = pools[i % len(pools)]
        fk.indexer_launch_score(**pi, max_bound=mb, topk=p.topk, workspace=ws)
        if ev_mid is not None:
            ev_mid.record(stream)
        fk.indexer_launch_select(pi["row_bound"], max_bound=mb, topk=p.topk, out_idx=outs, workspace=ws)
        if ev_end is not None:
            ev_end.record(stream)

    for i in range(args.warmup):
        staged(i)
    # the reference launch time, right before the staged block (same state)
    launch_ref_us = block_us(step, n_k)
    evs[0].record(stream)
    for i in range(n_k):
        staged(i, evs[2 * i + 1], evs[2 * i + 2])
    torch.cuda.synchronize()
    score_iv = float(np.mean([evs[2 * i].elapsed_time(evs[2 * i + 1]) for i in range(n_k)])) * 1e3
    select_iv = float(np.mean([evs[2 * i + 1].elapsed_time(evs[2 * i + 2]) for i in range(n_k)])) * 1e3
    marker_us = max(0.0, (score_iv + select_iv - launch_ref_us) / 2)
    score_ms = (score_iv - marker_us) * 1e-3
    # the same stage back to back (its digit counts pile up in a workspace of
    # its own, cleared afterwards), for comparison
    ws_t = fk.new_workspace(prob, True, dev)

    def score_stage(i):
        fk.indexer_launch_score(**pools[i % len(pools)], max_bound=mb, topk=p.topk, workspace=ws_t)

    for i in range(args.warmup):
        score_stage(i)
    score_b2b_us = block_us(score_stage, n_k)
    fk.workspace_init(ws_t)
    # indexer_score's kernel (scores only, no digit counts), for comparison
    for i in range(args.warmup):
        fk.indexer_score(**pools[i % len(pools)], max_bound=mb, scores=scores)
    score_only_us = block_us(lambda i: fk.indexer_score(**pools[i % len(pools)], max_bound=mb, scores=scores),
                             n_k)

    key_rows = p.key_rows()
    flops = FLOP_PER_KEY_ROW * key_rows
    abytes = algorithmic_bytes(p)
    ach_tflops = flops / (score_ms * 1e-3) / 1e12
    ach_gbs = abytes / (score_ms * 1e-3) / 1e9
    mfma_bound = flops / (PEAK_BF16_TFLOPS * 1e12) >= abytes / (PEAK_HBM_GBS * 1e9)
    prof = profile_figures(p.name)
    traffic = prof.get("traffic")
    roof = ({"bound": "mfma", "achieved": round(ach_tflops, 2), "peak": PEAK_BF16_TFLOPS,
             "unit": "TFLOP/s", "frac": round(ach_tflops / PEAK_BF16_TFLOPS, 4), "traffic": traffic}
            if mfma_bound else
            {"bound": "hbm", "achieved": round(ach_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
             "frac": round(ach_gbs / PEAK_HBM_GBS, 4), "traffic": traffic})
    roof.update({"kernel": "the scoring kernel of indexer_launch (with the selection's digit counts), "
                           "timed inside launches run as their two stages: the scoring interval between "
                           "events, less one event marker's overhead",
                 "kernel_us": round(score_ms * 1e3, 2), "traffic_unit": "bytes per launch",
                 "algorithmic_flops": flops, "algorithmic_bytes": abytes,
                 "hbm_gbs_at_kernel_time": round(ach_gbs, 1),
                 "mfma_busy_frac": prof.get("mfma_busy_frac"),
                 "score_only_kernel_us": round(score_only_us, 2),
                 "score_stage_interval_us": round(score_iv, 2), "select_stage_interval_us": round(select_iv, 2),
                 "marker_overhead_us": round(marker_us, 2), "launch_ref_us": round(launch_ref_us, 2),
                 "score_stage_back_to_back_us": round(score_b2b_us, 2)})
    if peaks is not None:
        mpeak = peaks["bf16_mfma_TFLOPs"] if mfma_bound else peaks["hbm_read_GBs"]
        roof.update({"measured_peak": mpeak, "frac_of_measured_peak": round(roof["achieved"] / mpeak, 4),
                     "measured_peaks": peaks})
    step_roof_s = max(flops / (PEAK_BF16_TFLOPS * 1e12), abytes / (PEAK_HBM_GBS * 1e9))

    res = {
        "metric": METRIC,
        "value": key_rows / (ms_step * 1e-3),
        "unit": "keys/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "settle_launches": n_settle,
        "settle_s": round(t_settle, 3),
        "us_per_launch": ms_step * 1e3,
        "us_per_launch_hot": ms_step_hot * 1e3,
        "us_per_launch_graph": None if us_graph is None else round(us_graph, 2),
        "us_per_launch_trials": {"n": n_trials, "median": round(trial_us[n_trials // 2], 2),
                                 "min": round(trial_us[0], 2), "max": round(trial_us[-1], 2),
                                 "over_1.1x_median": sum(t > 1.1 * trial_us[n_trials // 2] for t in trial_us)},
        "us_per_launch_rounds": rounds,
        "launch_roofline_frac": round(step_roof_s / (ms_step * 1e-3), 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": p.name, "rows": p.rows, "keys": int(p.max_bound), "key_rows": key_rows,
                   "heads": 64, "head_dim": 128, "page": 64, "topk": p.topk, "kv": "e4m3",
                   "pools_rotated": len(pools)},
        "roofline": roof,
    }
    if cpu is not None:
        res["cpu_baseline"] = cpu
    print(json.dumps(res))


if __name__ == "__main__":
    main()
