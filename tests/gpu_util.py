"""Helpers for the GPU parity tests: run the HIP path through the C ABI and
compare with the CPU oracle (sharded over host processes for big rows)."""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor
import os
import sys

import numpy as np

import oracle
import synthetic as syn

TOL_REL = 1e-3
TOL_ABS = 1e-6
OVERLAP_MIN = 0.999


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def oracle_rows(p: syn.Problem, rows, shard: int = 16384):
    """Full fp64 oracle scores and tolerance scales for the given rows.

    Shards run on threads (the C oracle is reentrant and ctypes releases the
    GIL), so no process is forked from a GPU-initialised interpreter."""
    tasks = []
    for r in rows:
        b = int(p.row_bound[r])
        for s0 in range(0, b, shard):
            tasks.append((r, s0, min(b, s0 + shard)))
    with ThreadPoolExecutor(workers()) as ex:
        res = list(ex.map(lambda t: oracle.score_range(p, *t), tasks))
    out = {r: ([], []) for r in rows}
    for (r, s0, s1), (sc, bd) in zip(tasks, res):
        out[r][0].append(sc)
        out[r][1].append(bd)
    return {r: (np.concatenate(v[0]) if v[0] else np.zeros(0), np.concatenate(v[1]) if v[1] else np.zeros(0))
            for r, v in out.items()}


def to_device(p: syn.Problem, device="cuda:0"):
    return syn.device_arrays(p, device)


def run_launch(p: syn.Problem, device="cuda:0", keep_scores=True, sentinel=float("nan"), workspace=None):
    import torch
    import fp8_key_scoring_amd as fk
    d = to_device(p, device)
    mb = p.max_bound
    scores = None
    if keep_scores:
        scores = torch.full((p.rows, max(1, mb)), sentinel, dtype=torch.float32, device=device)
    out = fk.indexer_launch(**d, max_bound=mb, topk=p.topk, scores=scores, workspace=workspace)
    torch.cuda.synchronize()
    return (scores.cpu().numpy() if scores is not None else None), out.cpu().numpy()


def check_scores_full(p, gpu_scores, ref, rows=None):
    rows = range(p.rows) if rows is None else rows
    worst = 0.0
    for r in rows:
        b = int(p.row_bound[r])
        sc, bd = ref[r]
        g = gpu_scores[r, :b].astype(np.float64)
        err = np.abs(g - sc)
        lim = TOL_REL * bd + TOL_ABS
        bad = np.nonzero(~(err <= lim))[0]
        assert bad.size == 0, f"row {r}: {bad.size} scores out of tolerance, first key {bad[0]}: gpu {g[bad[0]]} ref {sc[bad[0]]} B {bd[bad[0]]}"
        if b:
            worst = max(worst, float(np.max(err / lim)))
    return worst


def check_scores_sampled(p, gpu_scores, nsamp=4096, seed=0):
    rng = np.random.default_rng(seed)
    rows, keys = [], []
    for r in range(p.rows):
        b = int(p.row_bound[r])
        if b == 0:
            continue
        m = min(b, nsamp)
        ks = rng.choice(b, size=m, replace=False)
        ks = np.unique(np.concatenate([ks, [0, b - 1]]))   # include both ends
        rows.append(np.full(ks.size, r))
        keys.append(ks)
    rows = np.concatenate(rows)
    keys = np.concatenate(keys)
    sc, bd = oracle.score_samples(p, rows, keys)
    g = gpu_scores[rows, keys].astype(np.float64)
    err = np.abs(g - sc)
    lim = TOL_REL * bd + TOL_ABS
    bad = np.nonzero(~(err <= lim))[0]
    assert bad.size == 0, f"{bad.size} sampled scores out of tolerance, e.g. row {rows[bad[0]]} key {keys[bad[0]]}"
    return float(np.max(err / lim))


def check_untouched_past_bound(p, gpu_scores):
    for r in range(p.rows):
        b = int(p.row_bound[r])
        tail = gpu_scores[r, b:]
        assert np.all(np.isnan(tail)), f"row {r}: a score at or past the bound was written"


def check_topk_exact(p, gpu_scores, out_idx):
    """The selected set equals the oracle's top-k of the GPU's own scores; the
    output is in ascending index order with -1 padding."""
    k = p.topk
    for r in range(p.rows):
        b = int(p.row_bound[r])
        ref = oracle.topk(np.ascontiguousarray(gpu_scores[r, :b]), k)
        got = out_idx[r]
        m = min(k, b)
        assert np.all(got[m:] == -1), f"row {r}: padding"
        assert np.all(np.diff(got[:m]) > 0), f"row {r}: not ascending / duplicates"
        assert np.array_equal(np.sort(ref[:m]), got[:m]), f"row {r}: selection differs from the oracle's top-k of the GPU scores"


def overlap(p, ref, out_idx, rows=None):
    k = p.topk
    worst = 1.0
    rows = range(p.rows) if rows is None else rows
    for r in rows:
        b = int(p.row_bound[r])
        m = min(k, b)
        if m == 0:
            continue
        sel = oracle.topk(ref[r][0], k)[:m]
        got = out_idx[r][:m]
        ov = np.intersect1d(sel, got).size / m
        worst = min(worst, ov)
    return worst
