"""Short rows (every row of the launch at most 16,384 keys) on MI355X: the
selection of one workgroup per row that holds the row in registers
(select_small_kernel), against the oracle and against the multi-workgroup
chain that longer launches take.

  * caller-given scores through indexer_topk (the kernel counts the first
    digit itself): value sets with heavy ties, NaN, +-inf and +-0, rows of
    0 .. 16,384 keys; the same scores one key wider (max_bound 16,385, so the
    chain runs) give the same selection;
  * fused launches (the first digit from the scoring pass, cleared by the
    selection): all-equal keys, many requests of mixed lengths; the
    workspace's zero block is zero after every launch, also when the launch
    runs as its two stages (indexer_launch_score, indexer_launch_select).
"""
import numpy as np
import pytest
import torch

import fp8_key_scoring_amd as fk
import oracle
import synthetic as syn
from gpu_util import run_launch, say
from test_gpu_invariants import _zero_block_bytes
from test_gpu_parity import full_check

pytestmark = pytest.mark.gpu

SHORT = 16384


def _topk_rows(rows, bounds, k):
    return [np.sort(oracle.topk(np.ascontiguousarray(rows[r, :bounds[r]]), k)[:min(k, bounds[r])])
            for r in range(rows.shape[0])]


@pytest.mark.parametrize("k", [2048, 100, 1])
def test_caller_scores_with_ties_nan_inf_zero(k):
    rng = np.random.default_rng(90 + k)
    width = SHORT + 1
    vals = np.array([np.nan, -np.inf, np.inf, -0.0, 0.0, 1.0, -1.0, 0.5, 0.25, 3.0, 2.0 ** -20, 7.5],
                    np.float32)
    bounds = np.array([SHORT, SHORT - 1, 9000, 4097, 2049, 2048, 100, 1, 0, 12345], np.int32)
    R = bounds.size
    rows = vals[rng.integers(0, vals.size, size=(R, width))].astype(np.float32)
    rows[2] = rng.standard_normal(width).astype(np.float32)        # distinct values
    rows[3] = np.float32(1.0)                                       # all equal
    rows[9, ::7] = np.float32(3.0)                                  # a heavy tie at the top
    want = _topk_rows(rows, bounds, k)
    say(f"[gpu] short rows, caller scores: k={k}")
    for mb in (SHORT, width):   # the short-row kernel, then the chain
        sc = torch.from_numpy(np.ascontiguousarray(rows[:, :mb])).to("cuda:0")
        rb = torch.from_numpy(np.minimum(bounds, mb)).to("cuda:0")
        prob = fk.make_problem(rows=R, num_pages=1, pt_rows=1, pt_stride=(mb + 63) // 64, max_bound=mb, topk=k,
                               score_stride=mb)
        ws = fk.new_workspace(prob, False, "cuda:0")
        for rep in range(2):
            out = fk.indexer_topk(sc, rb, max_bound=mb, topk=k, workspace=ws).cpu().numpy()
            torch.cuda.synchronize()
            for r in range(R):
                m = min(k, int(bounds[r]))
                assert np.array_equal(out[r, :m], want[r]), (mb, rep, r)
                assert np.all(out[r, m:] == -1), (mb, rep, r)
            assert not ws[:_zero_block_bytes(R)].any(), "counters left non-zero"


def test_all_equal_keys_short_rows():
    p = syn.build_problem("short_all_equal", 4, [SHORT], [(0, SHORT), (0, 9000), (0, 2049), (0, 4096)],
                          key_mode="all_equal")
    _, out = full_check(p, "short all-equal")
    for r in range(p.rows):
        assert np.array_equal(out[r], np.arange(2048)), r


def test_many_short_requests():
    lens = [2049 + 1187 * i for i in range(12)] + [SHORT]
    p = syn.build_problem("short_many", 6, lens, [rw for i, n in enumerate(lens) for rw in syn.verify_rows(i, n)],
                          dup_frac=0.02)
    full_check(p, "short many")


def test_short_launch_leaves_the_workspace_clean():
    p = syn.build_problem("short_ws", 8, [SHORT, 7000], syn.verify_rows(0, SHORT) + syn.verify_rows(1, 7000))
    say("[gpu] short rows: zero block after fused launches")
    d = syn.device_arrays(p, "cuda:0")
    prob = fk._problem_from(d["q"], d["k_e4m3"], d["page_table"], p.max_bound, p.topk, 0)
    ws = fk.new_workspace(prob, True, "cuda:0")
    ref = None
    for rep in range(3):
        out = fk.indexer_launch(**d, max_bound=p.max_bound, topk=p.topk, workspace=ws).cpu().numpy()
        torch.cuda.synchronize()
        assert not ws[:_zero_block_bytes(p.rows)].any(), f"counters left non-zero after launch {rep}"
        if ref is None:
            ref = out
        assert np.array_equal(out, ref)
    _, want = run_launch(p)
    assert np.array_equal(ref, want)


def test_short_launch_in_two_stages():
    # indexer_launch_score then indexer_launch_select: the short-row selection
    # takes the first-digit counts the scoring stage left and clears them
    p = syn.build_problem("short_stages", 9, [SHORT, 5000], syn.verify_rows(0, SHORT) + syn.verify_rows(1, 5000),
                          dup_frac=0.01)
    say("[gpu] short rows: launch vs its two stages")
    s1, o1 = run_launch(p)
    d = syn.device_arrays(p, "cuda:0")
    mb = p.max_bound
    prob = fk._problem_from(d["q"], d["k_e4m3"], d["page_table"], mb, p.topk, 0)
    for own in (False, True):
        ws = fk.new_workspace(prob, own, "cuda:0")
        for rep in range(2):
            sc = None if own else torch.full((p.rows, mb), float("nan"), dtype=torch.float32, device="cuda:0")
            fk.indexer_launch_score(**d, max_bound=mb, topk=p.topk, scores=sc, workspace=ws)
            o2 = fk.indexer_launch_select(d["row_bound"], max_bound=mb, topk=p.topk, scores=sc, workspace=ws)
            torch.cuda.synchronize()
            if sc is not None:
                assert np.array_equal(s1.view(np.uint32), sc.cpu().numpy().view(np.uint32))
            assert np.array_equal(o1, o2.cpu().numpy()), (own, rep)
            assert not ws[:_zero_block_bytes(p.rows)].any(), (own, rep)
