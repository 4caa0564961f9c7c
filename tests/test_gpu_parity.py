"""Parity of the HIP path (through the C ABI) with the CPU oracle, on MI355X.

Acceptance per row:
  * scores: |gpu - ref| <= 1e-3 * B + 1e-6, B = scale * sum_h |w_h| |q_h . k|;
  * selection: the set equals the oracle's exact top-k of the GPU's own scores
    (ties to the lower index), in ascending index order, -1 padded;
  * overlap with the oracle's top-k of its own fp64 scores >= 99.9%;
  * entries at or past a row's bound are never written.
"""
import numpy as np
import pytest

import synthetic as syn
from gpu_util import (OVERLAP_MIN, check_scores_full, check_scores_sampled, check_topk_exact,
                      check_untouched_past_bound, oracle_rows, overlap, run_launch, say)

pytestmark = pytest.mark.gpu


def full_check(p, label):
    say(f"[gpu] {label}: rows={p.rows} max_bound={p.max_bound} topk={p.topk}")
    scores, out = run_launch(p)
    check_untouched_past_bound(p, scores)
    ref = oracle_rows(p, range(p.rows))
    worst = check_scores_full(p, scores, ref)
    check_topk_exact(p, scores, out)
    ov = overlap(p, ref, out)
    say(f"[gpu] {label}: worst err/tol {worst:.3g}, worst overlap {ov:.5f}")
    assert ov >= OVERLAP_MIN
    return scores, out


def test_c1_one_row_8k():
    full_check(syn.make_config(1), "c1")


def test_c2_four_rows_128k():
    full_check(syn.make_config(2), "c2")


SMALL = [
    ("r1_ragged", [5000], [(0, 5000)]),
    ("r4_ragged", [8983], syn.verify_rows(0, 8983)),
    ("r2", [7777], [(0, 7777), (0, 7770)]),
    ("r3", [6000], [(0, 6000), (0, 5999), (0, 5998)]),
    ("r5_same_request", [10000], [(0, 10000 - j) for j in range(5)]),
    ("interleaved_requests", [6000, 7000], [(0, 6000), (1, 7000), (0, 5999), (1, 6999)]),
    ("unaligned_groups", [3000, 9000], [(0, 3000), (0, 2999), (1, 9000), (1, 8999), (1, 8998), (1, 8997)]),
    ("many_requests", [2500 + 977 * i for i in range(10)],
     [rw for i in range(10) for rw in syn.verify_rows(i, 2500 + 977 * i)]),
    # one request's run of 70 rows: groups of rows 64.. find their run start
    # more than 60 rows back
    ("long_run_70_rows", [2200], [(0, 2200 - j) for j in range(70)]),
    # runs of 1, 3, 5 and 2 rows: blocks of four rows holding several group
    # starts, groups reaching into the next block
    ("mixed_runs", [3100, 4100, 5100, 2600],
     [(0, 3100), (1, 4100), (1, 4099), (1, 4098)] + [(2, 5100 - j) for j in range(5)] + [(3, 2600), (3, 2599)]),
]


@pytest.mark.parametrize("name,lens,rows", SMALL, ids=[s[0] for s in SMALL])
def test_small_shapes(name, lens, rows):
    full_check(syn.build_problem(name, 77, lens, rows), name)


def test_edge_bounds():
    bounds = [0, 1, 63, 64, 65, 2047, 2048, 2049, 3000]
    p = syn.build_problem("edge_bounds", 5, [3000], [(0, b) for b in bounds])
    scores, out = full_check(p, "edge_bounds")
    assert np.all(out[0] == -1)
    assert out[1].tolist()[:2] == [0, -1]
    assert out[4].tolist()[:65] == list(range(65)) and np.all(out[4][65:] == -1)
    assert out[6].tolist() == list(range(2048))


@pytest.mark.parametrize("k", [1, 100, 2047])
def test_smaller_topk(k):
    p = syn.build_problem(f"topk{k}", 9, [20000], syn.verify_rows(0, 20000), topk=k)
    full_check(p, f"topk{k}")


def test_all_equal_keys_take_the_lowest_indices():
    # every score of a row is equal: the exact answer is keys 0..k-1, reached
    # through the heavy-tie path (the prefix bin holds more than the candidate cap)
    p = syn.build_problem("all_equal", 3, [20000], [(0, 20000), (0, 19000)], key_mode="all_equal")
    scores, out = full_check(p, "all_equal")
    for r in range(p.rows):
        assert np.unique(scores[r, :p.row_bound[r]]).size == 1
        assert out[r].tolist() == list(range(2048))


def test_heavy_tie_fallback_rows_through_topk():
    # rows whose prefix bin at the threshold holds far more keys than the
    # selection keeps in LDS, so the exact fallback decides them: (a) one
    # value everywhere plus 1,500 larger keys scattered; (b) three adjacent
    # floats over 150,000 keys with 900 larger ones (several distinct last
    # digits); (c) the same as (a) in a score buffer whose rows are not
    # 16-byte aligned (offset by one float, odd stride)
    import torch
    import fp8_key_scoring_amd as fk
    import oracle
    rng = np.random.default_rng(17)
    n = 200000
    a = np.ones(n, np.float32)
    a[rng.choice(n, 1500, replace=False)] = 2.0
    b = np.array([1.0, np.nextafter(np.float32(1.0), np.float32(2.0)),
                  np.nextafter(np.nextafter(np.float32(1.0), np.float32(2.0)), np.float32(2.0))], np.float32)
    bb = b[rng.integers(0, 3, size=n)].astype(np.float32)
    bb[150000:] = np.nan                      # past the row's bound (never read)
    bb[rng.choice(150000, 900, replace=False)] = 3.0
    rows = np.stack([a, bb, a])
    bounds = np.array([n, 150000, n], np.int32)
    say("[gpu] heavy-tie fallback through indexer_topk (aligned and unaligned rows)")
    for offset in (0, 1):
        buf = torch.full((3, n + 1 + offset), float("nan"), dtype=torch.float32, device="cuda:0")
        sc = buf[:, offset:offset + n] if offset == 0 else buf[:, offset:offset + n + 1]
        sc[:, :n] = torch.from_numpy(rows).to("cuda:0")
        rb = torch.from_numpy(bounds).to("cuda:0")
        out = fk.indexer_topk(sc, rb, max_bound=n).cpu().numpy()
        for r in range(3):
            want = np.sort(oracle.topk(np.ascontiguousarray(rows[r, :bounds[r]]), 2048))
            assert np.array_equal(out[r], want), (offset, r)


def test_ties_straddling_the_threshold():
    p = syn.scale_tie_problem(n=12000)
    scores, out = full_check(p, "scale_ties")
    vals = np.unique(scores[0, :12000])
    assert vals.size == 3
    s = scores[0, :12000]
    top = np.nonzero(s == vals[2])[0]
    mid = np.nonzero(s == vals[1])[0]
    expect = np.sort(np.concatenate([top, mid[:2048 - top.size]]))
    assert np.array_equal(out[0], expect)


def test_ties_ranked_inside_the_last_bin():
    # 1500 keys above the threshold value and 900 keys equal to it: the 900
    # fit the candidate slices, so the ties are ranked (by index) inside the
    # third-digit bin rather than by the full rescan
    p = syn.scale_tie_problem(n=12000, counts=(1500, 900))
    scores, out = full_check(p, "scale_ties_ranked")
    s = scores[0, :12000]
    vals = np.unique(s)
    top = np.nonzero(s == vals[2])[0]
    mid = np.nonzero(s == vals[1])[0]
    assert top.size == 1500 and mid.size == 900
    expect = np.sort(np.concatenate([top, mid[:2048 - top.size]]))
    assert np.array_equal(out[0], expect)


def test_extreme_codes():
    p = syn.build_problem("extreme", 4, [9000], syn.verify_rows(0, 9000), key_mode="extreme")
    full_check(p, "extreme")


def _big(idx, overlap_rows=None):
    p = syn.make_config(idx)
    say(f"[gpu] {p.name}: rows={p.rows} max_bound={p.max_bound}")
    scores, out = run_launch(p)
    check_untouched_past_bound(p, scores)
    w = check_scores_sampled(p, scores)
    check_topk_exact(p, scores, out)
    rows = range(p.rows) if overlap_rows is None else overlap_rows
    ref = oracle_rows(p, rows)
    check_scores_full(p, scores, ref, rows)
    ov = overlap(p, ref, out, rows)
    say(f"[gpu] {p.name}: sampled worst err/tol {w:.3g}, worst overlap {ov:.5f}")
    assert ov >= OVERLAP_MIN


def test_c3_four_rows_512k():
    _big(3)


def test_c4_two_requests_8_rows():
    _big(4)


def test_c5_batch_256_rows():
    _big(5, overlap_rows=[0, 1, 2, 3, 100, 101, 254, 255])


def test_c6_one_row_512k():
    # a lone row over a long context: every wave scores one row (HBM-bound)
    _big(6)


def test_c7_two_rows_512k():
    # a two-row group over a long context
    _big(7)


def test_c8_all_equal_keys_512k():
    # every score of each 524,288-key row equal: the exact answer is keys
    # 0..2047, reached through the heavy-tie fallback at full length
    _big(8, overlap_rows=[0, 3])
    p = syn.make_config(8)
    scores, out = run_launch(p)
    for r in range(p.rows):
        assert out[r].tolist() == list(range(2048))


def test_one_row_1200k_multi_step_slices():
    # a row longer than 64 x 8,192 keys: each selection workgroup scans
    # several 8K-key steps of its slice (refine's and gather's step loop
    # past the first step), and the scoring grid has 293 chunks of 4,096
    n = 1_200_000
    p = syn.build_problem("row_1200k", 37, [n], [(0, n)], dup_frac=0.01)
    scores, out = full_check(p, "row_1200k")
    # the selection alone (its own first-digit pass over several steps per
    # workgroup) on the same scores gives the same bytes
    import torch
    import fp8_key_scoring_amd as fk
    sc = torch.from_numpy(np.ascontiguousarray(scores)).to("cuda:0")
    rb = torch.from_numpy(p.row_bound.copy()).to("cuda:0")
    o2 = fk.indexer_topk(sc, rb, max_bound=p.max_bound, topk=p.topk)
    torch.cuda.synchronize()
    assert np.array_equal(o2.cpu().numpy(), out)


def test_1100_rows_more_than_the_zero_block_layout():
    # more rows than the 256 the workspace's zero block is laid out for by
    # default: the block is then sized by the row count
    lens = [300 + (i * 37) % 2900 for i in range(275)]
    rows = []
    for i, n in enumerate(lens):
        rows += syn.verify_rows(i, n)
    p = syn.build_problem("rows_1100", 38, lens, rows)
    assert p.rows == 1100
    full_check(p, "rows_1100")


def test_every_row_empty():
    # max_bound 0: nothing is scored, every output slot is -1, and the
    # workspace is left as it was found (zero), so a next launch is right
    import torch
    import fp8_key_scoring_amd as fk
    p0 = syn.build_problem("all_empty", 39, [640], [(0, 0), (0, 0), (0, 0)])
    assert p0.max_bound == 0
    d = syn.device_arrays(p0, "cuda:0")
    prob = fk._problem_from(d["q"], d["k_e4m3"], d["page_table"], 0, p0.topk, 0)
    ws = fk.new_workspace(prob, True, "cuda:0")
    out = fk.indexer_launch(**d, max_bound=0, topk=p0.topk, workspace=ws)
    torch.cuda.synchronize()
    assert np.all(out.cpu().numpy() == -1)
    assert not ws.any()
