"""Two-row launches on MI355X (the row-group scoring kernel with groups of
one or two rows), against the oracle:

  * two verify rows of one request (one page-table row: one group of two
    rows, each key read and converted once for both) with bounds anywhere in
    a 16-key group, a page or a chunk, equal or far apart, one of them 0;
    scores at or past a row's bound are never written;
  * two rows of two requests (different page-table rows: two groups of one
    row), in both orders of their lengths;
  * an out-of-range page-table row scores its row NaN and leaves the other
    row exact;
  * indexer_score (no first-digit count) writes the launch's scores bit for
    bit.
"""
import numpy as np
import pytest
import torch

import fp8_key_scoring_amd as fk
import synthetic as syn
from gpu_util import check_scores_full, check_topk_exact, oracle_rows, say

pytestmark = pytest.mark.gpu

MB = 20000
LENS = [3000, 9000, MB]


def _launch(p, max_bound=MB):
    d = syn.device_arrays(p, "cuda:0")
    sc = torch.full((p.rows, max_bound), float("nan"), dtype=torch.float32, device="cuda:0")
    out = fk.indexer_launch(**d, max_bound=max_bound, topk=p.topk, scores=sc)
    torch.cuda.synchronize()
    return sc.cpu().numpy(), out.cpu().numpy()


def _check(p, scores, out):
    for r in range(p.rows):
        b = int(p.row_bound[r])
        assert np.all(np.isnan(scores[r, b:])), f"row {r}: a score at or past the bound was written"
    live = [r for r in range(p.rows) if p.row_bound[r] > 0]
    if live:
        check_scores_full(p, scores, oracle_rows(p, live), rows=live)
    check_topk_exact(p, scores, out)


@pytest.mark.parametrize("b0,b1", [(MB - 1, MB), (1, MB), (0, 17), (2048, 2049), (4097, 15),
                                   (9001, 9001), (MB, 63)])
def test_two_verify_rows(b0, b1):
    p = syn.build_problem(f"two_rows_{b0}_{b1}", 200 + (b0 + 3 * b1) % 89, LENS, [(2, b0), (2, b1)],
                          dup_frac=0.01)
    say(f"[gpu] two rows of one request: bounds {b0}, {b1}, max_bound {MB}")
    scores, out = _launch(p)
    _check(p, scores, out)


@pytest.mark.parametrize("rows", [[(1, 9000), (2, MB)], [(2, MB - 5), (0, 3000)], [(1, 5000), (1, 0)]])
def test_two_rows_of_two_requests(rows):
    p = syn.build_problem("two_requests", 211 + rows[0][1] % 7, LENS, rows, dup_frac=0.01)
    say(f"[gpu] two rows, page-table rows {p.row_pt.tolist()}, bounds {p.row_bound.tolist()}")
    scores, out = _launch(p)
    _check(p, scores, out)


def test_two_rows_bad_page_table_row():
    p = syn.build_problem("two_rows_badpt", 223, LENS, [(2, 12000), (1, 9000)])
    p.row_pt[1] = 7                          # past the page table's three rows
    say("[gpu] two rows: the second row's page-table row out of range")
    scores, out = _launch(p)
    assert np.all(np.isnan(scores[1, :9000]))
    check_scores_full(p, scores, oracle_rows(p, [0]), rows=[0])
    check_topk_exact(p, scores, out)


@pytest.mark.parametrize("same_request", [True, False])
def test_two_rows_score_equals_launch(same_request):
    rows = [(2, 17777), (2, 16001)] if same_request else [(2, 17777), (1, 9000)]
    p = syn.build_problem("two_rows_score", 233, LENS, rows, dup_frac=0.02)
    say(f"[gpu] two rows: indexer_score vs the fused launch (same request: {same_request})")
    s_launch, _ = _launch(p)
    d = syn.device_arrays(p, "cuda:0")
    sc = torch.full((2, MB), float("nan"), dtype=torch.float32, device="cuda:0")
    fk.indexer_score(**d, max_bound=MB, scores=sc)
    torch.cuda.synchronize()
    assert np.array_equal(s_launch.view(np.uint32), sc.cpu().numpy().view(np.uint32))
