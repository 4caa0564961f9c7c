"""One-row launches on MI355X (one query row: the launch's scoring runs the
one-row kernel, eight waves per workgroup), against the oracle:

  * the row's bound anywhere in a 16-key group, a page or a chunk, below the
    launch's max_bound (whole chunks then hold none of the row's keys), and
    0; scores at or past the bound are never written;
  * the row reading the last of three page-table rows;
  * a bound above max_bound is clamped to it, a negative one to 0;
  * out-of-range page ids, and an out-of-range page-table row, score NaN;
  * indexer_score (no first-digit count) writes the launch's scores bit for
    bit; the longest chunk (4,096 keys: 64 pages, 8 per wave) is covered by
    the 1.2M-key row of the parity tests.
"""
import numpy as np
import pytest
import torch

import fp8_key_scoring_amd as fk
import synthetic as syn
from gpu_util import check_scores_full, check_topk_exact, oracle_rows, say

pytestmark = pytest.mark.gpu

MB = 20000
LENS = [3000, 5000, MB]


def _launch(p, row_bound=None, max_bound=MB):
    d = syn.device_arrays(p, "cuda:0")
    if row_bound is not None:
        d["row_bound"] = torch.tensor(row_bound, dtype=torch.int32, device="cuda:0")
    sc = torch.full((p.rows, max_bound), float("nan"), dtype=torch.float32, device="cuda:0")
    out = fk.indexer_launch(**d, max_bound=max_bound, topk=p.topk, scores=sc)
    torch.cuda.synchronize()
    return sc.cpu().numpy(), out.cpu().numpy()


@pytest.mark.parametrize("b", [0, 1, 15, 17, 63, 65, 255, 257, 2048, 4097, 9001, MB])
def test_one_row_bound_below_max_bound(b):
    p = syn.build_problem(f"one_row_{b}", 100 + b % 97, LENS, [(2, b)], dup_frac=0.01)
    say(f"[gpu] one row: bound {b}, max_bound {MB}")
    scores, out = _launch(p)
    assert np.all(np.isnan(scores[0, b:])), "a score at or past the bound was written"
    if b:
        check_scores_full(p, scores, oracle_rows(p, [0]))
    check_topk_exact(p, scores[:, :max(b, 1)], out)
    m = min(b, p.topk)
    assert np.all(out[0, m:] == -1)
    if b <= p.topk:
        assert out[0, :b].tolist() == list(range(b))


def test_one_row_bound_clamped():
    p = syn.build_problem("one_row_clamp", 131, LENS, [(2, MB)])
    say("[gpu] one row: bounds clamped to [0, max_bound]")
    s_ref, o_ref = _launch(p)
    s_hi, o_hi = _launch(p, row_bound=[MB + 777])
    assert np.array_equal(s_ref.view(np.uint32), s_hi.view(np.uint32))
    assert np.array_equal(o_ref, o_hi)
    s_neg, o_neg = _launch(p, row_bound=[-5])
    assert np.all(np.isnan(s_neg)) and np.all(o_neg == -1)


def test_one_row_bad_pages_score_nan():
    p = syn.build_problem("one_row_badpage", 132, LENS, [(2, 9000)])
    p.page_table[2, 3] = p.num_pages + 5     # keys 192..255
    p.page_table[2, 70] = -1                 # keys 4480..4543 (a later chunk)
    say("[gpu] one row: out-of-range page ids")
    scores, out = _launch(p)
    bad = np.zeros(9000, bool)
    bad[192:256] = True
    bad[4480:4544] = True
    assert np.all(np.isnan(scores[0, :9000][bad]))
    assert np.all(np.isfinite(scores[0, :9000][~bad]))
    check_topk_exact(p, scores[:, :9000], out)
    assert not np.any(bad[out[out >= 0]])
    p.row_pt[0] = 3                          # past the page table's three rows
    say("[gpu] one row: out-of-range page-table row")
    scores, out = _launch(p)
    assert np.all(np.isnan(scores))
    check_topk_exact(p, scores, out)


def test_one_row_score_equals_launch():
    p = syn.build_problem("one_row_score", 133, LENS, [(2, 17777)], dup_frac=0.02)
    say("[gpu] one row: indexer_score vs the fused launch")
    s_launch, _ = _launch(p)
    d = syn.device_arrays(p, "cuda:0")
    sc = torch.full((1, MB), float("nan"), dtype=torch.float32, device="cuda:0")
    fk.indexer_score(**d, max_bound=MB, scores=sc)
    torch.cuda.synchronize()
    assert np.array_equal(s_launch.view(np.uint32), sc.cpu().numpy().view(np.uint32))
