"""Sparse attention over each row's selected keys on MI355X against the
oracle (oracle_sparse_attention; the reading is stated there and in the
kernel's header): 16 heads of 576 dims over the row's index list in a paged
bf16 latent cache, softmax of sm_scale * q . c, output the weighted mean of
the first 512 dims, plus the log-sum-exp.

Tolerance, from the arithmetic: bf16 inputs are exact; a logit is a sum of
576 exact products accumulated in fp32 (relative error of the sum of |terms|
below 576 * 2^-24 ~ 3.4e-5), the weights are split into bf16 hi + lo (2^-17
relative), the weighted sum of up to 2,048 values is accumulated in fp32
(2,048 * 2^-24 ~ 1.2e-4 of the weighted sum of |values|).  So per output
element |gpu - ref| <= 3e-4 * A + 1e-5 with A = sum_j p_j |c_j[d]| / sum_j p_j
(plus the logit error times the spread of the values, covered by A at the
logit scales used), and |lse_gpu - lse_ref| <= 3e-4 * (1 + |lse_ref|).
"""
import numpy as np
import pytest
import torch

import fp8_key_scoring_amd as fk
import oracle
import synthetic as syn
from gpu_util import say

pytestmark = pytest.mark.gpu

H, D, DV = 16, 576, 512


def _case(name, seed, req_lens, rows, sel_fn, topk=2048, scale=None):
    p = syn.build_problem(name, seed, req_lens, rows, topk=topk)
    rng = np.random.default_rng(seed + 7)
    kv = syn.bf16_bits_rne(rng.standard_normal((p.num_pages, 64, D), dtype=np.float32))
    q = syn.bf16_bits_rne(rng.standard_normal((p.rows, H, D), dtype=np.float32))
    sel = sel_fn(p, rng)
    sm = float(1.0 / np.sqrt(192.0)) if scale is None else scale
    return p, q, kv, sel, sm


def _gpu(p, q, kv, sel, sm):
    dev = "cuda:0"
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    qd = t(q.view(np.int16)).view(torch.bfloat16)
    kvd = t(kv.view(np.int16)).view(torch.bfloat16)
    out, lse = fk.indexer_sparse_attention(qd, kvd, t(p.page_table), t(p.row_pt), t(sel.astype(np.int32)),
                                           max_bound=p.max_bound, sm_scale=sm)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def _check(p, q, kv, sel, sm, label):
    say(f"[gpu] attention {label}: rows={p.rows} topk={sel.shape[1]}")
    out, lse = _gpu(p, q, kv, sel, sm)
    ref, rlse = oracle.sparse_attention(q, kv, p.page_table, p.row_pt, sel, p.max_bound, sm)
    kvf = syn.bf16_bits_to_f32(kv).astype(np.float64)
    qf = syn.bf16_bits_to_f32(q).astype(np.float64)
    worst = 0.0
    for r in range(p.rows):
        # the selected rows' values and weights (for the tolerance scale only)
        rowsel = []
        for s in sel[r]:
            if 0 <= s < p.max_bound:
                pg = int(p.page_table[p.row_pt[r]][s // 64])
                if 0 <= pg < p.num_pages:
                    rowsel.append(kvf[pg, s % 64])
        if not rowsel:
            assert not out[r].any() and np.all(np.isneginf(lse[r])), f"row {r}: empty selection"
            assert np.all(np.isneginf(rlse[r]))
            continue
        c = np.stack(rowsel)
        lg = sm * (qf[r] @ c.T)                        # [H, n]
        w = np.exp(lg - lg.max(axis=1, keepdims=True))
        w /= w.sum(axis=1, keepdims=True)
        A = w @ np.abs(c[:, :DV])                      # [H, 512]
        err = np.abs(out[r] - ref[r])
        lim = 3e-4 * A + 1e-5
        bad = np.argwhere(~(err <= lim))
        assert bad.size == 0, f"{label} row {r}: {bad.shape[0]} outputs out of tolerance, e.g. head/dim {bad[0]}: gpu {out[r][tuple(bad[0])]} ref {ref[r][tuple(bad[0])]}"
        lerr = np.abs(lse[r] - rlse[r])
        assert np.all(lerr <= 3e-4 * (1 + np.abs(rlse[r]))), f"{label} row {r}: lse {lse[r]} vs {rlse[r]}"
        worst = max(worst, float(np.max(err / lim)))
    say(f"[gpu] attention {label}: worst err/tol {worst:.3g}")


def _indexer_sel(p, rng):
    """The indexer's own selection for the rows (the launch's output)."""
    d = syn.device_arrays(p, "cuda:0")
    out = fk.indexer_launch(**d, max_bound=p.max_bound, topk=p.topk)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def test_attention_over_the_indexer_selection():
    # four verify rows of a 60,000-key request: the selection the indexer
    # launch itself returns (2,048 per row)
    p, q, kv, sel, sm = _case("attn_idx", 61, [60000], syn.verify_rows(0, 60000), _indexer_sel)
    _check(p, q, kv, sel, sm, "indexer selection")


def test_attention_ragged_padded_and_empty_rows():
    # rows with fewer keys than k (the selection padded with -1), a row with
    # nothing selected, two requests, duplicated positions, positions past
    # max_bound and an out-of-range page id (skipped)
    def sel_fn(p, rng):
        s = np.full((p.rows, p.topk), -1, np.int32)
        s[0, :1500] = rng.choice(int(p.row_bound[0]), 1500, replace=False)
        s[1, :] = rng.integers(0, int(p.row_bound[1]), size=p.topk)          # duplicates
        s[3, :70] = np.arange(70)
        s[3, 70] = p.max_bound + 5                                            # skipped
        s[4, :2048] = rng.choice(int(p.row_bound[4]), 2048, replace=False)
        return s
    p, q, kv, sel, sm = _case("attn_ragged", 62, [9000, 20000],
                              [(0, 1600), (0, 9000), (1, 0), (1, 100), (1, 20000)], sel_fn)
    p.page_table[1, 0] = -3                                                   # row 3's positions 0..63: skipped
    _check(p, q, kv, sel, sm, "ragged")


@pytest.mark.parametrize("topk", [1, 100, 777])
def test_attention_short_index_lists(topk):
    def sel_fn(p, rng):
        return np.stack([rng.choice(int(b), topk, replace=False) for b in p.row_bound]).astype(np.int32)
    p, q, kv, sel, sm = _case(f"attn_k{topk}", 63, [5000], syn.verify_rows(0, 5000), sel_fn, topk=topk, scale=0.05)
    _check(p, q, kv, sel, sm, f"topk {topk}")


def test_attention_many_rows():
    # 64 rows: a single split per row (the other path of the split choice)
    lens = [3000 + 211 * i for i in range(16)]
    rows = [rw for i, n in enumerate(lens) for rw in syn.verify_rows(i, n)]
    def sel_fn(p, rng):
        return np.stack([rng.choice(int(b), 2048, replace=False) for b in p.row_bound]).astype(np.int32)
    p, q, kv, sel, sm = _case("attn_many", 64, lens, rows, sel_fn)
    _check(p, q, kv, sel, sm, "64 rows")


def test_attention_one_split_per_row_writes_directly():
    # 300 rows (more than the 256 workgroups a launch aims at): one split per
    # row, so the attention kernel normalises and writes out and lse itself
    # (no combine); 320-entry index lists, some rows short of 320 valid keys
    lens = [400 + 97 * i for i in range(75)]
    rows = [rw for i, n in enumerate(lens) for rw in syn.verify_rows(i, n)]
    def sel_fn(p, rng):
        s = np.full((p.rows, p.topk), -1, np.int32)
        for r, b in enumerate(p.row_bound):
            m = min(int(b), p.topk) - (r % 7 == 3) * 50
            s[r, :m] = rng.choice(int(b), m, replace=False)
        return s
    p, q, kv, sel, sm = _case("attn_direct", 65, lens, rows, sel_fn, topk=320)
    assert p.rows == 300
    _check(p, q, kv, sel, sm, "one split per row")
