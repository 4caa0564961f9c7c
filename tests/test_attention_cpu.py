"""Pins of the sparse-attention oracle (oracle_sparse_attention in oracle.c),
the step after the indexer: each row's 16 heads attend over its selected key
positions in a paged latent cache (the reading is stated in oracle.c; the
pages give no formula, so every pin here is a closed form of softmax
attention, not a restatement of the oracle's code):

  * one selected key returns that key's first 512 values, lse = its logit;
  * equal logits return the mean of the values, lse = log(count);
  * logits l and l + ln 3 weigh 1 : 3;  a repeated position counts twice;
  * the order of the selection does not matter;
  * -1 slots, positions at or past max_bound and page ids out of range are
    skipped; a row with nothing selected gives 0 and -inf;
  * heads are independent (each uses its own query);
  * huge logits do not overflow (the result is the dominant key's value).
"""
import math

import numpy as np
import pytest

import oracle
import synthetic as syn

H, D, DV, PAGE = oracle.ATTN_HEADS, oracle.ATTN_DIM, oracle.ATTN_VDIM, 64


def bf(x):
    return syn.bf16_bits_rne(np.asarray(x, np.float32))


def cache(pages=3, seed=0):
    """A small cache of bf16 latent vectors: page p slot o holds values that
    are exact in bf16 (multiples of 1/8 in [-4, 4))."""
    rng = np.random.default_rng(seed)
    vals = rng.integers(-32, 32, size=(pages, PAGE, D)).astype(np.float32) / 8.0
    return vals, bf(vals)


def run(q_vals, kv_bits, sel, sm_scale=1.0, page_table=None, row_pt=0, max_bound=None):
    q = bf(np.asarray(q_vals, np.float32).reshape(1, H, D))
    pt = np.arange(kv_bits.shape[0], dtype=np.int32)[None, :] if page_table is None else np.asarray(page_table, np.int32)
    mb = pt.shape[1] * PAGE if max_bound is None else max_bound
    out, lse = oracle.sparse_attention(q, kv_bits, pt, np.array([row_pt], np.int32),
                                       np.asarray(sel, np.int32)[None, :], mb, sm_scale)
    return out[0], lse[0]


def test_one_key_returns_its_value(oracle_lib):
    vals, kv = cache()
    rng = np.random.default_rng(1)
    q = rng.integers(-8, 8, size=(H, D)).astype(np.float32) / 4.0
    out, lse = run(q, kv, [70, -1, -1, -1])          # position 70: page 1, slot 6
    for h in range(H):
        assert np.array_equal(out[h], vals[1, 6, :DV].astype(np.float64))
        assert lse[h] == pytest.approx(float(np.dot(q[h].astype(np.float64), vals[1, 6].astype(np.float64))),
                                       rel=1e-12, abs=1e-12)


def test_equal_logits_give_the_mean(oracle_lib):
    vals, kv = cache()
    sel = [3, 64, 100, 130, 191]
    out, lse = run(np.zeros((H, D)), kv, sel)          # q = 0: every logit 0
    pos = [(s // PAGE, s % PAGE) for s in sel]
    mean = np.mean([vals[p, o, :DV].astype(np.float64) for p, o in pos], axis=0)
    assert np.allclose(out, mean[None, :], rtol=0, atol=1e-12)
    assert np.allclose(lse, math.log(len(sel)), rtol=0, atol=1e-12)


def test_ln3_apart_weighs_one_to_three_and_repeats_count(oracle_lib):
    vals = np.zeros((2, PAGE, D), np.float32)
    vals[0, 0, 0] = 1.0                      # key 0: dim 0 = 1  (logit sm_scale)
    vals[0, 0, 1:DV] = 2.0
    vals[0, 1, 1:DV] = -1.0                  # key 1: dim 0 = 0  (logit 0)
    kv = bf(vals)
    q = np.zeros((H, D), np.float32)
    q[:, 0] = 1.0
    out, lse = run(q, kv, [0, 1], sm_scale=math.log(3.0))
    want = (3.0 * vals[0, 0, :DV].astype(np.float64) + vals[0, 1, :DV]) / 4.0
    assert np.allclose(out, want[None, :], rtol=1e-13, atol=1e-13)
    assert np.allclose(lse, math.log(4.0), rtol=1e-13)   # log(e^{ln 3} + e^0)
    # key 1 listed twice: weights 3 : 2
    out2, _ = run(q, kv, [1, 0, 1], sm_scale=math.log(3.0))
    want2 = (3.0 * vals[0, 0, :DV].astype(np.float64) + 2.0 * vals[0, 1, :DV]) / 5.0
    assert np.allclose(out2, want2[None, :], rtol=1e-13, atol=1e-13)


def test_selection_order_does_not_matter(oracle_lib):
    vals, kv = cache(seed=3)
    rng = np.random.default_rng(4)
    q = rng.integers(-8, 8, size=(H, D)).astype(np.float32) / 16.0
    sel = rng.choice(3 * PAGE, 40, replace=False)
    a, la = run(q, kv, sel, sm_scale=0.1)
    b, lb = run(q, kv, sel[::-1].copy(), sm_scale=0.1)
    assert np.allclose(a, b, rtol=1e-12, atol=1e-12) and np.allclose(la, lb, rtol=1e-12)


def test_skipped_slots_and_empty_rows(oracle_lib):
    vals, kv = cache(pages=2, seed=5)
    q = np.zeros((H, D), np.float32)
    # -1, a position at max_bound, and a position whose page id is -7: all
    # skipped, so only positions 5 and 9 count (equal logits: their mean)
    pt = np.array([[0, -7, 1]], np.int32)
    out, lse = run(q, kv, [5, -1, 100, 9, 130], page_table=pt, max_bound=128)
    want = (vals[0, 5, :DV].astype(np.float64) + vals[0, 9, :DV]) / 2.0
    assert np.allclose(out, want[None, :], rtol=0, atol=1e-12)
    assert np.allclose(lse, math.log(2.0), rtol=0, atol=1e-12)
    out0, lse0 = run(q, kv, [-1, -1, 200], max_bound=128)
    assert not out0.any() and np.all(np.isneginf(lse0))


def test_heads_use_their_own_query(oracle_lib):
    vals = np.zeros((1, PAGE, D), np.float32)
    vals[0, 0, 0] = 1.0
    vals[0, 0, 1:DV] = 1.0
    vals[0, 1, 1:DV] = -1.0
    kv = bf(vals)
    q = np.zeros((H, D), np.float32)
    c = np.arange(H, dtype=np.float32) / 4.0     # head h: logit difference h/4 (exact)
    q[:, 0] = c
    out, lse = run(q, kv, [0, 1])
    for h in range(H):
        e = math.exp(float(c[h]))
        w0, w1 = e / (e + 1.0), 1.0 / (e + 1.0)
        assert np.allclose(out[h, 1:DV], w0 - w1, rtol=1e-13, atol=1e-13)
        assert out[h, 0] == pytest.approx(w0, rel=1e-13)
        assert lse[h] == pytest.approx(math.log(e + 1.0), rel=1e-13)


def test_huge_logits_do_not_overflow(oracle_lib):
    vals = np.zeros((1, PAGE, D), np.float32)
    vals[0, 0, 0] = 4.0
    vals[0, 0, 1:DV] = 0.5
    vals[0, 1, 0] = 3.0
    vals[0, 1, 1:DV] = -0.5
    kv = bf(vals)
    q = np.zeros((H, D), np.float32)
    q[:, 0] = 256.0                              # logits 1024 and 768
    out, lse = run(q, kv, [1, 0])
    assert np.all(np.isfinite(out)) and np.allclose(out[:, 1:DV], 0.5, rtol=0, atol=1e-12)
    assert np.allclose(lse, 1024.0 + math.log1p(math.exp(-256.0)), rtol=1e-15)
