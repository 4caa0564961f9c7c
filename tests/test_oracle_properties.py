"""Property tests of the oracle's top-k (CPU, hypothesis).

The selection's definition (the sglang pull request page
"sgl-project/sglang#48224", sgl-amd-mono #86 commit body, Motivation: each
row's exact top-k; ties to the lower key index, NaN below every number, -0
equal to +0) checked on many tiny rows drawn with heavy ties, NaN, infinities
and signed zeros:
  * the result equals a brute-force ranking written here with Python's sort
    on a key that states the order directly;
  * invariants: min(k, n) distinct valid indices, then -1; the threshold cut
    (every unselected key ranks below every selected one);
  * the key-sharded merge of the shards' own top-k sets equals the top-k of
    the whole row for any shard count.
"""
import math

import numpy as np
from hypothesis import given, settings, strategies as st

import oracle

VALUES = st.sampled_from([0.0, -0.0, 1.0, -1.0, 2.5, -2.5, 1e-30, -1e-30, 7.0, math.inf, -math.inf,
                          math.nan, 3.25, 3.25, 1.0])
ROWS = st.lists(VALUES, min_size=0, max_size=40)


def _rank_key(v, i):
    # larger first; NaN after every number; -0 == +0; then the lower index
    if math.isnan(v):
        return (1, 0.0, i)
    return (0, -(v + 0.0), i)


def _brute(vals, k):
    order = sorted(range(len(vals)), key=lambda i: _rank_key(vals[i], i))
    sel = order[:min(k, len(vals))]
    return sel + [-1] * (k - len(sel))


@settings(max_examples=300, deadline=None)
@given(ROWS, st.integers(min_value=1, max_value=12))
def test_topk_matches_brute_force_ranking(vals, k):
    a = np.array(vals, dtype=np.float32)
    got = oracle.topk(a, k).tolist()
    want = _brute([float(x) for x in a], k)
    assert got == want


@settings(max_examples=300, deadline=None)
@given(ROWS, st.integers(min_value=1, max_value=12))
def test_topk_invariants(vals, k):
    a = np.array(vals, dtype=np.float32)
    got = oracle.topk(a, k)
    m = min(k, a.size)
    sel = got[:m]
    assert np.all(got[m:] == -1)
    assert len(set(sel.tolist())) == m and np.all((sel >= 0) & (sel < a.size))
    keys = [_rank_key(float(a[i]), int(i)) for i in range(a.size)]
    worst_sel = max((keys[i] for i in sel), default=None)
    for i in range(a.size):
        if i not in set(sel.tolist()):
            assert keys[i] > worst_sel      # the threshold cut


@settings(max_examples=150, deadline=None)
@given(st.lists(VALUES, min_size=1, max_size=300), st.integers(min_value=1, max_value=6),
       st.integers(min_value=1, max_value=40))
def test_merge_of_shard_topk_is_the_row_topk(vals, shards, k):
    # keys are split by 4-key "pages" interleaved over the shards (the same
    # rule as the 64-key pages of the sharded launch, at a tiny page size)
    a = np.array(vals, dtype=np.float32)
    page = 4
    cs, ci = [], []
    for g in range(shards):
        idx = np.array([s for s in range(a.size) if (s // page) % shards == g], dtype=np.int64)
        loc = a[idx] if idx.size else np.zeros(0, np.float32)
        sel = oracle.topk(loc, k)
        sel = sel[sel >= 0]
        cs.append(np.concatenate([loc[sel], np.zeros(k - sel.size, np.float32)]))
        ci.append(np.concatenate([idx[sel], np.full(k - sel.size, -1)]))
    merged = oracle.merge_topk(np.concatenate(cs), np.concatenate(ci), k).tolist()
    want = sorted(x for x in _brute([float(x) for x in a], k) if x >= 0)
    assert merged == want + [-1] * (k - len(want))
