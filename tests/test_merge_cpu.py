"""Pins of the key-sharded selection's oracle and input layout (CPU only).

The context of a request is split over G shards by page (the GLM-5.2 release
test-suite page: 64-key pages interleaved over ranks, each rank's top-k
merged by owner).  Checked here without the GPU:
  * oracle.merge_topk on hand-computed cases (ties across shards, NaN, -0/+0,
    fewer than k candidates);
  * the merge property: the top-k of the union of the shards' own top-k sets
    equals the row's top-k over all its keys (oracle.topk on the full row);
  * synthetic.shard_problem: the shard's page table and bounds hold exactly
    the keys 64*(g + G*j) + o of the request below each row's bound.
"""
import numpy as np
import pytest

import oracle
import synthetic as syn


def test_merge_hand_cases():
    nan = float("nan")
    # two shards, k = 3: 5.0 at indices 10 and 4 (both taken), 3.0 at 2 and 70
    # (the lower index wins), an empty slot
    s = [5.0, 3.0, 1.0, 5.0, 3.0, 0.0]
    i = [10, 2, 7, 4, 70, -1]
    assert oracle.merge_topk(s, i, 3).tolist() == [2, 4, 10]
    # NaN ranks below every number
    assert oracle.merge_topk([nan, 1.0], [0, 5], 1).tolist() == [5]
    assert oracle.merge_topk([nan, 1.0], [0, 5], 2).tolist() == [0, 5]
    # -0 equals +0: the lower index wins
    assert oracle.merge_topk([-0.0, 0.0], [9, 3], 1).tolist() == [3]
    # fewer than k candidates: all of them, then -1
    assert oracle.merge_topk([2.0, 1.0, 0.0], [6, 1, -1], 4).tolist() == [1, 6, -1, -1]
    # -inf still ranks above NaN
    assert oracle.merge_topk([nan, -np.inf], [1, 2], 1).tolist() == [2]


def _global_of_shard(n, g, G):
    """Global keys of shard g (pages g, g+G, ...), in the shard's order."""
    keys = []
    for page in range(g, -(-n // 64), G):
        keys.extend(range(64 * page, min(64 * page + 64, n)))
    return np.array(keys, dtype=np.int64)


@pytest.mark.parametrize("n,G,k", [(1000, 2, 100), (5003, 3, 2048), (20000, 8, 2048),
                                   (20000, 8, 100), (130, 4, 50), (64 * 9, 8, 2048)])
def test_union_of_shard_topk_is_the_global_topk(n, G, k):
    rng = np.random.default_rng(n + G + k)
    full = rng.standard_normal(n).astype(np.float32)
    dup = rng.integers(0, n, size=n // 20)             # repeated values: ties across shards
    full[dup] = full[rng.integers(0, n, size=dup.size)]
    full[rng.integers(0, n, size=3)] = np.nan
    cs, ci = [], []
    for g in range(G):
        gk = _global_of_shard(n, g, G)
        local = full[gk]
        sel = oracle.topk(local, k)
        sel = sel[sel >= 0]                            # a shard may hold no key at all
        cs.append(np.concatenate([local[sel], np.zeros(k - sel.size, np.float32)]))
        ci.append(np.concatenate([gk[sel], np.full(k - sel.size, -1)]))
    merged = oracle.merge_topk(np.concatenate(cs), np.concatenate(ci), k)
    want = np.sort(oracle.topk(full, k))
    want = np.concatenate([want[want >= 0], want[want < 0]])
    assert merged.tolist() == want.tolist()


@pytest.mark.parametrize("G", [1, 2, 3, 8])
def test_shard_problem_holds_the_interleaved_pages(G):
    n = 64 * 37 + 13
    p = syn.build_problem("shardmap", 5, [n, 700], [(0, n), (0, n - 70), (1, 700), (1, 64), (0, 0)])
    seen = {r: [] for r in range(p.rows)}
    for g in range(G):
        ps = syn.shard_problem(p, g, G)
        for r in range(p.rows):
            b = int(ps.row_bound[r])
            pt = ps.page_table[int(ps.row_pt[r])]
            for s in range(b):
                page = int(pt[s // 64])
                glob = 64 * (g + G * (s // 64)) + s % 64
                # the physical page of the shard's key is the request's page of its global key
                assert page == int(p.page_table[int(p.row_pt[r])][glob // 64])
                seen[r].append(glob)
    for r in range(p.rows):
        assert sorted(seen[r]) == list(range(int(p.row_bound[r])))
