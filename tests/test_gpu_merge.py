"""Key-sharded selection on MI355X: the context split over G shards by page
(pages g, g+G, ... in shard g), each shard's own launch, its candidates, and
the exact merge.  Every key scores bit for bit the same in its shard as in
the unsharded launch, so the merged selection must equal the unsharded one as
a set, and equal the oracle's merge of the same candidates; the merge writes
it in candidate-slot order."""
import numpy as np
import pytest
import torch

import fp8_key_scoring_amd as fk
import oracle
import synthetic as syn
from gpu_util import run_launch, say, to_device

pytestmark = pytest.mark.gpu


def _sharded(p, G):
    """Per-shard launches (scores kept), candidates, merge; returns the merged
    selection and the candidates on the host."""
    k = p.topk
    cand_s = torch.empty((p.rows, G * k), dtype=torch.float32, device="cuda:0")
    cand_i = torch.empty((p.rows, G * k), dtype=torch.int32, device="cuda:0")
    for g in range(G):
        ps = syn.shard_problem(p, g, G)
        d = to_device(ps)
        mb = ps.max_bound
        scores = torch.full((ps.rows, max(1, mb)), float("nan"), dtype=torch.float32, device="cuda:0")
        out = fk.indexer_launch(**d, max_bound=mb, topk=k, scores=scores)
        fk.indexer_shard_candidates(scores, out, shard=g, shards=G, max_bound=mb,
                                    cand_score=cand_s, cand_idx=cand_i)
    merged = fk.indexer_merge_topk(cand_s, cand_i, shards=G, topk=k)
    torch.cuda.synchronize()
    return merged.cpu().numpy(), cand_s.cpu().numpy(), cand_i.cpu().numpy()


def _canon(x):
    """A selection as a set: its indices ascending, then the -1 padding."""
    x = np.asarray(x)
    return np.concatenate([np.sort(x[x >= 0]), x[x < 0]])


def _check(p, G):
    say(f"[gpu] sharded {p.name}: rows={p.rows} max_bound={p.max_bound} shards={G}")
    full_scores, full_out = run_launch(p)
    merged, cs, ci = _sharded(p, G)
    for r in range(p.rows):
        assert np.array_equal(_canon(merged[r]), full_out[r]), f"row {r}: merged selection differs"
        assert np.array_equal(_canon(merged[r]), oracle.merge_topk(cs[r], ci[r], p.topk)), f"row {r}: oracle merge"
        # output order: grouped by shard in candidate-slot order
        slot = {int(v): j for j, v in enumerate(ci[r]) if v >= 0}
        pos = [slot[int(v)] for v in merged[r] if v >= 0]
        assert pos == sorted(pos), f"row {r}: not in slot order"
        assert (merged[r][len(pos):] == -1).all()
        ok = ci[r] >= 0
        # a candidate's score is the unsharded launch's score of its global key, bit for bit
        assert np.array_equal(cs[r][ok].view(np.uint32), full_scores[r][ci[r][ok]].view(np.uint32))


@pytest.mark.parametrize("G", [2, 4, 8])
def test_sharded_four_rows_128k(G):
    _check(syn.make_config(2), G)


def test_sharded_ragged_rows_and_short_rows():
    # bounds that end inside a page, rows with fewer keys than k in some or
    # all shards, two requests
    n, m = 9000, 2100
    p = syn.build_problem("shard_ragged", 17, [n, m], syn.verify_rows(0, n) + syn.verify_rows(1, m),
                          dup_frac=0.02)
    for G in (3, 8):
        _check(p, G)


def test_sharded_c3_eight_shards():
    _check(syn.make_config(3), 8)


def test_sharded_smaller_topk():
    # k = 1000 (G * k a multiple of 16, as the merge requires): the
    # candidate blocks and the merge at a k other than 2048
    n = 30000
    p = syn.build_problem("shard_k1000", 19, [n], syn.verify_rows(0, n), topk=1000, dup_frac=0.02)
    _check(p, 8)
