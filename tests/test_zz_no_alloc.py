"""indexer_launch_static (the launch on the library's static per-GPU scratch,
no workspace, no allocation in the call) against indexer_launch, on MI355X.

Two calls in a row on the same GPU, the second with a smaller problem (fewer
rows, shorter context): each call's selection must equal indexer_launch's on
the same inputs bit for bit, and its scores must be the same bytes.  The
second call reuses the scratch the first left behind, so it also shows that
every call leaves the counters clear.  A problem over the scratch's limits is
rejected before anything is enqueued."""
import numpy as np
import pytest
import torch

import fp8_key_scoring_amd as fk
import synthetic as syn
from gpu_util import check_topk_exact, say, to_device

pytestmark = pytest.mark.gpu


def _both(p, own_scores):
    d = to_device(p)
    mb = p.max_bound
    ref_sc = torch.full((p.rows, mb), float("nan"), dtype=torch.float32, device="cuda:0")
    ref = fk.indexer_launch(**d, max_bound=mb, topk=p.topk, scores=ref_sc)
    out = torch.full((p.rows, p.topk), -7, dtype=torch.int32, device="cuda:0")
    sc = None if own_scores else torch.full((p.rows, mb), float("nan"), dtype=torch.float32, device="cuda:0")
    fk.indexer_launch_static(**d, max_bound=mb, topk=p.topk, scores=sc, out_idx=out)
    torch.cuda.synchronize()
    ref_np = ref.cpu().numpy()
    out_np = out.cpu().numpy()
    assert np.array_equal(out_np, ref_np), "static launch selection differs from indexer_launch"
    if sc is not None:
        assert np.array_equal(sc.cpu().numpy().view(np.uint32), ref_sc.cpu().numpy().view(np.uint32))
    check_topk_exact(p, ref_sc.cpu().numpy(), out_np)


def test_static_launch_two_calls_second_smaller():
    big = syn.build_problem("static_big", 41, [200000, 90000],
                            syn.verify_rows(0, 200000) + syn.verify_rows(1, 90000), dup_frac=0.01)
    small = syn.build_problem("static_small", 42, [30000], syn.verify_rows(0, 30000, 3), dup_frac=0.01)
    say(f"[gpu] static launch: {big.rows} rows x {big.max_bound}, then {small.rows} rows x {small.max_bound}")
    _both(big, own_scores=False)
    _both(small, own_scores=False)


def test_static_launch_scores_in_scratch_and_ties():
    # scores kept in the scratch; then a heavy-tie row set (the selection's
    # exact fallback) and a short problem again
    p1 = syn.build_problem("static_own", 43, [120000], syn.verify_rows(0, 120000), dup_frac=0.01)
    p2 = syn.build_problem("static_ties", 44, [20000], syn.verify_rows(0, 20000), key_mode="all_equal")
    p3 = syn.build_problem("static_short", 45, [5000, 3000], [(0, 5000), (1, 3000), (1, 0)])
    say("[gpu] static launch: scores in the scratch, heavy ties, short rows")
    _both(p1, own_scores=True)
    _both(p2, own_scores=True)
    _both(p3, own_scores=False)


def test_static_launch_rejects_oversize():
    d = dict(q=torch.zeros((fk.STATIC_MAX_ROWS + 1, 64, 128), dtype=torch.bfloat16, device="cuda:0"))
    R = fk.STATIC_MAX_ROWS + 1
    q = d["q"]
    w = torch.zeros((R, 64), dtype=torch.float32, device="cuda:0")
    k8 = torch.zeros((4, 64, 128), dtype=torch.uint8, device="cuda:0")
    ks = torch.ones((4, 64), dtype=torch.float32, device="cuda:0")
    pt = torch.zeros((1, 4), dtype=torch.int32, device="cuda:0")
    rp = torch.zeros(R, dtype=torch.int32, device="cuda:0")
    rb = torch.full((R,), 256, dtype=torch.int32, device="cuda:0")
    with pytest.raises(fk.Fp8IdxError) as e:
        fk.indexer_launch_static(q, w, k8, ks, pt, rp, rb, max_bound=256)
    assert e.value.code == -5
