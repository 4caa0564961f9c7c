"""The fused launch captured in a HIP graph (torch.cuda.CUDAGraph on the
launch stream) and replayed: every replay, with new inputs copied into the
captured buffers eagerly in between, gives the bytes of an eager launch on
those inputs.  The launch enqueues kernels only (no memset, no allocation), so
a caller may capture it; the workspace it leaves zeroed is what the next
replay needs."""
import numpy as np
import pytest
import torch

import fp8_key_scoring_amd as fk
import synthetic as syn
from gpu_util import say, to_device

pytestmark = pytest.mark.gpu


def _problem(seed):
    n = 40000
    return syn.build_problem("graph", seed, [n, n // 2], syn.verify_rows(0, n) + syn.verify_rows(1, n // 2),
                             dup_frac=0.01)


def test_captured_launch_replays_like_eager_launches():
    say("[gpu] graph capture of indexer_launch")
    p = _problem(51)
    d = to_device(p)
    mb, k = p.max_bound, p.topk
    prob = fk._problem_from(d["q"], d["k_e4m3"], d["page_table"], mb, k, 0)
    ws = fk.new_workspace(prob, True, "cuda:0")
    out = torch.empty((p.rows, k), dtype=torch.int32, device="cuda:0")
    side = torch.cuda.Stream()              # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):           # warm-up outside the capture
        fk.indexer_launch(**d, max_bound=mb, topk=k, out_idx=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fk.indexer_launch(**d, max_bound=mb, topk=k, out_idx=out, workspace=ws)
    torch.cuda.synchronize()
    for trial in range(4):
        p2 = _problem(60 + trial)           # same shapes, new values
        d2 = to_device(p2)
        ref = fk.indexer_launch(**d2, max_bound=mb, topk=k)   # eager, own buffers
        torch.cuda.synchronize()
        for name in ("q", "w", "k_e4m3", "k_scale", "page_table", "row_pt", "row_bound"):
            d[name].copy_(d2[name])
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), ref.cpu().numpy()), f"replay {trial}"
        assert not ws[:1 << 20].any()       # the zero block's start is left zero
