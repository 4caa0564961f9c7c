"""Bitwise invariants of the HIP path on MI355X: determinism, the fused launch
against the separate calls, scores kept in the workspace, physical page
relabelling, row-set independence, workspace reuse and out-of-range page ids."""
import numpy as np
import pytest
import torch

import fp8_key_scoring_amd as fk
import synthetic as syn
from gpu_util import check_topk_exact, run_launch, say, to_device

pytestmark = pytest.mark.gpu


def _prob(seed=21, n=40000):
    return syn.build_problem("inv", seed, [n, n // 2], syn.verify_rows(0, n) + syn.verify_rows(1, n // 2),
                             dup_frac=0.01)


def test_two_launches_are_bitwise_equal():
    p = _prob()
    say("[gpu] determinism")
    s1, o1 = run_launch(p)
    s2, o2 = run_launch(p)
    assert np.array_equal(s1.view(np.uint32), s2.view(np.uint32))
    assert np.array_equal(o1, o2)


def test_launch_equals_score_then_topk():
    p = _prob(22)
    say("[gpu] launch vs score + topk")
    s1, o1 = run_launch(p)
    d = to_device(p)
    sc = torch.full((p.rows, p.max_bound), float("nan"), dtype=torch.float32, device="cuda:0")
    fk.indexer_score(**d, max_bound=p.max_bound, scores=sc)
    o2 = fk.indexer_topk(sc, d["row_bound"], max_bound=p.max_bound, topk=p.topk)
    torch.cuda.synchronize()
    assert np.array_equal(s1.view(np.uint32), sc.cpu().numpy().view(np.uint32))
    assert np.array_equal(o1, o2.cpu().numpy())



def test_launch_equals_its_two_stages():
    # indexer_launch_score then indexer_launch_select, with caller scores and
    # with scores in the workspace, twice in a row on one workspace
    p = _prob(25)
    say("[gpu] launch vs its two stages")
    s1, o1 = run_launch(p)
    d = to_device(p)
    mb = p.max_bound
    for own in (False, True):
        prob = fk._problem_from(d["q"], d["k_e4m3"], d["page_table"], mb, p.topk, 0)
        ws = fk.new_workspace(prob, own, "cuda:0")
        for rep in range(2):
            sc = None if own else torch.full((p.rows, mb), float("nan"), dtype=torch.float32, device="cuda:0")
            fk.indexer_launch_score(**d, max_bound=mb, topk=p.topk, scores=sc, workspace=ws)
            o2 = fk.indexer_launch_select(d["row_bound"], max_bound=mb, topk=p.topk, scores=sc, workspace=ws)
            torch.cuda.synchronize()
            if sc is not None:
                assert np.array_equal(s1.view(np.uint32), sc.cpu().numpy().view(np.uint32))
            assert np.array_equal(o1, o2.cpu().numpy()), (own, rep)
        assert not ws[:_zero_block_bytes(p.rows)].any(), "counters left non-zero"

def test_launch_plan_follows_new_contents():
    # a LaunchPlan on fixed buffers: new problem contents copied in between
    # calls give each problem's own launch, byte for byte (scores too)
    pa, pb = _prob(26), _prob(27)
    say("[gpu] launch plan over new contents")
    da, db = to_device(pa), to_device(pb)
    assert all(da[n].shape == db[n].shape for n in da)
    mb = pa.max_bound
    buf = {n: t.clone() for n, t in da.items()}
    sc = torch.full((pa.rows, mb), float("nan"), dtype=torch.float32, device="cuda:0")
    plan = fk.LaunchPlan(**buf, max_bound=mb, topk=pa.topk, scores=sc)
    for p, d in ((pa, da), (pb, db), (pa, da)):
        ref_s, ref_o = run_launch(p)
        for n in buf:
            buf[n].copy_(d[n])
        sc.fill_(float("nan"))
        out = plan()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), ref_o)
        assert np.array_equal(sc.cpu().numpy().view(np.uint32), ref_s.view(np.uint32))


def test_scores_in_workspace():
    p = _prob(23)
    say("[gpu] scores kept in the workspace")
    _, o1 = run_launch(p)
    _, o2 = run_launch(p, keep_scores=False)
    assert np.array_equal(o1, o2)


def test_page_relabel_invariance():
    p = _prob(24)
    say("[gpu] page relabel")
    s1, o1 = run_launch(p)
    relabel = np.random.default_rng(5).permutation(p.num_pages)
    k8 = np.empty_like(p.k_e4m3)
    ks = np.empty_like(p.k_scale)
    k8[relabel] = p.k_e4m3
    ks[relabel] = p.k_scale
    pt = np.where(p.page_table >= 0, relabel[np.maximum(p.page_table, 0)], -1).astype(np.int32)
    p2 = syn.Problem(**{**p.__dict__, "k_e4m3": k8, "k_scale": ks, "page_table": pt})
    s2, o2 = run_launch(p2)
    assert np.array_equal(s1.view(np.uint32), s2.view(np.uint32))
    assert np.array_equal(o1, o2)


def test_rows_scored_alone_match_rows_scored_together():
    p = _prob(25)
    say("[gpu] row-set independence")
    s_all, o_all = run_launch(p)
    for r in (0, 2, 5):
        sub = syn.Problem(**{**p.__dict__, "q_bf16": p.q_bf16[r:r + 1].copy(), "w": p.w[r:r + 1].copy(),
                             "row_pt": p.row_pt[r:r + 1].copy(), "row_bound": p.row_bound[r:r + 1].copy()})
        s1, o1 = run_launch(sub)
        b = int(p.row_bound[r])
        assert np.array_equal(s1[0, :b].view(np.uint32), s_all[r, :b].view(np.uint32))
        assert np.array_equal(o1[0], o_all[r])


def test_workspace_reuse_across_problems():
    say("[gpu] workspace reuse")
    big = _prob(26, n=60000)
    small = syn.build_problem("small", 27, [5000], syn.verify_rows(0, 5000))
    prob = fk.make_problem(rows=8, num_pages=big.num_pages, pt_rows=2, pt_stride=big.pt_stride,
                           max_bound=big.max_bound, topk=2048)
    ws = fk.new_workspace(prob, True, "cuda:0")
    ref_big = run_launch(big)[1]
    ref_small = run_launch(small)[1]
    for p, ref in [(big, ref_big), (small, ref_small), (big, ref_big), (small, ref_small), (big, ref_big)]:
        _, o = run_launch(p, keep_scores=False, workspace=ws)
        assert np.array_equal(o, ref)


def test_out_of_range_page_ids_score_nan():
    p = syn.build_problem("badpage", 28, [4096], syn.verify_rows(0, 4096))
    p.page_table[0, 3] = p.num_pages + 100     # keys 192..255
    p.page_table[0, 10] = -7                   # keys 640..703
    say("[gpu] out-of-range page ids")
    scores, out = run_launch(p)
    bad = np.zeros(4096, bool)
    bad[192:256] = True
    bad[640:704] = True
    for r in range(p.rows):
        b = int(p.row_bound[r])
        assert np.all(np.isnan(scores[r, :b][bad[:b]]))
        assert np.all(np.isfinite(scores[r, :b][~bad[:b]]))
    check_topk_exact(p, scores, out)
    assert not np.any(bad[out[out >= 0]])


def test_validate_reports_each_kind_of_bad_array():
    import torch
    p = syn.build_problem("validate", 41, [3000, 700], [(0, 3000), (0, 2999), (1, 700), (1, 64)])
    def status(pt, rp, rb, mb=None):
        st = fk.indexer_validate(torch.from_numpy(pt).to("cuda:0"), torch.from_numpy(rp).to("cuda:0"),
                                 torch.from_numpy(rb).to("cuda:0"), max_bound=p.max_bound if mb is None else mb,
                                 num_pages=p.num_pages)
        return int(st.item())
    pt, rp, rb = p.page_table.copy(), p.row_pt.copy(), p.row_bound.copy()
    assert status(pt, rp, rb) == 0
    rb2 = rb.copy(); rb2[3] = -5
    assert status(pt, rp, rb2) == fk.VALID_BOUND
    rb3 = rb.copy(); rb3[0] = p.max_bound + 1                 # past max_bound
    assert status(pt, rp, rb3) == fk.VALID_BOUND
    rp2 = rp.copy(); rp2[2] = pt.shape[0]
    assert status(pt, rp2, rb) == fk.VALID_ROW_PT
    pt2 = pt.copy(); pt2[1, 5] = p.num_pages                  # row 2 reads page 5 of request 1
    assert status(pt2, rp, rb) == fk.VALID_PAGE
    pt3 = pt.copy(); pt3[1, 10] = -1                          # page 10 of request 1 (keys 640..699)
    assert status(pt3, rp, rb) == fk.VALID_PAGE               # row 2 (bound 700) reads it
    rb4 = rb.copy(); rb4[2] = 640
    assert status(pt3, rp, rb4) == 0                          # with bound 640 no row reads it
    both = rb.copy(); both[1] = -1
    assert status(pt2, rp2, both) == fk.VALID_BOUND | fk.VALID_ROW_PT   # row 2's pages are not read: its pt row is bad


def _zero_block_bytes(rows):
    """Bytes of the workspace's zero block (the three digit histograms, the
    heavy-tie counters and the finalize arrival counters), the part every
    launch must find zero and leaves zero; the rest is scratch a launch
    writes before it reads (sizes as the library lays them out)."""
    al = lambda x: (x + 255) // 256 * 256
    rz = max(rows, 256)
    return al(rz * 16 * 64 * 4) + al(rz * 8 * 256 * 4) + al(rz * 256 * 4) + al(rz * 1024 * 4) + al(rz * 4)


def test_poisoned_scratch_gives_the_same_bytes():
    # 0xFF in every scratch byte (NaN scores, huge counts, garbage lists):
    # the launch must not read scratch it has not written
    say("[gpu] poisoned scratch")
    for p in (_prob(28, n=70000), syn.build_problem("poison_ties", 29, [9000], syn.verify_rows(0, 9000),
                                                    dup_frac=0.3)):
        ref_scores, ref = run_launch(p)
        prob = fk.make_problem(rows=p.rows, num_pages=p.num_pages, pt_rows=p.page_table.shape[0],
                               pt_stride=p.pt_stride, max_bound=p.max_bound, topk=p.topk)
        ws = fk.new_workspace(prob, True, "cuda:0")
        z = _zero_block_bytes(p.rows)
        assert ws.numel() > z
        for _ in range(2):
            ws[z:].fill_(255)
            _, o = run_launch(p, keep_scores=False, workspace=ws)
            assert np.array_equal(o, ref)
            assert not ws[:z].any()            # the zero block is left zero


def test_heavy_tie_rows_leave_the_workspace_clean():
    # rows whose threshold bin overflows the ranked ties: several finalize
    # workgroups per row count the bin's last digits, the last one to arrive
    # writes the selection and clears the row's counters.  Two launches on
    # one workspace give the same bytes, the zero block (histograms, heavy-tie
    # counters, arrival counters) is zero after each, and a normal problem on
    # the same workspace afterwards is unaffected.
    import oracle
    say("[gpu] heavy-tie rows: workspace left clean")
    rng = np.random.default_rng(41)
    n = 300000                                  # five finalize workgroups per row
    vals = np.array([1.0, np.nextafter(np.float32(1.0), np.float32(2.0))], np.float32)
    rows = np.stack([vals[rng.integers(0, 2, size=n)] for _ in range(3)]).astype(np.float32)
    rows[1, rng.choice(n, 700, replace=False)] = 4.0
    bounds = np.array([n, n - 1, 123457], np.int32)
    sc = torch.from_numpy(rows).to("cuda:0")
    rb = torch.from_numpy(bounds).to("cuda:0")
    prob = fk.make_problem(rows=3, num_pages=1, pt_rows=1, pt_stride=(n + 63) // 64, max_bound=n, topk=2048,
                           score_stride=n)
    ws = fk.new_workspace(prob, False, "cuda:0")
    want = [np.sort(oracle.topk(np.ascontiguousarray(rows[r, :bounds[r]]), 2048)) for r in range(3)]
    for rep in range(2):
        out = fk.indexer_topk(sc, rb, max_bound=n, workspace=ws).cpu().numpy()
        torch.cuda.synchronize()
        for r in range(3):
            assert np.array_equal(out[r], want[r]), (rep, r)
        assert not ws[:_zero_block_bytes(3)].any(), "counters left non-zero"
    p = _prob(42)
    ref_scores, ref = run_launch(p)
    d = to_device(p)
    o = fk.indexer_topk(torch.from_numpy(ref_scores).to("cuda:0"), d["row_bound"], max_bound=p.max_bound,
                        topk=p.topk, workspace=ws)
    assert np.array_equal(o.cpu().numpy(), ref)
