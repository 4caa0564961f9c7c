"""The new-key write on MI355X against the oracle.

Each row's own key (bf16) is quantized to E4M3 codes plus a scale and written
at the row's last position (bound - 1); the rows of its request then score the
cache with it (the sglang pull request page "sgl-project/sglang#48224",
sgl-amd-mono #86 commit body, Modifications row 2 and the Reviewer notes on
new keys).  Checked: the whole cache after the write equals the oracle's write
byte for byte (codes) and bit for bit (scales), with nothing else touched;
the scores of the combined call are within tolerance of the oracle's scores
of the written cache, the selection is bit-exact on the GPU's own scores and
the combined call equals a write followed by the ordinary launch.
"""
import dataclasses

import numpy as np
import pytest
import torch

import fp8_key_scoring_amd as fk
import oracle
import synthetic as syn
from gpu_util import (check_scores_full, check_topk_exact, check_untouched_past_bound, oracle_rows,
                      overlap, say, to_device, OVERLAP_MIN)

pytestmark = pytest.mark.gpu


def _kn_dev(kn):
    return torch.from_numpy(np.ascontiguousarray(kn).view(np.int16)).to("cuda:0").view(torch.bfloat16)


def _write_on_gpu(p, kn):
    d = to_device(p)
    fk.indexer_write_keys(_kn_dev(kn), d["k_e4m3"], d["k_scale"], d["page_table"], d["row_pt"],
                          d["row_bound"], max_bound=p.max_bound)
    torch.cuda.synchronize()
    return d["k_e4m3"].cpu().numpy(), d["k_scale"].cpu().numpy()


def _check_cache(p, kn):
    k8, ks = _write_on_gpu(p, kn)
    k8o, kso = oracle.write_new_keys(p, kn)
    diff = np.argwhere(np.any(k8 != k8o, axis=2))
    assert diff.size == 0, f"codes differ at (page, slot) {diff[:4].tolist()}"
    assert np.array_equal(ks.view(np.uint32), kso.view(np.uint32)), "scales differ"
    return k8o, kso


def test_write_many_keys_bytes_match_oracle():
    # 300 rows of one request at consecutive positions (distinct slots over
    # five pages), edge keys first: all zeros, subnormal codes, ties, -0
    n = 9000
    p = syn.build_problem("newkeys_many", 31, [n], syn.verify_rows(0, n, 300))
    kn = syn.new_keys(p, 3)
    say(f"[gpu] new-key write: rows={p.rows} n={n}")
    _check_cache(p, kn)


def test_write_positions_and_skips():
    # page starts and ends, bound 1, bound 0 (no write), two requests, a
    # page-table row whose page ids at the written positions are out of range
    n, m = 64 * 6, 700
    p = syn.build_problem("newkeys_pos", 32, [n, m],
                          [(0, 1), (0, 64), (0, 65), (0, 128), (0, n), (1, 0), (1, 700), (1, 640)])
    p.page_table[1, 699 // 64] = p.num_pages + 5    # row 6 (position 699) writes nothing
    p.page_table[1, 639 // 64] = -3                  # nor does row 7 (position 639)
    kn = syn.new_keys(p, 4)
    say(f"[gpu] new-key write positions: rows={p.rows}")
    k8o, kso = _check_cache(p, kn)
    changed = np.argwhere(np.any(k8o != p.k_e4m3, axis=2) | (kso.view(np.uint32) != p.k_scale.view(np.uint32)))
    assert len(changed) == 5                          # rows 0-4 write; 5, 6 and 7 do not


def _launch_case(p, kn):
    d = to_device(p)
    mb = p.max_bound
    scores = torch.full((p.rows, mb), float("nan"), dtype=torch.float32, device="cuda:0")
    out = fk.indexer_launch_new_keys(d["q"], d["w"], _kn_dev(kn), d["k_e4m3"], d["k_scale"], d["page_table"],
                                     d["row_pt"], d["row_bound"], max_bound=mb, topk=p.topk, scores=scores)
    torch.cuda.synchronize()
    # the same as a write followed by the ordinary launch
    d2 = to_device(p)
    fk.indexer_write_keys(_kn_dev(kn), d2["k_e4m3"], d2["k_scale"], d2["page_table"], d2["row_pt"],
                          d2["row_bound"], max_bound=mb)
    scores2 = torch.full_like(scores, float("nan"))
    out2 = fk.indexer_launch(**d2, max_bound=mb, topk=p.topk, scores=scores2)
    torch.cuda.synchronize()
    g, o = scores.cpu().numpy(), out.cpu().numpy()
    assert np.array_equal(g.view(np.uint32), scores2.cpu().numpy().view(np.uint32))
    assert np.array_equal(o, out2.cpu().numpy())
    assert np.array_equal(d["k_e4m3"].cpu().numpy(), d2["k_e4m3"].cpu().numpy())
    # against the oracle on the written cache
    k8o, kso = oracle.write_new_keys(p, kn)
    assert np.array_equal(d["k_e4m3"].cpu().numpy(), k8o)
    pw = dataclasses.replace(p, k_e4m3=k8o, k_scale=kso)
    ref = oracle_rows(pw, range(p.rows))
    worst = check_scores_full(pw, g, ref)
    check_untouched_past_bound(pw, g)
    check_topk_exact(pw, g, o)
    ov = overlap(pw, ref, o)
    say(f"[gpu] {p.name}: worst err/tol {worst:.3f}, min overlap {ov:.5f}")
    assert ov >= OVERLAP_MIN
    return pw, g


def test_launch_new_keys_four_verify_rows():
    n = 20000
    p = syn.build_problem("newkeys_launch4", 33, [n], syn.verify_rows(0, n))
    kn = syn.new_keys(p, 5, special=False)
    # make the new keys large so they are selected: their scores must come
    # from the written codes, not from what the slots held before
    kn = syn.bf16_bits_rne(((kn.astype(np.uint32) << 16).view(np.float32) * 4).astype(np.float32))
    pw, g = _launch_case(p, kn)
    # the check is sensitive to the write: at the new keys' positions the
    # oracle's scores of the written cache differ from those of the old one
    r = p.rows - 1
    pos = p.row_bound.astype(np.int64) - 1
    new_sc, _ = oracle.score_samples(pw, np.full(pos.size, r), pos)
    old_sc, _ = oracle.score_samples(p, np.full(pos.size, r), pos)
    assert np.all(new_sc != old_sc)


def test_launch_new_keys_eight_row_request_and_a_second():
    # an 8-row request is scored as two groups of four: the second group must
    # see the first group's new keys too; a second request alongside
    n, m = 30000, 5000
    p = syn.build_problem("newkeys_launch8", 34, [n, m], syn.verify_rows(0, n, 8) + syn.verify_rows(1, m, 3))
    kn = syn.new_keys(p, 6)
    _launch_case(p, kn)


def test_launch_new_keys_many_requests():
    # a batch of 24 requests of 4 verify rows each, lengths from 300 to
    # 12,000 keys, one pool: every request's rows write and score their own
    # new keys only
    rng = np.random.default_rng(35)
    lens = [int(x) for x in rng.integers(300, 12000, size=24)]
    rows = []
    for i, n in enumerate(lens):
        rows += syn.verify_rows(i, n)
    p = syn.build_problem("newkeys_batch", 35, lens, rows)
    kn = syn.new_keys(p, 7)
    say(f"[gpu] new keys, batch: rows={p.rows} requests={len(lens)}")
    _launch_case(p, kn)


def test_write_hand_worked_cases():
    # the hand-worked quantizations of tests/golden/quant_hand_cases.json,
    # written by the GPU and read back from the cache
    import json, os
    cases = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "quant_hand_cases.json")))["cases"]
    n = 64 * 4
    p = syn.build_problem("newkeys_hand", 36, [n], [(0, 10 + 70 * i) for i in range(len(cases))])
    kn = np.zeros((p.rows, 128), np.uint16)
    for r, case in enumerate(cases):
        for i, bits in case["k_bf16_bits"].items():
            kn[r, int(i)] = int(bits, 16)
    k8, ks = _write_on_gpu(p, kn)
    for r, case in enumerate(cases):
        pos = int(p.row_bound[r]) - 1
        page = int(p.page_table[0][pos // 64])
        want = np.zeros(128, np.uint8)
        for i, c in case["codes"].items():
            want[int(i)] = int(c, 16)
        assert np.array_equal(k8[page, pos % 64], want), case["name"]
        assert int(ks[page, pos % 64:pos % 64 + 1].view(np.uint32)[0]) == int(case["scale_bits"], 16), case["name"]


def test_write_hand_worked_positions():
    # the literal positions of tests/golden/new_key_positions.json, written by the GPU
    from golden_cases import check_new_key_positions, new_key_positions
    p, kn, want = new_key_positions()
    say(f"[gpu] new-key write, hand-worked positions: rows={p.rows}")
    k8, ks = _write_on_gpu(p, kn)
    check_new_key_positions(k8, ks, want, p.k_e4m3, p.k_scale)
