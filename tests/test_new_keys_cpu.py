"""Pins of the oracle's new-key quantizer and write step (CPU only).

The new-key write (the sglang pull request page "sgl-project/sglang#48224",
sgl-amd-mono #86 commit body, Modifications row 2 and the Reviewer notes on
new keys): each row's own key is quantized to E4M3 codes plus one fp32 scale
and written at the row's last position, and the rows of its request score it.
The quantizer is pinned to the OCP E4M3FN table, to torch's float8_e4m3fn
conversion (a library routine, round to nearest even) on many values, to
hand-worked ties, and to the bounds the rule implies; the write step to hand
positions, page crossings and the skip cases.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import synthetic as syn


def _torch_e4m3(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_every_finite_code_encodes_to_itself(oracle_lib):
    for c in list(range(0x00, 0x7F)) + list(range(0x80, 0xFF)):
        v = oracle_lib.e4m3_decode(c)
        assert oracle_lib.e4m3_nearest(v) == c, hex(c)


def test_hand_ties_and_saturation(oracle_lib):
    f = oracle_lib.e4m3_nearest
    assert f(1.0625) == 0x38            # 1 + 1/16: between 1.0 (even) and 1.125
    assert f(1.1875) == 0x3A            # between 1.125 (odd) and 1.25 (even)
    assert f(2.0 ** -10) == 0x00        # half the smallest subnormal: to zero
    assert f(3 * 2.0 ** -10) == 0x02    # between 2^-9 (odd) and 2^-8 (even)
    assert f(-(2.0 ** -10)) == 0x80     # a negative value rounding to zero keeps its sign
    assert f(0.9688) == 0x38            # above the 0.9375 / 1.0 midpoint
    assert f(448.0) == 0x7E and f(-448.0) == 0xFE
    assert f(470.0) == 0x7E and f(1e6) == 0x7E and f(-1e6) == 0xFE   # saturation
    assert f(-0.0) == 0x80 and f(0.0) == 0x00


def test_matches_torch_on_random_values(oracle_lib):
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.uniform(-448, 448, 4000), rng.standard_normal(4000) * 4,
                        rng.uniform(-2.0 ** -5, 2.0 ** -5, 4000)]).astype(np.float32)
    want = _torch_e4m3(x)
    got = np.array([oracle_lib.e4m3_nearest(float(v)) for v in x], dtype=np.uint8)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(x[i]), hex(got[i]), hex(want[i])) for i in bad[:5]]


def test_quantize_key_rule(oracle_lib):
    rng = np.random.default_rng(11)
    for trial in range(40):
        kf = (rng.standard_normal(128) * rng.uniform(0.01, 50)).astype(np.float32)
        kb = syn.bf16_bits_rne(kf)
        k = (kb.astype(np.uint32) << 16).view(np.float32)
        codes, sc = oracle_lib.quantize_key(kb)
        amax = np.max(np.abs(k))
        assert sc == np.float32(amax) / np.float32(448.0)          # one fp32 division
        i = int(np.argmax(np.abs(k)))
        assert codes[i] == (0xFE if k[i] < 0 else 0x7E)             # the largest element maps to 448
        want = _torch_e4m3(k / sc)                                   # fp32 quotients, then RNE
        assert np.array_equal(codes, want)
        dec = np.array([oracle_lib.e4m3_decode(c) for c in codes]) * float(sc)
        err = np.abs(dec - k.astype(np.float64))
        assert np.all(err <= 2.0 ** -4 * np.abs(k) + 2.0 ** -10 * float(sc) * (1 + 1e-6))


def test_quantize_key_zero_and_edges(oracle_lib):
    codes, sc = oracle_lib.quantize_key(np.zeros(128, np.uint16))
    assert sc == 1.0 and not codes.any()
    neg0 = np.full(128, 0x8000, np.uint16)                           # all -0: amax 0
    codes, sc = oracle_lib.quantize_key(neg0)
    assert sc == 1.0 and not codes.any()
    # amax 448: scale exactly 1, the codes are the elements' own nearest codes
    k = np.full(128, 1.0625, np.float32); k[0] = 448.0; k[1] = 1.1875; k[2] = -(2.0 ** -10); k[3] = -0.0
    codes, sc = oracle_lib.quantize_key(syn.bf16_bits_rne(k))
    assert sc == 1.0
    assert codes[0] == 0x7E and codes[1] == 0x3A and codes[2] == 0x80 and codes[3] == 0x80
    assert (codes[4:] == 0x38).all()


def test_write_step_positions_and_skips(oracle_lib):
    n = 64 * 5 + 3
    p = syn.build_problem("newkeys", 3, [n, 200], [(0, n), (0, n - 1), (0, 64), (1, 200), (1, 0), (0, 65)])
    kn = syn.new_keys(p, 1, special=False)
    k8, ks = oracle_lib.write_new_keys(p, kn)
    changed = set(map(tuple, np.argwhere(np.any(k8 != p.k_e4m3, axis=2) | (ks != p.k_scale))))
    want = set()
    for r in range(p.rows):
        b = int(p.row_bound[r])
        if b == 0:
            continue
        page = int(p.page_table[int(p.row_pt[r])][(b - 1) // 64])
        codes, sc = oracle_lib.quantize_key(kn[r])
        assert np.array_equal(k8[page, (b - 1) % 64], codes) and ks[page, (b - 1) % 64] == sc
        want.add((page, (b - 1) % 64))
    assert changed == want                        # nothing else is touched
    # two rows naming one slot: the later row's key lands
    p2 = syn.build_problem("newkeys2", 4, [500], [(0, 300), (0, 300)])
    kn2 = syn.new_keys(p2, 2, special=False)
    k8b, ksb = oracle_lib.write_new_keys(p2, kn2)
    page = int(p2.page_table[0][299 // 64])
    codes, sc = oracle_lib.quantize_key(kn2[1])
    assert np.array_equal(k8b[page, 299 % 64], codes) and ksb[page, 299 % 64] == sc


def test_new_key_generator_edges():
    p = syn.build_problem("nk", 5, [1000], [(0, 1000)] * 6)
    kn = syn.new_keys(p, 0)
    assert kn.shape == (6, 128) and kn.dtype == np.uint16
    assert not (kn[0] & 0x7FFF).any()                              # the all-zero key
    assert ((kn[3] == 0x8000).sum()) >= 40                          # negative zeros


def test_hand_worked_quantizations(oracle_lib):
    """tests/golden/quant_hand_cases.json: quantizations worked out by hand
    from the rule (the arithmetic is in each case's 'why')."""
    path = os.path.join(os.path.dirname(__file__), "golden", "quant_hand_cases.json")
    for case in json.load(open(path))["cases"]:
        k = np.zeros(128, np.uint16)
        for i, bits in case["k_bf16_bits"].items():
            k[int(i)] = int(bits, 16)
        codes, sc = oracle_lib.quantize_key(k)
        assert int(np.array([sc], np.float32).view(np.uint32)[0]) == int(case["scale_bits"], 16), case["name"]
        want = np.zeros(128, np.uint8)
        for i, c in case["codes"].items():
            want[int(i)] = int(c, 16)
        assert np.array_equal(codes, want), case["name"]


def test_hand_worked_positions(oracle_lib):
    """tests/golden/new_key_positions.json: literal (page, slot) positions of
    the new keys for bounds 1, 64, 65, 128, 130 and 100 over a hand-written
    page table, and three rows that write nothing (bound 0, a page id of -1,
    a page-table row that does not exist)."""
    from golden_cases import check_new_key_positions, new_key_positions
    p, kn, want = new_key_positions()
    k8, ks = oracle_lib.write_new_keys(p, kn)
    check_new_key_positions(k8, ks, want, p.k_e4m3, p.k_scale)
