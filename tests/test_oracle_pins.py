"""Pins of the CPU oracle against things other than itself (no GPU).

Decoders: the OCP E4M3FN spec table and torch's float8_e4m3fn / bfloat16
dtypes (library routines).  Scores: hand-worked fixtures (tests/golden), a
special case that reduces to a GEMV checked with numpy, exact power-of-two
scalings, invariance under a permutation of the head dims and under a
relabelling of physical pages.  Top-k: hand-worked fixtures, brute force with
Python's sort on small rows, invariants (threshold cut) and closed forms.
Each pin is chosen so that a plausible slip in the oracle (a dropped ReLU,
scale or weight, a wrong sign, a transposed q, a wrong page lookup, ties by
the higher index, an off-by-one bound) fails at least one of them.
"""
import math

import numpy as np
import pytest
import torch

import golden_cases as gc
import synthetic as syn


# ------------------------------------------------------------------ decode
SPEC_E4M3 = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0,
             0x39: 1.125, 0x40: 2.0, 0x7E: 448.0, 0x80: -0.0, 0xB8: -1.0, 0xFE: -448.0}


def test_e4m3_spec_table(oracle_lib):
    for code, v in SPEC_E4M3.items():
        got = oracle_lib.e4m3_decode(code)
        assert got == v and math.copysign(1, got) == math.copysign(1, v), hex(code)
    assert math.isnan(oracle_lib.e4m3_decode(0x7F)) and math.isnan(oracle_lib.e4m3_decode(0xFF))


def test_e4m3_all_codes_match_torch(oracle_lib):
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    for c in range(256):
        got = oracle_lib.e4m3_decode(c)
        if math.isnan(ref[c]):
            assert math.isnan(got)
        else:
            assert got == float(ref[c]) and math.copysign(1, got) == math.copysign(1, ref[c]), hex(c)


def test_bf16_decode_matches_torch(oracle_lib):
    rng = np.random.default_rng(0)
    bits = np.concatenate([rng.integers(0, 65536, 4000), [0x0000, 0x8000, 0x3F80, 0x7F80, 0xFF80, 0x0001, 0x807F]])
    ref = torch.from_numpy(bits.astype(np.int16)).view(torch.bfloat16).float().numpy()
    for b, r in zip(bits, ref):
        got = oracle_lib.bf16_decode(int(b))
        assert (math.isnan(got) and math.isnan(r)) or got == float(r), hex(int(b))


def test_generator_encoder_matches_torch():
    # the data-side quantiser of the generator (not the oracle) against torch's RNE cast
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(20000) * s for s in (1e-4, 0.01, 1, 30, 300)]).astype(np.float32)
    x = x[np.abs(x) <= 448]
    ours = syn.e4m3_encode_rne(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)
    b = syn.bf16_bits_rne(x)
    refb = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(b, refb)


# ------------------------------------------------------------------ scores
@pytest.mark.parametrize("case", gc.load("score_hand_cases.json")["cases"], ids=lambda c: c["name"])
def test_score_hand_cases(oracle_lib, case):
    p = gc.score_case_problem(case)
    for r, s, score, bnd in case["expected"]:
        got, gotb = oracle_lib.score_range(p, r, s, s + 1)
        assert got[0] == score, (r, s, got[0], score)
        assert gotb[0] == bnd, (r, s, gotb[0], bnd)
    for r in range(p.rows):   # nothing at or past the bound
        sc, _ = oracle_lib.score_range(p, r, 0, 10 ** 6)
        assert sc.size == p.row_bound[r]


def _decoded(p):
    q = syn.bf16_bits_to_f32(p.q_bf16).astype(np.float64)
    lut = np.array([0.0 if (c & 0x7F) == 0x7F else
                    ((-1) ** (c >> 7)) * ((c & 7) / 8 * 2.0 ** -6 if ((c >> 3) & 15) == 0
                                          else (1 + (c & 7) / 8) * 2.0 ** (((c >> 3) & 15) - 7))
                    for c in range(256)])
    return q, lut


def _small_problem(seed, n=300, rows=2, **kw):
    return syn.build_problem("small", seed, [n], [(0, n - j) for j in range(rows)], **kw)


def test_score_reduces_to_gemv_when_relu_inactive(oracle_lib):
    # q >= 0, codes >= 0, w >= 0: every d_h >= 0, so the score is
    # scale * (sum_h w_h q_h) . k -- one GEMV, checked with numpy fp64.
    p = _small_problem(3, n=200, rows=1)
    p.q_bf16 &= 0x7FFF
    p.w = np.abs(p.w)
    p.k_e4m3 &= 0x7F
    p.k_e4m3[p.k_e4m3 == 0x7F] = 0x7E
    q, lut = _decoded(p)
    u = (p.w[0].astype(np.float64)[:, None] * q[0]).sum(0)           # [128]
    b = int(p.row_bound[0])
    pt = p.page_table[0]
    s = np.arange(b)
    keys = lut[p.k_e4m3[pt[s // 64], s % 64]]                           # [b, 128]
    scale = p.k_scale[pt[s // 64], s % 64].astype(np.float64)
    ref = scale * (keys @ u)
    got, _ = oracle_lib.score_range(p, 0)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=0)


def test_score_difference_with_negated_key_is_linear(oracle_lib):
    # relu(d) - relu(-d) = d, so score(k) - score(-k) = scale * sum_h w_h (q_h . k):
    # a GEMV that holds for any signs; it exposes a ReLU put in the wrong place.
    p = _small_problem(4, n=130, rows=2)
    neg = syn.Problem(**{**p.__dict__, "k_e4m3": p.k_e4m3 ^ 0x80})
    q, lut = _decoded(p)
    for r in range(p.rows):
        b = int(p.row_bound[r])
        s = np.arange(b)
        pt = p.page_table[p.row_pt[r]]
        keys = lut[p.k_e4m3[pt[s // 64], s % 64]]
        scale = p.k_scale[pt[s // 64], s % 64].astype(np.float64)
        lin = scale * (keys @ (p.w[r].astype(np.float64) @ q[r]))
        a, bnd = oracle_lib.score_range(p, r)
        c, bndn = oracle_lib.score_range(neg, r)
        np.testing.assert_allclose(a - c, lin, rtol=1e-9, atol=1e-12 * np.abs(bnd).max())
        # and the tolerance scale is symmetric: sum_h |w_h| |d_h| does not see the sign
        np.testing.assert_allclose(bnd, bndn, rtol=1e-12)


def test_score_exact_power_of_two_scalings(oracle_lib):
    p = _small_problem(5, n=100)
    base, _ = oracle_lib.score_range(p, 0)
    p2 = syn.Problem(**{**p.__dict__, "w": (p.w * np.float32(4.0)).astype(np.float32)})
    got, _ = oracle_lib.score_range(p2, 0)
    assert np.array_equal(got, base * 4.0)
    p3 = syn.Problem(**{**p.__dict__, "k_scale": (p.k_scale * np.float32(0.5)).astype(np.float32)})
    got, _ = oracle_lib.score_range(p3, 0)
    assert np.array_equal(got, base * 0.5)


def test_score_invariant_under_head_dim_permutation(oracle_lib):
    p = _small_problem(6, n=90, rows=1)
    perm = np.random.default_rng(0).permutation(128)
    p2 = syn.Problem(**{**p.__dict__, "q_bf16": p.q_bf16[:, :, perm].copy(),
                        "k_e4m3": p.k_e4m3[:, :, perm].copy()})
    a, _ = oracle_lib.score_range(p, 0)
    b, _ = oracle_lib.score_range(p2, 0)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12 * np.abs(a).max())


def test_score_invariant_under_page_relabel(oracle_lib):
    p = _small_problem(7, n=400, rows=2)
    P = p.num_pages
    relabel = np.random.default_rng(1).permutation(P)      # old physical -> new physical
    k8 = np.empty_like(p.k_e4m3)
    ks = np.empty_like(p.k_scale)
    k8[relabel] = p.k_e4m3
    ks[relabel] = p.k_scale
    pt = np.where(p.page_table >= 0, relabel[np.maximum(p.page_table, 0)], -1).astype(np.int32)
    p2 = syn.Problem(**{**p.__dict__, "k_e4m3": k8, "k_scale": ks, "page_table": pt})
    for r in range(p.rows):
        a, _ = oracle_lib.score_range(p, r)
        b, _ = oracle_lib.score_range(p2, r)
        assert np.array_equal(a, b)


def test_score_samples_agree_with_range(oracle_lib):
    p = _small_problem(8, n=256, rows=3)
    rows = np.array([0, 1, 2, 0, 2], dtype=np.int32)
    keys = np.array([0, 5, 253, 255, 100], dtype=np.int64)
    got, gotb = oracle_lib.score_samples(p, rows, keys)
    for i, (r, s) in enumerate(zip(rows, keys)):
        a, b = oracle_lib.score_range(p, int(r), int(s), int(s) + 1)
        assert got[i] == a[0] and gotb[i] == b[0]


def test_score_rejects_bad_page(oracle_lib):
    p = _small_problem(9, n=128, rows=1)
    p.page_table[0, 1] = p.num_pages + 5
    with pytest.raises(RuntimeError):
        oracle_lib.score_range(p, 0)


# ------------------------------------------------------------------- top-k
@pytest.mark.parametrize("case", gc.load("topk_hand_cases.json")["cases"], ids=lambda c: c["name"])
def test_topk_hand_cases(oracle_lib, case):
    v = gc.topk_case_scores(case)
    for arr in (v, v.astype(np.float32)):
        got = oracle_lib.topk(arr, case["k"])
        assert got.tolist() == case["expected"]


def _brute(v, k):
    # Python's sort with an explicit key: (is NaN, -value, index); -0.0 == 0.0 already
    order = sorted(range(len(v)), key=lambda i: (math.isnan(v[i]), 0.0 if math.isnan(v[i]) else -v[i], i))
    out = order[:k]
    return out + [-1] * (k - len(out))


def test_topk_matches_python_sort_on_small_rows(oracle_lib):
    rng = np.random.default_rng(11)
    for trial in range(300):
        n = int(rng.integers(0, 60))
        k = int(rng.integers(1, 70))
        v = rng.integers(-4, 5, size=n).astype(np.float32) * np.float32(0.5)   # many ties
        if n and trial % 5 == 0:
            v[rng.integers(0, n, size=3)] = np.nan
        if n and trial % 7 == 0:
            v[rng.integers(0, n, size=2)] = -0.0
        got = oracle_lib.topk(v, k).tolist()
        assert got == _brute(v.tolist(), k), (v, k)


def check_topk_invariants(v, k, sel):
    n = len(v)
    m = min(k, n)
    chosen = [int(i) for i in sel[:m]]
    assert all(int(i) == -1 for i in sel[m:])
    assert len(set(chosen)) == m and all(0 <= i < n for i in chosen)
    if m == 0 or m == n:
        return
    key = lambda i: (-np.inf if np.isnan(v[i]) else v[i])
    T = min(key(i) for i in chosen)
    cs = set(chosen)
    max_eq_sel = max(i for i in chosen if key(i) == T)
    for i in range(n):
        if i in cs:
            continue
        assert key(i) <= T
        if key(i) == T:
            assert i > max_eq_sel   # ties went to the lower indices


def test_topk_threshold_cut_invariant(oracle_lib):
    rng = np.random.default_rng(12)
    for _ in range(40):
        n = int(rng.integers(1, 5000))
        k = int(rng.integers(1, 2049))
        v = np.round(rng.standard_normal(n) * 3, 1).astype(np.float32)
        check_topk_invariants(v, k, oracle_lib.topk(v, k))


def test_topk_closed_forms(oracle_lib):
    n, k = 5000, 2048
    assert oracle_lib.topk(np.full(n, 1.5, np.float32), k).tolist() == list(range(k))
    inc = np.arange(n, dtype=np.float32)
    assert sorted(oracle_lib.topk(inc, k).tolist()) == list(range(n - k, n))
    small = np.random.default_rng(2).standard_normal(100).astype(np.float32)
    got = oracle_lib.topk(small, k).tolist()
    assert sorted(got[:100]) == list(range(100)) and got[100:] == [-1] * (k - 100)
