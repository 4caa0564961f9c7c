"""Builds synthetic.Problem instances from the hand-worked fixtures in tests/golden."""
import json
import os

import numpy as np

from synthetic import D, H, PAGE, Problem

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _w_row(spec):
    w = np.zeros(H, dtype=np.float32)
    for h in range(H):
        if "all" in spec:
            w[h] = spec["all"]
        else:
            w[h] = spec["even"] if h % 2 == 0 else spec["odd"]
    return w


def score_case_problem(case) -> Problem:
    R = len(case["row_pt"])
    q = np.zeros((R, H, D), dtype=np.uint16)
    for heads, dim, bits in case["q"]:
        hs = range(H) if heads == "all" else [int(heads)]
        for h in hs:
            d = 2 * h if dim == "2h" else int(dim)
            q[:, h, d] = int(bits, 16)
    if "w_rows" in case:
        w = np.stack([_w_row(s) for s in case["w_rows"]])
    else:
        w = np.stack([_w_row(case["w"])] * R)
    P = case["pages"]
    k8 = np.zeros((P, PAGE, D), dtype=np.uint8)
    ks = np.ones((P, PAGE), dtype=np.float32)
    for page, slot, dims, scale in case["keys"]:
        for dk, code in dims.items():
            ds = range(0, D, 2) if dk == "even" else [int(dk)]
            for d in ds:
                k8[page, slot, d] = int(code, 16)
        ks[page, slot] = scale
    return Problem(name=case["name"], q_bf16=q, w=w, k_e4m3=k8, k_scale=ks,
                   page_table=np.array(case["page_table"], dtype=np.int32),
                   row_pt=np.array(case["row_pt"], dtype=np.int32),
                   row_bound=np.array(case["row_bound"], dtype=np.int32), topk=4)


def topk_case_scores(case):
    vals = [float(v) for v in case["scores"]]
    return np.array(vals, dtype=np.float64)


def new_key_positions():
    """The problem, new keys and expected writes of golden/new_key_positions.json:
    (Problem, k_new uint16 [rows, 128], list of (page, slot, scale_bits) or None)."""
    case = load("new_key_positions.json")
    rows = case["rows"]
    R = len(rows)
    P = case["num_pages"]
    k8 = np.full((P, PAGE, D), 0x11, dtype=np.uint8)
    ks = np.full((P, PAGE), 0.5, dtype=np.float32)
    p = Problem(name="new_key_positions", q_bf16=np.zeros((R, H, D), np.uint16),
                w=np.zeros((R, H), np.float32), k_e4m3=k8, k_scale=ks,
                page_table=np.array(case["page_table"], dtype=np.int32),
                row_pt=np.array([r["row_pt"] for r in rows], dtype=np.int32),
                row_bound=np.array([r["bound"] for r in rows], dtype=np.int32))
    kn = np.zeros((R, D), dtype=np.uint16)
    for r in range(R):
        kn[r, 0] = 0x4060 + (r << 7)      # bf16 of 3.5 * 2^r
    want = [None if r["write"] is None else
            (r["write"]["page"], r["write"]["slot"], int(r["write"]["scale_bits"], 16)) for r in rows]
    return p, kn, want


def check_new_key_positions(k8, ks, want, k8_before, ks_before):
    """The cache after the write holds each listed row's codes (0x7E, then
    zeros) and scale bits at its (page, slot), and nothing else changed."""
    expect8 = k8_before.copy()
    expects = ks_before.copy()
    for w in want:
        if w is None:
            continue
        page, slot, bits = w
        expect8[page, slot, :] = 0
        expect8[page, slot, 0] = 0x7E
        expects[page, slot] = np.array([bits], np.uint32).view(np.float32)[0]
    bad = np.argwhere(np.any(k8 != expect8, axis=2))
    assert bad.size == 0, f"codes differ from the hand-worked placement at (page, slot) {bad[:4].tolist()}"
    assert np.array_equal(ks.view(np.uint32), expects.view(np.uint32)), "scales differ from the hand-worked placement"
