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
