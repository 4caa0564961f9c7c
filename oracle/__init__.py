"""ctypes binding of the plain CPU oracle (``oracle/oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.  It shares no code
with the HIP library; both are fed the same seeded inputs from ``synthetic``.

Every function here is argument marshalling around the C file, which states
the definition it follows (the paged FP8 indexer of the sglang pull request
page "sgl-project/sglang#48224", sgl-amd-mono #86 commit body).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (fp64, -O2, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fno-fast-math",
                               "-ffp-contract=off", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        I = ctypes.c_int
        lib.oracle_e4m3_decode.restype = ctypes.c_double
        lib.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
        lib.oracle_bf16_decode.restype = ctypes.c_double
        lib.oracle_bf16_decode.argtypes = [ctypes.c_uint16]
        lib.oracle_score_range.restype = I
        lib.oracle_score_range.argtypes = [I, I64, I64, P, P, P, P, I, P, I, I, P, P, P, P]
        lib.oracle_score_samples.restype = I
        lib.oracle_score_samples.argtypes = [I64, P, P, P, P, P, P, I, P, I, I, P, P, P, P]
        lib.oracle_quantize_key.restype = I
        lib.oracle_quantize_key.argtypes = [P, P, P]
        lib.oracle_e4m3_nearest.restype = ctypes.c_uint8
        lib.oracle_e4m3_nearest.argtypes = [ctypes.c_float]
        lib.oracle_topk_f32.restype = I
        lib.oracle_topk_f32.argtypes = [P, I64, I, P]
        lib.oracle_topk_f64.restype = I
        lib.oracle_topk_f64.argtypes = [P, I64, I, P]
        lib.oracle_sparse_attention.restype = I
        lib.oracle_sparse_attention.argtypes = [P, P, I, P, I, I, I, P, I, I, ctypes.c_double, P, P]
        _lib = lib
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def e4m3_decode(code: int) -> float:
    return float(_load().oracle_e4m3_decode(int(code) & 0xFF))


def bf16_decode(bits: int) -> float:
    return float(_load().oracle_bf16_decode(int(bits) & 0xFFFF))


def _arrays(p):
    return (np.ascontiguousarray(p.q_bf16, dtype=np.uint16),
            np.ascontiguousarray(p.w, dtype=np.float32),
            np.ascontiguousarray(p.k_e4m3, dtype=np.uint8),
            np.ascontiguousarray(p.k_scale, dtype=np.float32),
            np.ascontiguousarray(p.page_table, dtype=np.int32),
            np.ascontiguousarray(p.row_pt, dtype=np.int32),
            np.ascontiguousarray(p.row_bound, dtype=np.int32))


def score_range(p, r: int, s0: int = 0, s1: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
    """fp64 scores and tolerance scales of row r for keys [s0, s1) ∩ [0, bound)."""
    q, w, k8, ks, pt, rp, rb = _arrays(p)
    b = int(rb[r])
    s1 = b if s1 is None else min(int(s1), b)
    n = max(0, s1 - s0)
    sc = np.empty(max(n, 1), dtype=np.float64)
    bd = np.empty(max(n, 1), dtype=np.float64)
    rc = _load().oracle_score_range(int(r), int(s0), int(s1), _p(q), _p(w), _p(k8), _p(ks),
                                    int(k8.shape[0]), _p(pt), int(pt.shape[0]), int(pt.shape[1]),
                                    _p(rp), _p(rb), _p(sc), _p(bd))
    if rc != 0:
        raise RuntimeError(f"oracle_score_range failed: {rc}")
    return sc[:n], bd[:n]


def score_samples(p, rows: np.ndarray, keys: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """fp64 scores and tolerance scales for explicit (row, key) samples."""
    q, w, k8, ks, pt, rp, rb = _arrays(p)
    rows = np.ascontiguousarray(rows, dtype=np.int32)
    keys = np.ascontiguousarray(keys, dtype=np.int64)
    n = rows.size
    sc = np.empty(max(n, 1), dtype=np.float64)
    bd = np.empty(max(n, 1), dtype=np.float64)
    rc = _load().oracle_score_samples(int(n), _p(rows), _p(keys), _p(q), _p(w), _p(k8), _p(ks),
                                      int(k8.shape[0]), _p(pt), int(pt.shape[0]), int(pt.shape[1]),
                                      _p(rp), _p(rb), _p(sc), _p(bd))
    if rc != 0:
        raise RuntimeError(f"oracle_score_samples failed: {rc}")
    return sc[:n], bd[:n]


def topk(scores: np.ndarray, k: int) -> np.ndarray:
    """Exact top-k of one row (fp32 or fp64 values), ties to the lower index,
    NaN last; returns int32[k] padded with -1 (order: selection order)."""
    out = np.empty(k, dtype=np.int32)
    if scores.dtype == np.float32:
        a = np.ascontiguousarray(scores)
        rc = _load().oracle_topk_f32(_p(a), int(a.size), int(k), _p(out))
    else:
        a = np.ascontiguousarray(scores, dtype=np.float64)
        rc = _load().oracle_topk_f64(_p(a), int(a.size), int(k), _p(out))
    if rc != 0:
        raise RuntimeError(f"oracle_topk failed: {rc}")
    return out


def merge_topk(cand_scores: np.ndarray, cand_idx: np.ndarray, k: int) -> np.ndarray:
    """Exact top-k of one row over candidate (score, global index) pairs, the
    union of the shards' own top-k sets when the context is split over shards
    by page (the GLM-5.2 release test-suite page: 64-key pages interleaved
    over ranks, top-k merged by owner).  Order as for the unsharded top-k:
    larger score first, NaN below every number, equal scores (and -0 == +0)
    to the lower global index.  Candidates with index -1 are empty.  Returns
    the selected global indices ascending, int32[k] padded with -1.

    The plain definition, written out: a stable sort of the valid pairs by
    (-score, index), the first k."""
    s = np.asarray(cand_scores, dtype=np.float32).ravel()
    i = np.asarray(cand_idx, dtype=np.int64).ravel()
    keep = i >= 0
    s, i = s[keep], i[keep]
    order = np.lexsort((i, -s.astype(np.float64)))   # NaN sorts last in either sign
    sel = np.sort(i[order[:k]])
    out = np.full(k, -1, dtype=np.int32)
    out[:sel.size] = sel
    return out


def e4m3_nearest(x: float) -> int:
    """The E4M3 code of one fp32 value: nearest finite code, ties to the even
    mantissa, saturating at +-448 (oracle.c states the rule)."""
    return int(_load().oracle_e4m3_nearest(ctypes.c_float(float(x))))


def quantize_key(k_bf16: np.ndarray) -> Tuple[np.ndarray, np.float32]:
    """One new key (128 raw bf16 patterns) -> its 128 E4M3 codes and fp32
    scale (amax / 448; oracle.c states the rule)."""
    k = np.ascontiguousarray(k_bf16, dtype=np.uint16).reshape(-1)
    if k.size != 128:
        raise ValueError("a key has 128 elements")
    codes = np.empty(128, dtype=np.uint8)
    sc = np.empty(1, dtype=np.float32)
    rc = _load().oracle_quantize_key(_p(k), _p(codes), _p(sc))
    if rc != 0:
        raise RuntimeError(f"oracle_quantize_key failed: {rc}")
    return codes, sc[0]


def write_new_keys(p, k_new_bf16: np.ndarray):
    """The launch's new-key write applied to host copies of the cache: row r
    (in row order, so a later row wins a slot two rows name) writes its key
    k_new[r] at logical position bound[r] - 1 of its page-table row, i.e.
    page page_table[row_pt[r]][(bound - 1) // 64], slot (bound - 1) % 64.
    A row with bound 0, a page-table row or page id out of range writes
    nothing.  Returns (k_e4m3, k_scale) copies with the keys written; the
    scores of the launch are then those of the written cache (the same page,
    Reviewer notes "New keys": every row of the request that reaches the
    position scores the new key)."""
    k8 = np.array(p.k_e4m3, dtype=np.uint8, copy=True)
    ks = np.array(p.k_scale, dtype=np.float32, copy=True)
    kn = np.asarray(k_new_bf16, dtype=np.uint16).reshape(p.rows, 128)
    pt = np.asarray(p.page_table)
    for r in range(p.rows):
        b = min(max(int(p.row_bound[r]), 0), int(p.max_bound))
        pr = int(p.row_pt[r])
        if b == 0 or pr < 0 or pr >= pt.shape[0]:
            continue
        page = int(pt[pr][(b - 1) // 64])
        if page < 0 or page >= k8.shape[0]:
            continue
        codes, sc = quantize_key(kn[r])
        k8[page, (b - 1) % 64, :] = codes
        ks[page, (b - 1) % 64] = sc
    return k8, ks


ATTN_HEADS = 16
ATTN_DIM = 576
ATTN_VDIM = 512


def sparse_attention(q_bf16: np.ndarray, kv_bf16: np.ndarray, page_table: np.ndarray, row_pt: np.ndarray,
                     sel: np.ndarray, max_bound: int, sm_scale: float, rows=None) -> Tuple[np.ndarray, np.ndarray]:
    """Sparse attention of each row's 16 heads over its selected key
    positions (oracle.c states the reading): returns (out [rows, 16, 512]
    fp64, lse [rows, 16] fp64) for the given rows (all by default).

    q_bf16 [R, 16, 576] and kv_bf16 [pages, 64, 576] are raw bf16 patterns
    (uint16); sel [R, topk] int32 logical positions, -1 for none."""
    q = np.ascontiguousarray(q_bf16, dtype=np.uint16)
    kv = np.ascontiguousarray(kv_bf16, dtype=np.uint16)
    pt = np.ascontiguousarray(page_table, dtype=np.int32)
    sl = np.ascontiguousarray(sel, dtype=np.int32)
    rows = range(q.shape[0]) if rows is None else rows
    rows = list(rows)
    out = np.zeros((len(rows), ATTN_HEADS, ATTN_VDIM), np.float64)
    lse = np.zeros((len(rows), ATTN_HEADS), np.float64)
    for i, r in enumerate(rows):
        o = np.zeros((ATTN_HEADS, ATTN_VDIM), np.float64)
        l = np.zeros(ATTN_HEADS, np.float64)
        rc = _load().oracle_sparse_attention(_p(q[r]), _p(kv), int(kv.shape[0]), _p(pt), int(pt.shape[0]),
                                             int(pt.shape[1]), int(row_pt[r]), _p(sl[r]), int(sl.shape[1]),
                                             int(max_bound), float(sm_scale), _p(o), _p(l))
        if rc != 0:
            raise RuntimeError(f"oracle_sparse_attention failed: {rc}")
        out[i] = o
        lse[i] = l
    return out, lse
