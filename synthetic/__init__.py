"""Seeded synthetic inputs for the paged FP8-E4M3 decode indexer.

This module only *generates* inputs: query rows, head weights, a paged E4M3 key
cache with a per-key fp32 scale, page tables and row bounds.  It holds none of
the scoring or selection arithmetic, so the CPU oracle and the HIP path can both
be fed from it without sharing any of the method's code.

The workloads follow the decode indexer launch described on the sglang pull
request page "sgl-project/sglang#48224" (the sgl-amd-mono #86 commit body,
Motivation and Speed Tests sections): one request's multi-token-prediction
verify rows at consecutive positions (4 rows), long contexts (8K to 512K keys),
page size 64 and an exact top-2048 per row.  The distributions are the plain
ones stated for the workloads: q ~ N(0,1) rounded to bf16, w ~ N(0,1)/8 in
fp32, keys ~ N(0,1) in fp32 quantised to E4M3 with scale = amax/448 per key.

Draw order for one problem (numpy PCG64, ``default_rng(seed)``):
request lengths (only for the log-uniform batch) -> q -> w -> keys (page blocks
in physical order) -> duplicated keys -> page permutation.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence, Tuple

import numpy as np

H = 64          # index heads
D = 128         # head dim
PAGE = 64       # keys per page
TOPK = 2048

E4M3_MAX = 448.0


# --------------------------------------------------------------------------
# data-side codecs (quantisation of the cache write; not the scoring path)
# --------------------------------------------------------------------------
def bf16_bits_rne(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even. NaN kept NaN."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    out = r.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = (u[nan] >> 16).astype(np.uint16) | 0x0040
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def e4m3_encode_rne(x: np.ndarray) -> np.ndarray:
    """fp32 -> OCP E4M3FN codes, round to nearest even, saturating at +-448.

    Normal codes: (e+7)<<3 | m for values (1+m/8)*2^e, e in [-6, 8];
    subnormal codes: m for values m*2^-9.  NaN -> 0x7F.
    """
    x = np.asarray(x, dtype=np.float32)
    sign = np.signbit(x).astype(np.uint8) << 7
    a = np.abs(x).astype(np.float64)
    out = np.zeros(x.shape, dtype=np.uint8)
    sub = a < 2.0 ** -6
    # subnormal grid 2^-9 (rint is round-half-even); m == 8 is code 0x08 = 2^-6
    out[sub] = np.rint(a[sub] * 512.0).astype(np.uint8)
    nrm = ~sub
    an = np.minimum(a[nrm], E4M3_MAX)
    m, e = np.frexp(an)                 # an = m * 2^e, m in [0.5, 1)
    e = e - 1                           # an in [2^e, 2^(e+1))
    mant = np.rint(an / np.ldexp(1.0, e - 3))  # in [8, 16]
    carry = mant >= 16
    e = np.where(carry, e + 1, e)
    mant = np.where(carry, 8, mant)
    code = ((e + 7) << 3) | (mant.astype(np.int64) - 8)
    code = np.minimum(code, 0x7E)
    out[nrm] = code.astype(np.uint8)
    out |= sign
    out[np.isnan(x)] = 0x7F
    return out


def quantize_keys(kf: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Per-key quantisation: scale = amax/448 (fp32), code = E4M3(k/scale).

    kf: float32 [..., D].  An all-zero key gets scale 1 and zero codes.
    """
    amax = np.max(np.abs(kf), axis=-1).astype(np.float32)
    scale = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    scale = np.where(amax > 0, scale, np.float32(1.0)).astype(np.float32)
    codes = e4m3_encode_rne((kf / scale[..., None]).astype(np.float32))
    return codes, scale


# --------------------------------------------------------------------------
# the problem container
# --------------------------------------------------------------------------
@dataclasses.dataclass
class Problem:
    name: str
    q_bf16: np.ndarray       # uint16 [R, 64, 128]
    w: np.ndarray            # float32 [R, 64]
    k_e4m3: np.ndarray       # uint8 [P, 64, 128]
    k_scale: np.ndarray      # float32 [P, 64]
    page_table: np.ndarray   # int32 [T, stride]
    row_pt: np.ndarray       # int32 [R]
    row_bound: np.ndarray    # int32 [R]
    topk: int = TOPK
    seed: int = 0

    @property
    def rows(self) -> int:
        return int(self.q_bf16.shape[0])

    @property
    def num_pages(self) -> int:
        return int(self.k_e4m3.shape[0])

    @property
    def max_bound(self) -> int:
        return int(self.row_bound.max()) if self.rows else 0

    @property
    def pt_stride(self) -> int:
        return int(self.page_table.shape[1])

    def key_rows(self) -> int:
        """Sum over rows of the row bound (key-row pairs scored)."""
        return int(self.row_bound.astype(np.int64).sum())

    def distinct_keys(self) -> int:
        """Keys streamed once per request (max bound over each page-table row)."""
        best = {}
        for r in range(self.rows):
            p = int(self.row_pt[r])
            best[p] = max(best.get(p, 0), int(self.row_bound[r]))
        return int(sum(best.values()))


# --------------------------------------------------------------------------
# builders
# --------------------------------------------------------------------------
def _gen_keys(rng: np.random.Generator, num_pages: int, key_mode: str,
              block_pages: int = 512) -> Tuple[np.ndarray, np.ndarray]:
    k8 = np.empty((num_pages, PAGE, D), dtype=np.uint8)
    ks = np.empty((num_pages, PAGE), dtype=np.float32)
    if key_mode == "all_equal":
        v = rng.standard_normal(D, dtype=np.float32)
        c, s = quantize_keys(v[None, :])
        k8[:] = c[0]
        ks[:] = s[0]
        return k8, ks
    if key_mode == "extreme":
        # every finite code (max-magnitude +-448 and the subnormals included),
        # scales spread over ten binades
        finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
        k8[:] = finite[rng.integers(0, finite.size, size=k8.shape)]
        ks[:] = np.exp2(rng.uniform(-12.0, -2.0, size=ks.shape)).astype(np.float32)
        return k8, ks
    if key_mode != "normal":
        raise ValueError(key_mode)
    for p0 in range(0, num_pages, block_pages):
        p1 = min(num_pages, p0 + block_pages)
        kf = rng.standard_normal((p1 - p0, PAGE, D), dtype=np.float32)
        c, s = quantize_keys(kf)
        k8[p0:p1] = c
        ks[p0:p1] = s
    return k8, ks


def build_problem(name: str, seed: int, req_lens: Sequence[int],
                  rows: Sequence[Tuple[int, int]], topk: int = TOPK,
                  dup_frac: float = 0.0, key_mode: str = "normal",
                  permute: bool = True, pt_fill: int = -1,
                  w_nonneg: bool = False) -> Problem:
    """General builder.

    req_lens: keys per request (each request owns one page-table row).
    rows:     (request index, row bound) per query row, in launch order.
    Each request's pages come from one shared pool; the pool is laid out in
    request order and then (optionally) relabelled by a seeded permutation.
    Unused page-table entries hold ``pt_fill``.
    """
    rng = np.random.default_rng(seed)
    R = len(rows)
    q = rng.standard_normal((R, H, D), dtype=np.float32)
    q_bits = bf16_bits_rne(q)
    w = (rng.standard_normal((R, H), dtype=np.float32) / np.float32(8.0)).astype(np.float32)
    if w_nonneg:
        w = np.abs(w)
    req_pages = [max(1, math.ceil(n / PAGE)) for n in req_lens]
    num_pages = int(sum(req_pages))
    k8, ks = _gen_keys(rng, num_pages, key_mode)
    # logical page j of request i sits at pool slot start_i + j (before relabel)
    starts = np.concatenate([[0], np.cumsum(req_pages)[:-1]]).astype(np.int64)
    if dup_frac > 0:
        for i, n in enumerate(req_lens):
            ndup = int(round(dup_frac * n))
            if ndup == 0:
                continue
            perm = rng.permutation(n)
            dst = perm[:ndup]
            src = perm[ndup:][rng.integers(0, n - ndup, size=ndup)]
            dp, ds = starts[i] + dst // PAGE, dst % PAGE
            sp, ss = starts[i] + src // PAGE, src % PAGE
            k8[dp, ds] = k8[sp, ss]
            ks[dp, ds] = ks[sp, ss]
    if permute:
        relabel = rng.permutation(num_pages)      # pool slot -> physical page id
    else:
        relabel = np.arange(num_pages)
    phys_k8 = np.empty_like(k8)
    phys_ks = np.empty_like(ks)
    phys_k8[relabel] = k8
    phys_ks[relabel] = ks
    stride = max(req_pages)
    pt = np.full((len(req_lens), stride), pt_fill, dtype=np.int32)
    for i, npg in enumerate(req_pages):
        pt[i, :npg] = relabel[starts[i]:starts[i] + npg]
    row_pt = np.array([r for r, _ in rows], dtype=np.int32)
    row_bound = np.array([b for _, b in rows], dtype=np.int32)
    for (ri, b) in rows:
        if not (0 <= b <= req_lens[ri]):
            raise ValueError("row bound beyond its request")
    return Problem(name=name, q_bf16=q_bits, w=w, k_e4m3=phys_k8, k_scale=phys_ks,
                   page_table=pt, row_pt=row_pt, row_bound=row_bound, topk=topk, seed=seed)


def verify_rows(req: int, n: int, count: int = 4) -> List[Tuple[int, int]]:
    """MTP verify rows of one request at positions n-count+1..n (bounds exclusive)."""
    return [(req, n - count + 1 + j) for j in range(count)]


# --------------------------------------------------------------------------
# the five workloads
# --------------------------------------------------------------------------
CONFIG_NAMES = ["c1_1row_8k", "c2_4rows_128k", "c3_4rows_512k", "c4_8rows_512k_384k",
                "c5_256rows_loguniform",
                # small-row groups over a long context (HBM-bound): one row, and
                # two verify rows, of one 524,288-key request
                "c6_1row_512k", "c7_2rows_512k",
                # heavy ties at full length: four verify rows over 524,288
                # copies of one key (every score of a row equal)
                "c8_4rows_512k_all_equal"]


def c5_lengths(rng: np.random.Generator, nreq: int = 64,
               lo: int = 8192, hi: int = 262144) -> List[int]:
    u = rng.uniform(math.log(lo), math.log(hi), size=nreq)
    return [int(round(math.exp(v))) for v in u]


def make_config(idx: int) -> Problem:
    """Workload idx in 1..8 (seed 1000 + idx)."""
    seed = 1000 + idx
    if idx == 1:
        return build_problem(CONFIG_NAMES[0], seed, [8192], [(0, 8192)])
    if idx == 2:
        n = 131072
        return build_problem(CONFIG_NAMES[1], seed, [n], verify_rows(0, n))
    if idx == 3:
        n = 524288
        return build_problem(CONFIG_NAMES[2], seed, [n], verify_rows(0, n), dup_frac=0.01)
    if idx == 4:
        na, nb = 524288, 393216
        return build_problem(CONFIG_NAMES[3], seed, [na, nb],
                             verify_rows(0, na) + verify_rows(1, nb))
    if idx == 5:
        rng = np.random.default_rng(seed)
        lens = c5_lengths(rng)
        rows = []
        for i, n in enumerate(lens):
            rows += verify_rows(i, n)
        return build_problem(CONFIG_NAMES[4], seed + 10_000, lens, rows)
    if idx == 6:
        n = 524288
        return build_problem(CONFIG_NAMES[5], seed, [n], [(0, n)])
    if idx == 7:
        n = 524288
        return build_problem(CONFIG_NAMES[6], seed, [n], verify_rows(0, n, 2))
    if idx == 8:
        n = 524288
        return build_problem(CONFIG_NAMES[7], seed, [n], verify_rows(0, n), key_mode="all_equal")
    raise ValueError(idx)


def scale_tie_problem(n: int = 12000, topk: int = TOPK, seed: int = 7,
                      counts: Tuple[int, int] = (1000, 3000)) -> Problem:
    """Keys that share one E4M3 vector and differ only by scale in {3,2,1}*c.

    With non-negative q, codes and weights every score is a positive multiple of
    one common factor, so the row has exactly three distinct score values and
    the top-k boundary falls inside the middle group (a tie that straddles the
    threshold).  The middle-group keys are spread over random positions.
    """
    rng = np.random.default_rng(seed)
    q = np.abs(rng.standard_normal((1, H, D), dtype=np.float32))
    q_bits = bf16_bits_rne(q)
    w = np.abs(rng.standard_normal((1, H), dtype=np.float32) / np.float32(8.0)).astype(np.float32)
    npg = math.ceil(n / PAGE)
    v = np.abs(rng.standard_normal(D, dtype=np.float32))
    c, s = quantize_keys(v[None, :])
    k8 = np.broadcast_to(c[0], (npg, PAGE, D)).copy()
    base = np.float32(s[0])
    mult = np.ones(npg * PAGE, dtype=np.float32)
    pos = rng.permutation(n)
    mult[pos[:counts[0]]] = 3.0
    mult[pos[counts[0]:counts[0] + counts[1]]] = 2.0
    ks = (mult * base).astype(np.float32).reshape(npg, PAGE)
    relabel = rng.permutation(npg)
    pk8 = np.empty_like(k8)
    pks = np.empty_like(ks)
    pk8[relabel] = k8
    pks[relabel] = ks
    pt = relabel[None, :].astype(np.int32)
    return Problem(name="scale_tie", q_bf16=q_bits, w=w, k_e4m3=pk8, k_scale=pks,
                   page_table=pt, row_pt=np.zeros(1, np.int32),
                   row_bound=np.array([n], np.int32), topk=topk, seed=seed)


def shard_problem(p: Problem, g: int, shards: int) -> Problem:
    """Shard g of `shards` of a problem split by page: the shard holds pages
    g, g+shards, g+2*shards, ... of every request (the same pool; its page
    table lists them in that order), so its logical key s is the request's key
    64 * (g + shards * (s // 64)) + s % 64.  Row bounds become the number of
    the shard's keys below the row's bound."""
    pt = np.asarray(p.page_table)
    stride = pt.shape[1]
    sub = pt[:, g::shards]
    if sub.shape[1] == 0:
        sub = np.full((pt.shape[0], 1), -1, dtype=np.int32)
    bounds = []
    for r in range(p.rows):
        b = int(p.row_bound[r])
        full, rem = divmod(b, PAGE)              # whole pages below the bound, keys of the next
        nfull = max(0, -(-(full - g) // shards)) if full > g else 0   # shard pages among them
        part = rem if (rem and full % shards == g) else 0
        bounds.append(nfull * PAGE + part)
    return Problem(name=f"{p.name}_shard{g}of{shards}", q_bf16=p.q_bf16, w=p.w, k_e4m3=p.k_e4m3,
                   k_scale=p.k_scale, page_table=np.ascontiguousarray(sub, dtype=np.int32),
                   row_pt=p.row_pt, row_bound=np.array(bounds, dtype=np.int32), topk=p.topk,
                   seed=p.seed)


def device_arrays(p: Problem, device):
    """Torch tensors of a problem on ``device`` (plumbing for tests and bench)."""
    import torch
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device)
    return dict(q=t(p.q_bf16.view(np.int16)).view(torch.bfloat16), w=t(p.w),
                k_e4m3=t(p.k_e4m3), k_scale=t(p.k_scale), page_table=t(p.page_table),
                row_pt=t(p.row_pt), row_bound=t(p.row_bound))


def new_keys(p: Problem, seed: int = 0, special: bool = True) -> np.ndarray:
    """The launch's new keys, one per row: uint16 [rows, 128] raw bf16 of
    fp32 N(0,1) draws (round to nearest even).  With `special`, the first rows
    are edge keys: all zeros, one large element with tiny others (their
    quotients fall into the E4M3 subnormals and below), exact E4M3 ties
    after scaling (amax 448 makes the scale 1), and negative zeros."""
    rng = np.random.default_rng(9000 + seed)
    kf = rng.standard_normal((p.rows, 128)).astype(np.float32)
    if special:
        edge = []
        edge.append(np.zeros(128, np.float32))                                  # amax 0
        t = (rng.standard_normal(128) * 1e-3).astype(np.float32); t[5] = 300.0  # subnormal codes
        edge.append(t)
        t = np.full(128, 1.0625, np.float32); t[0] = 448.0                      # scale 1: ties
        t[1:64:2] = 1.1875; t[2:64:4] = 3 * 2.0 ** -10; t[3:64:4] = -(2.0 ** -10)
        edge.append(t)
        t = rng.standard_normal(128).astype(np.float32); t[::3] = -0.0           # -0 elements
        edge.append(t)
        for i, e in enumerate(edge[:p.rows]):
            kf[i] = e
    return bf16_bits_rne(kf)


# --------------------------------------------------------------------------
# inputs of the sparse attention after the indexer
# --------------------------------------------------------------------------
ATTN_HEADS = 16     # query heads per row (absorbed MLA decode)
ATTN_DIM = 576      # latent (512) + rotary (64) values per cache row


def attention_inputs_device(p: Problem, seed: int, device):
    """Seeded inputs of the sparse attention for problem ``p``, drawn on the
    device with torch's generator (sizes the numpy path would take seconds
    for): q_attn [rows, 16, 576] and a latent cache [num_pages, 64, 576], both
    N(0,1) rounded to bf16 by torch's cast.  The cache shares ``p``'s page
    table."""
    import torch
    g = torch.Generator(device=device).manual_seed(seed)
    q = torch.randn((p.rows, ATTN_HEADS, ATTN_DIM), generator=g, device=device).to(torch.bfloat16)
    kv = torch.empty((p.num_pages, PAGE, ATTN_DIM), dtype=torch.bfloat16, device=device)
    step = 1024   # pages per draw, so the fp32 draw stays small
    for p0 in range(0, p.num_pages, step):
        p1 = min(p.num_pages, p0 + step)
        kv[p0:p1] = torch.randn((p1 - p0, PAGE, ATTN_DIM), generator=g, device=device).to(torch.bfloat16)
    return q, kv


def random_selections_device(p: Problem, seed: int, count: int, device):
    """``count`` seeded selections [rows, topk] int32 for problem ``p``: row r
    takes topk distinct positions below its bound (all of them, then -1, when
    the bound is smaller), in random order."""
    import torch
    g = torch.Generator(device=device).manual_seed(seed)
    out = []
    for _ in range(count):
        s = torch.full((p.rows, p.topk), -1, dtype=torch.int32, device=device)
        for r in range(p.rows):
            b = int(p.row_bound[r])
            n = min(b, p.topk)
            if n:
                s[r, :n] = torch.randperm(b, generator=g, device=device)[:n].to(torch.int32)
        out.append(s)
    return out
