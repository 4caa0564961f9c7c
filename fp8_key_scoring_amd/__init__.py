"""Python binding of libfp8idx, the MI355X (gfx950) paged FP8 decode indexer.

Argument marshalling only: every step (scoring, masking, first-digit counting,
selection) runs in the HIP kernels behind the C ABI declared in
``include/fp8idx.h``.  PyTorch is used for device memory and the current
stream.  If the compiled library is missing the import of any entry point
raises; there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfp8idx.so")

HEADS = 64
HEAD_DIM = 128
PAGE = 64
MAX_TOPK = 2048

EXPORTED = ("fp8idx_abi_version", "fp8idx_strerror", "fp8idx_workspace_size",
            "fp8idx_workspace_init", "indexer_score", "indexer_topk", "indexer_launch",
            "indexer_launch_score", "indexer_launch_select", "indexer_launch_static",
            "fp8idx_attention_workspace_size", "indexer_sparse_attention",
            "indexer_shard_candidates", "indexer_merge_topk", "indexer_write_keys",
            "indexer_launch_new_keys", "indexer_validate")


class Problem(ctypes.Structure):
    """Mirror of fp8idx_problem_t."""
    _fields_ = [("rows", ctypes.c_int32), ("num_pages", ctypes.c_int32),
                ("pt_rows", ctypes.c_int32), ("pt_stride", ctypes.c_int32),
                ("max_bound", ctypes.c_int32), ("topk", ctypes.c_int32),
                ("score_stride", ctypes.c_int64)]


class Fp8IdxError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"fp8idx error {code}: {msg}")
        self.code = code


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the compiled library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with fp8_key_scoring_amd/build.py "
                          "(or __graft_entry__.build()); there is no fallback path")
    # torch first: the library then binds to the HIP runtime torch already
    # loaded, so both see the same devices, streams and allocations
    import torch  # noqa: F401
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    lib.fp8idx_abi_version.restype = ctypes.c_int
    lib.fp8idx_abi_version.argtypes = []
    lib.fp8idx_strerror.restype = ctypes.c_char_p
    lib.fp8idx_strerror.argtypes = [ctypes.c_int]
    lib.fp8idx_workspace_size.restype = ctypes.c_int
    lib.fp8idx_workspace_size.argtypes = [ctypes.POINTER(Problem), ctypes.c_int,
                                          ctypes.POINTER(ctypes.c_size_t)]
    lib.fp8idx_workspace_init.restype = ctypes.c_int
    lib.fp8idx_workspace_init.argtypes = [P, ctypes.c_size_t, P]
    lib.indexer_score.restype = ctypes.c_int
    lib.indexer_score.argtypes = [ctypes.POINTER(Problem), P, P, P, P, P, P, P, P, P]
    lib.indexer_topk.restype = ctypes.c_int
    lib.indexer_topk.argtypes = [ctypes.POINTER(Problem), P, P, P, P, ctypes.c_size_t, P]
    lib.indexer_launch.restype = ctypes.c_int
    lib.indexer_launch.argtypes = [ctypes.POINTER(Problem), P, P, P, P, P, P, P, P, P, P,
                                   ctypes.c_size_t, P]
    lib.indexer_launch_score.restype = ctypes.c_int
    lib.indexer_launch_score.argtypes = [ctypes.POINTER(Problem), P, P, P, P, P, P, P, P, P,
                                         ctypes.c_size_t, P]
    lib.indexer_launch_select.restype = ctypes.c_int
    lib.indexer_launch_select.argtypes = [ctypes.POINTER(Problem), P, P, P, P, ctypes.c_size_t, P]
    lib.indexer_launch_static.restype = ctypes.c_int
    lib.indexer_launch_static.argtypes = [ctypes.POINTER(Problem), P, P, P, P, P, P, P, P, P, P]
    lib.fp8idx_attention_workspace_size.restype = ctypes.c_int
    lib.fp8idx_attention_workspace_size.argtypes = [ctypes.POINTER(Problem), ctypes.POINTER(ctypes.c_size_t)]
    lib.indexer_sparse_attention.restype = ctypes.c_int
    lib.indexer_sparse_attention.argtypes = [ctypes.POINTER(Problem), P, P, P, P, P, ctypes.c_float, P, P, P,
                                             ctypes.c_size_t, P]
    lib.indexer_validate.restype = ctypes.c_int
    lib.indexer_validate.argtypes = [ctypes.POINTER(Problem), P, P, P, P, P]
    lib.indexer_write_keys.restype = ctypes.c_int
    lib.indexer_write_keys.argtypes = [ctypes.POINTER(Problem), P, P, P, P, P, P, P]
    lib.indexer_launch_new_keys.restype = ctypes.c_int
    lib.indexer_launch_new_keys.argtypes = [ctypes.POINTER(Problem), P, P, P, P, P, P, P, P, P, P,
                                            P, ctypes.c_size_t, P]
    lib.indexer_shard_candidates.restype = ctypes.c_int
    lib.indexer_shard_candidates.argtypes = [ctypes.POINTER(Problem), ctypes.c_int, ctypes.c_int,
                                             P, P, P, P, P]
    lib.indexer_merge_topk.restype = ctypes.c_int
    lib.indexer_merge_topk.argtypes = [ctypes.POINTER(Problem), ctypes.c_int, P, P, P, P]
    _lib = lib
    return lib


def _check(rc: int) -> None:
    if rc != 0:
        msg = load_library().fp8idx_strerror(rc).decode()
        raise Fp8IdxError(rc, msg)


def abi_version() -> int:
    return int(load_library().fp8idx_abi_version())


def make_problem(rows: int, num_pages: int, pt_rows: int, pt_stride: int, max_bound: int,
                 topk: int = MAX_TOPK, score_stride: int = 0) -> Problem:
    return Problem(rows, num_pages, pt_rows, pt_stride, max_bound, topk, score_stride)


def workspace_size(prob: Problem, scores_in_workspace: bool) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().fp8idx_workspace_size(ctypes.byref(prob), int(bool(scores_in_workspace)),
                                                ctypes.byref(n)))
    return int(n.value)


def _stream(device) -> int:
    import torch
    return torch.cuda.current_stream(device).cuda_stream


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def new_workspace(prob: Problem, scores_in_workspace: bool, device):
    """A zero-filled workspace tensor (uint8, 256-byte aligned base)."""
    import torch
    n = workspace_size(prob, scores_in_workspace)
    ws = torch.empty(n + 256, dtype=torch.uint8, device=device)
    off = (-ws.data_ptr()) % 256
    ws = ws[off:off + n]
    _check(load_library().fp8idx_workspace_init(ws.data_ptr(), n, _stream(ws.device)))
    return ws



def workspace_init(ws) -> None:
    """Zero-fills a workspace tensor on its device's current stream (restores
    one whose counters a misuse left non-zero)."""
    _check(load_library().fp8idx_workspace_init(ws.data_ptr(), ws.numel(), _stream(ws.device)))

def _problem_from(q, k_e4m3, page_table, max_bound: int, topk: int, score_stride: int) -> Problem:
    return make_problem(rows=q.shape[0], num_pages=k_e4m3.shape[0], pt_rows=page_table.shape[0],
                        pt_stride=page_table.shape[1], max_bound=max_bound, topk=topk,
                        score_stride=score_stride)


def _check_inputs(q, w, k_e4m3, k_scale, page_table, row_pt, row_bound):
    # (torch.Size compares equal to a tuple; one chained condition per
    # tensor keeps the per-call cost low for launch-rate callers)
    import torch
    qs = q.shape
    R = qs[0]
    assert q.dtype == torch.bfloat16 and qs[1:] == (HEADS, HEAD_DIM) and q.is_contiguous()
    assert w.dtype == torch.float32 and w.shape == (R, HEADS) and w.is_contiguous()
    ks = k_e4m3.shape
    assert k_e4m3.dtype == torch.uint8 and ks[1:] == (PAGE, HEAD_DIM) and k_e4m3.is_contiguous()
    assert k_scale.dtype == torch.float32 and k_scale.shape == (ks[0], PAGE) and k_scale.is_contiguous()
    assert page_table.dtype == torch.int32 and page_table.dim() == 2 and page_table.is_contiguous()
    assert row_pt.dtype == torch.int32 and row_pt.shape == (R,) and row_pt.is_contiguous()
    assert row_bound.dtype == torch.int32 and row_bound.shape == (R,) and row_bound.is_contiguous()
    _on_one_gpu(q, w, k_e4m3, k_scale, page_table, row_pt, row_bound)


def _on_one_gpu(first, *others) -> None:
    """The library takes raw device pointers: every tensor given (None
    skipped) must live on the first one's GPU."""
    dev = first.device
    assert dev.type == "cuda" and all(t is None or t.device == dev for t in others), \
        "every input must be on one GPU"


def _check_scores(scores, rows: int, max_bound: int, device) -> None:
    """scores must be an fp32 [>= rows, >= max_bound] matrix with unit inner
    stride on the inputs' device: the kernels write row r at scores + r *
    stride(0) for every key below the row's bound."""
    import torch
    assert scores.dtype == torch.float32, "scores must be float32"
    assert scores.dim() == 2 and scores.stride(1) == 1, "scores must be 2-D with unit inner stride"
    assert scores.shape[0] >= rows and scores.shape[1] >= max_bound, \
        f"scores {tuple(scores.shape)} too small for {rows} rows x {max_bound} keys"
    assert scores.device == device, "scores must be on the inputs' device"


def _check_out(out_idx, rows: int, topk: int, device) -> None:
    """out_idx must be a contiguous int32 [rows, topk] tensor on the inputs' device."""
    import torch
    assert out_idx.dtype == torch.int32 and out_idx.is_contiguous(), "out_idx must be contiguous int32"
    assert out_idx.shape == (rows, topk), f"out_idx must be ({rows}, {topk}), got {tuple(out_idx.shape)}"
    assert out_idx.device == device, "out_idx must be on the inputs' device"


def indexer_score(q, w, k_e4m3, k_scale, page_table, row_pt, row_bound, *, max_bound: int,
                  scores=None):
    """Scores [rows, score_stride] fp32; entries at or past a row's bound untouched."""
    import torch
    _check_inputs(q, w, k_e4m3, k_scale, page_table, row_pt, row_bound)
    if scores is None:
        scores = torch.full((q.shape[0], max(1, max_bound)), float("nan"), dtype=torch.float32,
                            device=q.device)
    _check_scores(scores, q.shape[0], max_bound, q.device)
    prob = _problem_from(q, k_e4m3, page_table, max_bound, MAX_TOPK, scores.stride(0))
    _check(load_library().indexer_score(ctypes.byref(prob), _ptr(q), _ptr(w), _ptr(k_e4m3),
                                        _ptr(k_scale), _ptr(page_table), _ptr(row_pt),
                                        _ptr(row_bound), _ptr(scores), _stream(q.device)))
    return scores


def indexer_topk(scores, row_bound, *, max_bound: int, topk: int = MAX_TOPK, out_idx=None,
                 workspace=None):
    """Exact top-k indices [rows, topk] int32 (ascending index order, -1 padded)."""
    import torch
    R = row_bound.shape[0]
    assert row_bound.dtype == torch.int32 and row_bound.is_contiguous()
    _check_scores(scores, R, max_bound, scores.device)
    _on_one_gpu(scores, row_bound, out_idx, workspace)
    prob = make_problem(rows=R, num_pages=1, pt_rows=1, pt_stride=max(1, (max_bound + 63) // 64),
                        max_bound=max_bound, topk=topk, score_stride=scores.stride(0))
    if out_idx is None:
        out_idx = torch.empty((R, topk), dtype=torch.int32, device=scores.device)
    _check_out(out_idx, R, topk, scores.device)
    if workspace is None:
        workspace = new_workspace(prob, False, scores.device)
    _check(load_library().indexer_topk(ctypes.byref(prob), _ptr(scores), _ptr(row_bound),
                                       _ptr(out_idx), _ptr(workspace), workspace.numel(),
                                       _stream(scores.device)))
    return out_idx


def indexer_launch(q, w, k_e4m3, k_scale, page_table, row_pt, row_bound, *, max_bound: int,
                   topk: int = MAX_TOPK, scores=None, out_idx=None, workspace=None):
    """Fused scoring + exact top-k.  Returns out_idx [rows, topk] int32."""
    import torch
    _check_inputs(q, w, k_e4m3, k_scale, page_table, row_pt, row_bound)
    R = q.shape[0]
    if scores is not None:
        _check_scores(scores, R, max_bound, q.device)
    sstride = scores.stride(0) if scores is not None else 0
    prob = _problem_from(q, k_e4m3, page_table, max_bound, topk, sstride)
    if out_idx is None:
        out_idx = torch.empty((R, topk), dtype=torch.int32, device=q.device)
    _check_out(out_idx, R, topk, q.device)
    if workspace is None:
        workspace = new_workspace(prob, scores is None, q.device)
    _on_one_gpu(q, workspace)
    _check(load_library().indexer_launch(ctypes.byref(prob), _ptr(q), _ptr(w), _ptr(k_e4m3),
                                         _ptr(k_scale), _ptr(page_table), _ptr(row_pt),
                                         _ptr(row_bound), _ptr(scores), _ptr(out_idx),
                                         _ptr(workspace), workspace.numel(), _stream(q.device)))
    return out_idx



class LaunchPlan:
    """indexer_launch with its arguments checked and marshalled once, for
    loops that launch on the same buffers again and again (new contents
    copied in between, as a serving step does): each call is then one C call
    on the device's current stream.  The tensors are kept alive by the plan;
    their shapes, dtypes and storage must not change while it is used.
    Arguments as for indexer_launch; ``plan()`` returns out_idx."""

    def __init__(self, q, w, k_e4m3, k_scale, page_table, row_pt, row_bound, *, max_bound: int,
                 topk: int = MAX_TOPK, scores=None, out_idx=None, workspace=None):
        import torch
        _check_inputs(q, w, k_e4m3, k_scale, page_table, row_pt, row_bound)
        R = q.shape[0]
        if scores is not None:
            _check_scores(scores, R, max_bound, q.device)
        sstride = scores.stride(0) if scores is not None else 0
        self._prob = _problem_from(q, k_e4m3, page_table, max_bound, topk, sstride)
        if out_idx is None:
            out_idx = torch.empty((R, topk), dtype=torch.int32, device=q.device)
        _check_out(out_idx, R, topk, q.device)
        if workspace is None:
            workspace = new_workspace(self._prob, scores is None, q.device)
        _on_one_gpu(q, workspace)
        self.out_idx = out_idx
        self._keep = (q, w, k_e4m3, k_scale, page_table, row_pt, row_bound, scores, out_idx, workspace)
        self._device = q.device
        self._fn = load_library().indexer_launch
        vp = ctypes.c_void_p
        self._args = (ctypes.byref(self._prob),) + tuple(
            vp(_ptr(t)) for t in (q, w, k_e4m3, k_scale, page_table, row_pt, row_bound, scores, out_idx,
                                  workspace)) + (ctypes.c_size_t(workspace.numel()),)

    def __call__(self):
        import torch
        rc = self._fn(*self._args, torch.cuda.current_stream(self._device).cuda_stream)
        if rc != 0:
            _check(rc)
        return self.out_idx


def indexer_launch_score(q, w, k_e4m3, k_scale, page_table, row_pt, row_bound, *, max_bound: int,
                         topk: int = MAX_TOPK, scores=None, workspace):
    """The scoring stage of indexer_launch: scores (into the workspace when
    `scores` is None) and the selection's digit counts added into the
    workspace.  Exactly one indexer_launch_select with the same arguments
    must follow before the workspace is used again."""
    _check_inputs(q, w, k_e4m3, k_scale, page_table, row_pt, row_bound)
    R = q.shape[0]
    if scores is not None:
        _check_scores(scores, R, max_bound, q.device)
    sstride = scores.stride(0) if scores is not None else 0
    prob = _problem_from(q, k_e4m3, page_table, max_bound, topk, sstride)
    _on_one_gpu(q, workspace)
    _check(load_library().indexer_launch_score(ctypes.byref(prob), _ptr(q), _ptr(w), _ptr(k_e4m3),
                                               _ptr(k_scale), _ptr(page_table), _ptr(row_pt),
                                               _ptr(row_bound), _ptr(scores), _ptr(workspace),
                                               workspace.numel(), _stream(q.device)))


def indexer_launch_select(row_bound, *, max_bound: int, topk: int = MAX_TOPK, scores=None, out_idx=None,
                          workspace, rows: Optional[int] = None):
    """The selection stage of indexer_launch, from the scores and counts an
    indexer_launch_score call left (same scores tensor or None, same
    workspace).  Returns out_idx [rows, topk] int32."""
    import torch
    R = row_bound.shape[0] if rows is None else rows
    assert row_bound.dtype == torch.int32 and tuple(row_bound.shape) == (R,) and row_bound.is_contiguous()
    if scores is not None:
        _check_scores(scores, R, max_bound, row_bound.device)
    if out_idx is None:
        out_idx = torch.empty((R, topk), dtype=torch.int32, device=row_bound.device)
    _check_out(out_idx, R, topk, row_bound.device)
    _on_one_gpu(row_bound, workspace)
    prob = make_problem(rows=R, num_pages=1, pt_rows=1, pt_stride=max(1, (max_bound + 63) // 64),
                        max_bound=max_bound, topk=topk,
                        score_stride=scores.stride(0) if scores is not None else 0)
    _check(load_library().indexer_launch_select(ctypes.byref(prob), _ptr(scores), _ptr(row_bound),
                                                _ptr(out_idx), _ptr(workspace), workspace.numel(),
                                                _stream(row_bound.device)))
    return out_idx


STATIC_MAX_ROWS = 256
STATIC_SCRATCH_BYTES = 64 << 20


def indexer_launch_static(q, w, k_e4m3, k_scale, page_table, row_pt, row_bound, *, max_bound: int,
                          topk: int = MAX_TOPK, scores=None, out_idx=None):
    """indexer_launch on the library's static per-GPU scratch (no workspace;
    the C call allocates nothing).  Pass `out_idx` (and `scores`) to allocate
    nothing here either.  Calls that may overlap on one GPU race.  Returns
    out_idx [rows, topk] int32."""
    import torch
    _check_inputs(q, w, k_e4m3, k_scale, page_table, row_pt, row_bound)
    R = q.shape[0]
    if scores is not None:
        _check_scores(scores, R, max_bound, q.device)
    sstride = scores.stride(0) if scores is not None else 0
    prob = _problem_from(q, k_e4m3, page_table, max_bound, topk, sstride)
    if out_idx is None:
        out_idx = torch.empty((R, topk), dtype=torch.int32, device=q.device)
    _check_out(out_idx, R, topk, q.device)
    _check(load_library().indexer_launch_static(ctypes.byref(prob), _ptr(q), _ptr(w), _ptr(k_e4m3),
                                                _ptr(k_scale), _ptr(page_table), _ptr(row_pt),
                                                _ptr(row_bound), _ptr(scores), _ptr(out_idx),
                                                _stream(q.device)))
    return out_idx

VALID_BOUND, VALID_ROW_PT, VALID_PAGE = 1, 2, 4


def indexer_validate(page_table, row_pt, row_bound, *, max_bound: int, num_pages: int, status=None):
    """Checks row_bound, row_pt and the page ids the rows would read; returns
    the status tensor (one int32 on the device; bits VALID_BOUND,
    VALID_ROW_PT, VALID_PAGE, 0 when every array is within range).  Nothing
    synchronises: read it with ``.item()`` when needed."""
    import torch
    R = row_pt.shape[0]
    assert page_table.dtype == torch.int32 and page_table.dim() == 2 and page_table.is_contiguous()
    assert row_pt.dtype == torch.int32 and row_pt.is_contiguous()
    assert row_bound.dtype == torch.int32 and tuple(row_bound.shape) == (R,) and row_bound.is_contiguous()
    if status is None:
        status = torch.empty(1, dtype=torch.int32, device=row_pt.device)
    _on_one_gpu(row_pt, page_table, row_bound, status)
    prob = make_problem(rows=R, num_pages=num_pages, pt_rows=page_table.shape[0], pt_stride=page_table.shape[1],
                        max_bound=max_bound, topk=MAX_TOPK, score_stride=0)
    _check(load_library().indexer_validate(ctypes.byref(prob), _ptr(page_table), _ptr(row_pt), _ptr(row_bound),
                                           _ptr(status), _stream(row_pt.device)))
    return status


def _check_new_keys(k_new, rows):
    import torch
    assert k_new.dtype == torch.bfloat16 and tuple(k_new.shape) == (rows, HEAD_DIM) and k_new.is_contiguous()


def indexer_write_keys(k_new, k_e4m3, k_scale, page_table, row_pt, row_bound, *, max_bound: int):
    """Quantizes each row's new key k_new [rows, 128] bf16 to E4M3 codes and a
    scale and writes them in place into k_e4m3 / k_scale at the row's last
    position (bound - 1).  Returns nothing."""
    import torch
    R = k_new.shape[0]
    _check_new_keys(k_new, R)
    assert k_e4m3.dtype == torch.uint8 and tuple(k_e4m3.shape[1:]) == (PAGE, HEAD_DIM) and k_e4m3.is_contiguous()
    assert k_scale.dtype == torch.float32 and tuple(k_scale.shape) == (k_e4m3.shape[0], PAGE) and k_scale.is_contiguous()
    assert page_table.dtype == torch.int32 and page_table.dim() == 2 and page_table.is_contiguous()
    assert row_pt.dtype == torch.int32 and tuple(row_pt.shape) == (R,) and row_pt.is_contiguous()
    assert row_bound.dtype == torch.int32 and tuple(row_bound.shape) == (R,) and row_bound.is_contiguous()
    _on_one_gpu(k_new, k_e4m3, k_scale, page_table, row_pt, row_bound)
    prob = make_problem(rows=R, num_pages=k_e4m3.shape[0], pt_rows=page_table.shape[0],
                        pt_stride=page_table.shape[1], max_bound=max_bound, topk=MAX_TOPK, score_stride=0)
    _check(load_library().indexer_write_keys(ctypes.byref(prob), _ptr(k_new), _ptr(k_e4m3), _ptr(k_scale),
                                             _ptr(page_table), _ptr(row_pt), _ptr(row_bound),
                                             _stream(k_new.device)))


def indexer_launch_new_keys(q, w, k_new, k_e4m3, k_scale, page_table, row_pt, row_bound, *,
                            max_bound: int, topk: int = MAX_TOPK, scores=None, out_idx=None,
                            workspace=None):
    """The new-key write (k_e4m3 / k_scale updated in place) followed by the
    fused scoring + exact top-k.  Returns out_idx [rows, topk] int32."""
    import torch
    _check_inputs(q, w, k_e4m3, k_scale, page_table, row_pt, row_bound)
    R = q.shape[0]
    _check_new_keys(k_new, R)
    if scores is not None:
        _check_scores(scores, R, max_bound, q.device)
    sstride = scores.stride(0) if scores is not None else 0
    prob = _problem_from(q, k_e4m3, page_table, max_bound, topk, sstride)
    if out_idx is None:
        out_idx = torch.empty((R, topk), dtype=torch.int32, device=q.device)
    _check_out(out_idx, R, topk, q.device)
    if workspace is None:
        workspace = new_workspace(prob, scores is None, q.device)
    _on_one_gpu(q, k_new, workspace)
    _check(load_library().indexer_launch_new_keys(ctypes.byref(prob), _ptr(q), _ptr(w), _ptr(k_new),
                                                  _ptr(k_e4m3), _ptr(k_scale), _ptr(page_table),
                                                  _ptr(row_pt), _ptr(row_bound), _ptr(scores),
                                                  _ptr(out_idx), _ptr(workspace), workspace.numel(),
                                                  _stream(q.device)))
    return out_idx


def indexer_shard_candidates(scores, out_idx, *, shard: int, shards: int, max_bound: int,
                             cand_score=None, cand_idx=None):
    """Shard `shard` of `shards` (pages interleaved): its selection out_idx
    [rows, topk] (logical indices) and scores [rows, stride] become (score,
    global index) candidates in block `shard` of cand_score / cand_idx
    [rows, shards * topk]."""
    import torch
    R, k = out_idx.shape
    assert scores.dtype == torch.float32 and scores.dim() == 2 and scores.stride(1) == 1
    assert out_idx.dtype == torch.int32 and out_idx.is_contiguous()
    if cand_score is None:
        cand_score = torch.empty((R, shards * k), dtype=torch.float32, device=scores.device)
    if cand_idx is None:
        cand_idx = torch.empty((R, shards * k), dtype=torch.int32, device=scores.device)
    assert scores.shape[0] >= R and scores.shape[1] >= max_bound, "scores too small for the shard's rows"
    assert cand_score.dtype == torch.float32 and cand_idx.dtype == torch.int32
    assert cand_score.shape == (R, shards * k) and cand_idx.shape == (R, shards * k)
    assert cand_score.is_contiguous() and cand_idx.is_contiguous()
    _on_one_gpu(scores, out_idx, cand_score, cand_idx)
    prob = make_problem(rows=R, num_pages=1, pt_rows=1, pt_stride=max(1, (max_bound + 63) // 64),
                        max_bound=max_bound, topk=k, score_stride=scores.stride(0))
    _check(load_library().indexer_shard_candidates(ctypes.byref(prob), shard, shards, _ptr(scores),
                                                   _ptr(out_idx), _ptr(cand_score), _ptr(cand_idx),
                                                   _stream(scores.device)))
    return cand_score, cand_idx


def indexer_merge_topk(cand_score, cand_idx, *, shards: int, topk: int = MAX_TOPK, out_idx=None):
    """Exact top-k per row of the shards' candidates: global indices grouped
    by shard (each group ascending), -1 padded.  Returns out_idx [rows, topk]
    int32."""
    import torch
    R = cand_idx.shape[0]
    assert cand_score.dtype == torch.float32 and cand_idx.dtype == torch.int32
    assert cand_score.is_contiguous() and cand_idx.is_contiguous()
    assert cand_idx.numel() == R * shards * topk and cand_score.numel() == R * shards * topk
    if out_idx is None:
        out_idx = torch.empty((R, topk), dtype=torch.int32, device=cand_idx.device)
    assert out_idx.dtype == torch.int32 and out_idx.shape == (R, topk) and out_idx.is_contiguous()
    _on_one_gpu(cand_idx, cand_score, out_idx)
    prob = make_problem(rows=R, num_pages=1, pt_rows=1, pt_stride=1, max_bound=0, topk=topk)
    _check(load_library().indexer_merge_topk(ctypes.byref(prob), shards, _ptr(cand_score), _ptr(cand_idx),
                                             _ptr(out_idx), _stream(cand_idx.device)))
    return out_idx


ATTN_HEADS = 16
ATTN_DIM = 576
ATTN_VDIM = 512


def attention_workspace(rows: int, topk: int, device):
    """Workspace tensor (uint8, 256-byte aligned) for indexer_sparse_attention."""
    import torch
    prob = make_problem(rows=rows, num_pages=1, pt_rows=1, pt_stride=1, max_bound=0, topk=topk)
    n = ctypes.c_size_t(0)
    _check(load_library().fp8idx_attention_workspace_size(ctypes.byref(prob), ctypes.byref(n)))
    ws = torch.empty(int(n.value) + 256, dtype=torch.uint8, device=device)
    off = (-ws.data_ptr()) % 256
    return ws[off:off + int(n.value)]


def indexer_sparse_attention(q_attn, kv, page_table, row_pt, sel, *, max_bound: int, sm_scale: float,
                             out=None, lse=None, workspace=None):
    """Attention of each row's 16 heads (q_attn [rows, 16, 576] bf16) over its
    selected positions sel [rows, topk] int32 (-1: none) in the paged latent
    cache kv [pages, 64, 576] bf16 (same page table as the index keys).
    Returns (out [rows, 16, 512] fp32, lse [rows, 16] fp32)."""
    import torch
    R = q_attn.shape[0]
    assert q_attn.dtype == torch.bfloat16 and tuple(q_attn.shape[1:]) == (ATTN_HEADS, ATTN_DIM) and q_attn.is_contiguous()
    assert kv.dtype == torch.bfloat16 and tuple(kv.shape[1:]) == (PAGE, ATTN_DIM) and kv.is_contiguous()
    assert page_table.dtype == torch.int32 and page_table.dim() == 2 and page_table.is_contiguous()
    assert row_pt.dtype == torch.int32 and tuple(row_pt.shape) == (R,) and row_pt.is_contiguous()
    assert sel.dtype == torch.int32 and sel.dim() == 2 and sel.shape[0] == R and sel.is_contiguous()
    topk = sel.shape[1]
    if out is None:
        out = torch.empty((R, ATTN_HEADS, ATTN_VDIM), dtype=torch.float32, device=q_attn.device)
    if lse is None:
        lse = torch.empty((R, ATTN_HEADS), dtype=torch.float32, device=q_attn.device)
    assert out.dtype == torch.float32 and tuple(out.shape) == (R, ATTN_HEADS, ATTN_VDIM) and out.is_contiguous()
    assert lse.dtype == torch.float32 and tuple(lse.shape) == (R, ATTN_HEADS) and lse.is_contiguous()
    if workspace is None:
        workspace = attention_workspace(R, topk, q_attn.device)
    _on_one_gpu(q_attn, kv, page_table, row_pt, sel, out, lse, workspace)
    prob = make_problem(rows=R, num_pages=kv.shape[0], pt_rows=page_table.shape[0], pt_stride=page_table.shape[1],
                        max_bound=max_bound, topk=topk)
    _check(load_library().indexer_sparse_attention(ctypes.byref(prob), _ptr(q_attn), _ptr(kv), _ptr(page_table),
                                                   _ptr(row_pt), _ptr(sel), float(sm_scale), _ptr(out), _ptr(lse),
                                                   _ptr(workspace), workspace.numel(), _stream(q_attn.device)))
    return out, lse
