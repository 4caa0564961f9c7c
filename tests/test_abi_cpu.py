"""The C-ABI library loads, exports every function include/fp8idx.h declares,
and rejects bad arguments on the host before touching any device (no GPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8idx.h")


@pytest.fixture(scope="module")
def lib():
    import fp8_key_scoring_amd as fk
    if not os.path.exists(fk.LIB_PATH):
        from fp8_key_scoring_amd import build
        build.build()
    return fk.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "while")))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("indexer_score", "indexer_topk", "indexer_launch", "fp8idx_workspace_size",
              "fp8idx_workspace_init", "fp8idx_abi_version", "fp8idx_strerror",
              "indexer_shard_candidates", "indexer_merge_topk", "indexer_write_keys",
              "indexer_launch_new_keys", "indexer_validate", "indexer_launch_score",
              "indexer_launch_select", "indexer_launch_static", "fp8idx_attention_workspace_size",
              "indexer_sparse_attention"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for n in declared_functions():
        assert hasattr(lib, n), n


def test_abi_version_and_strerror(lib):
    import fp8_key_scoring_amd as fk
    assert fk.abi_version() == 1
    for code in (0, -1, -2, -3, -4, -5, 7):
        assert lib.fp8idx_strerror(code)


def test_problem_struct_layout():
    import fp8_key_scoring_amd as fk
    assert ctypes.sizeof(fk.Problem) == 32
    assert fk.Problem.score_stride.offset == 24


def test_workspace_size(lib):
    import fp8_key_scoring_amd as fk
    p = fk.make_problem(rows=4, num_pages=8192, pt_rows=1, pt_stride=8192, max_bound=524288)
    a = fk.workspace_size(p, False)
    b = fk.workspace_size(p, True)
    assert 0 < a < b and b - a >= 4 * 524288 * 4
    with pytest.raises(fk.Fp8IdxError):
        fk.workspace_size(fk.make_problem(0, 1, 1, 1, 0), False)


def _call_score(lib, prob, ptrs):
    import fp8_key_scoring_amd as fk
    return lib.indexer_score(ctypes.byref(prob), *ptrs, None)


def test_host_side_argument_errors(lib):
    import fp8_key_scoring_amd as fk
    good = [0x1000, 0x2000, 0x3000, 0x4000, 0x5000, 0x6000, 0x7000, 0x8000]   # never dereferenced
    base = dict(rows=4, num_pages=16, pt_rows=1, pt_stride=16, max_bound=1024, topk=2048,
                score_stride=1024)
    bad = [dict(rows=0), dict(rows=70000), dict(topk=0), dict(topk=2049), dict(max_bound=-1),
           dict(max_bound=16 * 64 + 1), dict(num_pages=0), dict(pt_stride=0), dict(score_stride=1000)]
    for b in bad:
        p = fk.make_problem(**{**base, **b})
        assert _call_score(lib, p, good) == -1, b
    p = fk.make_problem(**base)
    for i in range(len(good)):
        ptrs = list(good)
        ptrs[i] = None
        assert _call_score(lib, p, ptrs) == -1
    misaligned = list(good)
    misaligned[0] = 0x1008   # q must be 16-byte aligned
    assert _call_score(lib, p, misaligned) == -1
    # workspace too small / missing
    rc = lib.indexer_topk(ctypes.byref(p), 0x1000, 0x2000, 0x3000, None, 0, None)
    assert rc == -2
    rc = lib.indexer_topk(ctypes.byref(p), 0x1000, 0x2000, 0x3000, 0x100000, 16, None)
    assert rc == -2
    rc = lib.indexer_launch(ctypes.byref(p), *good[:7], None, None, 0x100000, 1 << 30, None)
    assert rc == -1   # out_idx missing
    assert lib.fp8idx_workspace_init(None, 256, None) == -1
    assert lib.fp8idx_workspace_init(0x100001, 256, None) == -1



def test_launch_stage_argument_errors(lib):
    """indexer_launch_score / indexer_launch_select reject bad arguments on the host."""
    import fp8_key_scoring_amd as fk
    good = [0x1000, 0x2000, 0x3000, 0x4000, 0x5000, 0x6000, 0x7000]   # q .. row_bound, never dereferenced
    p = fk.make_problem(rows=4, num_pages=16, pt_rows=1, pt_stride=16, max_bound=1024, topk=2048,
                        score_stride=1024)
    ws_need = fk.workspace_size(p, False)
    for i in range(len(good)):
        ptrs = list(good)
        ptrs[i] = None
        assert lib.indexer_launch_score(ctypes.byref(p), *ptrs, 0x9000, 0x100000, 1 << 30, None) == -1
    # workspace missing, too small, misaligned
    assert lib.indexer_launch_score(ctypes.byref(p), *good, 0x9000, None, 1 << 30, None) == -2
    assert lib.indexer_launch_score(ctypes.byref(p), *good, 0x9000, 0x100000, ws_need - 4, None) == -2
    assert lib.indexer_launch_score(ctypes.byref(p), *good, 0x9000, 0x100010, 1 << 30, None) == -2
    # scores given with a stride below max_bound
    p2 = fk.make_problem(rows=4, num_pages=16, pt_rows=1, pt_stride=16, max_bound=1024, topk=2048,
                         score_stride=1000)
    assert lib.indexer_launch_score(ctypes.byref(p2), *good, 0x9000, 0x100000, 1 << 30, None) == -1
    # select: out_idx and row_bound required; the workspace as for the launch
    assert lib.indexer_launch_select(ctypes.byref(p), 0x9000, 0x7000, None, 0x100000, 1 << 30, None) == -1
    assert lib.indexer_launch_select(ctypes.byref(p), 0x9000, None, 0xA000, 0x100000, 1 << 30, None) == -1
    assert lib.indexer_launch_select(ctypes.byref(p), 0x9000, 0x7000, 0xA000, 0x100000, ws_need - 4, None) == -2
    # without caller scores the workspace must also hold them
    ws_own = fk.workspace_size(p, True)
    assert lib.indexer_launch_select(ctypes.byref(p), None, 0x7000, 0xA000, 0x100000, ws_own - 4, None) == -2


def test_static_launch_host_errors(lib):
    """indexer_launch_static rejects a problem over its scratch's limits (more
    than 256 rows, or a layout over 64 MiB) with -5, and bad arguments with
    -1, before touching any device."""
    import fp8_key_scoring_amd as fk
    good = [0x1000, 0x2000, 0x3000, 0x4000, 0x5000, 0x6000, 0x7000]
    p = fk.make_problem(rows=fk.STATIC_MAX_ROWS + 1, num_pages=16, pt_rows=1, pt_stride=16, max_bound=1024)
    assert lib.indexer_launch_static(ctypes.byref(p), *good, None, 0x9000, None) == -5
    # 8 rows x 2M keys with the scores in the scratch: 64 MiB of scores alone
    p = fk.make_problem(rows=8, num_pages=32768, pt_rows=1, pt_stride=32768, max_bound=1 << 21)
    assert lib.indexer_launch_static(ctypes.byref(p), *good, None, 0x9000, None) == -5
    p = fk.make_problem(rows=0, num_pages=16, pt_rows=1, pt_stride=16, max_bound=1024)
    assert lib.indexer_launch_static(ctypes.byref(p), *good, None, 0x9000, None) == -1

def test_sharded_selection_argument_errors(lib):
    """Host-side checks of the key-sharded calls (nothing is launched: every
    case fails before the device check)."""
    import fp8_key_scoring_amd as fk
    P = [0x1000, 0x2000, 0x3000, 0x4000]   # never dereferenced
    ok = fk.make_problem(rows=4, num_pages=1, pt_rows=1, pt_stride=2048, max_bound=131072, topk=2048,
                         score_stride=131072)
    sc = lambda p, g, G, ptrs: lib.indexer_shard_candidates(ctypes.byref(p), g, G, *ptrs, None)
    mg = lambda p, G, ptrs: lib.indexer_merge_topk(ctypes.byref(p), G, *ptrs, None)
    for g, G in ((-1, 8), (8, 8), (0, 0), (0, 9)):        # shard outside [0, G); G * topk > 16384
        assert sc(ok, g, G, P) == -1, (g, G)
    for i in range(4):
        ptrs = list(P)
        ptrs[i] = None
        assert sc(ok, 0, 8, ptrs) == -1
    big = fk.make_problem(rows=4, num_pages=1, pt_rows=1, pt_stride=1 << 24, max_bound=(1 << 28),
                          topk=2048, score_stride=1 << 28)
    assert sc(big, 0, 8, P) == -1                          # global indices past int32
    short = fk.make_problem(rows=4, num_pages=1, pt_rows=1, pt_stride=2048, max_bound=131072, topk=2048,
                            score_stride=1000)
    assert sc(short, 0, 8, P) == -1                        # score_stride < max_bound
    assert mg(ok, 0, P[:3]) == -1 and mg(ok, 9, P[:3]) == -1
    assert mg(ok, 8, [0x1004, 0x2000, 0x3000]) == -1       # candidates must be 16-byte aligned
    odd = fk.make_problem(rows=4, num_pages=1, pt_rows=1, pt_stride=1, max_bound=0, topk=5)
    assert mg(odd, 3, P[:3]) == -1                         # shards * topk not a multiple of 16
    for i in range(3):
        ptrs = list(P[:3])
        ptrs[i] = None
        assert mg(ok, 8, ptrs) == -1


def test_new_key_argument_errors(lib):
    """Host-side checks of the new-key calls (every case fails before the
    device check, so nothing is launched)."""
    import fp8_key_scoring_amd as fk
    P = [0x1000, 0x2000, 0x3000, 0x4000, 0x5000, 0x6000]   # k_new, k8, scale, pt, row_pt, bound
    ok = fk.make_problem(rows=4, num_pages=16, pt_rows=1, pt_stride=16, max_bound=1024, topk=2048,
                         score_stride=1024)
    wk = lambda p, ptrs: lib.indexer_write_keys(ctypes.byref(p), *ptrs, None)
    for i in range(6):
        ptrs = list(P)
        ptrs[i] = None
        assert wk(ok, ptrs) == -1, i
    for i, a in ((0, 0x1002), (1, 0x2008), (2, 0x3002)):    # k_new 4-, k_e4m3 16-, k_scale 4-byte aligned
        ptrs = list(P)
        ptrs[i] = a
        assert wk(ok, ptrs) == -1, i
    for b in (dict(rows=0), dict(num_pages=0), dict(pt_stride=0), dict(max_bound=16 * 64 + 1)):
        assert wk(fk.make_problem(**{**dict(rows=4, num_pages=16, pt_rows=1, pt_stride=16, max_bound=1024,
                                            topk=2048, score_stride=1024), **b}), P) == -1, b
    # the combined call checks everything of both steps first
    q, w = 0x7000, 0x8000
    L = lambda p, kn, out, ws, wsb: lib.indexer_launch_new_keys(ctypes.byref(p), q, w, kn, *P[1:], None, out,
                                                               ws, wsb, None)
    assert L(ok, None, 0x9000, 0x100000, 1 << 30) == -1      # k_new missing
    assert L(ok, 0x1002, 0x9000, 0x100000, 1 << 30) == -1    # k_new misaligned
    assert L(ok, 0x1000, None, 0x100000, 1 << 30) == -1      # out_idx missing
    assert L(ok, 0x1000, 0x9000, 0x100000, 16) == -2         # workspace too small


def test_validate_argument_errors(lib):
    import fp8_key_scoring_amd as fk
    P = [0x1000, 0x2000, 0x3000, 0x4000]   # page_table, row_pt, row_bound, status (never dereferenced)
    ok = fk.make_problem(rows=4, num_pages=16, pt_rows=1, pt_stride=16, max_bound=1024, topk=2048)
    v = lambda p, ptrs: lib.indexer_validate(ctypes.byref(p), *ptrs, None)
    for i in range(4):
        ptrs = list(P)
        ptrs[i] = None
        assert v(ok, ptrs) == -1, i
    ptrs = list(P)
    ptrs[3] = 0x4002                                      # status must be 4-byte aligned
    assert v(ok, ptrs) == -1
    bad = fk.make_problem(rows=4, num_pages=16, pt_rows=1, pt_stride=16, max_bound=16 * 64 + 1, topk=2048)
    assert v(bad, P) == -1


def test_attention_argument_errors(lib):
    import fp8_key_scoring_amd as fk
    ok = fk.make_problem(rows=4, num_pages=16, pt_rows=1, pt_stride=16, max_bound=1024, topk=2048)
    n = ctypes.c_size_t(0)
    assert lib.fp8idx_attention_workspace_size(ctypes.byref(ok), ctypes.byref(n)) == 0
    # 4 rows: 32 splits of 64 entries (4 waves x 16); partial outputs 4*32*16*512 fp32 + maxima and sums
    assert n.value == 4 * 32 * 16 * 512 * 4 + 4 * 32 * 2 * 16 * 4
    assert lib.fp8idx_attention_workspace_size(ctypes.byref(ok), None) == -1
    one = fk.make_problem(rows=1000, num_pages=16, pt_rows=1, pt_stride=16, max_bound=1024, topk=2048)
    assert lib.fp8idx_attention_workspace_size(ctypes.byref(one), ctypes.byref(n)) == 0
    assert n.value == 1000 * 16 * 512 * 4 + 1000 * 2 * 16 * 4 + (-(1000 * 16 * 512 * 4)) % 256
    big = n.value
    # q, kv, page_table, row_pt, sel, out, lse: never dereferenced
    P = [0x1000, 0x2000, 0x3000, 0x4000, 0x5000, 0x6000, 0x7000]
    a = lambda p, ptrs, sm=0.1, ws=0x100000, wsb=1 << 30: lib.indexer_sparse_attention(
        ctypes.byref(p), *ptrs[:5], ctypes.c_float(sm), *ptrs[5:], ws, wsb, None)
    for i in range(7):
        ptrs = list(P)
        ptrs[i] = None
        assert a(ok, ptrs) == -1, i
    for i, al in ((0, 0x1008), (1, 0x2008), (4, 0x5002)):   # q, kv 16-byte; sel 4-byte
        ptrs = list(P)
        ptrs[i] = al
        assert a(ok, ptrs) == -1, i
    for sm in (float("nan"), float("inf"), float("-inf")):
        assert a(ok, P, sm=sm) == -1
    assert a(ok, P, ws=None) == -2
    assert a(ok, P, ws=0x100080) == -2                      # 256-byte alignment
    assert a(ok, P, wsb=16) == -2
    assert a(one, P, wsb=big - 4) == -2
    bad = fk.make_problem(rows=4, num_pages=16, pt_rows=1, pt_stride=16, max_bound=16 * 64 + 1, topk=2048)
    assert a(bad, P) == -1
    for kw in (dict(rows=0), dict(topk=0), dict(topk=2049)):
        args = dict(rows=4, num_pages=16, pt_rows=1, pt_stride=16, max_bound=1024, topk=2048)
        args.update(kw)
        assert a(fk.make_problem(**args), P) == -1, kw


def test_header_is_plain_c_and_links(tmp_path):
    """include/fp8idx.h compiles as C99 with gcc (no HIP or C++ types in the
    boundary), and a C program taking the address of every entry point links
    against the built library."""
    import shutil
    import subprocess
    import fp8_key_scoring_amd as fk
    if shutil.which("gcc") is None:
        pytest.skip("gcc not installed")
    src = tmp_path / "use_abi.c"
    names = declared_functions()
    body = "\n".join(f"    p[{i}] = (void (*)(void))&{n};" for i, n in enumerate(names))
    src.write_text('#include "fp8idx.h"\n#include <stdio.h>\n'
                   f"int main(void) {{\n    void (*p[{len(names)}])(void);\n{body}\n"
                   "    fp8idx_problem_t prob = {0};\n    (void)prob;\n"
                   '    printf("%d\\n", fp8idx_abi_version());\n    return p[0] == 0;\n}\n')
    exe = tmp_path / "use_abi"
    lib = fk.LIB_PATH
    cmd = ["gcc", "-std=c99", "-Wall", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"), str(src),
           "-o", str(exe), lib, "-Wl,-rpath," + os.path.dirname(lib)]
    out = subprocess.run(cmd, capture_output=True, text=True)
    assert out.returncode == 0, out.stderr[-2000:]


def test_binding_rejects_host_tensors_before_any_call(lib):
    """The binding passes raw pointers: inputs that are not all on one GPU
    (here host tensors) are refused before the library is called."""
    import torch
    import fp8_key_scoring_amd as fk
    R = 2
    q = torch.zeros(R, fk.HEADS, fk.HEAD_DIM, dtype=torch.bfloat16)
    w = torch.zeros(R, fk.HEADS)
    k = torch.zeros(4, fk.PAGE, fk.HEAD_DIM, dtype=torch.uint8)
    ks = torch.zeros(4, fk.PAGE)
    pt = torch.zeros(1, 4, dtype=torch.int32)
    rp = torch.zeros(R, dtype=torch.int32)
    rb = torch.full((R,), 100, dtype=torch.int32)
    for fn in (fk.indexer_score, fk.indexer_launch, fk.indexer_launch_static):
        with pytest.raises(AssertionError, match="one GPU"):
            fn(q, w, k, ks, pt, rp, rb, max_bound=100)
    with pytest.raises(AssertionError, match="one GPU"):
        fk.indexer_launch_score(q, w, k, ks, pt, rp, rb, max_bound=100, workspace=torch.zeros(256, dtype=torch.uint8))
    sc = torch.zeros(R, 128)
    with pytest.raises(AssertionError, match="one GPU"):
        fk.indexer_topk(sc, rb, max_bound=100)
    with pytest.raises(AssertionError, match="one GPU"):
        fk.indexer_launch_select(rb, max_bound=100, scores=sc, workspace=torch.zeros(256, dtype=torch.uint8))
    with pytest.raises(AssertionError, match="one GPU"):
        fk.indexer_validate(pt, rp, rb, max_bound=100, num_pages=4)
    with pytest.raises(AssertionError, match="one GPU"):
        fk.indexer_write_keys(torch.zeros(R, fk.HEAD_DIM, dtype=torch.bfloat16), k, ks, pt, rp, rb, max_bound=100)
    with pytest.raises(AssertionError, match="one GPU"):
        fk.indexer_merge_topk(torch.zeros(R, 2 * 8), torch.zeros(R, 2 * 8, dtype=torch.int32), shards=2, topk=8)
    sel = torch.zeros(R, 8, dtype=torch.int32)
    with pytest.raises(AssertionError, match="one GPU"):
        fk.indexer_shard_candidates(sc, sel, shard=0, shards=2, max_bound=100)
    with pytest.raises(AssertionError, match="one GPU"):
        fk.indexer_sparse_attention(torch.zeros(R, fk.ATTN_HEADS, fk.ATTN_DIM, dtype=torch.bfloat16),
                                    torch.zeros(4, fk.PAGE, fk.ATTN_DIM, dtype=torch.bfloat16), pt, rp, sel,
                                    max_bound=100, sm_scale=0.1)


def test_launch_plan_rejects_host_tensors(lib):
    import torch
    import fp8_key_scoring_amd as fk
    R = 2
    args = (torch.zeros(R, fk.HEADS, fk.HEAD_DIM, dtype=torch.bfloat16), torch.zeros(R, fk.HEADS),
            torch.zeros(4, fk.PAGE, fk.HEAD_DIM, dtype=torch.uint8), torch.zeros(4, fk.PAGE),
            torch.zeros(1, 4, dtype=torch.int32), torch.zeros(R, dtype=torch.int32),
            torch.full((R,), 100, dtype=torch.int32))
    with pytest.raises(AssertionError, match="one GPU"):
        fk.LaunchPlan(*args, max_bound=100)
