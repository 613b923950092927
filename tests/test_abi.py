"""The C ABI on the CPU: the library loads, exports what include/solattn.h
declares, and rejects bad arguments before any HIP call (so these run on a
machine without a GPU).  No compute call is made here."""

import ctypes
import math
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "solattn.h")


@pytest.fixture(scope="module")
def sa():
    from free_dynamic_sparse_amd import solattn
    return solattn


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(solattn_\w+)\s*\(", text, re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for want in ("solattn_pool", "solattn_moments", "solattn_fwd", "solattn_dense_fwd",
                 "solattn_strerror", "solattn_version"):
        assert want in names


def test_library_exports_every_declared_symbol(sa):
    for name in declared_functions():
        assert hasattr(sa.LIB, name), name
    assert set(declared_functions()) == set(sa.EXPORTS)


def test_problem_struct_layout_matches_header(sa):
    # int64 x4, int32 x2, float x2, uint32 x2 -> 56 bytes, no padding
    assert ctypes.sizeof(sa.Problem) == 56
    assert sa.Problem.beta.offset == 40 and sa.Problem.reserved.offset == 52


def test_version_and_strerror(sa):
    assert sa.LIB.solattn_version() == 300
    for code in (0, -1, -2, -3, -4, 7):
        assert isinstance(sa.LIB.solattn_strerror(code), bytes)
    assert b"workspace" in sa.LIB.solattn_strerror(-4)


FAKE = 1 << 20  # a 256-byte aligned address that is never dereferenced
WS = 1024        # solattn_fwd_workspace_bytes of every non-empty problem


def call_fwd(sa, p, ptr=FAKE, ws_bytes=WS, **over):
    args = dict(q=ptr, k=ptr, v=ptr, qbar=ptr, kbar=ptr, vhat=ptr, tau=ptr, out=ptr,
                workspace=ptr, sel_mask=None, sel_count=None)
    args.update(over)
    vals = [ctypes.c_void_p(args[n]) if args[n] is not None else None
            for n in ("q", "k", "v", "qbar", "kbar", "vhat", "tau", "out", "workspace",
                      "sel_mask", "sel_count")]
    return sa.LIB.solattn_fwd(ctypes.byref(p), *vals[:9], ws_bytes, *vals[9:], None)


@pytest.mark.parametrize("field,value,code", [
    ("head_dim", 96, -2), ("head_dim", 256, -2), ("block", 32, -2), ("block", 256, -2),
    ("chunk", 0, -2), ("chunk", 65, -2), ("beta", float("nan"), -1), ("scale", float("nan"), -1),
    ("scale", float("inf"), -1), ("seq_len", -1, -1), ("batch", -2, -1), ("heads", -1, -1),
    ("seq_len", (1 << 22) + 1, -1), ("reserved", 1, -1), ("flags", 2, -1),
])
def test_fwd_rejects_bad_problem(sa, field, value, code):
    p = sa.problem(1, 2, 1000, 128, 128, 32, 1.0)
    setattr(p, field, value)
    assert call_fwd(sa, p) == code


@pytest.mark.parametrize("which", ["q", "k", "v", "qbar", "kbar", "vhat", "tau", "out"])
def test_fwd_rejects_null_and_misaligned_pointers(sa, which):
    p = sa.problem(1, 2, 1000, 128, 128, 32, 1.0)
    assert call_fwd(sa, p, **{which: None}) == -1
    assert call_fwd(sa, p, **{which: FAKE + 8}) == -1


def test_fwd_workspace_size_and_checks(sa):
    p = sa.problem(1, 2, 1000, 128, 128, 32, 1.0)
    assert sa.solattn_fwd_workspace_bytes(p) == WS
    assert sa.solattn_fwd_workspace_bytes(sa.problem(0, 2, 1000, 128)) == 0
    assert sa.solattn_fwd_workspace_bytes(sa.problem(1, 2, 1000, 96)) == 0
    assert sa.LIB.solattn_fwd_workspace_bytes(None) == 0
    assert call_fwd(sa, p, workspace=None) == -4
    assert call_fwd(sa, p, workspace=FAKE + 16) == -4      # 16- but not 256-byte aligned
    assert call_fwd(sa, p, ws_bytes=WS - 1) == -4
    # argument errors are reported before workspace errors
    assert call_fwd(sa, p, q=None, workspace=None) == -1
    # an empty problem needs no workspace
    assert call_fwd(sa, sa.problem(1, 0, 1000, 128), ptr=None, ws_bytes=0) == 0


def test_fwd_rejects_misaligned_debug_outputs(sa):
    p = sa.problem(1, 2, 1000, 128, 128, 32, 1.0)
    assert call_fwd(sa, p, sel_mask=FAKE + 4) == -1
    assert call_fwd(sa, p, sel_count=FAKE + 4) == -1


def test_null_problem_is_rejected(sa):
    nul = ctypes.POINTER(sa.Problem)()
    assert sa.LIB.solattn_pool(nul, None, None, None, None, None, None, None) == -1
    assert sa.LIB.solattn_moments(nul, None, None, None, None, None, None, None, None) == -1
    assert sa.LIB.solattn_dense_fwd(nul, None, None, None, None, None) == -1


@pytest.mark.parametrize("B,H,L", [(0, 4, 100), (2, 0, 100), (1, 1, 0)])
def test_empty_problems_are_no_ops(sa, B, H, L):
    p = sa.problem(B, H, L, 64, 64, 16, 1.0)
    assert sa.LIB.solattn_pool(ctypes.byref(p), None, None, None, None, None, None, None) == 0
    assert sa.LIB.solattn_moments(ctypes.byref(p), None, None, None, None, None, None, None,
                                  None) == 0
    assert call_fwd(sa, p, ptr=None) == 0
    assert sa.LIB.solattn_dense_fwd(ctypes.byref(p), None, None, None, None, None) == 0


def test_empty_problem_still_checks_beta_and_chunk(sa):
    p = sa.problem(0, 4, 100, 64, 64, 16, float("nan"))
    assert call_fwd(sa, p, ptr=None) == -1
    p = sa.problem(0, 4, 100, 64, 64, 99, 1.0)
    assert call_fwd(sa, p, ptr=None) == -2


def test_fused_block_limit(sa):
    # the fused kernel keeps at most 8192 blocks of selection bits on chip
    assert call_fwd(sa, sa.problem(1, 1, 8192 * 128 + 1, 128, 128, 32, 1.0)) == -2
    assert call_fwd(sa, sa.problem(1, 1, 8192 * 64 + 1, 64, 64, 16, 1.0)) == -2


def test_grid_limit(sa):
    # B*H*N must fit a 1-D grid (< 2^31)
    p = sa.problem(1 << 20, 1 << 10, 4096, 64, 64, 16, 1.0)
    assert call_fwd(sa, p) == -1


def test_moments_and_pool_reject_bad_pointers(sa):
    p = sa.problem(1, 1, 256, 64, 64, 16, 1.0)
    f = ctypes.c_void_p(FAKE)
    bad = ctypes.c_void_p(FAKE + 4)
    assert sa.LIB.solattn_pool(ctypes.byref(p), f, f, f, f, f, bad, None) == -1
    assert sa.LIB.solattn_moments(ctypes.byref(p), f, f, f, f, None, None, None, None) == -1
    assert sa.LIB.solattn_moments(ctypes.byref(p), f, f, f, f, f, bad, None, None) == -1
    p.beta = math.nan
    assert sa.LIB.solattn_moments(ctypes.byref(p), f, f, f, f, f, None, None, None) == -1


# ------------------------------------------------------------ routing baselines

def test_baseline_entry_points_reject_bad_arguments(sa):
    p = sa.problem(1, 2, 4096, 128, 128, 32, 1.0)
    P = lambda x: ctypes.c_void_p(x)
    lib = sa.LIB
    # proxy map: null / misaligned pointers
    assert lib.solattn_proxy_map(ctypes.byref(p), None, P(FAKE), P(FAKE), None) == -1
    assert lib.solattn_proxy_map(ctypes.byref(p), P(FAKE), P(FAKE + 4), P(FAKE), None) == -1
    # top-k: k < 1, null mask, misaligned count
    assert lib.solattn_select_topk(ctypes.byref(p), P(FAKE), 0, P(FAKE), None, None) == -1
    assert lib.solattn_select_topk(ctypes.byref(p), P(FAKE), 3, None, None, None) == -1
    assert lib.solattn_select_topk(ctypes.byref(p), P(FAKE), 3, P(FAKE), P(FAKE + 8), None) == -1
    # top-p: p outside (0, 1], NaN
    for bad in (0.0, -0.5, 1.5, math.nan):
        assert lib.solattn_select_topp(ctypes.byref(p), P(FAKE), bad, P(FAKE), None, None) == -1
    # rows longer than the on-chip sort holds
    big = sa.problem(1, 1, 128 * 8193, 128, 128, 32, 1.0)
    assert lib.solattn_select_topk(ctypes.byref(big), P(FAKE), 3, P(FAKE), None, None) == -2
    assert lib.solattn_select_topp(ctypes.byref(big), P(FAKE), 0.5, P(FAKE), None, None) == -2
    # unsupported head dim, and empty problems (nothing launched)
    bad_d = sa.problem(1, 1, 4096, 96, 128, 32, 1.0)
    assert lib.solattn_proxy_map(ctypes.byref(bad_d), P(FAKE), P(FAKE), P(FAKE), None) == -2
    empty = sa.problem(0, 4, 4096, 128, 128, 32, 1.0)
    assert lib.solattn_proxy_map(ctypes.byref(empty), None, None, None, None) == 0
    assert lib.solattn_select_topk(ctypes.byref(empty), None, 5, None, None, None) == 0
    assert lib.solattn_select_topp(ctypes.byref(empty), None, 0.5, None, None, None) == 0


def test_masked_forward_rejects_bad_arguments(sa):
    p = sa.problem(1, 2, 4096, 128, 128, 32, 1.0)
    P = lambda x: ctypes.c_void_p(x)
    lib = sa.LIB
    # q, k, v, kbar, vhat, sel_in, out: each null or misaligned in turn
    ws = [P(FAKE), WS]
    for i in range(7):
        args = [P(FAKE)] * 7
        args[i] = None
        assert lib.solattn_fwd_masked(ctypes.byref(p), *args, *ws, None) == -1
        args[i] = P(FAKE + 8)
        assert lib.solattn_fwd_masked(ctypes.byref(p), *args, *ws, None) == -1
    big = sa.problem(1, 1, 128 * 8193, 128, 128, 32, 1.0)
    assert lib.solattn_fwd_masked(ctypes.byref(big), *([P(FAKE)] * 7), *ws, None) == -2
    empty = sa.problem(2, 0, 4096, 128, 128, 32, 1.0)
    assert lib.solattn_fwd_masked(ctypes.byref(empty), *([None] * 7), None, 0, None) == 0
    # the workspace: missing, misaligned, too small
    for bad in ([None, WS], [P(FAKE + 128), WS], [P(FAKE), WS - 4]):
        assert lib.solattn_fwd_masked(ctypes.byref(p), *([P(FAKE)] * 7), *bad, None) == -4


def test_first_order_workspace_size(sa):
    lib = sa.LIB
    p = sa.problem(2, 3, 1000, 128, 128, 32, 1.0)   # N = 8, one bitmap word per row
    up = lambda x: (x + 255) // 256 * 256
    # queue counters, bitmaps, log denominators, float32 O
    want = WS + up(2 * 3 * 8 * 1 * 8) + up(2 * 3 * 1000 * 4) + up(2 * 3 * 1000 * 128 * 4)
    assert lib.solattn_fwd_first_order_workspace(ctypes.byref(p)) == want
    assert sa.solattn_fwd_first_order_workspace(p) == want
    assert lib.solattn_fwd_first_order_workspace(ctypes.byref(sa.problem(0, 3, 1000, 128))) == 0
    assert lib.solattn_fwd_first_order_workspace(ctypes.byref(sa.problem(1, 1, 1000, 96))) == 0
    assert lib.solattn_fwd_first_order_workspace(None) == 0


def test_first_order_entry_points_reject_bad_arguments(sa):
    lib = sa.LIB
    P = lambda x: ctypes.c_void_p(x)
    p = sa.problem(1, 2, 4096, 128, 128, 32, 1.0)
    need = lib.solattn_fwd_first_order_workspace(ctypes.byref(p))

    def fo(prob, ptrs, size=need):
        # ptrs: q, k, v, qbar, kbar, vhat, kvc, tau, out, workspace
        return lib.solattn_fwd_first_order(ctypes.byref(prob), *ptrs, size, None)

    for i in range(10):   # each pointer null, then misaligned
        ptrs = [P(FAKE)] * 10
        ptrs[i] = None
        assert fo(p, ptrs) == (-4 if i == 9 else -1), i
        ptrs[i] = P(FAKE + 8)
        assert fo(p, ptrs) == (-4 if i == 9 else -1), i
    ok = [P(FAKE)] * 10
    assert fo(p, ok, need - 1) == -4                        # workspace too small
    exact = sa.problem(1, 2, 4096, 128, 128, 32, 1.0, exact_only=True)
    assert fo(exact, ok) == -1                              # exact-only is refused
    nan = sa.problem(1, 2, 4096, 128, 128, 32, math.nan)
    assert fo(nan, ok) == -1
    big = sa.problem(1, 1, 128 * 8193, 128, 128, 32, 1.0)
    assert fo(big, ok, 1 << 40) == -2
    assert fo(sa.problem(1, 2, 4096, 96, 128, 32, 1.0), ok) == -2
    empty = sa.problem(1, 0, 4096, 128, 128, 32, 1.0)
    assert fo(empty, [None] * 10, 0) == 0
    # kv moments: k, v, kbar, vhat, kvc
    for i in range(5):
        ptrs = [P(FAKE)] * 5
        ptrs[i] = None
        assert lib.solattn_kv_moments(ctypes.byref(p), *ptrs, None) == -1
        ptrs[i] = P(FAKE + 8)
        assert lib.solattn_kv_moments(ctypes.byref(p), *ptrs, None) == -1
    assert lib.solattn_kv_moments(ctypes.byref(empty), *[None] * 5, None) == 0
    assert lib.solattn_kv_moments(ctypes.byref(sa.problem(1, 1, 64, 128, 32)),
                                  *[P(FAKE)] * 5, None) == -2
