"""The allocation-free forward (solattn_fwd_noalloc) against solattn_fwd
(GPU, through the C ABI).

Both run the same kernels; only where the work-queue counters live differs
(the library's per-device scratch array against a caller's workspace), so
outputs, selections and counts must be equal bit for bit.  Two calls in a
row, the second on a smaller problem, check that the counters the first call
left behind in the shared array do not leak into the second.
"""

import ctypes

import numpy as np
import pytest
import torch

from free_dynamic_sparse_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sa():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible to torch")
    from free_dynamic_sparse_amd import solattn
    return solattn


def _inputs(w):
    return tuple(torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).cuda()
                 for b in synth.make_inputs_bf16_bits(w))


def _prepare(sa, w, beta):
    q, k, v = _inputs(w)
    p = sa.problem(w.B, w.H, w.L, w.d, w.block, w.chunk, beta)
    ws = sa.Workspace(p, debug=True)
    sa.solattn_pool(p, q, k, v, ws.qbar, ws.kbar, ws.vhat)
    sa.solattn_moments(p, ws.qbar, ws.kbar, ws.kmean, ws.kcov, ws.tau)
    return p, q, k, v, ws


def _noalloc_through_abi(sa, p, q, k, v, ws, out, mask, count):
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    rc = sa.LIB.solattn_fwd_noalloc(ctypes.byref(p), P(q), P(k), P(v), P(ws.qbar), P(ws.kbar),
                                    P(ws.vhat), P(ws.tau), P(out), P(mask), P(count),
                                    ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0, sa.LIB.solattn_strerror(rc)


def test_noalloc_forward_equals_workspace_forward(sa):
    big = synth.Workload("noalloc_big", B=1, H=6, L=4096 + 300, d=128, block=128, chunk=32,
                         seed=41, kind="pos", grid=(1, 1, 4096 + 300))
    small = synth.Workload("noalloc_small", B=1, H=2, L=1000, d=64, block=64, chunk=16, seed=42,
                           kind="pos", grid=(1, 1, 1000))
    for w, beta in ((big, 1.0), (small, 0.5)):
        print(f"noalloc {w.name} beta={beta}", flush=True)
        p, q, k, v, ws = _prepare(sa, w, beta)
        N = w.N
        out_ref = torch.empty_like(q)
        sa.solattn_fwd(p, q, k, v, ws.qbar, ws.kbar, ws.vhat, ws.tau, out_ref, ws.queue,
                       ws.sel_mask, ws.sel_count)
        out = torch.full_like(q, float("nan"))
        mask = torch.zeros_like(ws.sel_mask)
        count = torch.full_like(ws.sel_count, -1)
        _noalloc_through_abi(sa, p, q, k, v, ws, out, mask, count)
        torch.cuda.synchronize()
        assert torch.equal(out, out_ref)
        assert torch.equal(mask, ws.sel_mask)
        assert torch.equal(count, ws.sel_count)
        assert 0 < count.sum().item() < w.B * w.H * N * N


def test_noalloc_forward_rejects_bad_arguments(sa):
    # checked before any HIP call, as for solattn_fwd
    P = lambda x: ctypes.c_void_p(x)
    p = sa.problem(1, 2, 1000, 128, 128, 32, 1.0)
    args = [P(1 << 20)] * 8
    args[3] = None
    assert sa.LIB.solattn_fwd_noalloc(ctypes.byref(p), *args, None, None, None) == -1
    empty = sa.problem(1, 0, 1000, 128, 128, 32, 1.0)
    assert sa.LIB.solattn_fwd_noalloc(ctypes.byref(empty), *([None] * 8), None, None,
                                      None) == 0


def test_noalloc_forward_replays_from_a_graph(sa):
    # Code under graph capture is one of the callers this entry point is for:
    # a captured call, replayed three times with cleared outputs, eager work
    # and an eager allocation-free call on another problem (which shares the
    # scratch array) between replays, equals the eager call bit for bit.
    w = synth.Workload("noalloc_graph", B=1, H=4, L=3000, d=128, block=128, chunk=32, seed=43,
                       kind="pos", grid=(1, 1, 3000))
    other = synth.Workload("noalloc_other", B=1, H=2, L=1000, d=64, block=64, chunk=16, seed=44,
                           kind="pos", grid=(1, 1, 1000))
    p, q, k, v, ws = _prepare(sa, w, 1.0)
    po, qo, ko, vo, wso = _prepare(sa, other, 0.5)
    eager = torch.empty_like(q)
    mask0, count0 = torch.zeros_like(ws.sel_mask), torch.zeros_like(ws.sel_count)
    _noalloc_through_abi(sa, p, q, k, v, ws, eager, mask0, count0)
    torch.cuda.synchronize()
    out = torch.empty_like(q)
    mask, count = torch.zeros_like(ws.sel_mask), torch.zeros_like(ws.sel_count)
    out_o = torch.empty_like(qo)
    mask_o, count_o = torch.zeros_like(wso.sel_mask), torch.zeros_like(wso.sel_count)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # one eager call on a side stream first
        _noalloc_through_abi(sa, p, q, k, v, ws, out, mask, count)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _noalloc_through_abi(sa, p, q, k, v, ws, out, mask, count)
    torch.cuda.synchronize()
    noise = torch.randn(1 << 20, device="cuda")
    for replay in range(3):
        print(f"noalloc graph replay {replay}", flush=True)
        out.zero_()
        mask.zero_()
        count.fill_(-1)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {replay}: output"
        assert torch.equal(mask, mask0), f"replay {replay}: selections"
        assert torch.equal(count, count0), f"replay {replay}: counts"
        noise.mul_(1.5).add_(0.25)  # eager work between replays
        _noalloc_through_abi(sa, po, qo, ko, vo, wso, out_o, mask_o, count_o)
        torch.cuda.synchronize()
    assert 0 < count0.sum().item() < w.B * w.H * w.N * w.N
