"""The forward pass on other streams and replayed from a HIP graph.

The library only enqueues kernels on the stream it is given and never
synchronises or allocates, so a whole forward call (pool, moments and
thresholds, fused kernel) can run on any stream and can be captured once
into a graph and replayed.  Both must give the eager result bit for bit.
"""

import math

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


def inputs(w):
    q, k, v = synth.make_inputs(w)
    dev = lambda x: torch.from_numpy(synth.bf16_bits(x).view(np.int16)).view(torch.bfloat16).cuda()
    return dev(q), dev(k), dev(v)


WORK = synth.Workload("streams", B=1, H=4, L=3000, d=128, block=128, chunk=32, seed=31,
                      kind="pos", grid=(1, 50, 60))


def test_forward_on_a_side_stream_is_bitwise_equal(sa):
    q, k, v = inputs(WORK)
    base = sa.forward(q, k, v, beta=1.0, block=WORK.block, chunk=WORK.chunk)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        out = sa.forward(q, k, v, beta=1.0, block=WORK.block, chunk=WORK.chunk)
    side.synchronize()
    assert torch.equal(out, base)


@pytest.mark.parametrize("first_order,beta", [(False, 1.0), (False, -math.inf), (True, 1.0)])
def test_forward_replayed_from_a_graph_is_bitwise_equal(sa, first_order, beta):
    q, k, v = inputs(WORK)
    B, H, L, d = q.shape
    p = sa.problem(B, H, L, d, WORK.block, WORK.chunk, beta)
    kw = dict(beta=beta, block=WORK.block, chunk=WORK.chunk)
    fwd = sa.forward_first_order if first_order else sa.forward
    eager = fwd(q, k, v, **kw)
    torch.cuda.synchronize()
    # every buffer of the captured call is allocated before capture
    bufs = dict(out=torch.empty_like(q), ws=sa.Workspace(p, "cuda"))
    if first_order:
        bufs["fws"] = sa.FirstOrderWorkspace(p, "cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # one eager call on a side stream first
        fwd(q, k, v, **kw, **bufs)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fwd(q, k, v, **kw, **bufs)
    torch.cuda.synchronize()
    out, ws = bufs["out"], bufs["ws"]
    noise = torch.randn(1 << 20, device="cuda")
    for replay in range(3):
        out.zero_()
        ws.tau.fill_(float("nan"))  # the replay must recompute what the fused kernel reads
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {replay} differs from the eager call"
        noise.mul_(1.5).add_(0.25)  # eager work between replays
        torch.cuda.synchronize()
