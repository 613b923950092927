"""Guard regions around every buffer the library writes (GPU, through the C ABI).

Each output is a view into the middle of a larger allocation whose head and
tail hold a sentinel pattern.  After a forward call on ragged shapes (a last
block with fewer valid tokens than the block size, so padded rows exist in
the kernels' tiles but not in the buffers), every sentinel must be intact:
no kernel writes a row past L, a block past N, a bitmap word past
ceil(N/64), a workspace byte past its size, or anything before a buffer's
start.  The outputs inside the guards must equal those of a call on plain
allocations bit for bit.
"""

import math

import numpy as np
import pytest
import torch

from free_dynamic_sparse_amd import synth

pytestmark = pytest.mark.gpu

GUARD_BYTES = 4096  # a multiple of 256, so every view keeps the allocation's alignment


@pytest.fixture(scope="module")
def sa():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible to torch")
    from free_dynamic_sparse_amd import solattn
    return solattn


class Guarded:
    """A buffer of `shape` and `dtype` with GUARD_BYTES of sentinel on each side."""

    def __init__(self, shape, dtype):
        esize = torch.empty(0, dtype=dtype).element_size()
        self.g = GUARD_BYTES // esize
        n = int(np.prod(shape)) if len(shape) else 1
        self.raw = torch.empty(2 * GUARD_BYTES + n * esize, dtype=torch.uint8, device="cuda")
        # sentinel: every byte 0xA5
        self.raw.fill_(0xA5)
        self.view = self.raw[GUARD_BYTES:GUARD_BYTES + n * esize].view(dtype).view(shape)
        self.n_bytes = n * esize

    def intact(self) -> bool:
        head = self.raw[:GUARD_BYTES]
        tail = self.raw[GUARD_BYTES + self.n_bytes:]
        return bool((head == 0xA5).all().item() and (tail == 0xA5).all().item())


def _forward_guarded(sa, q, k, v, p, first_order=False):
    B, H, L, d = q.shape
    N = sa.num_blocks(L, p.block)
    bufs = {
        "qbar": Guarded((B, H, N, d), torch.float32),
        "kbar": Guarded((B, H, N, d), torch.float32),
        "vhat": Guarded((B, H, N, d), torch.float32),
        "kmean": Guarded((B, H, d), torch.float32),
        "kcov": Guarded((B, H, d, d), torch.float32),
        "tau": Guarded((B, H, N), torch.float32),
        "mu": Guarded((B, H, N), torch.float32),
        "sigma": Guarded((B, H, N), torch.float32),
        "out": Guarded((B, H, L, d), torch.bfloat16),
    }
    x = {n: b.view for n, b in bufs.items()}
    sa.solattn_pool(p, q, k, v, x["qbar"], x["kbar"], x["vhat"])
    sa.solattn_moments(p, x["qbar"], x["kbar"], x["kmean"], x["kcov"], x["tau"], x["mu"],
                       x["sigma"])
    if first_order:
        bufs["kvc"] = Guarded((B, H, N, d, d), torch.bfloat16)
        bufs["workspace"] = Guarded((sa.solattn_fwd_first_order_workspace(p),), torch.uint8)
        sa.solattn_kv_moments(p, k, v, x["kbar"], x["vhat"], bufs["kvc"].view)
        sa.solattn_fwd_first_order(p, q, k, v, x["qbar"], x["kbar"], x["vhat"], bufs["kvc"].view,
                                   x["tau"], x["out"], bufs["workspace"].view)
    else:
        bufs["workspace"] = Guarded((sa.solattn_fwd_workspace_bytes(p),), torch.uint8)
        bufs["sel_mask"] = Guarded((B, H, N, (N + 63) // 64), torch.int64)
        bufs["sel_count"] = Guarded((B, H, N), torch.int32)
        sa.solattn_fwd(p, q, k, v, x["qbar"], x["kbar"], x["vhat"], x["tau"], x["out"],
                       bufs["workspace"].view, bufs["sel_mask"].view, bufs["sel_count"].view)
    torch.cuda.synchronize()
    return bufs


def _forward_plain(sa, q, k, v, p, first_order=False):
    ws = sa.Workspace(p, debug=True)
    out = torch.empty_like(q)
    sa.solattn_pool(p, q, k, v, ws.qbar, ws.kbar, ws.vhat)
    sa.solattn_moments(p, ws.qbar, ws.kbar, ws.kmean, ws.kcov, ws.tau, ws.mu, ws.sigma)
    if first_order:
        fws = sa.FirstOrderWorkspace(p)
        sa.solattn_kv_moments(p, k, v, ws.kbar, ws.vhat, fws.kvc)
        sa.solattn_fwd_first_order(p, q, k, v, ws.qbar, ws.kbar, ws.vhat, fws.kvc, ws.tau, out,
                                   fws.scratch)
    else:
        sa.solattn_fwd(p, q, k, v, ws.qbar, ws.kbar, ws.vhat, ws.tau, out, ws.queue, ws.sel_mask,
                       ws.sel_count)
    torch.cuda.synchronize()
    res = dict(out=out, qbar=ws.qbar, kbar=ws.kbar, vhat=ws.vhat, tau=ws.tau, kcov=ws.kcov)
    if not first_order:
        res.update(sel_mask=ws.sel_mask, sel_count=ws.sel_count)
    return res


# ragged L for every (d, block) instantiation; N = 8 .. 16, and one row of
# more than 64 blocks (two bitmap words, the second partial)
CASES = [(128, 128, 1000, 1.0), (128, 64, 1000, 0.5), (64, 128, 1000, 1.5),
         (64, 64, 1000, 1.0), (128, 128, 64 * 128 + 77, 1.0), (128, 128, 1000, -math.inf),
         (128, 128, 1000, math.inf)]


@pytest.mark.parametrize("d,block,L,beta", CASES)
def test_guards_intact_around_forward_outputs(sa, d, block, L, beta):
    print(f"canary d={d} block={block} L={L} beta={beta}", flush=True)
    w = synth.Workload("canary", B=2, H=2, L=L, d=d, block=block, chunk=16, seed=31, kind="pos",
                       grid=(1, 1, L))
    q, k, v = (torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).cuda()
               for b in synth.make_inputs_bf16_bits(w))
    p = sa.problem(w.B, w.H, L, d, block, 16, beta)
    bufs = _forward_guarded(sa, q, k, v, p)
    for name, b in bufs.items():
        assert b.intact(), f"{name}: a sentinel byte was overwritten"
    plain = _forward_plain(sa, q, k, v, p)
    for name, t in plain.items():
        assert torch.equal(bufs[name].view, t), f"{name} differs from the unguarded call"


@pytest.mark.parametrize("d,block,L", [(128, 128, 1000), (64, 64, 1000), (128, 64, 700)])
def test_guards_intact_around_first_order_outputs(sa, d, block, L):
    print(f"canary first-order d={d} block={block} L={L}", flush=True)
    w = synth.Workload("canary_fo", B=1, H=3, L=L, d=d, block=block, chunk=16, seed=32,
                       kind="pos", grid=(1, 1, L))
    q, k, v = (torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).cuda()
               for b in synth.make_inputs_bf16_bits(w))
    p = sa.problem(w.B, w.H, L, d, block, 16, 1.0)
    bufs = _forward_guarded(sa, q, k, v, p, first_order=True)
    for name, b in bufs.items():
        assert b.intact(), f"{name}: a sentinel byte was overwritten"
    plain = _forward_plain(sa, q, k, v, p, first_order=True)
    for name, t in plain.items():
        assert torch.equal(bufs[name].view, t), f"{name} differs from the unguarded call"
