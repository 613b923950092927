"""GPU parity of the routing baselines (top-k and top-p over the proxy map)
against the oracle, through the C ABI.

Tolerances: the proxy map is a float32 dot product of pooled float32
vectors, so each entry may differ from the float64 oracle by its rounding
bound eps_ij = (d + 2 (n + 2) + 4) 2^-24 scale sum_d |Qbar_id| |Kbar_jd|
(the dot product plus both pooled operands).  A selection may differ from
the oracle's only where the order it rests on is within that bound:
  * top-k: the count is exact; a block may be in one set and not the other
    only if its score lies within 2 eps of the row's k-th largest score;
  * top-p: the count c must be valid for the oracle's masses within the
    float32 summation bound delta (the c - 1 largest keep mass < p + delta,
    the c largest reach >= p - delta), and the set is the oracle's top-c set
    up to the same near-tie rule.
"""

import math

import numpy as np
import pytest
import torch

from free_dynamic_sparse_amd import synth
from oracle import solattn_ref as ref

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sa():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible to torch")
    from free_dynamic_sparse_amd import solattn
    return solattn


def log(msg):
    print(msg, flush=True)


def dev_bf16(x):
    return torch.from_numpy(synth.bf16_bits(x).view(np.int16)).view(torch.bfloat16).cuda()


def gpu_map_and_selections(sa, w, ks=(), ps=()):
    q, k, v = synth.make_inputs(w)
    B, H, L, d = q.shape
    p = sa.problem(B, H, L, d, w.block, w.chunk, 1.0)
    ws = sa.Workspace(p)
    sa.solattn_pool(p, dev_bf16(q), dev_bf16(k), dev_bf16(v), ws.qbar, ws.kbar, ws.vhat)
    N = w.N
    shat = torch.empty((B, H, N, N), dtype=torch.float32, device="cuda")
    sa.solattn_proxy_map(p, ws.qbar, ws.kbar, shat)
    W64 = (N + 63) // 64
    sels = {}
    for kk in ks:
        m = torch.empty((B, H, N, W64), dtype=torch.int64, device="cuda")
        c = torch.empty((B, H, N), dtype=torch.int32, device="cuda")
        sa.solattn_select_topk(p, shat, kk, m, c)
        sels[("k", kk)] = (m, c)
    for pp in ps:
        m = torch.empty((B, H, N, W64), dtype=torch.int64, device="cuda")
        c = torch.empty((B, H, N), dtype=torch.int32, device="cuda")
        sa.solattn_select_topp(p, shat, pp, m, c)
        sels[("p", pp)] = (m, c)
    torch.cuda.synchronize()
    out = {key: (sa.mask_to_bool(m, N).numpy(), c.cpu().numpy()) for key, (m, c) in sels.items()}
    return q, k, v, shat.cpu().numpy(), out


def map_tolerance(qbar, kbar, scale, d, n):
    return (d + 2 * (n + 2) + 4) * 2.0 ** -24 * scale * (np.abs(qbar) @ np.abs(kbar).T) + 1e-30


def check_set_against_order(got_row, shat_row, eps_row, count, tag):
    """got_row must be the oracle's top-`count` set of shat_row up to near-ties
    with the count-th largest score."""
    order = ref.order_row(shat_row)
    want = np.zeros_like(got_row)
    want[order[:count]] = True
    diff = np.flatnonzero(got_row != want)
    if diff.size:
        t = shat_row[order[count - 1]]
        far = diff[np.abs(shat_row[diff] - t) > 2 * eps_row[diff]]
        assert far.size == 0, f"{tag}: blocks {far[:5]} differ away from the boundary"
    return int(diff.size)


def check_workload(sa, w, ks, ps, rows=None):
    q, k, v, g_shat, g = gpu_map_and_selections(sa, w, ks, ps)
    N = w.N
    scale = ref.default_scale(w.d)
    n_tok = min(w.block, w.L)
    flips = 0
    for b in range(w.B):
        for h in range(w.H):
            qbar, kbar, _ = ref.pool(q[b, h], k[b, h], v[b, h], w.block)
            shat = ref.proxy_scores(qbar, kbar, scale)
            eps = map_tolerance(qbar, kbar, scale, w.d, n_tok)
            rs = np.arange(N) if rows is None else np.asarray(rows)
            err = np.abs(g_shat[b, h][rs] - shat[rs])
            assert np.all(err <= eps[rs]), f"{w.name} h{h}: map error {err.max():.3g}"
            for kk in ks:
                sel, cnt = g[("k", kk)]
                want_k = min(kk, N)
                assert np.all(cnt[b, h] == want_k)
                assert np.all(sel[b, h].sum(axis=1) == want_k)
                for i in rs:
                    flips += check_set_against_order(sel[b, h, i], shat[i], eps[i], want_k,
                                                     f"{w.name} h{h} i{i} top-{kk}")
            for pp in ps:
                sel, cnt = g[("p", pp)]
                assert np.all(sel[b, h].sum(axis=1) == cnt[b, h])
                delta = 4 * N * 2.0 ** -24 + 1e-6
                for i in rs:
                    c = int(cnt[b, h, i])
                    assert 1 <= c <= N
                    order = ref.order_row(shat[i])
                    w_ = np.exp(shat[i][order] - shat[i][order[0]])
                    frac = np.cumsum(w_) / w_.sum()
                    if pp >= 1.0:
                        assert c == N
                    else:
                        assert frac[c - 1] >= pp - delta, f"{w.name} h{h} i{i} top-p {pp}: short"
                        if c > 1:
                            assert frac[c - 2] < pp + delta, f"{w.name} h{h} i{i} top-p {pp}: long"
                    flips += check_set_against_order(sel[b, h, i], shat[i], eps[i], c,
                                                     f"{w.name} h{h} i{i} top-p {pp}")
    log(f"{w.name}: baselines match the oracle ({flips} near-tie differences)")
    return g


def test_baselines_tiny_and_image(sa):
    check_workload(sa, synth.WORKLOADS["tiny"], ks=(1, 10, 64, 70), ps=(0.1, 0.5, 0.9, 1.0))
    check_workload(sa, synth.WORKLOADS["image"], ks=(1, 5, 32), ps=(0.3, 0.9))


@pytest.mark.parametrize("d,block,L", [(128, 128, 3000), (64, 64, 50), (64, 128, 1900),
                                       (128, 64, 4160)])
def test_baselines_ragged_shapes(sa, d, block, L):
    w = synth.Workload("ragged_sel", B=2, H=2, L=L, d=d, block=block, chunk=16, seed=23,
                       kind="pos", grid=(1, 1, L))
    N = w.N
    check_workload(sa, w, ks=(1, max(1, N // 7), N), ps=(0.2, 0.75, 1.0))


@pytest.mark.timeout(300)
def test_baselines_wan_shape(sa):
    # the Wan shape (8 of its 40 heads, every row); k and p near the
    # threshold router's mean density at beta = 1
    w = synth.WORKLOADS["wan"].replace(H=8)
    check_workload(sa, w, ks=(80,), ps=(0.5,), rows=None)


@pytest.mark.timeout(300)
def test_baselines_longest_rows(sa):
    # N = 8192, the on-chip sort's limit; sampled rows
    w = synth.Workload("n8192", B=1, H=1, L=64 * 8192, d=64, block=64, chunk=16, seed=29,
                       kind="pos", grid=(8, 256, 256))
    check_workload(sa, w, ks=(1100,), ps=(0.4,), rows=[0, 1, 4095, 8190, 8191])
