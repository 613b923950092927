"""GPU parity of the first-order term (solattn_kv_moments and
solattn_fwd_first_order, through the C ABI) against the oracle.

Tolerances.
  * Block moments C_j = K_j^T V_j - Kbar_j Vhat_j^T: exact bf16 products
    accumulated in float32 (error <= 2^-24 (n + 2) S[a][b] with
    S[a][b] = sum_t |k_t[a]| |v_t[b]|), the float32 pooled Kbar_j and Vhat_j
    (each within 2^-24 (n + 2) of the sums of absolute values they come
    from), one float32 product and subtraction, then one bf16 rounding (unit
    roundoff u = 2^-8).  So each element is within
        u |C_j[a][b]| + 2^-24 (3 n + 8) (S[a][b] + mean_t |k_t[a]| sum_t |v_t[b]|).
  * Outputs: the bf16 output bounds of the zeroth-order path (max-abs 2e-2,
    mean-relative 5e-3), after checking the selection as for solattn_fwd
    (in-band flips only; the oracle then takes the GPU's selection).
  * The correction itself: where the first-order change is at least 5% of
    the output, the GPU's first-order output must lie within 10% of that
    change from the oracle's (the correction is formed from bf16 operands,
    relative error about 2^-7, plus the output's bf16 rounding), so a wrong
    sign, scale or operand in the kernel cannot pass.
"""

import math
import sys
import time

import numpy as np
import pytest
import torch

from free_dynamic_sparse_amd import synth
from oracle import solattn_ref as ref
from tests import parity

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sa():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible to torch")
    from free_dynamic_sparse_amd import solattn
    return solattn


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev_bf16(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(synth.bf16_bits(x).view(np.int16)).view(torch.bfloat16).cuda()


def bits_to_dev(b: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).cuda()


def run_both(sa, q, k, v, beta, block, chunk=16, want_kvc=False):
    """Zeroth-order forward (with its selection) and first-order forward on
    the same inputs.  q, k, v: numpy float32 (bf16-representable) or bf16
    CUDA tensors [B, H, L, d]."""
    if isinstance(q, np.ndarray):
        q, k, v = to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v)
    B, H, L, d = q.shape
    N = sa.num_blocks(L, block)
    p = sa.problem(B, H, L, d, block, chunk, beta)
    ws = sa.Workspace(p, debug=True)
    fws = sa.FirstOrderWorkspace(p)
    out0 = torch.empty_like(q)
    out1 = torch.empty_like(q)
    sa.solattn_pool(p, q, k, v, ws.qbar, ws.kbar, ws.vhat)
    sa.solattn_moments(p, ws.qbar, ws.kbar, ws.kmean, ws.kcov, ws.tau, ws.mu, ws.sigma)
    sa.solattn_fwd(p, q, k, v, ws.qbar, ws.kbar, ws.vhat, ws.tau, out0, ws.queue, ws.sel_mask,
                   ws.sel_count)
    sa.solattn_kv_moments(p, k, v, ws.kbar, ws.vhat, fws.kvc)
    sa.solattn_fwd_first_order(p, q, k, v, ws.qbar, ws.kbar, ws.vhat, fws.kvc, ws.tau, out1,
                               fws.scratch)
    torch.cuda.synchronize()
    res = dict(out0=out0.float().cpu().numpy(), out1=out1.float().cpu().numpy(),
               sel=sa.mask_to_bool(ws.sel_mask, N).numpy())
    for name in ("kbar", "tau", "mu", "sigma"):
        res[name] = getattr(ws, name).cpu().numpy()
    if want_kvc:
        res["kvc"] = fws.kvc.float().cpu().numpy()
    return res


def check_kvc(kvc_gpu, k, v, block, tag):
    """kvc_gpu: [N, d(value), d(key)] for one head."""
    L, d = k.shape
    want = ref.kv_moments(k, v, block)              # [N, d(key), d(value)]
    u = 2.0 ** -8
    worst = 0.0
    for j in range(ref.num_blocks(L, block)):
        a, b = ref.block_range(L, block, j)
        n = b - a
        kj = np.abs(k[a:b].astype(np.float64))
        vj = np.abs(v[a:b].astype(np.float64))
        S = kj.T @ vj
        pooled = kj.mean(axis=0)[:, None] * vj.sum(axis=0)[None, :]
        tol = u * np.abs(want[j]) + 2.0 ** -24 * (3 * n + 8) * (S + pooled) + 1e-30
        err = np.abs(kvc_gpu[j].T - want[j])
        assert np.all(err <= tol), f"{tag}: block {j}, max excess {(err - tol).max():.3g}"
        worst = max(worst, float((err / tol).max()))
    return worst


def check_first_order(g, q, k, v, beta, block, rows=None, tag="", scaled_abs=False):
    """One head: selection as for solattn_fwd, then the first-order output
    against the oracle with the GPU's selection.  scaled_abs: the max-abs bar
    applies to |err| / max(1, |ref|) (for outputs far outside the unit range,
    where bf16 rounding alone exceeds the absolute bar)."""
    L = q.shape[0]
    r = ref.solattn_head(q, k, v, beta, block, rows=[])
    st = parity.selection_check(g["sel"], r)
    assert st.hard == 0, f"{tag}: {st.hard} selection mismatches outside the tie band"
    sel = g["sel"]
    rows = range(ref.num_blocks(L, block)) if rows is None else rows
    want1 = np.full(q.shape, np.nan)
    want0 = np.full(q.shape, np.nan)
    for i in rows:
        a, b = ref.block_range(L, block, i)
        want1[a:b] = ref.forward_block(q, k, v, r.kbar, r.vhat, sel[i], i, block, r.scale,
                                       first_order=True)
        want0[a:b] = ref.forward_block(q, k, v, r.kbar, r.vhat, sel[i], i, block, r.scale)
    ok = np.isfinite(want1)
    if scaled_abs:
        scale_ref = np.maximum(1.0, np.abs(np.where(ok, want1, 0.0)))
        max_abs, mean_rel, finite = parity.output_errors(g["out1"] / scale_ref, want1 / scale_ref)
        mean_rel = parity.output_errors(g["out1"], want1)[1]
    else:
        max_abs, mean_rel, finite = parity.output_errors(g["out1"], want1)
    change = float(np.abs(want1[ok] - want0[ok]).mean())
    size = float(np.abs(want1[ok]).mean())
    err1 = float(np.abs(g["out1"][ok] - want1[ok]).mean())
    mean_rel0 = parity.output_errors(g["out0"], want0)[1]
    rep = dict(tag=tag, density=float(sel.mean()), flips=st.in_band, max_abs=max_abs,
               mean_rel=mean_rel, mean_rel_zeroth=mean_rel0, change_rel=change / size,
               err_over_change=err1 / max(change, 1e-30))
    log(f"  {rep}")
    assert finite, f"{tag}: non-finite output"
    assert max_abs <= parity.MAX_ABS, f"{tag}: max-abs {max_abs}"
    assert mean_rel <= parity.MEAN_REL, f"{tag}: mean-rel {mean_rel}"
    if change >= 0.05 * size:
        assert err1 <= 0.1 * change, f"{tag}: first-order change not reproduced ({rep})"
    return rep


def check_workload(sa, w, beta, kvc=True):
    q, k, v = synth.make_inputs(w)
    g = run_both(sa, q, k, v, beta, w.block, w.chunk, want_kvc=kvc)
    reps = []
    for b in range(w.B):
        for h in range(w.H):
            tag = f"{w.name} b{b} h{h} beta={beta}"
            if kvc:
                check_kvc(g["kvc"][b, h], k[b, h], v[b, h], w.block, tag)
            gh = {key: val[b, h] for key, val in g.items() if key != "kvc"}
            reps.append(check_first_order(gh, q[b, h], k[b, h], v[b, h], beta, w.block, tag=tag))
    return reps


@pytest.mark.parametrize("beta", [math.inf, 1.0, 0.0])
def test_tiny_config(sa, beta):
    # i.i.d. inputs: the first-order change is 30-70% of the output
    reps = check_workload(sa, synth.WORKLOADS["tiny"], beta)
    assert reps[0]["change_rel"] > 0.05


def test_image_config(sa):
    check_workload(sa, synth.WORKLOADS["image"].replace(H=4), 1.0)


@pytest.mark.parametrize("d,block,L", [(64, 64, 50), (64, 128, 1900), (128, 64, 4160),
                                       (128, 128, 3000), (64, 64, 2113)])
@pytest.mark.parametrize("beta", [1.0, math.inf])
def test_ragged_shapes(sa, d, block, L, beta):
    # every (d, block) instantiation, ragged tails, N from 1 to 65 (one and
    # several 32-block groups, one and two bitmap words per row)
    w = synth.Workload("ragged_fo", B=2, H=2, L=L, d=d, block=block, chunk=16, seed=31,
                       kind="iid" if beta == math.inf else "pos", grid=(1, 1, L))
    check_workload(sa, w, beta)


@pytest.mark.parametrize("d,block,L,grid", [(64, 64, 1000, (1, 1, 1000)),
                                            (128, 128, 4096, (1, 64, 64))])
def test_peaked_heads_at_beta_plus_inf(sa, d, block, L, grid):
    # Peaked positional heads with every block approximated: the first-order
    # term dominates (outputs reach about 30, several times the dense
    # output's norm away from it) and the kernel must still follow the oracle.
    w = synth.Workload("peaked_fo", B=1, H=2, L=L, d=d, block=block, chunk=16, seed=4,
                       kind="pos", grid=grid, alpha=4.0)
    q, k, v = synth.make_inputs(w)
    g = run_both(sa, q, k, v, math.inf, block, want_kvc=True)
    for h in range(w.H):
        check_kvc(g["kvc"][0, h], k[0, h], v[0, h], block, f"peaked h{h}")
        gh = {key: val[0, h] for key, val in g.items() if key != "kvc"}
        rep = check_first_order(gh, q[0, h], k[0, h], v[0, h], math.inf, block,
                                tag=f"peaked d{d} h{h}", scaled_abs=True)
        assert rep["change_rel"] > 0.5
        assert rep["mean_rel_zeroth"] <= parity.MEAN_REL


@pytest.mark.parametrize("case", range(4))
def test_random_shapes(sa, case):
    # the first four of the seeded random problems of the zeroth-order tests
    from tests.test_gpu_parity import RANDOM_SHAPES
    B, H, L, d, block, chunk, beta, kind = RANDOM_SHAPES[case]
    w = synth.Workload(f"random{case}", B=B, H=H, L=L, d=d, block=block, chunk=chunk,
                       seed=100 + case, kind=kind, grid=(1, 1, L))
    check_workload(sa, w, beta)


def test_beta_minus_inf_leaves_the_output_unchanged(sa):
    # nothing is unselected: the first-order forward is the zeroth-order one
    w = synth.WORKLOADS["tiny"]
    q, k, v = synth.make_inputs(w)
    g = run_both(sa, q, k, v, -math.inf, w.block, w.chunk)
    assert g["sel"].all()
    np.testing.assert_array_equal(g["out1"], g["out0"])


def test_block_constant_keys_give_zero_moments(sa):
    # keys constant within each block: C_j = 0 (the two float32 sums of
    # K_j^T V_j - Kbar_j Vhat_j^T cancel up to their rounding), so the
    # correction is below 2^-20 of the output's scale: each bf16 output moves
    # by at most one unit in its last place or by that absolute amount
    rng = np.random.default_rng(12)
    B, H, L, d, block = 1, 2, 1000, 128, 128
    N = ref.num_blocks(L, block)
    kb = synth.round_bf16(rng.standard_normal((B, H, N, d)).astype(np.float32))
    k = np.repeat(kb, block, axis=2)[:, :, :L]
    q = synth.round_bf16(rng.standard_normal((B, H, L, d)).astype(np.float32))
    v = synth.round_bf16(rng.standard_normal((B, H, L, d)).astype(np.float32))
    g = run_both(sa, q, k, v, 1.0, block, want_kvc=True)
    for h in range(H):
        check_kvc(g["kvc"][0, h], k[0, h], v[0, h], block, f"constant keys h{h}")
    np.testing.assert_allclose(g["out1"], g["out0"], rtol=2.0 ** -7,
                               atol=2.0 ** -20 * float(np.abs(g["out0"]).max()))


def test_repeat_calls_are_bitwise_identical(sa):
    w = synth.WORKLOADS["image"].replace(H=2)
    q, k, v = synth.make_inputs(w)
    a = run_both(sa, q, k, v, 1.0, w.block, w.chunk)
    b = run_both(sa, q, k, v, 1.0, w.block, w.chunk)
    assert np.array_equal(a["out1"].view(np.uint32), b["out1"].view(np.uint32))


@pytest.mark.timeout(300)
def test_wan_full_size(sa):
    # the Wan shape in the bench's launch configuration: every head's
    # selection, two heads' sampled query blocks against the oracle
    w = synth.WORKLOADS["wan"]
    t0 = time.time()
    qb, kb, vb = synth.make_inputs_bf16_bits(w)
    log(f"wan: inputs generated in {time.time() - t0:.1f}s")
    q, k, v = bits_to_dev(qb), bits_to_dev(kb), bits_to_dev(vb)
    g = run_both(sa, q, k, v, 1.0, w.block, w.chunk)
    del q, k, v
    torch.cuda.empty_cache()
    log(f"wan: GPU done, density {g['sel'].mean():.4f}")
    rows = [0, 1, w.N // 2, w.N - 1]
    for h in (0, w.H - 1):
        qh, kh, vh = (synth.bits_to_f32(x[0, h]) for x in (qb, kb, vb))
        gh = {key: val[0, h] for key, val in g.items()}
        check_first_order(gh, qh, kh, vh, 1.0, w.block, rows=rows, tag=f"wan h{h}")
