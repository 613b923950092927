"""Pins of the CPU oracle against what the mathematics fixes (CPU only).

Each test checks the oracle against something other than itself: a library
routine (torch SDPA, numpy reductions), a closed form, a brute-force
materialisation, or an invariant the method states.  Together they are
chosen so that a dropped term, a wrong sign, a wrong weight or a transposed
operand in the oracle fails at least one of them.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

from free_dynamic_sparse_amd import synth
from oracle import solattn_ref as ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def sdpa(q, k, v, scale, mask=None):
    """torch's scaled-dot-product attention on CPU in float64 (library routine)."""
    t = lambda x: torch.as_tensor(np.asarray(x, np.float64))[None, None]
    m = None if mask is None else torch.as_tensor(mask)[None, None]
    o = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), attn_mask=m,
                                                         scale=scale)
    return o[0, 0].numpy()


def small(L=1000, d=64, block=64, seed=11, kind="iid", grid=None):
    w = synth.Workload("t", B=1, H=1, L=L, d=d, block=block, chunk=16, seed=seed, kind=kind,
                       grid=grid)
    q, k, v = synth.make_head(w, 0, 0)
    return w, q, k, v


def phi_sf(beta):
    """1 - Phi(beta) for the standard normal."""
    return 0.5 * math.erfc(beta / math.sqrt(2.0))


# ---------------------------------------------------------------- pooling

@pytest.mark.parametrize("L", [4096, 1000, 65])
def test_pool_matches_numpy_segment_reductions(L):
    _, q, k, v = small(L=L)
    block = 64
    qbar, kbar, vhat = ref.pool(q, k, v, block)
    starts = np.arange(0, L, block)
    n = np.diff(np.append(starts, L)).astype(np.float64)
    for x, got, is_mean in ((q, qbar, True), (k, kbar, True), (v, vhat, False)):
        s = np.add.reduceat(x.astype(np.float64), starts, axis=0)
        want = s / n[:, None] if is_mean else s
        np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(ref.block_sizes(L, block), n.astype(np.int64))


# ---------------------------------------------------------------- moments

@pytest.mark.parametrize("case", ["iid_ragged", "pos"])
def test_row_stats_equal_bruteforce_proxy_rows(case):
    if case == "iid_ragged":
        w, q, k, v = small(L=1000)
    else:
        w, q, k, v = small(L=4096, d=128, block=128, kind="pos", grid=(1, 64, 64))
    scale = 1.0 / math.sqrt(w.d)
    qbar, kbar, _ = ref.pool(q, k, v, w.block)
    m, cov = ref.key_moments(kbar)
    mu, sigma = ref.row_stats(qbar, m, cov, scale)
    shat = ref.proxy_scores(qbar, kbar, scale)
    # brute force: materialise every proxy row and take numpy's mean / std (ddof=0)
    np.testing.assert_allclose(mu, shat.mean(axis=1), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(sigma, shat.std(axis=1, ddof=0), rtol=1e-9, atol=1e-12)
    # brute force of the moments themselves
    np.testing.assert_allclose(m, kbar.mean(axis=0), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(cov, np.cov(kbar.T, bias=True), rtol=1e-9, atol=1e-13)


def test_thresholds_special_values():
    mu = np.array([0.5, 1.0, -2.0])
    sigma = np.array([1.0, 0.0, 2.0])
    assert np.all(ref.thresholds(mu, sigma, -math.inf) == -np.inf)
    assert np.all(ref.thresholds(mu, sigma, math.inf) == np.inf)
    tau = ref.thresholds(mu, sigma, 1.5)
    assert tau[0] == 2.0 and tau[1] == -np.inf and tau[2] == 1.0
    with pytest.raises(ValueError):
        ref.thresholds(mu, sigma, float("nan"))


@pytest.mark.parametrize("beta", [0.5, 1.0, 1.5, 2.0])
def test_mean_density_tracks_gaussian_tail(beta):
    # iid N(0,1) Q and K: given Qbar_i, the proxy row is an iid Gaussian sample,
    # so the mean selected density approaches rho_G(beta) = 1 - Phi(beta).
    dens = []
    for seed in range(12):
        w = synth.Workload("t", B=1, H=1, L=4096, d=64, block=64, chunk=16, seed=100 + seed)
        q, k, v = synth.make_head(w, 0, 0)
        r = ref.solattn_head(q, k, v, beta, 64, rows=[])
        dens.append(r.sel.mean())
    assert abs(np.mean(dens) - phi_sf(beta)) <= 0.01


def test_mean_density_tracks_gaussian_tail_long_row():
    # N = 591 blocks (the Wan block count): tighter tolerance.
    w = synth.Workload("t", B=1, H=1, L=591 * 128, d=128, block=128, chunk=32, seed=7)
    q, k, v = synth.make_head(w, 0, 0)
    r = ref.solattn_head(q, k, v, 1.0, 128, rows=[])
    assert abs(r.sel.mean() - phi_sf(1.0)) <= 0.003


def test_two_blocks_put_tau_on_the_larger_score():
    # A proxy row of two entries a < b has mean (a + b) / 2 and population
    # std (b - a) / 2, so at beta = 1 the threshold is exactly b: the larger
    # block passes the >= test and the smaller does not.  Small integers keep
    # every step exact in float64.
    q = np.array([[1.0], [1.0]])
    k = np.array([[1.0], [3.0]])
    v = np.array([[1.0], [2.0]])
    r = ref.solattn_head(q, k, v, 1.0, 1, scale=1.0)
    assert np.all(r.shat == [[1.0, 3.0], [1.0, 3.0]])
    assert np.all(r.tau == 3.0)
    assert r.sel.tolist() == [[False, True], [False, True]]


def test_selection_invariances():
    w, q, k, v = small(L=4096, d=64, block=64, kind="pos", grid=(1, 64, 64))
    base = ref.solattn_head(q, k, v, 1.0, 64, rows=[])
    # (a) any positive softmax scale gives the same selection
    for s in (0.01, 1.0, 3.0):
        r = ref.solattn_head(q, k, v, 1.0, 64, scale=s, rows=[])
        band = np.abs(base.shat - base.tau[:, None]) < 1e-6 * base.sigma[:, None]
        assert np.all((r.sel == base.sel) | band)
    # (b) permuting key blocks (with their values) permutes the selection and
    #     leaves every output unchanged
    N = w.N
    perm = np.random.default_rng(0).permutation(N)
    kp = k.reshape(N, 64, -1)[perm].reshape(k.shape)
    vp = v.reshape(N, 64, -1)[perm].reshape(v.shape)
    full = ref.solattn_head(q, k, v, 1.0, 64)
    permd = ref.solattn_head(q, kp, vp, 1.0, 64)
    np.testing.assert_array_equal(permd.sel, full.sel[:, perm])
    np.testing.assert_allclose(permd.out, full.out, rtol=1e-10, atol=1e-12)


# ---------------------------------------------------------------- streaming

@pytest.mark.parametrize("chunk", [1, 5, 16, 64, 70])
def test_streaming_selection_equals_full_row(chunk):
    w, q, k, v = small(L=4000, d=64, block=64, kind="pos", grid=(1, 50, 80))
    scale = 1.0 / 8.0
    r = ref.solattn_head(q, k, v, 1.0, 64, rows=[])
    s = ref.select_streaming(q, r.kbar, r.tau, 64, chunk, scale)
    np.testing.assert_array_equal(s, r.sel)


def test_tile_column_means_are_proxy_scores():
    # The column means of the token-to-block tile (Eq. 11) are the proxy scores.
    w, q, k, v = small(L=1000, d=64, block=64)
    scale = 0.125
    qbar, kbar, _ = ref.pool(q, k, v, 64)
    shat = ref.proxy_scores(qbar, kbar, scale)
    for i in range(w.N):
        a, b = ref.block_range(w.L, 64, i)
        tile = scale * (q[a:b].astype(np.float64) @ kbar.T)
        np.testing.assert_allclose(tile.mean(axis=0), shat[i], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("chunk", [1, 7, 16, 64])
@pytest.mark.parametrize("beta", [0.5, 1.0])
def test_streaming_forward_equals_direct_forward(chunk, beta):
    w, q, k, v = small(L=1500, d=64, block=64, kind="pos", grid=(1, 30, 50))
    r = ref.solattn_head(q, k, v, beta, 64)
    out, sel = ref.forward_streaming(q, k, v, r.tau, 64, chunk, r.scale)
    np.testing.assert_array_equal(sel, r.sel)
    np.testing.assert_allclose(out, r.out, rtol=1e-10, atol=1e-12)


# ---------------------------------------------------------------- forward

@pytest.mark.parametrize("L", [1000, 4096])
def test_beta_minus_inf_is_dense_attention(L):
    w, q, k, v = small(L=L)
    r = ref.solattn_head(q, k, v, -math.inf, 64)
    assert r.sel.all()
    want = sdpa(q, k, v, r.scale)
    np.testing.assert_allclose(r.out, want, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(ref.dense(q, k, v, r.scale), want, rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("beta", [0.0, 0.5, 1.0, 2.0, math.inf])
def test_block_constant_keys_make_the_approximation_exact(beta):
    # If every key of block j equals Kbar_j, the zeroth-order term is exact, so
    # the output is dense attention whatever is selected.  The ragged last
    # block (n_j < block) checks the n_j weight; Vhat as a sum is checked too.
    w, q, _, v = small(L=1000)
    rng = np.random.default_rng(5)
    kb = rng.standard_normal((w.N, w.d))
    k = np.repeat(kb, 64, axis=0)[:w.L]
    r = ref.solattn_head(q, k, v, beta, 64)
    if beta not in (0.0, math.inf):
        assert 0 < r.sel.mean() < 1
    np.testing.assert_allclose(r.out, sdpa(q, k, v, r.scale), rtol=1e-10, atol=1e-12)


def _denominator_probe(L=1000, block=64, constant_keys=False, beta=1.0):
    """Outputs that expose the softmax denominator row by row.

    Values are zero except on one selected block j0, whose tokens all carry
    e_0.  Then coordinate 0 of every output row is the exact mass of block j0
    divided by the row's whole denominator, for the oracle's forward
    (approximate unselected blocks) and for dense attention alike, so their
    ratio dense / oracle is D_approx / D_exact, row by row."""
    w, q, k, _ = small(L=L, block=block)
    if constant_keys:
        rng = np.random.default_rng(5)
        k = np.repeat(rng.standard_normal((w.N, w.d)), block, axis=0)[:L]
    r = ref.solattn_head(q, k, np.zeros_like(q), beta, block)
    sel = r.sel.copy()
    j0 = 1
    sel[:, j0] = True
    v = np.zeros_like(q)
    v[j0 * block:(j0 + 1) * block, 0] = 1.0
    approx = ref.forward(q, k, v, sel, block, r.scale)[:, 0]
    exact = ref.dense(q, k, v, r.scale)[:, 0]
    return sel, exact / approx


def test_approx_denominator_is_below_the_exact_one():
    # Jensen: exp of a block's mean logit is at most the mean of exp over the
    # block's logits, so n_j exp(scale q.Kbar_j) <= sum_c exp(scale q.k_c) for
    # every unselected block, and the approximate denominator never exceeds
    # the exact one; with non-constant keys the bound is strict.
    sel, ratio = _denominator_probe()
    assert (~sel).any(axis=1).all()
    assert np.all(ratio <= 1.0 + 1e-12)
    assert np.all(ratio < 1.0 - 1e-6)
    # equality for block-constant keys (each block's logits are constant)
    _, ratio_c = _denominator_probe(constant_keys=True)
    np.testing.assert_allclose(ratio_c, 1.0, rtol=1e-12)


def test_beta_plus_inf_is_attention_over_pooled_keys():
    # Nothing selected: each block contributes n_j exp(scale q.Kbar_j) and
    # exp(scale q.Kbar_j) Vhat_j, i.e. attention over the pooled keys with an
    # additive bias log n_j and values Vhat_j / n_j.
    w, q, k, v = small(L=1000)
    r = ref.solattn_head(q, k, v, math.inf, 64)
    assert not r.sel.any()
    nj = ref.block_sizes(w.L, 64).astype(np.float64)
    bias = np.broadcast_to(np.log(nj)[None, :], (w.L, w.N)).copy()
    want = sdpa(q, r.kbar, r.vhat / nj[:, None], r.scale, mask=bias)
    np.testing.assert_allclose(r.out, want, rtol=1e-10, atol=1e-12)


def test_exact_only_is_block_masked_attention():
    w, q, k, v = small(L=1000)
    r = ref.solattn_head(q, k, v, 1.0, 64)
    out = ref.forward(q, k, v, r.sel, 64, r.scale, exact_only=True)
    blk = np.arange(w.L) // 64
    mask = r.sel[blk][:, blk]  # token-level: query token's block row, key token's block
    np.testing.assert_allclose(out, sdpa(q, k, v, r.scale, mask=mask), rtol=1e-10, atol=1e-12)


def test_hand_worked_example():
    with open(os.path.join(GOLDEN, "worked_example.json")) as f:
        g = json.load(f)
    q, k, v = (np.array(g[x], np.float64) for x in ("q", "k", "v"))
    block, scale = g["block"], g["scale"]
    env = {"__builtins__": {}}
    ev = lambda s: float(eval(s, env, {"e": math.e, "inf": math.inf}))
    for case in g["cases"]:
        beta = ev(case["beta"])
        first = case.get("first_order", False)
        r = ref.solattn_head(q, k, v, beta, block, scale=scale, exact_only=case["exact_only"],
                             first_order=first)
        np.testing.assert_allclose(r.mu, [ev(x) for x in g["mu"]], rtol=1e-14)
        np.testing.assert_allclose(r.sigma, [ev(x) for x in g["sigma"]], rtol=1e-14)
        if "tau" in case:
            np.testing.assert_allclose(r.tau, [ev(x) for x in case["tau"]], rtol=1e-14)
        np.testing.assert_array_equal(r.sel, np.array(case["selected"]))
        want = np.array([[ev(x) for x in row] for row in case["out"]])
        np.testing.assert_allclose(r.out, want, rtol=1e-13)
        if not case["exact_only"] and not first:
            out_s, _ = ref.forward_streaming(q, k, v, r.tau, block, 1, scale)
            np.testing.assert_allclose(out_s, want, rtol=1e-13)


def test_executed_flops_counts():
    # Dense selection: 4 L^2 d exact, plus the tile 2 L d N, and no approximate term.
    L, d, b = 1000, 64, 64
    N = ref.num_blocks(L, b)
    sel = np.ones((N, N), bool)
    assert ref.executed_flops(L, d, b, sel) == 4.0 * L * L * d + 2.0 * L * d * N
    none = np.zeros((N, N), bool)
    assert ref.executed_flops(L, d, b, none) == 2.0 * L * d * N + 2.0 * L * d * N


def _flops_by_enumeration(L, d, block, sel, exact_only=False):
    """Multiply-adds counted one query token at a time (2 FLOPs each).

    For every valid query token r of block i: d for q_r . k_c and d for
    p_rc v_c, per key token c of each selected block; d per pooled key (all
    N of them: the token-to-block tile); d per unselected block for the
    p_rj Vhat_j product."""
    N = ref.num_blocks(L, block)
    macs = 0
    for r in range(L):
        i = r // block
        for j in range(N):
            macs += d  # tile entry q_r . Kbar_j
            if sel[i, j]:
                for c in range(j * block, min(L, (j + 1) * block)):
                    macs += 2 * d
            elif not exact_only:
                macs += d
    return 2.0 * macs


@pytest.mark.parametrize("L,block", [(300, 64), (1000, 128), (129, 64)])
def test_executed_flops_equal_enumeration_at_a_partial_selection(L, block):
    # A partial selection with a ragged last block, selected for some query
    # blocks and not for others (so n_i and n_j both differ from the block
    # size somewhere): the closed form must equal the token-by-token count.
    d = 32
    N = ref.num_blocks(L, block)
    rng = np.random.default_rng(L + block)
    sel = rng.random((N, N)) < 0.4
    sel[0, N - 1] = True
    sel[N - 1, N - 1] = False
    sel[N - 1, 0] = True
    for eo in (False, True):
        assert ref.executed_flops(L, d, block, sel, exact_only=eo) == \
            _flops_by_enumeration(L, d, block, sel, exact_only=eo)


def test_exact_only_with_nothing_selected_outputs_zero():
    w, q, k, v = small(L=200)
    r = ref.solattn_head(q, k, v, math.inf, 64, exact_only=True)
    assert not r.sel.any()
    assert np.all(r.out == 0.0)


# ---------------------------------------------------------------- routing baselines
# top-k and top-p over the materialised proxy map: the baselines the page
# compares threshold routing with.

def _rows(seed, n_rows=12, N=37):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((n_rows, N)) * rng.uniform(0.2, 3.0, (n_rows, 1))


@pytest.mark.parametrize("k", [1, 5, 36, 37, 50])
def test_topk_keeps_the_k_largest(k):
    shat = _rows(1)
    sel = ref.select_topk(shat, k)
    N = shat.shape[1]
    for i in range(shat.shape[0]):
        assert sel[i].sum() == min(k, N)
        if 0 < sel[i].sum() < N:
            assert shat[i][sel[i]].min() >= shat[i][~sel[i]].max()


def test_topk_breaks_ties_by_block_index():
    row = np.array([[1.0, 3.0, 2.0, 3.0, 2.0, 2.0, 0.0]])
    assert np.array_equal(np.flatnonzero(ref.select_topk(row, 3)[0]), [1, 2, 3])
    assert np.array_equal(np.flatnonzero(ref.select_topk(row, 4)[0]), [1, 2, 3, 4])


@pytest.mark.parametrize("beta", [-0.5, 0.5, 1.0, 2.0])
def test_topk_with_threshold_counts_is_threshold_routing(beta):
    # S_i = {j : shat_ij >= tau_i} is an upper set of row i, so the top-|S_i|
    # entries of the row are exactly S_i
    w = synth.Workload("pin_topk", B=1, H=1, L=64 * 40, d=64, block=64, chunk=8, seed=31,
                       kind="pos", grid=(1, 40, 64))
    q, k, v = synth.make_head(w, 0, 0)
    r = ref.solattn_head(q, k, v, beta, w.block, rows=[])
    got = ref.select_topk(r.shat, r.sel.sum(axis=1))
    assert np.array_equal(got, r.sel)


@pytest.mark.parametrize("p", [0.05, 0.3, 0.5, 0.9, 0.999])
def test_topp_is_the_shortest_prefix_reaching_p(p):
    shat = _rows(2)
    sel = ref.select_topp(shat, p)
    for i in range(shat.shape[0]):
        o = ref.order_row(shat[i])
        cnt = int(sel[i].sum())
        assert cnt >= 1 and sel[i][o[:cnt]].all()  # a prefix of the sorted order
        assert ref.topp_mass(shat[i], sel[i]) >= p - 1e-12
        if cnt > 1:
            shorter = sel[i].copy()
            shorter[o[cnt - 1]] = False
            assert ref.topp_mass(shat[i], shorter) < p


@pytest.mark.parametrize("p,N", [(0.3, 37), (0.62, 20), (0.999, 11)])
def test_topp_on_a_uniform_row_keeps_ceil_pN(p, N):
    # equal logits: every block has mass 1/N, so the shortest prefix with mass
    # >= p has ceil(p N) blocks (p N is not an integer here)
    sel = ref.select_topp(np.zeros((1, N)), p)
    assert sel.sum() == math.ceil(p * N)
    assert np.array_equal(np.flatnonzero(sel[0]), np.arange(math.ceil(p * N)))


def test_topp_special_cases():
    row = np.zeros((1, 16))
    row[0, 9] = 50.0  # one dominant logit holds mass 1 - 15 e^-50
    assert np.array_equal(np.flatnonzero(ref.select_topp(row, 0.9)[0]), [9])
    assert ref.select_topp(_rows(3), 1.0).all()
    with pytest.raises(ValueError):
        ref.select_topp(row, 0.0)


# ---------------------------------------------------------------- first-order term
# The next term of the page's Taylor expansion of an unselected block's
# exponential scores around the block's row-wise mean score.

def _near_mean_keys(L, d, block, eps, seed=3):
    """Keys within eps of their block mean: k_t = Kbar_j + eps delta_t with the
    deltas of each block centred, so Kbar_j does not depend on eps."""
    rng = np.random.default_rng(seed)
    N = ref.num_blocks(L, block)
    base = rng.standard_normal((N, d))
    delta = rng.standard_normal((L, d))
    k = np.empty((L, d))
    for j in range(N):
        a, b = ref.block_range(L, block, j)
        k[a:b] = base[j] + eps * (delta[a:b] - delta[a:b].mean(axis=0))
    q = rng.standard_normal((L, d))
    v = rng.standard_normal((L, d))
    return q, k, v


def test_first_order_error_is_second_order_in_the_key_spread():
    # All blocks approximated (beta = +inf).  Exact attention differs from
    # the zeroth-order output by O(eps) and from the first-order output by
    # O(eps^2): halving eps halves the one error and quarters the other.
    # A dropped scale, a sign error or a transposed moment breaks the eps^2.
    L, d, block = 45, 6, 8   # ragged last block of 5 tokens
    N = ref.num_blocks(L, block)
    none = np.zeros((N, N), bool)
    scale = 0.5
    errs0, errs1 = [], []
    for eps in (0.02, 0.01, 0.005):
        q, k, v = _near_mean_keys(L, d, block, eps)
        exact = ref.dense(q, k, v, scale)
        errs0.append(np.abs(ref.forward(q, k, v, none, block, scale) - exact).max())
        errs1.append(np.abs(ref.forward(q, k, v, none, block, scale, first_order=True)
                            - exact).max())
    for a, b in zip(errs0, errs0[1:]):
        assert 1.8 < a / b < 2.2, errs0
    for a, b in zip(errs1, errs1[1:]):
        assert 3.6 < a / b < 4.4, errs1
    assert errs1[-1] < 0.05 * errs0[-1]


def test_first_order_denominator_term_vanishes():
    _, q, k, v = small(L=300, d=16, block=64, kind="pos", grid=(1, 1, 300))
    qi = np.asarray(q[64:128], np.float64)
    kj, vj = np.asarray(k[128:192], np.float64), np.asarray(v[128:192], np.float64)
    scale = 0.25
    centre = scale * (qi @ kj.mean(axis=0))
    num, den = ref.first_order_terms(qi, kj, vj, centre, centre.max() * np.ones(64), scale)
    S = scale * (qi @ kj.T)
    size = (np.exp(centre - centre.max())[:, None] * np.abs(S - centre[:, None])).sum(axis=1)
    assert np.all(np.abs(den) <= 1e-13 * size)
    assert np.abs(num).max() > 1e-3


def test_kv_moments_is_n_times_numpy_cross_covariance():
    L, d, block = 150, 5, 64
    _, _, k, v = small(L=L, d=d, block=block)
    C = ref.kv_moments(k, v, block)
    for j in range(ref.num_blocks(L, block)):
        a, b = ref.block_range(L, block, j)
        cov = np.cov(np.asarray(k[a:b], np.float64).T, np.asarray(v[a:b], np.float64).T,
                     bias=True)[:d, d:]
        np.testing.assert_allclose(C[j], (b - a) * cov, rtol=1e-11, atol=1e-12)


def test_kv_moments_give_the_first_order_numerator():
    # scale * q_r^T C_j (the moment form the kernels use) equals the token
    # form sum_t (S_rt - c_r) v_t of first_order_terms.
    L, d, block = 200, 12, 64
    _, q, k, v = small(L=L, d=d, block=block, kind="pos", grid=(1, 1, L))
    scale = 0.3
    C = ref.kv_moments(k, v, block)
    qi = np.asarray(q[:64], np.float64)
    for j in range(ref.num_blocks(L, block)):
        a, b = ref.block_range(L, block, j)
        centre = scale * (qi @ np.asarray(k[a:b], np.float64).mean(axis=0))
        num, _ = ref.first_order_terms(qi, k[a:b], v[a:b], centre, centre, scale)
        np.testing.assert_allclose(num, scale * (qi @ C[j]), rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("beta", [-math.inf, 0.0, 1.0, math.inf])
def test_first_order_with_block_constant_keys_is_dense(beta):
    # Constant keys within each block make S - c = 0: the first-order term
    # adds nothing and the output is still dense attention.
    rng = np.random.default_rng(8)
    L, d, block = 200, 8, 64
    N = ref.num_blocks(L, block)
    kb = rng.standard_normal((N, d))
    k = np.repeat(kb, block, axis=0)[:L]
    q = rng.standard_normal((L, d))
    v = rng.standard_normal((L, d))
    r = ref.solattn_head(q, k, v, beta, block, first_order=True)
    np.testing.assert_allclose(r.out, sdpa(q, k, v, r.scale), rtol=1e-10, atol=1e-12)


def test_first_order_at_beta_minus_inf_is_dense():
    w, q, k, v = small(L=300, d=16, block=64, kind="pos", grid=(1, 1, 300))
    r = ref.solattn_head(q, k, v, -math.inf, 64, first_order=True)
    np.testing.assert_allclose(r.out, sdpa(q, k, v, r.scale), rtol=1e-10, atol=1e-12)


def test_first_order_refuses_exact_only():
    _, q, k, v = small(L=100, d=8, block=64)
    with pytest.raises(ValueError):
        ref.solattn_head(q, k, v, 1.0, 64, exact_only=True, first_order=True)


def test_first_order_flops():
    L, d, b = 1000, 64, 64
    N = ref.num_blocks(L, b)
    none = np.zeros((N, N), bool)
    base = ref.executed_flops(L, d, b, none)
    assert ref.executed_flops(L, d, b, none, first_order=True) == \
        base + 2.0 * d * d * L * N + 2.0 * d * d * L
