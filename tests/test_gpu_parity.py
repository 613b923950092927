"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded, bf16-rounded inputs.

Small cases run the oracle in full (several tiles, ragged tails, every
kernel instantiation); the full-size video cases run in the launch
configuration the bench times and compare every head's selection and
thresholds plus sampled query blocks' outputs.
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
    """bf16-representable float32 array -> bf16 CUDA tensor (exact)."""
    bits = synth.bf16_bits(x).view(np.int16)
    return torch.from_numpy(bits).view(torch.bfloat16).cuda()


def bits_to_dev(b: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).cuda()


def run_gpu(sa, q, k, v, beta, block, chunk, exact_only=False, scale=None):
    """Run pool, moments and the fused kernel with every debug output.

    q, k, v: float32 numpy [B, H, L, d] (bf16-representable) or bf16 CUDA tensors."""
    if isinstance(q, np.ndarray):
        q, k, v = to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v)
    B, H, L, d = q.shape
    p = sa.problem(B, H, L, d, block, chunk, beta, scale, exact_only)
    ws = sa.Workspace(p, debug=True)
    out = torch.empty_like(q)
    sa.solattn_pool(p, q, k, v, ws.qbar, ws.kbar, ws.vhat)
    sa.solattn_moments(p, ws.qbar, ws.kbar, ws.kmean, ws.kcov, ws.tau, ws.mu, ws.sigma)
    sa.solattn_fwd(p, q, k, v, ws.qbar, ws.kbar, ws.vhat, ws.tau, out, ws.queue, ws.sel_mask,
                   ws.sel_count)
    torch.cuda.synchronize()
    N = sa.num_blocks(L, block)
    res = dict(out=out.float().cpu().numpy(), sel=sa.mask_to_bool(ws.sel_mask, N).numpy(),
               count=ws.sel_count.cpu().numpy())
    for name in ("qbar", "kbar", "vhat", "kmean", "kcov", "tau", "mu", "sigma"):
        res[name] = getattr(ws, name).cpu().numpy()
    return res


def head_view(res, b, h):
    return {k: (v[b, h] if v.ndim >= 3 else v) for k, v in res.items()}


def check_head(g, q, k, v, beta, block, exact_only=False, scale=None, rows=None, pool=True,
               tag=""):
    """Oracle on one head vs the GPU's results for it; returns a report dict."""
    r = ref.solattn_head(q, k, v, beta, block, scale=scale, rows=[], exact_only=exact_only)
    if pool:
        parity.check_pool(g, q, k, v, r, block)
    np.testing.assert_allclose(g["kmean"], r.m, rtol=0, atol=4 * 2.0 ** -24 * np.abs(r.m).max()
                               + 1e-30)
    np.testing.assert_allclose(g["kcov"], r.cov, rtol=0,
                               atol=8 * 2.0 ** -24 * np.abs(r.cov).max() + 1e-30)
    tau_err = parity.check_stats(g, r, beta)
    st = parity.selection_check(g["sel"], r)
    assert st.hard == 0, f"{tag}: {st.hard} selection mismatches outside the tie band"
    np.testing.assert_array_equal(g["count"], g["sel"].sum(axis=1))
    sel = r.sel if st.mismatches == 0 else g["sel"]
    L = q.shape[0]
    if rows is None:
        want = ref.forward(q, k, v, sel, block, r.scale, exact_only)
        got = g["out"]
    else:
        want = np.full(q.shape, np.nan)
        for i in rows:
            a, b = ref.block_range(L, block, i)
            want[a:b] = ref.forward_block(q, k, v, r.kbar, r.vhat, sel[i], i, block, r.scale,
                                          exact_only)
        got = g["out"]
    max_abs, mean_rel, finite = parity.output_errors(got, want)
    rep = dict(tag=tag, density=float(g["sel"].mean()), flips=st.in_band, total=st.total,
               hard=st.hard, max_abs=max_abs, mean_rel=mean_rel, tau_err_sigma=tau_err)
    log(f"  {tag}: {rep}")
    assert finite, f"{tag}: non-finite output"
    assert max_abs <= parity.MAX_ABS, f"{tag}: max-abs {max_abs}"
    assert mean_rel <= parity.MEAN_REL, f"{tag}: mean-rel {mean_rel}"
    return rep


def check_all_heads(sa, w: synth.Workload, beta, chunk=None, exact_only=False, scale=None):
    q, k, v = synth.make_inputs(w)
    g = run_gpu(sa, q, k, v, beta, w.block, chunk or w.chunk, exact_only, scale)
    reps = []
    for b in range(w.B):
        for h in range(w.H):
            reps.append(check_head(head_view(g, b, h), q[b, h], k[b, h], v[b, h], beta, w.block,
                                   exact_only, scale, tag=f"{w.name} b{b} h{h} beta={beta}"))
    parity.summarise(f"{w.name}: B{w.B} H{w.H} L{w.L} d{w.d} block{w.block} "
                     f"C{chunk or w.chunk}" + (" exact-only" if exact_only else ""), beta, reps)
    return g


# ------------------------------------------------------------------ small cases

@pytest.mark.parametrize("beta", [1.0, -math.inf])
def test_tiny_config(sa, beta):
    log(f"tiny beta={beta}")
    check_all_heads(sa, synth.WORKLOADS["tiny"], beta)


@pytest.mark.parametrize("beta", [0.5, 1.0, 1.5])
def test_image_config(sa, beta):
    log(f"image beta={beta}")
    check_all_heads(sa, synth.WORKLOADS["image"], beta)


@pytest.mark.parametrize("d,block,L,chunk", [
    (64, 64, 1000, 7), (128, 128, 3000, 1), (128, 64, 2500, 64), (64, 128, 1900, 33),
    (128, 128, 4096 + 128 * 3 + 1, 16),
])
def test_ragged_shapes_and_chunks(sa, d, block, L, chunk):
    log(f"ragged d={d} block={block} L={L} chunk={chunk}")
    w = synth.Workload("ragged", B=2, H=2, L=L, d=d, block=block, chunk=chunk, seed=21,
                       kind="pos", grid=(1, 1, L))
    check_all_heads(sa, w, 1.0)


@pytest.mark.parametrize("L", [1, 50, 64])
def test_single_block_selects_everything(sa, L):
    # one block: the proxy row is constant (sigma = 0), so every block is
    # selected and the pass is dense attention
    log(f"single block L={L}")
    w = synth.Workload("one", B=1, H=2, L=L, d=64, block=64, chunk=16, seed=3)
    g = check_all_heads(sa, w, 1.0)
    assert g["sel"].all()


def test_two_blocks_put_tau_on_the_larger_score(sa):
    # N = 2 at beta = 1: mu and sigma are the midpoint and half-gap of the two
    # proxy scores, so tau_i equals the larger one; the >= decision sits on the
    # tie and may go either way (an in-band case), and everything else holds.
    log("two blocks")
    w = synth.Workload("two", B=1, H=4, L=100, d=64, block=64, chunk=16, seed=3)
    check_all_heads(sa, w, 1.0)


def test_beta_plus_inf_is_all_approximation(sa):
    log("beta=+inf")
    w = synth.Workload("none", B=1, H=3, L=2000, d=128, block=128, chunk=32, seed=4, kind="pos",
                       grid=(1, 40, 50))
    g = check_all_heads(sa, w, math.inf)
    assert not g["sel"].any()


@pytest.mark.parametrize("d,block,L,grid", [(64, 64, 1000, (1, 1, 1000)),
                                            (128, 128, 4096, (1, 64, 64))])
def test_peaked_heads_all_approximated(sa, d, block, L, grid):
    # Peaked positional heads (alpha = 4) at beta = +inf: every block is
    # approximated and the logits run to a few hundred, so the approximation
    # logits must keep more precision than a bf16 Kbar gives.
    w = synth.Workload("peaked", B=1, H=2, L=L, d=d, block=block, chunk=16, seed=4,
                       kind="pos", grid=grid, alpha=4.0)
    check_all_heads(sa, w, math.inf)


def random_shapes(n=12, seed=2026):
    """Seeded random problems: batch, heads, ragged L, d, block, chunk, beta
    and input kind, drawn once (the same list on every run)."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        out.append((int(rng.integers(1, 3)), int(rng.integers(1, 4)), int(rng.integers(1, 4500)),
                    int(rng.choice([64, 128])), int(rng.choice([64, 128])),
                    int(rng.integers(1, 65)), float(np.round(rng.uniform(-1.0, 3.0), 2)),
                    str(rng.choice(["iid", "pos"]))))
    return out


RANDOM_SHAPES = random_shapes()


@pytest.mark.parametrize("case", range(len(RANDOM_SHAPES)))
def test_random_shapes(sa, case):
    B, H, L, d, block, chunk, beta, kind = RANDOM_SHAPES[case]
    w = synth.Workload(f"random{case}", B=B, H=H, L=L, d=d, block=block, chunk=chunk,
                       seed=100 + case, kind=kind, grid=(1, 1, L))
    check_all_heads(sa, w, beta)


@pytest.mark.parametrize("beta", [0.5, 2.0])
def test_exact_only_mode(sa, beta):
    log(f"exact-only beta={beta}")
    w = synth.Workload("exact", B=1, H=3, L=3000, d=128, block=128, chunk=32, seed=5,
                       kind="pos", grid=(1, 50, 60))
    check_all_heads(sa, w, beta, exact_only=True)


def test_explicit_scale(sa):
    log("explicit scale")
    w = synth.Workload("scale", B=1, H=2, L=2048, d=64, block=64, chunk=16, seed=6)
    check_all_heads(sa, w, 1.0, scale=0.3)


def test_dense_kernel_matches_textbook_attention(sa):
    for w in (synth.WORKLOADS["image"].replace(H=4),
              synth.Workload("dr", B=2, H=1, L=1500, d=64, block=64, chunk=16, seed=8)):
        log(f"dense {w.name}")
        q, k, v = synth.make_inputs(w)
        out = sa.dense_forward(to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v), block=w.block)
        got = out.float().cpu().numpy()
        for b in range(w.B):
            for h in range(w.H):
                want = ref.dense(q[b, h], k[b, h], v[b, h], 1.0 / math.sqrt(w.d))
                max_abs, mean_rel, finite = parity.output_errors(got[b, h], want)
                log(f"  dense b{b} h{h}: max_abs={max_abs:.3g} mean_rel={mean_rel:.3g}")
                assert finite and max_abs <= parity.MAX_ABS and mean_rel <= parity.MEAN_REL


def test_fused_at_beta_minus_inf_equals_dense_kernel(sa):
    # every block selected: the fused kernel does the dense kernel's exact
    # work in the same order; the empty approximation steps change nothing
    w = synth.WORKLOADS["image"].replace(H=6)
    q, k, v = (to_dev_bf16(x) for x in synth.make_inputs(w))
    fused = sa.forward(q, k, v, beta=-math.inf, block=w.block, chunk=w.chunk)
    dense = sa.dense_forward(q, k, v, block=w.block)
    torch.cuda.synchronize()
    assert torch.equal(fused, dense)


def test_exact_only_at_the_beta_limits(sa):
    # beta = -inf: every block is exact, so dropping the approximation changes
    # nothing and the output equals the dense kernel's bit for bit; beta = +inf:
    # nothing is selected, and a row with no exact block outputs zeros
    w = synth.WORKLOADS["image"].replace(H=3, L=4000, grid=(1, 50, 80))
    q, k, v = (to_dev_bf16(x) for x in synth.make_inputs(w))
    every = sa.forward(q, k, v, beta=-math.inf, block=w.block, chunk=w.chunk, exact_only=True)
    dense = sa.dense_forward(q, k, v, block=w.block)
    none = torch.full_like(q, float("nan"))
    sa.forward(q, k, v, beta=math.inf, block=w.block, chunk=w.chunk, exact_only=True, out=none)
    torch.cuda.synchronize()
    assert torch.equal(every, dense)
    assert torch.count_nonzero(none).item() == 0


def test_chunk_size_does_not_change_the_result(sa):
    # C is validated but does not change the schedule: the kernel routes 64
    # pooled keys per step whatever C is, and the selected set is the union of
    # the chunks' sets whatever the chunking (the page's streaming identity),
    # so every output bit is the same for every C.
    w = synth.WORKLOADS["image"].replace(H=4)
    q, k, v = synth.make_inputs(w)
    base = run_gpu(sa, q, k, v, 1.0, w.block, 32)
    for chunk in (1, 8, 16, 33, 64):
        g = run_gpu(sa, q, k, v, 1.0, w.block, chunk)
        for name in ("sel", "count", "out", "tau"):
            np.testing.assert_array_equal(g[name], base[name], err_msg=f"chunk {chunk}: {name}")


def test_key_covariance_is_exactly_symmetric(sa):
    # each off-diagonal 32x32 tile of Sigma is computed once and written to
    # both halves; d = 128 (ten tiles) and d = 64 (three)
    for wname, H in (("image", 3), ("tiny", 1)):
        w = synth.WORKLOADS[wname].replace(H=H)
        q, k, v = synth.make_inputs(w)
        g = run_gpu(sa, q, k, v, 1.0, w.block, w.chunk)
        cov = g["kcov"]
        assert np.array_equal(cov, np.swapaxes(cov, -1, -2)), wname
        assert np.all(np.isfinite(cov)), wname


def test_repeat_calls_are_bitwise_identical(sa):
    w = synth.WORKLOADS["image"].replace(H=4)
    q, k, v = synth.make_inputs(w)
    a = run_gpu(sa, q, k, v, 1.0, w.block, w.chunk)
    b = run_gpu(sa, q, k, v, 1.0, w.block, w.chunk)
    for name in ("out", "sel", "tau", "kcov", "qbar"):
        np.testing.assert_array_equal(a[name], b[name])


# ------------------------------------------------------------------ full sizes

def sampled_rows(N, n=6):
    rows = {0, N - 1, N // 2, N // 3, (2 * N) // 3, 1}
    return sorted(r for r in rows if 0 <= r < N)[:n]


_INPUTS = {}


def full_size_inputs(w: synth.Workload):
    """bf16 bit patterns of a full-size workload, kept for the next test that
    asks for the same workload (several betas run on the same inputs)."""
    key = repr(w)
    if key not in _INPUTS:
        _INPUTS.clear()
        t0 = time.time()
        _INPUTS[key] = synth.make_inputs_bf16_bits(w)
        log(f"{w.name}: inputs generated in {time.time() - t0:.1f}s")
    return _INPUTS[key]


def full_size(sa, name, beta, heads_checked, n_rows=6):
    """name: a workload name or a synth.Workload.

    Every head: pooled arrays, thresholds and the whole selection against the
    oracle; heads_checked: also n_rows sampled query blocks' outputs."""
    w = synth.WORKLOADS[name] if isinstance(name, str) else name
    name = w.name
    qb, kb, vb = full_size_inputs(w)
    q, k, v = bits_to_dev(qb), bits_to_dev(kb), bits_to_dev(vb)
    g = run_gpu(sa, q, k, v, beta, w.block, w.chunk)
    del q, k, v
    torch.cuda.empty_cache()
    log(f"{name}: GPU done, density {g['sel'].mean():.4f}")
    reports = []
    for h in range(w.H):
        qh = synth.bits_to_f32(qb[0, h])
        kh = synth.bits_to_f32(kb[0, h])
        vh = synth.bits_to_f32(vb[0, h])
        gh = head_view(g, 0, h)
        if h in heads_checked:
            reports.append(check_head(gh, qh, kh, vh, beta, w.block, rows=sampled_rows(w.N, n_rows),
                                      tag=f"{name} h{h} beta={beta}"))
        else:
            # every head: pooling, thresholds and the whole selection
            r = ref.solattn_head(qh, kh, vh, beta, w.block, rows=[])
            parity.check_pool(gh, qh, kh, vh, r, w.block)
            tau_err = parity.check_stats(gh, r, beta)
            st = parity.selection_check(gh["sel"], r)
            assert st.hard == 0, f"{name} h{h}: {st.hard} hard selection mismatches"
            reports.append(dict(density=float(gh["sel"].mean()), flips=st.in_band,
                                total=st.total, hard=st.hard, tau_err_sigma=tau_err))
    e = parity.summarise(f"{name}: B{w.B} H{w.H} L{w.L} d{w.d} block{w.block} C{w.chunk}", beta,
                         reports, {"output_rows_per_head": n_rows})
    log(f"{name} beta={beta}: {e}")
    return g, reports


@pytest.mark.timeout(300)
@pytest.mark.parametrize("beta", [0.5, 1.0, 1.5])
def test_wan_full_size(sa, beta):
    g, reps = full_size(sa, "wan", beta, heads_checked=(0, 13, 26, 39))
    dens = g["sel"].mean()
    log(f"wan density {dens:.4f} (Gaussian reference {0.5 * math.erfc(beta / math.sqrt(2)):.4f})")


@pytest.mark.timeout(300)
def test_hunyuan_full_size(sa):
    full_size(sa, "hunyuan", 1.0, heads_checked=(0, 23), n_rows=4)


@pytest.mark.timeout(300)
@pytest.mark.parametrize("beta", [-math.inf, 0.0, 1.0, 2.0, 3.0])
def test_stress_full_size(sa, beta):
    # heads 0-3 peaked (alpha = 4), heads 4-7 flat (iid): outputs on one of each
    full_size(sa, "stress", beta, heads_checked=(0, 7), n_rows=3)


@pytest.mark.timeout(300)
@pytest.mark.parametrize("L,beta", [(16384, 2.0), (131072, 1.0)])
def test_seq_sweep_shapes(sa, L, beta):
    # the sequence-length sweep's shortest and longest shapes, in the
    # configuration the sweep times
    full_size(sa, synth.seq_workload(L), beta, heads_checked=(0, 7), n_rows=3)


def test_stats_returns_the_routing_statistics(sa):
    # the Python convenience entry: the same statistics as the oracle
    w = synth.WORKLOADS["image"].replace(H=3)
    q, k, v = synth.make_inputs(w)
    res = sa.stats(to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v), beta=1.0, block=w.block,
                   chunk=w.chunk)
    torch.cuda.synchronize()
    N = w.N
    sel = sa.mask_to_bool(res["sel_mask"], N).numpy()
    for h in range(w.H):
        r = ref.solattn_head(q[0, h], k[0, h], v[0, h], 1.0, w.block, rows=[])
        g = {"tau": res["tau"][0, h].cpu().numpy(), "mu": res["mu"][0, h].cpu().numpy(),
             "sigma": res["sigma"][0, h].cpu().numpy()}
        parity.check_stats(g, r, 1.0)
        st = parity.selection_check(sel[0, h], r)
        assert st.hard == 0
        np.testing.assert_array_equal(res["sel_count"][0, h].cpu().numpy(), sel[0, h].sum(axis=1))


@pytest.mark.timeout(300)
def test_wan_full_size_block64(sa):
    # the page's 64-token blocks at the Wan shape (N = 1182, tail 16): every
    # head's selection and statistics, sampled heads' outputs
    full_size(sa, synth.WORKLOADS["wan"].replace(block=64, H=16), 1.0, heads_checked=(0, 15),
              n_rows=4)


# ------------------------------------------------------------ given selections

@pytest.mark.parametrize("exact_only", [False, True])
def test_masked_forward_with_topk_selections(sa, exact_only):
    # the oracle's top-k sets (an upper set of each proxy row of a fixed
    # size) as the given selections: the fused kernel without routing against
    # the oracle's forward over the same sets
    for w, kk in ((synth.WORKLOADS["image"].replace(H=3), 6),
                  (synth.Workload("ragged_m", B=2, H=2, L=3000, d=128, block=128, chunk=32,
                                  seed=27, kind="pos", grid=(1, 1, 3000)), 5)):
        q, k, v = synth.make_inputs(w)
        sels = np.zeros((w.B, w.H, w.N, w.N), dtype=bool)
        for b in range(w.B):
            for h in range(w.H):
                qb, kb, _ = ref.pool(q[b, h], k[b, h], v[b, h], w.block)
                sels[b, h] = ref.select_topk(ref.proxy_scores(qb, kb, ref.default_scale(w.d)), kk)
        mask = sa.bool_to_mask(torch.from_numpy(sels)).cuda()
        out = sa.forward_masked(to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v), mask,
                                block=w.block, exact_only=exact_only)
        got = out.float().cpu().numpy()
        for b in range(w.B):
            for h in range(w.H):
                want = ref.forward(q[b, h], k[b, h], v[b, h], sels[b, h], w.block,
                                   ref.default_scale(w.d), exact_only)
                max_abs, mean_rel, finite = parity.output_errors(got[b, h], want)
                log(f"  masked {w.name} b{b} h{h} exact_only={exact_only}: max_abs={max_abs:.3g} "
                    f"mean_rel={mean_rel:.3g}")
                assert finite and max_abs <= parity.MAX_ABS and mean_rel <= parity.MEAN_REL


def test_masked_forward_reproduces_routed_forward(sa):
    # fed the routed kernel's own selections (with garbage in the bits past
    # N), the masked kernel does the same work in the same order: equal bits
    w = synth.Workload("mask_same", B=1, H=4, L=4096 + 200, d=128, block=128, chunk=32, seed=28,
                       kind="pos", grid=(1, 1, 4096 + 200))
    q, k, v = (to_dev_bf16(x) for x in synth.make_inputs(w))
    res = sa.stats(q, k, v, beta=1.0, block=w.block, chunk=w.chunk)
    mask = res["sel_mask"].clone()
    N = w.N
    assert N % 64 != 0
    junk = torch.tensor(-1 << (N % 64), dtype=torch.int64)  # every bit at or past N
    mask[..., -1] |= junk.cuda()
    out = sa.forward_masked(q, k, v, mask, block=w.block)
    torch.cuda.synchronize()
    assert torch.equal(out, res["out"])
