"""CPU oracle for the Sol-Attn sparse-attention forward pass.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
CPU-baseline leg may import this module.  The HIP path never imports it, and
it shares no code with the HIP path.

Source: "Sol-Attn: Accelerating Video Generation Inference via On-the-Fly
Attention Sparsification" (arXiv 2607.24027, HTML version), the method
section: block proxies (Eq. 3), query-dependent threshold routing (Eq. 4),
moment-based row statistics (the moment identity of Appendix B), chunk-wise
streaming thresholding (Eqs. 6-7), the zeroth-order Taylor approximation of
unselected blocks (the expansion before Eqs. 9-10), the combined denominator
and numerator (Eqs. 9-10), the token-to-block score tile (Eq. 11, Figure 4)
and the nested-loop kernel (Algorithm 3.2).  Beyond the page's method,
first_order_terms keeps the first-order term of the same Taylor expansion.

Everything is plain NumPy in float64 on one (batch, head) at a time, written
for a reader checking it against the page, not for speed.  Where the page
leaves a step open (its equation displays did not survive), the reading
taken is stated at the function that depends on it.

Pins (tests/test_oracle_*.py, CPU only):
  pool                 block means / sums vs numpy reshape reductions
  key_moments,
  row_stats            mean / std(ddof=0) of brute-force materialised proxy rows
  thresholds, select   Gaussian density 1 - Phi(beta) on iid inputs; scale and
                       block-permutation invariance
  select_streaming     equals full-row selection (the page's union identity)
  forward              beta = -inf -> dense softmax attention (torch SDPA);
                       block-constant keys -> dense attention for every beta;
                       beta = +inf -> SDPA over pooled keys with bias log n_j;
                       exact-only mode -> SDPA with a block mask;
                       hand-worked example in tests/golden
  forward_streaming    equals forward for every chunk size (C-invariance)
  dense                torch SDPA
  approx denominator   Jensen bound: never above the exact denominator, strictly
                       below it for non-constant keys, equal for block-constant
                       keys (read off the outputs with a one-block value probe)
  select_topk          k largest by construction (count, order and tie
                       invariants); with per-row counts |S_i| it reproduces
                       threshold routing, whose sets are upper sets of the row
  select_topp          mass reaches p and the prefix is the shortest such
                       (invariants); uniform rows keep ceil(p N) blocks, a
                       dominant score keeps one, p = 1 keeps the row
  first_order_terms    hand-worked first-order cases in tests/golden; the
                       error against exact attention falls as eps^2 when the
                       keys lie within eps of their block mean (the
                       zeroth-order error as eps); the denominator term
                       vanishes; block-constant keys and beta = -inf leave
                       the output unchanged
  kv_moments           n_j times numpy's cross-covariance (np.cov, bias=True);
                       scale * q^T C_j equals first_order_terms' numerator
  executed_flops       closed forms at all / none selected; equal to a
                       token-by-token multiply-add count at partial selections
                       with a ragged last block
No function here is "parity unpinned".
"""

from __future__ import annotations

import math
from typing import Optional, Tuple

import numpy as np

F64 = np.float64


# --------------------------------------------------------------------------
# Blocks
# --------------------------------------------------------------------------

def num_blocks(L: int, block: int) -> int:
    """N = ceil(L / block): the number of query blocks and of key blocks."""
    return (L + block - 1) // block


def block_range(L: int, block: int, j: int) -> Tuple[int, int]:
    """Token rows [start, stop) of block j; the last block may hold fewer rows."""
    return j * block, min(L, (j + 1) * block)


def block_sizes(L: int, block: int) -> np.ndarray:
    """n_j: the number of valid tokens in each block."""
    N = num_blocks(L, block)
    return np.array([block_range(L, block, j)[1] - block_range(L, block, j)[0]
                     for j in range(N)], dtype=np.int64)


# --------------------------------------------------------------------------
# Step 1: block pooling (Eq. 3 proxies; summed values of Eqs. 9-10)
# --------------------------------------------------------------------------

def pool(q: np.ndarray, k: np.ndarray, v: np.ndarray, block: int):
    """Pooled queries Qbar_i, pooled keys Kbar_j (means) and summed values Vhat_j.

    Qbar and Kbar are means over the block's tokens: the page's column-mean
    identity (Eq. 11) recovers the routing scores from the token-to-block tile
    "exactly" only when Qbar_i is the mean of Q_i's rows, and the approximation
    centres each unselected block on the row-wise mean score q_r . mean(K_j).
    Vhat_j is the sum of V_j along the token dimension (stated on the page).
    Reading: a ragged last block is pooled over its valid tokens only.
    """
    L, d = q.shape
    N = num_blocks(L, block)
    qbar = np.empty((N, d), F64)
    kbar = np.empty((N, d), F64)
    vhat = np.empty((N, d), F64)
    for j in range(N):
        a, b = block_range(L, block, j)
        qbar[j] = np.asarray(q[a:b], F64).mean(axis=0)
        kbar[j] = np.asarray(k[a:b], F64).mean(axis=0)
        vhat[j] = np.asarray(v[a:b], F64).sum(axis=0)
    return qbar, kbar, vhat


# --------------------------------------------------------------------------
# Step 2: moments of the pooled keys and row thresholds (Eq. 4, Appendix B)
# --------------------------------------------------------------------------

def key_moments(kbar: np.ndarray):
    """First moment m and centred second moment Sigma of the pooled keys.

    m = (1/N) sum_j Kbar_j;  Sigma = (1/N) sum_j (Kbar_j - m)(Kbar_j - m)^T.
    Reading: population (1/N) statistics, because mu_i and sigma_i are the mean
    and standard deviation of the whole proxy row.
    """
    N = kbar.shape[0]
    m = kbar.sum(axis=0) / N
    c = kbar - m[None, :]
    cov = (c.T @ c) / N
    return m, cov


def row_stats(qbar: np.ndarray, m: np.ndarray, cov: np.ndarray, scale: float):
    """mu_i and sigma_i of the proxy row shat_i = scale * Qbar_i Kbar^T, from moments.

    The row is a linear projection of the pooled keys, so its mean is
    scale * Qbar_i . m and its variance scale^2 * Qbar_i^T Sigma Qbar_i:
    O(N d^2) work, O(d^2) storage, no N x N map.
    """
    mu = scale * (qbar @ m)
    var = (scale * scale) * np.einsum("id,de,ie->i", qbar, cov, qbar)
    sigma = np.sqrt(np.maximum(var, 0.0))
    return mu, sigma


def thresholds(mu: np.ndarray, sigma: np.ndarray, beta: float) -> np.ndarray:
    """tau_i = mu_i + beta * sigma_i (Eq. 4).

    Readings: beta = -inf selects every block and beta = +inf selects none
    (the page states beta > 0; the formula is extended to both limits so that
    -inf * 0 never arises).  A degenerate row with sigma_i = 0 is constant, so
    every block passes the >= test in exact arithmetic; tau_i = -inf encodes
    that so rounding cannot split the tie.
    """
    if math.isnan(beta):
        raise ValueError("beta is NaN")
    if beta == -math.inf:
        return np.full(mu.shape, -np.inf)
    if beta == math.inf:
        return np.full(mu.shape, np.inf)
    tau = mu + beta * sigma
    return np.where(sigma == 0.0, -np.inf, tau)


def proxy_scores(qbar: np.ndarray, kbar: np.ndarray, scale: float) -> np.ndarray:
    """The full N x N proxy map shat_ij = scale * Qbar_i . Kbar_j (Eq. 3).

    The method never builds it; the oracle does, to check everything else.
    """
    return scale * (qbar @ kbar.T)


def select(shat: np.ndarray, tau: np.ndarray) -> np.ndarray:
    """S_i = {j : shat_ij >= tau_i} (Eq. 4).

    Reading: ">=".  The comparison is taken in float32, the precision the
    GPU kernel decides in, on values computed here in float64.
    """
    return shat.astype(np.float32) >= tau.astype(np.float32)[:, None]


# --------------------------------------------------------------------------
# Routing baselines the page compares threshold routing with: top-k and
# top-p over the materialised proxy map (the discussion after Eq. 4; the
# selection-latency comparison of Figure 5(b); the density spread of
# Figure 7).  They are not part of the method.
# --------------------------------------------------------------------------

def order_row(shat_row: np.ndarray) -> np.ndarray:
    """Block indices of one proxy row, largest score first.

    Reading: the page gives no tie rule; equal scores are taken in
    increasing block index.
    """
    n = len(shat_row)
    return np.lexsort((np.arange(n), -np.asarray(shat_row, F64)))


def select_topk(shat: np.ndarray, k) -> np.ndarray:
    """Top-k routing: S_i = the k_i largest entries of proxy row i.

    k is one count for every row or an array of per-row counts; counts of N
    or more select the whole row.  Every row keeps the same number of blocks
    (a fixed budget, the contrast the page draws with threshold routing).
    """
    n_rows, N = shat.shape
    ks = np.broadcast_to(np.asarray(k, dtype=np.int64), (n_rows,))
    sel = np.zeros((n_rows, N), dtype=bool)
    for i in range(n_rows):
        kk = int(min(max(ks[i], 0), N))
        sel[i, order_row(shat[i])[:kk]] = True
    return sel


def select_topp(shat: np.ndarray, p: float) -> np.ndarray:
    """Top-p routing: the shortest run of a row's largest scores whose
    softmax mass reaches p (at least one block).

    Row i is sorted by score, largest first; its softmax distribution over
    the N blocks is w_j = exp(shat_ij) / sum_l exp(shat_il); S_i is the
    smallest prefix of the sorted order with sum_{j in prefix} w_j >= p.
    Reading: the softmax is over the proxy logits themselves, one term per
    block (not weighted by the block's token count), the plainest reading of
    the cumulative mass of the softmax-score distribution; 0 < p <= 1.
    """
    if not 0.0 < p <= 1.0:
        raise ValueError("top-p needs 0 < p <= 1")
    n_rows, N = shat.shape
    sel = np.zeros((n_rows, N), dtype=bool)
    for i in range(n_rows):
        o = order_row(shat[i])
        row = np.asarray(shat[i], F64)[o]
        w = np.exp(row - row[0])
        cum = np.cumsum(w)
        frac = cum / cum[-1]
        # p = 1 is reached only by the whole row (every w_j > 0 in exact
        # arithmetic), however small the tail's mass is in floating point
        count = N if p >= 1.0 else min(int(np.searchsorted(frac, p, side="left")) + 1, N)
        sel[i, o[:count]] = True
    return sel


def topp_mass(shat_row: np.ndarray, sel_row: np.ndarray) -> float:
    """Softmax mass of the selected entries of one proxy row."""
    x = np.asarray(shat_row, F64)
    w = np.exp(x - x.max())
    return float(w[sel_row].sum() / w.sum())


def select_streaming(q: np.ndarray, kbar: np.ndarray, tau: np.ndarray,
                     block: int, chunk: int, scale: float) -> np.ndarray:
    """Chunk-wise streaming thresholding (Eqs. 6-7) through the score tile (Eq. 11).

    For query block i and chunk t of C pooled keys, the token-to-block tile is
    scale * Q_i Kbar^(t)^T (n_i x C); its column means over the query tokens
    are the chunk's proxy scores, which are thresholded on the spot.  The
    union over chunks is the selected set.
    """
    L, _ = q.shape
    N = kbar.shape[0]
    T = (N + chunk - 1) // chunk
    sel = np.zeros((N, N), dtype=bool)
    for i in range(N):
        a, b = block_range(L, block, i)
        qi = np.asarray(q[a:b], F64)
        for t in range(T):
            js = np.arange(t * chunk, min(N, (t + 1) * chunk))
            tile = scale * (qi @ kbar[js].T)
            shat_t = tile.mean(axis=0)
            sel[i, js] = shat_t.astype(np.float32) >= np.float32(tau[i])
    return sel


# --------------------------------------------------------------------------
# Steps 3-4: attention with exact selected blocks and zeroth-order
# approximations of unselected blocks (Eqs. 8-10)
# --------------------------------------------------------------------------

def forward_block(q: np.ndarray, k: np.ndarray, v: np.ndarray, kbar: np.ndarray,
                  vhat: np.ndarray, sel_row: np.ndarray, i: int, block: int, scale: float,
                  exact_only: bool = False, first_order: bool = False) -> np.ndarray:
    """Output rows of query block i, O_i = N_i / D_i row by row (Eqs. 9-10).

    For a query token r of block i:
      exact terms, every key c of every selected block j in S_i:
          weight exp(scale * q_r . k_c), value v_c;
      zeroth-order terms, every unselected block j in U_i:
          the block's exponential score row is replaced by exp(centre) broadcast
          over its keys, with centre = the row-wise mean score within the block
          = scale * q_r . Kbar_j; summed over the block's n_j keys this gives
          n_j * exp(centre) in the denominator and exp(centre) * Vhat_j in the
          numerator.
    Readings: a selected block is exact only, an unselected block is
    approximate only; the ragged last block weighs n_j.  exact_only drops the
    approximate terms (plain keep-or-drop sparse attention, the page's
    exact-only comparison); a row with nothing selected then outputs 0.
    first_order keeps the next term of the same expansion for every
    unselected block (see first_order_terms); it needs the zeroth-order term
    and is refused together with exact_only.
    """
    if exact_only and first_order:
        raise ValueError("the first-order term extends the zeroth-order approximation; "
                         "it has no meaning in exact-only mode")
    L, d = q.shape
    nj = block_sizes(L, block).astype(F64)
    a, b = block_range(L, block, i)
    qi = np.asarray(q[a:b], F64)
    S = np.flatnonzero(sel_row)
    U = np.flatnonzero(~np.asarray(sel_row, bool))
    if exact_only:
        U = U[:0]
    keys = np.concatenate([np.arange(*block_range(L, block, j)) for j in S]) \
        if len(S) else np.zeros(0, np.int64)
    ex = scale * (qi @ np.asarray(k[keys], F64).T)          # n_i x |keys|
    ap = scale * (qi @ kbar[U].T)                           # n_i x |U|
    if ex.shape[1] + ap.shape[1] == 0:
        # Reading: exact-only with nothing selected attends to nothing; output 0.
        return np.zeros((b - a, d), F64)
    M = np.concatenate([ex, ap], axis=1).max(axis=1, keepdims=True)
    pe = np.exp(ex - M)
    pa = np.exp(ap - M)
    D = pe.sum(axis=1) + (pa * nj[U][None, :]).sum(axis=1)
    Num = pe @ np.asarray(v[keys], F64) + pa @ vhat[U]
    if first_order:
        for u, j in enumerate(U):
            ka, kb = block_range(L, block, j)
            num1, den1 = first_order_terms(qi, k[ka:kb], v[ka:kb], ap[:, u], M[:, 0], scale)
            Num += num1
            D += den1
    return Num / D[:, None]


def first_order_terms(qi: np.ndarray, kj: np.ndarray, vj: np.ndarray, centre: np.ndarray,
                      ref_max: np.ndarray, scale: float):
    """First-order terms of one unselected block j for the query rows qi.

    The page expands the block's exponential score matrix exp(S_ij), with
    S_ij = scale * q_r . k_t (rows r of block i, keys t of block j), around
    the row-wise mean score c_r = scale * q_r . Kbar_j broadcast along the
    keys: exp(S_ij) = exp(c) (1 + (S_ij - c) + ...), element-wise.  The
    zeroth-order term is what forward_block already adds.  The first-order
    term is exp(c_r) (S_rt - c_r); entering the numerator with the keys'
    values and the denominator with weight 1 per key, it gives, relative to
    the reference max ref_max_r,
        numerator   exp(c_r - ref_max_r) * sum_t (S_rt - c_r) v_t
        denominator exp(c_r - ref_max_r) * sum_t (S_rt - c_r)
    The denominator term is zero up to rounding, because c_r is the mean of
    S_rt over the block's keys; it is computed here all the same, from the
    definition, and the tests check that it vanishes.
    Returns (numerator terms n_i x d, denominator terms n_i).
    """
    S = scale * (np.asarray(qi, F64) @ np.asarray(kj, F64).T)   # n_i x n_j
    x = S - centre[:, None]
    w = np.exp(centre - ref_max)
    return w[:, None] * (x @ np.asarray(vj, F64)), w * x.sum(axis=1)


def kv_moments(k: np.ndarray, v: np.ndarray, block: int) -> np.ndarray:
    """Per-block key-value moments of the first-order term, N x d x d:
    C_j = sum over block j's valid tokens t of (k_t - Kbar_j) v_t^T, i.e. n_j
    times the block's key-value cross-covariance.  With it the first-order
    numerator term of first_order_terms is exp(c_r - ref_max_r) * scale *
    q_r^T C_j, with no pass over the block's keys; the kernels use this form.
    """
    L, d = k.shape
    N = num_blocks(L, block)
    out = np.zeros((N, d, d), F64)
    for j in range(N):
        a, b = block_range(L, block, j)
        kj = np.asarray(k[a:b], F64)
        out[j] = (kj - kj.mean(axis=0)).T @ np.asarray(v[a:b], F64)
    return out


def forward(q: np.ndarray, k: np.ndarray, v: np.ndarray, sel: np.ndarray,
            block: int, scale: float, exact_only: bool = False,
            first_order: bool = False) -> np.ndarray:
    """Output of every query block for a given selection (see forward_block)."""
    L, d = q.shape
    N = num_blocks(L, block)
    _, kbar, vhat = pool(q, k, v, block)
    out = np.zeros((L, d), F64)
    for i in range(N):
        a, b = block_range(L, block, i)
        out[a:b] = forward_block(q, k, v, kbar, vhat, sel[i], i, block, scale, exact_only,
                                 first_order)
    return out


def forward_streaming(q: np.ndarray, k: np.ndarray, v: np.ndarray, tau: np.ndarray,
                      block: int, chunk: int, scale: float):
    """The nested loop of Algorithm 3.2 with one online-softmax state per row.

    Outer loop over chunks of pooled keys: the token-to-block tile gives both
    the chunk's routing scores (column means) and, for unselected columns, the
    approximate logits; inner loop over the chunk's selected blocks: exact
    attention.  Both paths update the same running max, denominator and
    accumulator.  Returns (output, selection).
    """
    L, d = q.shape
    N = num_blocks(L, block)
    _, kbar, vhat = pool(q, k, v, block)
    nj = block_sizes(L, block).astype(F64)
    T = (N + chunk - 1) // chunk
    out = np.zeros((L, d), F64)
    sel = np.zeros((N, N), dtype=bool)
    for i in range(N):
        a, b = block_range(L, block, i)
        qi = np.asarray(q[a:b], F64)
        m = np.full(b - a, -np.inf)
        den = np.zeros(b - a)
        acc = np.zeros((b - a, d))

        def update(logits, weights, values):
            nonlocal m, den, acc
            if logits.shape[1] == 0:
                return
            m_new = np.maximum(m, logits.max(axis=1))
            alpha = np.exp(m - m_new)
            p = np.exp(logits - m_new[:, None])
            den = den * alpha + (p * weights[None, :]).sum(axis=1)
            acc = acc * alpha[:, None] + p @ values
            m = m_new

        for t in range(T):
            js = np.arange(t * chunk, min(N, (t + 1) * chunk))
            tile = scale * (qi @ kbar[js].T)
            chosen = tile.mean(axis=0).astype(np.float32) >= np.float32(tau[i])
            sel[i, js] = chosen
            u = ~chosen
            update(tile[:, u], nj[js[u]], vhat[js[u]])
            for j in js[chosen]:
                ka, kb = block_range(L, block, j)
                ex = scale * (qi @ np.asarray(k[ka:kb], F64).T)
                update(ex, np.ones(kb - ka), np.asarray(v[ka:kb], F64))
        out[a:b] = acc / den[:, None]
    return out, sel


def dense(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> np.ndarray:
    """Textbook softmax attention softmax(scale * Q K^T) V (one head)."""
    logits = scale * (np.asarray(q, F64) @ np.asarray(k, F64).T)
    logits -= logits.max(axis=1, keepdims=True)
    p = np.exp(logits)
    return (p @ np.asarray(v, F64)) / p.sum(axis=1, keepdims=True)


# --------------------------------------------------------------------------
# Whole pass on one head
# --------------------------------------------------------------------------

def default_scale(d: int) -> float:
    return 1.0 / math.sqrt(d)


class HeadResult:
    """Everything the oracle computes for one (batch, head)."""

    def __init__(self, **kw):
        self.__dict__.update(kw)


def solattn_head(q: np.ndarray, k: np.ndarray, v: np.ndarray, beta: float, block: int,
                 scale: Optional[float] = None, sel: Optional[np.ndarray] = None,
                 exact_only: bool = False, rows: Optional[np.ndarray] = None,
                 first_order: bool = False) -> HeadResult:
    """Pool, moments, thresholds, selection and output for one head.

    sel, if given, forces the selection (used to compare outputs when a GPU
    decision fell inside the tie band).  rows, if given, limits the output to
    those query blocks (for sampling very long sequences); other rows are NaN.
    """
    L, d = q.shape
    if scale is None:
        scale = default_scale(d)
    qbar, kbar, vhat = pool(q, k, v, block)
    m, cov = key_moments(kbar)
    mu, sigma = row_stats(qbar, m, cov, scale)
    tau = thresholds(mu, sigma, beta)
    shat = proxy_scores(qbar, kbar, scale)
    free_sel = select(shat, tau)
    use = free_sel if sel is None else np.asarray(sel, bool)
    if rows is None:
        out = forward(q, k, v, use, block, scale, exact_only, first_order)
    else:
        out = np.full((L, d), np.nan)
        for i in rows:
            a, b = block_range(L, block, int(i))
            out[a:b] = forward_block(q, k, v, kbar, vhat, use[int(i)], int(i), block, scale,
                                     exact_only, first_order)
    return HeadResult(qbar=qbar, kbar=kbar, vhat=vhat, m=m, cov=cov, mu=mu, sigma=sigma,
                      tau=tau, shat=shat, sel=free_sel, used_sel=use, out=out, scale=scale)


def executed_flops(L: int, d: int, block: int, sel: np.ndarray, exact_only: bool = False,
                   first_order: bool = False) -> float:
    """Algorithmic FLOPs of the fused pass on one head for a given selection.

    Per query block i: 4 n_i n_j d for each selected block (Q K^T and P V),
    2 n_i d N for the token-to-block score tile, 2 n_i d |U_i| for the
    approximate P Vhat product.  Valid tokens only.  With first_order, also
    2 n_i d^2 |U_i| for the products q_r^T C_j and 2 L d^2 for the moments
    C_j themselves.
    """
    nj = block_sizes(L, block).astype(F64)
    N = len(nj)
    s = np.asarray(sel, bool)
    exact = 4.0 * d * (nj[:, None] * nj[None, :] * s).sum()
    tile = 2.0 * d * nj.sum() * N
    approx = 0.0 if exact_only else 2.0 * d * (nj * (~s).sum(axis=1)).sum()
    first = 0.0
    if first_order:
        first = 2.0 * d * d * (nj * (~s).sum(axis=1)).sum() + 2.0 * d * d * L
    return float(exact + tile + approx + first)
