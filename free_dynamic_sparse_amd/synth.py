"""Seeded synthetic inputs for the Sol-Attn forward pass.

This module draws Q, K, V and nothing else: it holds none of the method's
arithmetic, so both the HIP path and the CPU oracle can take their inputs
from it without sharing any computation.

The pages evaluate on trained video/image DiTs (Wan2.1-14B, HunyuanVideo-13B,
...) whose weights and prompts are not available; these generators stand in
for those models' attention inputs at the same attention shapes.  Recipe:

* tokens are laid out on a (t, y, x) grid flattened row-major (x fastest);
* positional structure comes from F = 64 random Fourier features
  f_k(p) = sqrt(2) * sin(omega_k . p + phi_k), phi_k ~ U[0, 2pi),
  omega_k,a ~ N(0, 1/ell_a^2) with ell = 8 along y and x and ell = 2 along t,
  so that E[f(p).f(p')]/F ~= exp(-sum_a (p_a - p'_a)^2 / (2 ell_a^2)) and
  nearby blocks score higher;
* per head a projection W [d, F] with N(0, 1/F) entries;
* Q = 0.5 * eps_Q + alpha * f(p) W^T and K = 0.5 * eps_K + alpha * f(p) W^T
  (same W and f, independent eps ~ N(0, 1)); V ~ N(0, 1) iid;
* "iid" heads draw Q, K, V ~ N(0, 1) iid;
* everything is drawn in float32 from numpy's PCG64, seeded per
  (workload seed, stream, batch, head) so any head can be regenerated alone,
  then rounded to bfloat16 with round-to-nearest-even.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional, Tuple

import numpy as np

FEATURES = 64
_STREAM_FEATURES = 0xFEA7
_STREAM_W = 1
_STREAM_Q = 2
_STREAM_K = 3
_STREAM_V = 4


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic attention problem: shapes, routing parameters and recipe."""

    name: str
    B: int
    H: int
    L: int
    d: int
    block: int
    chunk: int
    seed: int
    kind: str = "iid"  # "iid", "pos" or "mixed" (first half of heads pos, second half iid)
    grid: Optional[Tuple[int, int, int]] = None  # (t, y, x) with t*y*x == L
    alpha: float = 1.0  # positional weight of "pos" heads
    mixed_alpha: float = 4.0  # positional weight of the peaked heads of a "mixed" workload
    betas: Tuple[float, ...] = (1.0,)

    @property
    def N(self) -> int:
        return -(-self.L // self.block)

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five attention shapes the method is exercised on.
WORKLOADS = {
    # B1 H1 L4096 d64, iid N(0,1): small enough for the oracle to run whole.
    "tiny": Workload("tiny", B=1, H=1, L=4096, d=64, block=64, chunk=16, seed=0,
                     kind="iid", betas=(1.0, -math.inf)),
    # Image DiT: 64x64 latent grid.
    "image": Workload("image", B=1, H=24, L=4096, d=128, block=128, chunk=16, seed=1,
                      kind="pos", grid=(1, 64, 64), betas=(0.5, 1.0, 1.5)),
    # Wan2.1-14B attention: 21x45x80 latent grid, 40 heads; the last block holds 80 tokens.
    "wan": Workload("wan", B=1, H=40, L=75600, d=128, block=128, chunk=32, seed=2,
                    kind="pos", grid=(21, 45, 80), betas=(0.5, 1.0, 1.5)),
    # HunyuanVideo-13B attention: 33x45x80 grid, 24 heads; the last block holds 16 tokens.
    "hunyuan": Workload("hunyuan", B=1, H=24, L=118800, d=128, block=128, chunk=32, seed=3,
                        kind="pos", grid=(33, 45, 80), betas=(1.0,)),
    # Load-imbalance stress: 64^3 grid, 8 heads; heads 0-3 peaked (alpha 4), 4-7 flat iid.
    "stress": Workload("stress", B=1, H=8, L=262144, d=128, block=128, chunk=32, seed=4,
                       kind="mixed", grid=(64, 64, 64),
                       betas=(-math.inf, 0.0, 1.0, 2.0, 3.0)),
}


# Sequence-length sweep (speedup over dense attention across length and
# sparsity): L tokens on an (L / 4096) x 64 x 64 latent grid, 8 heads.
SEQ_LENGTHS = (16384, 32768, 65536, 131072)


def seq_workload(L: int, H: int = 8) -> Workload:
    """Video-like sweep shape: L tokens on a (L / 4096, 64, 64) grid, d = 128."""
    if L <= 0 or L % 4096:
        raise ValueError("sweep lengths are whole 64x64 frames")
    return Workload(f"seq{L // 1024}k", B=1, H=H, L=L, d=128, block=128, chunk=32, seed=5,
                    kind="pos", grid=(L // 4096, 64, 64), betas=(0.5, 1.0, 1.5, 2.0))


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(x) for x in key])))


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that are already bfloat16-representable."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return (u >> np.uint32(16)).astype(np.uint16)


def bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Inverse of bf16_bits: widen bfloat16 bit patterns to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _grid(w: Workload) -> Tuple[int, int, int]:
    if w.grid is not None:
        t, y, x = w.grid
        if t * y * x != w.L:
            raise ValueError(f"grid {w.grid} does not hold L={w.L} tokens")
        return w.grid
    return (1, 1, w.L)


def positional_features(w: Workload) -> np.ndarray:
    """Random Fourier features f(p) for every token, float32 [L, F]."""
    gt, gy, gx = _grid(w)
    rng = _rng(w.seed, _STREAM_FEATURES)
    ell = np.array([2.0, 8.0, 8.0])
    omega = rng.standard_normal((FEATURES, 3)) / ell[None, :]
    phi = rng.uniform(0.0, 2.0 * math.pi, FEATURES)
    t, y, x = np.meshgrid(np.arange(gt), np.arange(gy), np.arange(gx), indexing="ij")
    pos = np.stack([t.ravel(), y.ravel(), x.ravel()], axis=1).astype(np.float64)
    return (math.sqrt(2.0) * np.sin(pos @ omega.T + phi[None, :])).astype(np.float32)


def head_kind(w: Workload, h: int) -> Tuple[str, float]:
    if w.kind == "mixed":
        return ("pos", w.mixed_alpha) if h < w.H // 2 else ("iid", 0.0)
    return (w.kind, w.alpha)


def make_head(w: Workload, b: int, h: int, feats: Optional[np.ndarray] = None,
              bf16: bool = True) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Q, K, V of one (batch, head), float32 [L, d] (bf16-representable if bf16)."""
    kind, alpha = head_kind(w, h)
    q = _rng(w.seed, _STREAM_Q, b, h).standard_normal((w.L, w.d), dtype=np.float32)
    k = _rng(w.seed, _STREAM_K, b, h).standard_normal((w.L, w.d), dtype=np.float32)
    v = _rng(w.seed, _STREAM_V, b, h).standard_normal((w.L, w.d), dtype=np.float32)
    if kind == "pos":
        if feats is None:
            feats = positional_features(w)
        wmat = (_rng(w.seed, _STREAM_W, h).standard_normal((w.d, FEATURES))
                / math.sqrt(FEATURES)).astype(np.float32)
        posterm = np.float32(alpha) * (feats @ wmat.T)
        q = np.float32(0.5) * q + posterm
        k = np.float32(0.5) * k + posterm
    if bf16:
        q, k, v = round_bf16(q), round_bf16(k), round_bf16(v)
    return q, k, v


def make_inputs(w: Workload, bf16: bool = True,
                heads: Optional[Tuple[int, ...]] = None) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Q, K, V float32 [B, H', L, d] for all heads (or the listed subset)."""
    hs = tuple(range(w.H)) if heads is None else tuple(heads)
    feats = positional_features(w) if w.kind in ("pos", "mixed") else None
    shape = (w.B, len(hs), w.L, w.d)
    q = np.empty(shape, np.float32)
    k = np.empty(shape, np.float32)
    v = np.empty(shape, np.float32)
    for b in range(w.B):
        for n, h in enumerate(hs):
            q[b, n], k[b, n], v[b, n] = make_head(w, b, h, feats, bf16)
    return q, k, v


def make_inputs_bf16_bits(w: Workload) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Q, K, V as bfloat16 bit patterns, uint16 [B, H, L, d]; built head by head."""
    feats = positional_features(w) if w.kind in ("pos", "mixed") else None
    shape = (w.B, w.H, w.L, w.d)
    out = [np.empty(shape, np.uint16) for _ in range(3)]
    for b in range(w.B):
        for h in range(w.H):
            for arr, x in zip(out, make_head(w, b, h, feats, bf16=True)):
                arr[b, h] = bf16_bits(x)
    return out[0], out[1], out[2]
