"""Python binding of libsolattn.so (argument marshalling only).

Each function below has the name of the C entry point it calls and takes
torch tensors for the device buffers; every step of the computation runs in
the HIP kernels behind the C ABI.  torch supplies device memory and the
current stream.  There is no fallback: if the library is missing the import
of this module fails.
"""

from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "_lib", "libsolattn.so")

SOLATTN_OK = 0
SOLATTN_E_INVALID_ARG = -1
SOLATTN_E_UNSUPPORTED = -2
SOLATTN_E_HIP = -3
SOLATTN_E_WORKSPACE = -4
SOLATTN_FLAG_EXACT_ONLY = 1

EXPORTS = ("solattn_pool", "solattn_moments", "solattn_fwd", "solattn_fwd_workspace_bytes",
           "solattn_fwd_noalloc", "solattn_fwd_masked", "solattn_dense_fwd",
           "solattn_proxy_map", "solattn_select_topk", "solattn_select_topp",
           "solattn_kv_moments", "solattn_fwd_first_order", "solattn_fwd_first_order_workspace",
           "solattn_strerror", "solattn_version")


class Problem(ctypes.Structure):
    """Mirror of solattn_problem_t."""

    _fields_ = [
        ("batch", ctypes.c_int64),
        ("heads", ctypes.c_int64),
        ("seq_len", ctypes.c_int64),
        ("head_dim", ctypes.c_int64),
        ("block", ctypes.c_int32),
        ("chunk", ctypes.c_int32),
        ("beta", ctypes.c_float),
        ("scale", ctypes.c_float),
        ("flags", ctypes.c_uint32),
        ("reserved", ctypes.c_uint32),
    ]


def load_library(path: str = _LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m free_dynamic_sparse_amd.build`")
    lib = ctypes.CDLL(path)
    vp = ctypes.c_void_p
    pp = ctypes.POINTER(Problem)
    lib.solattn_pool.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp]
    lib.solattn_moments.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.solattn_fwd.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp, vp,
                                vp]
    lib.solattn_fwd_noalloc.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.solattn_fwd_workspace_bytes.argtypes = [pp]
    lib.solattn_fwd_workspace_bytes.restype = ctypes.c_size_t
    lib.solattn_dense_fwd.argtypes = [pp, vp, vp, vp, vp, vp]
    lib.solattn_fwd_masked.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.solattn_proxy_map.argtypes = [pp, vp, vp, vp, vp]
    lib.solattn_select_topk.argtypes = [pp, vp, ctypes.c_int64, vp, vp, vp]
    lib.solattn_select_topp.argtypes = [pp, vp, ctypes.c_float, vp, vp, vp]
    lib.solattn_kv_moments.argtypes = [pp, vp, vp, vp, vp, vp, vp]
    lib.solattn_fwd_first_order_workspace.argtypes = [pp]
    lib.solattn_fwd_first_order_workspace.restype = ctypes.c_size_t
    lib.solattn_fwd_first_order.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                            ctypes.c_size_t, vp]
    for name in ("solattn_pool", "solattn_moments", "solattn_fwd", "solattn_fwd_noalloc",
                 "solattn_fwd_masked",
                 "solattn_dense_fwd", "solattn_proxy_map", "solattn_select_topk", "solattn_select_topp",
                 "solattn_kv_moments", "solattn_fwd_first_order"):
        getattr(lib, name).restype = ctypes.c_int
    lib.solattn_strerror.argtypes = [ctypes.c_int]
    lib.solattn_strerror.restype = ctypes.c_char_p
    lib.solattn_version.argtypes = []
    lib.solattn_version.restype = ctypes.c_int
    return lib


LIB = load_library()


class SolAttnError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {LIB.solattn_strerror(code).decode()} (code {code})")


def problem(B: int, H: int, L: int, d: int, block: int = 128, chunk: int = 32,
            beta: float = 1.0, scale: Optional[float] = None, exact_only: bool = False) -> Problem:
    return Problem(B, H, L, d, block, chunk, beta, 0.0 if scale is None else scale,
                   SOLATTN_FLAG_EXACT_ONLY if exact_only else 0, 0)


def num_blocks(L: int, block: int) -> int:
    return (L + block - 1) // block


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(rc: int, where: str) -> None:
    if rc != SOLATTN_OK:
        raise SolAttnError(rc, where)


def _need(t: torch.Tensor, dtype, shape, name: str) -> None:
    if t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous() or not t.is_cuda:
        raise ValueError(f"{name}: expected contiguous {dtype} CUDA tensor of shape {tuple(shape)}, "
                         f"got {t.dtype} {tuple(t.shape)} contiguous={t.is_contiguous()} "
                         f"cuda={t.is_cuda}")


def _dims(p: Problem):
    N = num_blocks(p.seq_len, p.block)
    return (p.batch, p.heads, p.seq_len, p.head_dim), (p.batch, p.heads, N, p.head_dim), N


def solattn_pool(p: Problem, q, k, v, qbar, kbar, vhat, stream=None) -> None:
    full, pooled, _ = _dims(p)
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, torch.bfloat16, full, n)
    for t, n in ((qbar, "qbar"), (kbar, "kbar"), (vhat, "vhat")):
        _need(t, torch.float32, pooled, n)
    _check(LIB.solattn_pool(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(qbar), _ptr(kbar),
                            _ptr(vhat), _stream(stream)), "solattn_pool")


def solattn_moments(p: Problem, qbar, kbar, kmean, kcov, tau, mu=None, sigma=None,
                    stream=None) -> None:
    _, pooled, N = _dims(p)
    B, H, d = p.batch, p.heads, p.head_dim
    _need(qbar, torch.float32, pooled, "qbar")
    _need(kbar, torch.float32, pooled, "kbar")
    _need(kmean, torch.float32, (B, H, d), "kmean")
    _need(kcov, torch.float32, (B, H, d, d), "kcov")
    _need(tau, torch.float32, (B, H, N), "tau")
    for t, n in ((mu, "mu"), (sigma, "sigma")):
        if t is not None:
            _need(t, torch.float32, (B, H, N), n)
    _check(LIB.solattn_moments(ctypes.byref(p), _ptr(qbar), _ptr(kbar), _ptr(kmean), _ptr(kcov),
                               _ptr(tau), _ptr(mu), _ptr(sigma), _stream(stream)),
           "solattn_moments")


def _need_workspace(ws, name: str = "workspace") -> None:
    if ws.dtype != torch.uint8 or ws.dim() != 1 or not ws.is_cuda or not ws.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous 1-D uint8 CUDA tensor")


def solattn_fwd_workspace_bytes(p: Problem) -> int:
    return int(LIB.solattn_fwd_workspace_bytes(ctypes.byref(p)))


def solattn_fwd(p: Problem, q, k, v, qbar, kbar, vhat, tau, out, workspace, sel_mask=None,
                sel_count=None, stream=None) -> None:
    """workspace: a contiguous uint8 CUDA tensor of at least
    solattn_fwd_workspace_bytes(p) bytes (the work-queue counters)."""
    full, pooled, N = _dims(p)
    _need_workspace(workspace)
    B, H = p.batch, p.heads
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (out, "out")):
        _need(t, torch.bfloat16, full, n)
    for t, n in ((qbar, "qbar"), (kbar, "kbar"), (vhat, "vhat")):
        _need(t, torch.float32, pooled, n)
    _need(tau, torch.float32, (B, H, N), "tau")
    if sel_mask is not None:
        _need(sel_mask, torch.int64, (B, H, N, (N + 63) // 64), "sel_mask")
    if sel_count is not None:
        _need(sel_count, torch.int32, (B, H, N), "sel_count")
    _check(LIB.solattn_fwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(qbar), _ptr(kbar),
                           _ptr(vhat), _ptr(tau), _ptr(out), _ptr(workspace), workspace.numel(),
                           _ptr(sel_mask), _ptr(sel_count), _stream(stream)), "solattn_fwd")


def solattn_fwd_noalloc(p: Problem, q, k, v, qbar, kbar, vhat, tau, out, sel_mask=None,
                        sel_count=None, stream=None) -> None:
    """solattn_fwd with the library's own per-device scratch array instead of
    a workspace (no allocation in the call; overlapping calls on one GPU race)."""
    full, pooled, N = _dims(p)
    B, H = p.batch, p.heads
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (out, "out")):
        _need(t, torch.bfloat16, full, n)
    for t, n in ((qbar, "qbar"), (kbar, "kbar"), (vhat, "vhat")):
        _need(t, torch.float32, pooled, n)
    _need(tau, torch.float32, (B, H, N), "tau")
    if sel_mask is not None:
        _need(sel_mask, torch.int64, (B, H, N, (N + 63) // 64), "sel_mask")
    if sel_count is not None:
        _need(sel_count, torch.int32, (B, H, N), "sel_count")
    _check(LIB.solattn_fwd_noalloc(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(qbar),
                                   _ptr(kbar), _ptr(vhat), _ptr(tau), _ptr(out), _ptr(sel_mask),
                                   _ptr(sel_count), _stream(stream)), "solattn_fwd_noalloc")


def solattn_fwd_masked(p: Problem, q, k, v, kbar, vhat, sel_in, out, workspace,
                       stream=None) -> None:
    full, pooled, N = _dims(p)
    _need_workspace(workspace)
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (out, "out")):
        _need(t, torch.bfloat16, full, n)
    for t, n in ((kbar, "kbar"), (vhat, "vhat")):
        _need(t, torch.float32, pooled, n)
    _need(sel_in, torch.int64, (p.batch, p.heads, N, (N + 63) // 64), "sel_in")
    _check(LIB.solattn_fwd_masked(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(kbar),
                                  _ptr(vhat), _ptr(sel_in), _ptr(out), _ptr(workspace),
                                  workspace.numel(), _stream(stream)), "solattn_fwd_masked")


def solattn_kv_moments(p: Problem, k, v, kbar, vhat, kvc, stream=None) -> None:
    full, pooled, N = _dims(p)
    _need(k, torch.bfloat16, full, "k")
    _need(v, torch.bfloat16, full, "v")
    _need(kbar, torch.float32, pooled, "kbar")
    _need(vhat, torch.float32, pooled, "vhat")
    _need(kvc, torch.bfloat16, (p.batch, p.heads, N, p.head_dim, p.head_dim), "kvc")
    _check(LIB.solattn_kv_moments(ctypes.byref(p), _ptr(k), _ptr(v), _ptr(kbar), _ptr(vhat),
                                  _ptr(kvc), _stream(stream)), "solattn_kv_moments")


def solattn_fwd_first_order_workspace(p: Problem) -> int:
    return int(LIB.solattn_fwd_first_order_workspace(ctypes.byref(p)))


def solattn_fwd_first_order(p: Problem, q, k, v, qbar, kbar, vhat, kvc, tau, out, workspace,
                            stream=None) -> None:
    """workspace: a contiguous uint8 CUDA tensor of at least
    solattn_fwd_first_order_workspace(p) bytes."""
    full, pooled, N = _dims(p)
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (out, "out")):
        _need(t, torch.bfloat16, full, n)
    for t, n in ((qbar, "qbar"), (kbar, "kbar"), (vhat, "vhat")):
        _need(t, torch.float32, pooled, n)
    _need(kvc, torch.bfloat16, (p.batch, p.heads, N, p.head_dim, p.head_dim), "kvc")
    _need(tau, torch.float32, (p.batch, p.heads, N), "tau")
    _need_workspace(workspace)
    _check(LIB.solattn_fwd_first_order(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(qbar),
                                       _ptr(kbar), _ptr(vhat), _ptr(kvc), _ptr(tau), _ptr(out),
                                       _ptr(workspace), workspace.numel(), _stream(stream)),
           "solattn_fwd_first_order")


def solattn_dense_fwd(p: Problem, q, k, v, out, stream=None) -> None:
    full, _, _ = _dims(p)
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (out, "out")):
        _need(t, torch.bfloat16, full, n)
    _check(LIB.solattn_dense_fwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(out),
                                 _stream(stream)), "solattn_dense_fwd")


def solattn_proxy_map(p: Problem, qbar, kbar, shat, stream=None) -> None:
    _, pooled, N = _dims(p)
    _need(qbar, torch.float32, pooled, "qbar")
    _need(kbar, torch.float32, pooled, "kbar")
    _need(shat, torch.float32, (p.batch, p.heads, N, N), "shat")
    _check(LIB.solattn_proxy_map(ctypes.byref(p), _ptr(qbar), _ptr(kbar), _ptr(shat),
                                 _stream(stream)), "solattn_proxy_map")


def _select_outputs(p: Problem, shat, sel_mask, sel_count):
    N = num_blocks(p.seq_len, p.block)
    _need(shat, torch.float32, (p.batch, p.heads, N, N), "shat")
    _need(sel_mask, torch.int64, (p.batch, p.heads, N, (N + 63) // 64), "sel_mask")
    if sel_count is not None:
        _need(sel_count, torch.int32, (p.batch, p.heads, N), "sel_count")


def solattn_select_topk(p: Problem, shat, k: int, sel_mask, sel_count=None, stream=None) -> None:
    _select_outputs(p, shat, sel_mask, sel_count)
    _check(LIB.solattn_select_topk(ctypes.byref(p), _ptr(shat), int(k), _ptr(sel_mask),
                                   _ptr(sel_count), _stream(stream)), "solattn_select_topk")


def solattn_select_topp(p: Problem, shat, top_p: float, sel_mask, sel_count=None,
                        stream=None) -> None:
    _select_outputs(p, shat, sel_mask, sel_count)
    _check(LIB.solattn_select_topp(ctypes.byref(p), _ptr(shat), float(top_p), _ptr(sel_mask),
                                   _ptr(sel_count), _stream(stream)), "solattn_select_topp")


class Workspace:
    """Device buffers for one problem shape (torch allocations)."""

    def __init__(self, p: Problem, device="cuda", debug: bool = False):
        B, H, L, d = p.batch, p.heads, p.seq_len, p.head_dim
        N = num_blocks(L, p.block)
        f32 = dict(dtype=torch.float32, device=device)
        self.qbar = torch.empty((B, H, N, d), **f32)
        self.kbar = torch.empty((B, H, N, d), **f32)
        self.vhat = torch.empty((B, H, N, d), **f32)
        self.kmean = torch.empty((B, H, d), **f32)
        self.kcov = torch.empty((B, H, d, d), **f32)
        self.tau = torch.empty((B, H, N), **f32)
        self.mu = torch.empty((B, H, N), **f32) if debug else None
        self.sigma = torch.empty((B, H, N), **f32) if debug else None
        self.sel_mask = (torch.empty((B, H, N, (N + 63) // 64), dtype=torch.int64, device=device)
                         if debug else None)
        self.sel_count = torch.empty((B, H, N), dtype=torch.int32, device=device) if debug else None
        # the fused kernel's work-queue counters
        self.queue = torch.empty(max(1, solattn_fwd_workspace_bytes(p)), dtype=torch.uint8,
                                 device=device)


def forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, beta: float = 1.0,
            block: int = 128, chunk: int = 32, scale: Optional[float] = None,
            exact_only: bool = False, out: Optional[torch.Tensor] = None,
            ws: Optional[Workspace] = None, stream=None) -> torch.Tensor:
    """The whole Sol-Attn forward: pool, moments/thresholds, fused kernel."""
    B, H, L, d = q.shape
    p = problem(B, H, L, d, block, chunk, beta, scale, exact_only)
    if ws is None:
        ws = Workspace(p, q.device)
    if out is None:
        out = torch.empty_like(q)
    solattn_pool(p, q, k, v, ws.qbar, ws.kbar, ws.vhat, stream)
    solattn_moments(p, ws.qbar, ws.kbar, ws.kmean, ws.kcov, ws.tau, ws.mu, ws.sigma, stream)
    solattn_fwd(p, q, k, v, ws.qbar, ws.kbar, ws.vhat, ws.tau, out, ws.queue, ws.sel_mask,
                ws.sel_count, stream)
    return out


class FirstOrderWorkspace:
    """Device buffers of the first-order forward for one problem shape: the
    block moments C_j and the scratch passed between its two kernels."""

    def __init__(self, p: Problem, device="cuda"):
        N = num_blocks(p.seq_len, p.block)
        self.kvc = torch.empty((p.batch, p.heads, N, p.head_dim, p.head_dim),
                               dtype=torch.bfloat16, device=device)
        self.scratch = torch.empty(max(1, solattn_fwd_first_order_workspace(p)),
                                   dtype=torch.uint8, device=device)


def forward_first_order(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, beta: float = 1.0,
                        block: int = 128, chunk: int = 32, scale: Optional[float] = None,
                        out: Optional[torch.Tensor] = None, ws: Optional[Workspace] = None,
                        fws: Optional[FirstOrderWorkspace] = None, stream=None) -> torch.Tensor:
    """The forward with the first-order term of every unselected block:
    pool, moments/thresholds, block moments C_j, fused kernel, correction."""
    B, H, L, d = q.shape
    p = problem(B, H, L, d, block, chunk, beta, scale)
    if ws is None:
        ws = Workspace(p, q.device)
    if fws is None:
        fws = FirstOrderWorkspace(p, q.device)
    if out is None:
        out = torch.empty_like(q)
    solattn_pool(p, q, k, v, ws.qbar, ws.kbar, ws.vhat, stream)
    solattn_moments(p, ws.qbar, ws.kbar, ws.kmean, ws.kcov, ws.tau, ws.mu, ws.sigma, stream)
    solattn_kv_moments(p, k, v, ws.kbar, ws.vhat, fws.kvc, stream)
    solattn_fwd_first_order(p, q, k, v, ws.qbar, ws.kbar, ws.vhat, fws.kvc, ws.tau, out,
                            fws.scratch, stream)
    return out


def stats(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, beta: float = 1.0,
          block: int = 128, chunk: int = 32, scale: Optional[float] = None,
          exact_only: bool = False, stream=None) -> dict:
    """The forward with every routing statistic returned: a dict of the
    output `out` and the thresholds `tau`, row means `mu` and standard
    deviations `sigma` [B, H, N], the selection bitmaps `sel_mask`
    [B, H, N, ceil(N/64)] (int64 words) and counts `sel_count` [B, H, N]."""
    B, H, L, d = q.shape
    p = problem(B, H, L, d, block, chunk, beta, scale, exact_only)
    ws = Workspace(p, q.device, debug=True)
    out = forward(q, k, v, beta, block, chunk, scale, exact_only, ws=ws, stream=stream)
    return dict(out=out, tau=ws.tau, mu=ws.mu, sigma=ws.sigma, sel_mask=ws.sel_mask,
                sel_count=ws.sel_count)


def forward_masked(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, sel_mask: torch.Tensor,
                   block: int = 128, scale: Optional[float] = None, exact_only: bool = False,
                   out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """The forward with given selections (int64 bitmaps [B, H, N, ceil(N/64)]):
    pool, then the fused kernel without routing."""
    B, H, L, d = q.shape
    p = problem(B, H, L, d, block, 32, 1.0, scale, exact_only)
    ws = Workspace(p, q.device)
    if out is None:
        out = torch.empty_like(q)
    solattn_pool(p, q, k, v, ws.qbar, ws.kbar, ws.vhat, stream)
    solattn_fwd_masked(p, q, k, v, ws.kbar, ws.vhat, sel_mask, out, ws.queue, stream)
    return out


def bool_to_mask(sel: torch.Tensor) -> torch.Tensor:
    """Pack bool [..., N] into the u64 row bitmaps [..., ceil(N/64)] (CPU,
    as int64 words)."""
    sel = sel.cpu().bool()
    N = sel.shape[-1]
    W = (N + 63) // 64
    padded = torch.zeros(*sel.shape[:-1], W * 64, dtype=torch.int64)
    padded[..., :N] = sel.to(torch.int64)
    bits = padded.reshape(*sel.shape[:-1], W, 64) << torch.arange(64, dtype=torch.int64)
    return bits.sum(dim=-1)


def dense_forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, block: int = 128,
                  scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                  stream=None) -> torch.Tensor:
    B, H, L, d = q.shape
    p = problem(B, H, L, d, block, 32, -math.inf, scale)
    if out is None:
        out = torch.empty_like(q)
    solattn_dense_fwd(p, q, k, v, out, stream)
    return out


def mask_to_bool(sel_mask: torch.Tensor, N: int) -> torch.Tensor:
    """Unpack the u64 row bitmaps [..., ceil(N/64)] into bool [..., N] (CPU)."""
    words = sel_mask.cpu().contiguous()
    bits = torch.arange(64, dtype=torch.int64)
    unpacked = ((words.unsqueeze(-1) >> bits) & 1).bool()
    return unpacked.reshape(*words.shape[:-1], -1)[..., :N]
