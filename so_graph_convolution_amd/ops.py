"""PyTorch-facing calls of the C ABI (same names as the library's entry points).

Tensors supply device memory, the current HIP stream orders the work; every
step of the convolution runs in libso2conv.so. Shapes are checked here before
any pointer is handed to a kernel.
"""
from __future__ import annotations

import ctypes
import dataclasses

import torch

from ._binding import (SO2_ACT_GATE, SO2_ACT_SWIGLU_S2, SO2_DEBUG_CHECKS, SO2_F32_NATIVE, SO2_FUSED_GATE, Cfg,
                       GraphC, So2Error, check, lib)

__all__ = ["SO2Config", "Graph", "so2conv_generator_table", "so2conv_graph_prepare", "so2conv_fwd", "so2conv_fwd_noalloc", "so2conv_bwd",
           "so2conv_dbwd",
           "so2conv_debug_rotate_gather", "so2conv_workspace_bytes", "so2conv_saved_bytes",
           "so2conv_saved_bwd_bytes", "weight_shapes",
           "so2conv_profile_enable", "so2conv_profile_reset", "so2conv_profile_read",
           "so2conv_chunked_workspace_bytes", "so2conv_debug_status"]


_DTYPES = {"f32": (0, torch.float32), "bf16": (1, torch.bfloat16)}
_ACTS = {"gate": SO2_ACT_GATE, "swiglu_s2": SO2_ACT_SWIGLU_S2}


@dataclasses.dataclass(frozen=True)
class SO2Config:
    """dtype "f32": every array float32. dtype "bf16": node features, weights and
    their gradients bfloat16 (positions, shifts, rbf and their gradients stay
    float32); the per-order products run on bfloat16 matrix cores with float32
    accumulation. debug_checks: validate the inputs on the device before
    computing (the call synchronises and raises on bad inputs). heads: the
    per-edge message weights `env` are [E] (heads = 1: a cutoff envelope) or
    [E, heads] (attention weights per head of channels/heads channels).
    f32_native: float32 per-order products on the float32 matrix cores
    instead of the default exact bfloat16-piece products.
    act: the Edge -> Edge activation, "gate" or "swiglu_s2" (the spherical-grid
    SwiGLU; the first linear then has 2C output channels per retained row,
    value half first). grid: for "swiglu_s2", the tables (G, P): CUDA float32
    tensors G [n_grid, q] (the retained basis at the grid points, rows of U in
    degree-major order) and P [q, n_grid] (the projection back).
    fused_gate: the forward gate in the first linear's epilogue (bitwise the
    same results; measured slower on MI355X, so off by default)."""
    lmax: int
    mmax: int
    channels: int
    n_rbf: int
    dtype: str = "f32"
    debug_checks: bool = False
    heads: int = 1
    f32_native: bool = False
    act: str = "gate"
    grid: tuple | None = dataclasses.field(default=None, compare=False, repr=False)
    fused_gate: bool = False

    def __post_init__(self):
        if self.dtype not in _DTYPES:
            raise ValueError(f"dtype must be one of {sorted(_DTYPES)}")
        if self.act not in _ACTS:
            raise ValueError(f"act must be one of {sorted(_ACTS)}")
        if self.act == "swiglu_s2":
            if self.grid is None:
                raise ValueError('act="swiglu_s2" needs grid=(G, P)')
            G, P = self.grid
            _dev(G, "grid G")
            if G.dim() != 2 or G.shape[1] != self.q:
                raise ValueError(f"grid G must be [n_grid, {self.q}]")
            _dev(P, "grid P", shape=(self.q, G.shape[0]))

    @property
    def q(self) -> int:
        L, M = self.lmax, self.mmax
        return (L + 1) * (2 * M + 1) - M * (M + 1)

    @property
    def n_grid(self) -> int:
        return 0 if self.grid is None else int(self.grid[0].shape[0])

    def c(self) -> Cfg:
        flags = (SO2_DEBUG_CHECKS if self.debug_checks else 0) | (SO2_F32_NATIVE if self.f32_native else 0) | \
            (SO2_FUSED_GATE if self.fused_gate else 0)
        G, P = self.grid if self.grid is not None else (None, None)
        return Cfg(self.lmax, self.mmax, self.channels, self.n_rbf, _DTYPES[self.dtype][0], flags, self.heads,
                   _ACTS[self.act], self.n_grid, None if G is None else G.data_ptr(),
                   None if P is None else P.data_ptr())

    def env_shape(self, n_edges):
        return (n_edges,) if self.heads == 1 else (n_edges, self.heads)

    @property
    def torch_dtype(self):
        return _DTYPES[self.dtype][1]

    @property
    def d(self) -> int:
        return (self.lmax + 1) ** 2


def weight_shapes(cfg: SO2Config):
    L, M, C = cfg.lmax, cfg.mmax, cfg.channels
    if cfg.act == "swiglu_s2":   # value and gate halves per retained row
        w1 = [((L + 1) * 2 * C, (L + 1) * 2 * C)] + \
            [((L - m + 1) * 2 * C, 2 * (L - m + 1) * 2 * C) for m in range(1, M + 1)]
    else:
        w1 = [((L + 1) * 2 * C, (L + 1) * C + L * C)] + \
            [((L - m + 1) * 2 * C, 2 * (L - m + 1) * C) for m in range(1, M + 1)]
    w2 = [((L + 1) * C, (L + 1) * C)] + [((L - m + 1) * C, 2 * (L - m + 1) * C) for m in range(1, M + 1)]
    return w1, w2


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev(t, name, dtype=torch.float32, shape=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t


def _ptr_array(ts, name, shapes, dtype):
    if ts is None:
        return None, []
    ts = list(ts)
    if len(ts) != len(shapes):
        raise ValueError(f"{name} needs {len(shapes)} blocks")
    keep = [_dev(t, f"{name}[{i}]", dtype=dtype, shape=shapes[i]) for i, t in enumerate(ts)]
    arr = (ctypes.c_void_p * len(ts))(*[None if t is None else t.data_ptr() for t in keep])
    return ctypes.cast(arr, ctypes.c_void_p), [arr, keep]


def _ws(nbytes, device):
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


class Graph:
    """Edges j -> i (src, dst int32, dst non-decreasing) plus the CSR arrays
    built on the device by so2conv_graph_prepare."""

    def __init__(self, n_nodes, src, dst, shift=None, dst_ptr=None, src_perm=None, src_ptr=None):
        self.n_nodes = int(n_nodes)
        self.src = _dev(src, "src", torch.int32)
        self.dst = _dev(dst, "dst", torch.int32)
        self.n_edges = int(self.src.shape[0])
        self.shift = _dev(shift, "shift", shape=(self.n_edges, 3))
        self.dst_ptr, self.src_perm, self.src_ptr = dst_ptr, src_perm, src_ptr

    def c(self) -> GraphC:
        return GraphC(self.n_nodes, self.n_edges, self.src.data_ptr(), self.dst.data_ptr(),
                      None if self.shift is None else self.shift.data_ptr(), self.dst_ptr.data_ptr(),
                      self.src_perm.data_ptr(), self.src_ptr.data_ptr())


def so2conv_graph_prepare(n_nodes, src, dst, shift=None, validate=True) -> Graph:
    g = Graph(n_nodes, src, dst, shift)
    dev = g.src.device
    g.dst_ptr = torch.empty(g.n_nodes + 1, dtype=torch.int32, device=dev)
    g.src_ptr = torch.empty(g.n_nodes + 1, dtype=torch.int32, device=dev)
    g.src_perm = torch.empty(max(g.n_edges, 1), dtype=torch.int32, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    ws = _ws(lib().so2conv_graph_workspace_bytes(g.n_nodes, g.n_edges), dev)
    check(lib().so2conv_graph_prepare(g.n_nodes, g.n_edges, _p(g.src), _p(g.dst), _p(g.dst_ptr), _p(g.src_perm),
                                      _p(g.src_ptr), _p(err) if validate else None, _p(ws), ws.numel(), _stream()),
          "so2conv_graph_prepare")
    if validate:
        e = int(err.item())
        if e:
            raise ValueError(f"invalid graph (error bits {e}: 1 src range, 2 dst range, 4 dst not sorted)")
    return g


def so2conv_workspace_bytes(cfg: SO2Config, n_nodes, n_edges, stage) -> int:
    c = cfg.c()
    return int(lib().so2conv_workspace_bytes(ctypes.byref(c), n_nodes, n_edges, stage))


def so2conv_saved_bytes(cfg: SO2Config, n_edges) -> int:
    c = cfg.c()
    return int(lib().so2conv_saved_bytes(ctypes.byref(c), n_edges))


def so2conv_saved_bwd_bytes(cfg: SO2Config, n_edges) -> int:
    c = cfg.c()
    return int(lib().so2conv_saved_bwd_bytes(ctypes.byref(c), n_edges))


def so2conv_generator_table() -> torch.Tensor:
    """The so(3) generator table compiled into the library (host memory, no
    GPU): float32 [3, n] for k = x, y, z, degree l's (2l+1)^2 block
    row-major at offset sum_{l' < l} (2l'+1)^2."""
    n = int(lib().so2conv_generator_table(None, 0))
    out = torch.empty(n, dtype=torch.float32)
    got = lib().so2conv_generator_table(ctypes.c_void_p(out.data_ptr()), n)
    if got != n:
        raise So2Error(f"so2conv_generator_table failed ({got})")
    return out.view(3, n // 3)


def _saved_bwd(cfg, g, saved_bwd, device, allocate):
    """The backward's kept-cotangent buffer: allocated for saved_bwd=True when
    `allocate` (the backward), else checked (dtype uint8, large enough)."""
    if saved_bwd is True and allocate:
        return _ws(so2conv_saved_bwd_bytes(cfg, g.n_edges), device)
    if saved_bwd is None:
        return None
    _dev(saved_bwd, "saved_bwd", dtype=torch.uint8)
    if saved_bwd.numel() < so2conv_saved_bwd_bytes(cfg, g.n_edges):
        raise ValueError("saved_bwd is smaller than so2conv_saved_bwd_bytes")
    return saved_bwd


def so2conv_chunked_workspace_bytes(cfg: SO2Config, n_nodes, n_edges, stage, chunk_edges) -> int:
    c = cfg.c()
    return int(lib().so2conv_chunked_workspace_bytes(ctypes.byref(c), n_nodes, n_edges, stage, chunk_edges))


def _ws_for(cfg, g, stage, saved, ws, chunk_edges, device):
    """Workspace of one stage: one chunk over all edges unless chunk_edges is given;
    with saved=None the forward state is recomputed inside the workspace."""
    if ws is not None:
        return ws
    if saved is None or chunk_edges is not None:
        ce = g.n_edges if chunk_edges is None else int(chunk_edges)
        if saved is None:
            nb = so2conv_chunked_workspace_bytes(cfg, g.n_nodes, g.n_edges, stage, max(1, ce))
        else:   # saved state given, chunked workspace for the remaining per-edge buffers
            nb = so2conv_chunked_workspace_bytes(cfg, g.n_nodes, g.n_edges, stage, max(1, ce)) - \
                so2conv_chunked_workspace_bytes(cfg, g.n_nodes, g.n_edges, 0, max(1, ce)) + \
                so2conv_workspace_bytes(cfg, g.n_nodes, g.n_edges, 0)
    else:
        nb = so2conv_workspace_bytes(cfg, g.n_nodes, g.n_edges, stage)
    return _ws(nb, device)


def _common(cfg, g, x, pos, rbf, w_rad, env=None):
    N, E, d, C = g.n_nodes, g.n_edges, cfg.d, cfg.channels
    _dev(x, "x", dtype=cfg.torch_dtype, shape=(N, d, C))
    _dev(pos, "pos", shape=(N, 3))
    _dev(rbf, "rbf", shape=(E, cfg.n_rbf))
    _dev(w_rad, "w_rad", dtype=cfg.torch_dtype, shape=(cfg.n_rbf, (cfg.lmax + 1) * 2 * C))
    _dev(env, "env", shape=cfg.env_shape(E))


def so2conv_fwd(cfg: SO2Config, g: Graph, x, pos, rbf, w_rad, w1, w2, saved=None, ws=None, chunk_edges=None,
                env=None):
    """Returns (y, saved). `saved=True` allocates the state for bwd/dbwd; with
    saved=None the state is not kept (chunks of chunk_edges edges). `env` [E]
    float32: optional per-edge cutoff envelope multiplying each message."""
    _common(cfg, g, x, pos, rbf, w_rad, env)
    s1, s2 = weight_shapes(cfg)
    dt = cfg.torch_dtype
    p1, k1 = _ptr_array(w1, "w1", s1, dt)
    p2, k2 = _ptr_array(w2, "w2", s2, dt)
    y = torch.empty_like(x)
    if saved is True:
        saved = _ws(so2conv_saved_bytes(cfg, g.n_edges), x.device)
    ws = _ws_for(cfg, g, 0, saved, ws, chunk_edges, x.device)
    c, gc = cfg.c(), g.c()
    check(lib().so2conv_fwd(ctypes.byref(c), ctypes.byref(gc), _p(x), _p(pos), _p(rbf), _p(env), _p(w_rad), p1, p2,
                            _p(y), _p(saved), _p(ws), ws.numel(), _stream()), "so2conv_fwd")
    return y, saved


def so2conv_fwd_noalloc(cfg: SO2Config, g: Graph, x, pos, rbf, w_rad, w1, w2, env=None, y=None):
    """Forward through the library's fixed device scratch (no workspace argument,
    no state kept). y: optional preallocated output."""
    _common(cfg, g, x, pos, rbf, w_rad, env)
    s1, s2 = weight_shapes(cfg)
    dt = cfg.torch_dtype
    p1, k1 = _ptr_array(w1, "w1", s1, dt)
    p2, k2 = _ptr_array(w2, "w2", s2, dt)
    y = torch.empty_like(x) if y is None else _dev(y, "y", dtype=dt, shape=x.shape)
    c, gc = cfg.c(), g.c()
    check(lib().so2conv_fwd_noalloc(ctypes.byref(c), ctypes.byref(gc), _p(x), _p(pos), _p(rbf), _p(env), _p(w_rad),
                                    p1, p2, _p(y), _stream()), "so2conv_fwd_noalloc")
    return y


GRAD_KEYS = ("x", "pos", "rbf", "w_rad", "w1", "w2", "edge", "env")


def so2conv_bwd(cfg: SO2Config, g: Graph, x, pos, rbf, w_rad, w1, w2, saved, gy, need=GRAD_KEYS, ws=None,
                chunk_edges=None, env=None, saved_bwd=None):
    """Returns dict gx, gpos, grbf, gw_rad, gw1, gw2, gedge and, with an envelope,
    genv (requested ones). saved=None recomputes the forward state chunk by chunk.
    saved_bwd=True (or a buffer of so2conv_saved_bwd_bytes) keeps the cotangents
    a double backward with the same inputs and gy can reuse (out["saved_bwd"])."""
    _common(cfg, g, x, pos, rbf, w_rad, env)
    dt = cfg.torch_dtype
    _dev(gy, "gy", dtype=dt, shape=x.shape)
    s1, s2 = weight_shapes(cfg)
    p1, k1 = _ptr_array(w1, "w1", s1, dt)
    p2, k2 = _ptr_array(w2, "w2", s2, dt)
    dev = x.device
    out = {}
    out["gx"] = torch.empty_like(x) if "x" in need else None
    out["gpos"] = torch.empty_like(pos) if "pos" in need else None
    out["grbf"] = torch.empty_like(rbf) if "rbf" in need else None
    out["gw_rad"] = torch.empty_like(w_rad) if "w_rad" in need else None
    out["gw1"] = [torch.empty(s, dtype=dt, device=dev) for s in s1] if "w1" in need else None
    out["gw2"] = [torch.empty(s, dtype=dt, device=dev) for s in s2] if "w2" in need else None
    out["gedge"] = torch.empty(g.n_edges, 3, device=dev) if "edge" in need else None
    out["genv"] = torch.empty_like(env) if ("env" in need and env is not None) else None
    q1, k3 = _ptr_array(out["gw1"], "gw1", s1, dt)
    q2, k4 = _ptr_array(out["gw2"], "gw2", s2, dt)
    out["saved_bwd"] = saved_bwd = _saved_bwd(cfg, g, saved_bwd, dev, allocate=True)
    ws = _ws_for(cfg, g, 1, saved, ws, chunk_edges, dev)
    c, gc = cfg.c(), g.c()
    check(lib().so2conv_bwd(ctypes.byref(c), ctypes.byref(gc), _p(x), _p(pos), _p(rbf), _p(env), _p(w_rad), p1, p2,
                            _p(saved), _p(gy), _p(out["gx"]), _p(out["gpos"]), _p(out["grbf"]), _p(out["genv"]),
                            _p(out["gw_rad"]), q1, q2, _p(out["gedge"]), _p(saved_bwd), _p(ws), ws.numel(),
                            _stream()), "so2conv_bwd")
    return out


DBWD_KEYS = ("gy", "x", "rbf", "w_rad", "w1", "w2")   # the force-training pattern; add "pos" for gpos2


def so2conv_dbwd(cfg: SO2Config, g: Graph, x, pos, rbf, w_rad, w1, w2, saved, gy, px=None, ppos=None, pedge=None,
                 prbf=None, pw_rad=None, pw1=None, pw2=None, need=DBWD_KEYS, ws=None, chunk_edges=None, env=None,
                 penv=None, saved_bwd=None):
    """Returns dict ggy, gx2, gpos2, grbf2, genv2, gw_rad2, gw1_2, gw2_2 (requested ones;
    gpos2 only when "pos" is in need, genv2 when "env" is and an envelope is given).
    saved_bwd: out["saved_bwd"] of so2conv_bwd on the same inputs and gy, or None."""
    _common(cfg, g, x, pos, rbf, w_rad, env)
    _dev(penv, "penv", shape=cfg.env_shape(g.n_edges))
    dt = cfg.torch_dtype
    _dev(gy, "gy", dtype=dt, shape=x.shape)
    _dev(px, "px", dtype=dt, shape=x.shape)
    _dev(ppos, "ppos", shape=pos.shape)
    _dev(pedge, "pedge", shape=(g.n_edges, 3))
    _dev(prbf, "prbf", shape=rbf.shape)
    _dev(pw_rad, "pw_rad", dtype=dt, shape=w_rad.shape)
    s1, s2 = weight_shapes(cfg)
    p1, k1 = _ptr_array(w1, "w1", s1, dt)
    p2, k2 = _ptr_array(w2, "w2", s2, dt)
    pp1, k5 = _ptr_array(pw1, "pw1", s1, dt)
    pp2, k6 = _ptr_array(pw2, "pw2", s2, dt)
    dev = x.device
    out = {}
    out["ggy"] = torch.empty_like(x) if "gy" in need else None
    out["gx2"] = torch.empty_like(x) if "x" in need else None
    out["gpos2"] = torch.empty_like(pos) if "pos" in need else None
    out["genv2"] = torch.empty_like(env) if ("env" in need and env is not None) else None
    out["grbf2"] = torch.empty_like(rbf) if "rbf" in need else None
    out["gw_rad2"] = torch.empty_like(w_rad) if "w_rad" in need else None
    out["gw1_2"] = [torch.empty(s, dtype=dt, device=dev) for s in s1] if "w1" in need else None
    out["gw2_2"] = [torch.empty(s, dtype=dt, device=dev) for s in s2] if "w2" in need else None
    q1, k3 = _ptr_array(out["gw1_2"], "gw1_2", s1, dt)
    q2, k4 = _ptr_array(out["gw2_2"], "gw2_2", s2, dt)
    saved_bwd = _saved_bwd(cfg, g, saved_bwd, dev, allocate=False)
    ws = _ws_for(cfg, g, 2, saved, ws, chunk_edges, dev)
    c, gc = cfg.c(), g.c()
    check(lib().so2conv_dbwd(ctypes.byref(c), ctypes.byref(gc), _p(x), _p(pos), _p(rbf), _p(env), _p(w_rad), p1,
                             p2, _p(saved), _p(gy), _p(px), _p(ppos), _p(pedge), _p(prbf), _p(penv), _p(pw_rad), pp1,
                             pp2, _p(out["ggy"]), _p(out["gx2"]), _p(out["gpos2"]), _p(out["grbf2"]),
                             _p(out["genv2"]), _p(out["gw_rad2"]), q1, q2, _p(saved_bwd),
                             _p(ws), ws.numel(), _stream()), "so2conv_dbwd")
    return out


def so2conv_profile_enable(on=True):
    check(lib().so2conv_profile_enable(1 if on else 0), "so2conv_profile_enable")


def so2conv_profile_reset():
    check(lib().so2conv_profile_reset(), "so2conv_profile_reset")


def so2conv_profile_read(kind=-1):
    """(launches, total_ms, total_flops, total_bytes) of the recorded GEMM launches of
    one kind (float32 operands 0: A B, 1: A B^T, 2: A^T B; bfloat16 operands
    3: A B^T, 4: A^T B; -1: all)."""
    n, ms, fl, by = ctypes.c_int64(), ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
    check(lib().so2conv_profile_read(kind, ctypes.byref(n), ctypes.byref(ms), ctypes.byref(fl), ctypes.byref(by)),
          "so2conv_profile_read")
    return int(n.value), float(ms.value), float(fl.value), float(by.value)


def so2conv_debug_rotate_gather(cfg: SO2Config, g: Graph, x, pos, rbf, w_rad):
    _common(cfg, g, x, pos, rbf, w_rad)
    L, M = cfg.lmax, cfg.mmax
    q = (L + 1) * (2 * M + 1) - M * (M + 1)
    T = torch.empty(g.n_edges, q * 2 * cfg.channels, dtype=cfg.torch_dtype, device=x.device)
    wS = (L + 1) * 2 * cfg.channels
    nb = g.n_edges * wS * 4 + 4096
    if cfg.dtype == "bf16":
        nb += (g.n_nodes * cfg.d * cfg.channels + cfg.n_rbf * wS) * 4 + 1024
    ws = _ws(nb, x.device)
    c, gc = cfg.c(), g.c()
    check(lib().so2conv_debug_rotate_gather(ctypes.byref(c), ctypes.byref(gc), _p(x), _p(pos), _p(rbf), _p(w_rad),
                                            _p(T), _p(ws), ws.numel(), _stream()), "so2conv_debug_rotate_gather")
    return T


def so2conv_debug_status():
    """Synchronise the current stream and raise So2Error (status -5) if the last
    call with debug_checks found bad inputs on this device."""
    check(lib().so2conv_debug_status(_stream()), "so2conv_debug_status")
