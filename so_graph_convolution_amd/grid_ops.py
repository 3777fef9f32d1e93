"""PyTorch-facing calls of the node-to-node spherical projection (C ABI
so2grid_*; TrimSO(2) page, Appendix B.4): per node U = sum_l G_l (X^(l) B_l)
with B_l = W_l A, and of the back-projection Z^(l) = (H_l Y) A from the grid
(so2grid_back_*), with their backward and double backward. Every step runs in
libso2conv.so; this module checks shapes and passes pointers and the stream."""
from __future__ import annotations

import ctypes
import dataclasses

import torch

from ._binding import GridCfg, check, lib
from .ops import _dev, _p, _stream, _ws

__all__ = ["GridConfig", "so2grid_fwd", "so2grid_bwd", "so2grid_dbwd", "so2grid_workspace_bytes",
           "so2grid_back_fwd", "so2grid_back_bwd", "so2grid_back_dbwd", "so2grid_back_workspace_bytes"]


@dataclasses.dataclass(frozen=True)
class GridConfig:
    lmax: int
    c_in: int
    c_h: int
    c_out: int
    n_grid: int

    def c(self) -> GridCfg:
        return GridCfg(self.lmax, self.c_in, self.c_h, self.c_out, self.n_grid, 0, 0)

    @property
    def d(self) -> int:
        return (self.lmax + 1) ** 2


def so2grid_workspace_bytes(cfg: GridConfig, n_nodes: int, stage: int) -> int:
    c = cfg.c()
    return int(lib().so2grid_workspace_bytes(ctypes.byref(c), n_nodes, stage))


def _check(cfg, x, G, W, A):
    N = x.shape[0]
    _dev(x, "x", shape=(N, cfg.d, cfg.c_in))
    _dev(G, "G", shape=(cfg.n_grid, cfg.d))
    _dev(W, "W", shape=(cfg.lmax + 1, cfg.c_in, cfg.c_h))
    _dev(A, "A", shape=(cfg.c_h, cfg.c_out))
    return N


def so2grid_fwd(cfg: GridConfig, x, G, W, A):
    """U [N, n_grid, c_out]."""
    N = _check(cfg, x, G, W, A)
    U = torch.empty(N, cfg.n_grid, cfg.c_out, device=x.device)
    ws = _ws(so2grid_workspace_bytes(cfg, N, 0), x.device)
    c = cfg.c()
    check(lib().so2grid_fwd(ctypes.byref(c), N, _p(x), _p(G), _p(W), _p(A), _p(U), _p(ws), ws.numel(), _stream()),
          "so2grid_fwd")
    return U


def so2grid_bwd(cfg: GridConfig, x, G, W, A, gU, need=("x", "W", "A")):
    """dict gx, gW, gA (requested ones)."""
    N = _check(cfg, x, G, W, A)
    _dev(gU, "gU", shape=(N, cfg.n_grid, cfg.c_out))
    out = {"gx": torch.empty_like(x) if "x" in need else None,
           "gW": torch.empty_like(W) if "W" in need else None,
           "gA": torch.empty_like(A) if "A" in need else None}
    ws = _ws(so2grid_workspace_bytes(cfg, N, 1), x.device)
    c = cfg.c()
    check(lib().so2grid_bwd(ctypes.byref(c), N, _p(x), _p(G), _p(W), _p(A), _p(gU), _p(out["gx"]), _p(out["gW"]),
                            _p(out["gA"]), _p(ws), ws.numel(), _stream()), "so2grid_bwd")
    return out


def so2grid_dbwd(cfg: GridConfig, x, G, W, A, gU, px=None, pW=None, pA=None, need=("gU", "x", "W", "A")):
    """dict ggU, gx2, gW2, gA2: derivatives of <px, gx> + <pW, gW> + <pA, gA>."""
    N = _check(cfg, x, G, W, A)
    _dev(gU, "gU", shape=(N, cfg.n_grid, cfg.c_out))
    _dev(px, "px", shape=x.shape)
    _dev(pW, "pW", shape=W.shape)
    _dev(pA, "pA", shape=A.shape)
    out = {"ggU": torch.empty_like(gU) if "gU" in need else None,
           "gx2": torch.empty_like(x) if "x" in need else None,
           "gW2": torch.empty_like(W) if "W" in need else None,
           "gA2": torch.empty_like(A) if "A" in need else None}
    ws = _ws(so2grid_workspace_bytes(cfg, N, 2), x.device)
    c = cfg.c()
    check(lib().so2grid_dbwd(ctypes.byref(c), N, _p(x), _p(G), _p(W), _p(A), _p(gU), _p(px), _p(pW), _p(pA),
                             _p(out["ggU"]), _p(out["gx2"]), _p(out["gW2"]), _p(out["gA2"]), _p(ws), ws.numel(),
                             _stream()), "so2grid_dbwd")
    return out


# ---------------------------------------------------------------- back-projection (so2grid_back_*)
def so2grid_back_workspace_bytes(cfg: GridConfig, n_nodes: int, stage: int) -> int:
    c = cfg.c()
    return int(lib().so2grid_back_workspace_bytes(ctypes.byref(c), n_nodes, stage))


def _check_back(cfg, Y, H, A):
    N = Y.shape[0]
    _dev(Y, "Y", shape=(N, cfg.n_grid, cfg.c_h))
    _dev(H, "H", shape=(cfg.d, cfg.n_grid))
    _dev(A, "A", shape=(cfg.c_h, cfg.c_out))
    return N


def so2grid_back_fwd(cfg: GridConfig, Y, H, A):
    """Z [N, (lmax+1)^2, c_out] = H_l (Y A) per degree, computed as (H_l Y) A."""
    N = _check_back(cfg, Y, H, A)
    Z = torch.empty(N, cfg.d, cfg.c_out, device=Y.device)
    ws = _ws(so2grid_back_workspace_bytes(cfg, N, 0), Y.device)
    c = cfg.c()
    check(lib().so2grid_back_fwd(ctypes.byref(c), N, _p(Y), _p(H), _p(A), _p(Z), _p(ws), ws.numel(), _stream()),
          "so2grid_back_fwd")
    return Z


def so2grid_back_bwd(cfg: GridConfig, Y, H, A, gZ, need=("Y", "A")):
    """dict gY, gA (requested ones)."""
    N = _check_back(cfg, Y, H, A)
    _dev(gZ, "gZ", shape=(N, cfg.d, cfg.c_out))
    out = {"gY": torch.empty_like(Y) if "Y" in need else None, "gA": torch.empty_like(A) if "A" in need else None}
    ws = _ws(so2grid_back_workspace_bytes(cfg, N, 1), Y.device)
    c = cfg.c()
    check(lib().so2grid_back_bwd(ctypes.byref(c), N, _p(Y), _p(H), _p(A), _p(gZ), _p(out["gY"]), _p(out["gA"]),
                                 _p(ws), ws.numel(), _stream()), "so2grid_back_bwd")
    return out


def so2grid_back_dbwd(cfg: GridConfig, Y, H, A, gZ, pY=None, pA=None, need=("gZ", "Y", "A")):
    """dict ggZ, gY2, gA2: derivatives of <pY, gY> + <pA, gA>."""
    N = _check_back(cfg, Y, H, A)
    _dev(gZ, "gZ", shape=(N, cfg.d, cfg.c_out))
    _dev(pY, "pY", shape=Y.shape)
    _dev(pA, "pA", shape=A.shape)
    out = {"ggZ": torch.empty_like(gZ) if "gZ" in need else None,
           "gY2": torch.empty_like(Y) if "Y" in need else None,
           "gA2": torch.empty_like(A) if "A" in need else None}
    ws = _ws(so2grid_back_workspace_bytes(cfg, N, 2), Y.device)
    c = cfg.c()
    check(lib().so2grid_back_dbwd(ctypes.byref(c), N, _p(Y), _p(H), _p(A), _p(gZ), _p(pY), _p(pA), _p(out["ggZ"]),
                                  _p(out["gY2"]), _p(out["gA2"]), _p(ws), ws.numel(), _stream()),
          "so2grid_back_dbwd")
    return out
