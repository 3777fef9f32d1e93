"""PyTorch-facing calls of the spherical-grid SwiGLU activation on edges (C ABI
so2s2_*; TrimSO(2) page, Table 2, Appendix C.1 and Appendix B.4): per edge and channel
z = P (SiLU(G u_g) * (G u_v)), its backward and double backward. Every step
runs in libso2conv.so; this module checks shapes and passes pointers and the
stream."""
from __future__ import annotations

import ctypes
import dataclasses

import torch

from ._binding import S2Cfg, check, lib
from .ops import _dev, _p, _stream

__all__ = ["S2Config", "so2s2_fwd", "so2s2_bwd", "so2s2_dbwd"]


@dataclasses.dataclass(frozen=True)
class S2Config:
    rows: int       # coefficient rows per edge (q)
    channels: int   # C: U carries 2C (value half, gate half), Z carries C
    n_grid: int

    def c(self) -> S2Cfg:
        return S2Cfg(self.rows, self.channels, self.n_grid, 0, 0)


def _check(cfg, U, G, P):
    E = U.shape[0]
    _dev(U, "U", shape=(E, cfg.rows, 2 * cfg.channels))
    _dev(G, "G", shape=(cfg.n_grid, cfg.rows))
    _dev(P, "P", shape=(cfg.rows, cfg.n_grid))
    return E


def so2s2_fwd(cfg: S2Config, U, G, P):
    """Z [E, rows, C]."""
    E = _check(cfg, U, G, P)
    Z = torch.empty(E, cfg.rows, cfg.channels, device=U.device)
    c = cfg.c()
    check(lib().so2s2_fwd(ctypes.byref(c), E, _p(U), _p(G), _p(P), _p(Z), _stream()), "so2s2_fwd")
    return Z


def so2s2_bwd(cfg: S2Config, U, G, P, gZ):
    """gU [E, rows, 2C]."""
    E = _check(cfg, U, G, P)
    _dev(gZ, "gZ", shape=(E, cfg.rows, cfg.channels))
    gU = torch.empty_like(U)
    c = cfg.c()
    check(lib().so2s2_bwd(ctypes.byref(c), E, _p(U), _p(G), _p(P), _p(gZ), _p(gU), _stream()), "so2s2_bwd")
    return gU


def so2s2_dbwd(cfg: S2Config, U, G, P, gZ, pU, need=("gZ", "U")):
    """dict ggZ, gU2: derivatives of <pU, gU> with respect to gZ and U."""
    E = _check(cfg, U, G, P)
    _dev(gZ, "gZ", shape=(E, cfg.rows, cfg.channels))
    _dev(pU, "pU", shape=U.shape)
    out = {"ggZ": torch.empty_like(gZ) if "gZ" in need else None,
           "gU2": torch.empty_like(U) if "U" in need else None}
    c = cfg.c()
    check(lib().so2s2_dbwd(ctypes.byref(c), E, _p(U), _p(G), _p(P), _p(gZ), _p(pU), _p(out["ggZ"]), _p(out["gU2"]),
                           _stream()), "so2s2_dbwd")
    return out
