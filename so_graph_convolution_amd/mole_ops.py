"""PyTorch-facing calls of the mixture-of-linear-experts entry points
(so2mole_*; same names as the library's). A batch of systems: system s owns
the receiver-sorted edges [sys_edge_ptr[s], sys_edge_ptr[s+1]) and uses the
weights sum_k coef[s, k] W^(k) of the expert stacks in both SO(2) linears.
Argument marshalling only: every step runs in libso2conv.so."""
from __future__ import annotations

import ctypes

import numpy as np
import torch

from ._binding import MoleCfg, check, lib
from .ops import (GRAD_KEYS, DBWD_KEYS, Graph, SO2Config, _common, _dev, _p, _ptr_array, _saved_bwd, _stream, _ws,
                  weight_shapes)

__all__ = ["Mixture", "so2mole_workspace_bytes", "so2mole_fwd", "so2mole_bwd", "so2mole_dbwd", "expert_shapes"]


class Mixture:
    """n_experts K and the host edge offsets of the systems (length S + 1)."""

    def __init__(self, n_experts, sys_edge_ptr):
        self.n_experts = int(n_experts)
        self.sys_edge_ptr = np.ascontiguousarray(np.asarray(sys_edge_ptr, dtype=np.int64))
        self.n_systems = int(self.sys_edge_ptr.shape[0] - 1)

    def c(self) -> MoleCfg:
        return MoleCfg(self.n_systems, self.n_experts, self.sys_edge_ptr.ctypes.data)


def expert_shapes(cfg: SO2Config, K):
    s1, s2 = weight_shapes(cfg)
    return [(K,) + s for s in s1], [(K,) + s for s in s2]


def so2mole_workspace_bytes(cfg: SO2Config, mix: Mixture, n_nodes, n_edges, stage, chunk_edges=0) -> int:
    c, m = cfg.c(), mix.c()
    return int(lib().so2mole_workspace_bytes(ctypes.byref(c), ctypes.byref(m), n_nodes, n_edges, stage,
                                             int(chunk_edges or 0)))


def _ws_for(cfg, mix, g, stage, saved, ws, chunk_edges, device):
    """One chunk over all edges using `saved`, else chunks of chunk_edges (all
    edges by default) that recompute the forward state."""
    if ws is not None:
        return ws
    if saved is not None and chunk_edges is None:
        return _ws(so2mole_workspace_bytes(cfg, mix, g.n_nodes, g.n_edges, stage, 0), device)
    ce = max(1, g.n_edges if chunk_edges is None else int(chunk_edges))
    return _ws(so2mole_workspace_bytes(cfg, mix, g.n_nodes, g.n_edges, stage, ce), device)


def _experts(cfg, mix, w1e, w2e, name1="w1e", name2="w2e"):
    s1, s2 = expert_shapes(cfg, mix.n_experts)
    dt = cfg.torch_dtype
    p1, k1 = _ptr_array(w1e, name1, s1, dt)
    p2, k2 = _ptr_array(w2e, name2, s2, dt)
    return p1, p2, [k1, k2]


def so2mole_fwd(cfg: SO2Config, g: Graph, mix: Mixture, x, pos, rbf, w_rad, w1e, w2e, coef, saved=None, ws=None,
                chunk_edges=None, env=None):
    """Returns (y, saved); as so2conv_fwd with expert stacks and coef [S, K] float32."""
    from .ops import so2conv_saved_bytes
    _common(cfg, g, x, pos, rbf, w_rad, env)
    _dev(coef, "coef", shape=(mix.n_systems, mix.n_experts))
    p1, p2, keep = _experts(cfg, mix, w1e, w2e)
    y = torch.empty_like(x)
    if saved is True:
        saved = _ws(so2conv_saved_bytes(cfg, g.n_edges), x.device)
    ws = _ws_for(cfg, mix, g, 0, saved, ws, chunk_edges, x.device)
    c, gc, m = cfg.c(), g.c(), mix.c()
    check(lib().so2mole_fwd(ctypes.byref(c), ctypes.byref(gc), ctypes.byref(m), _p(x), _p(pos), _p(rbf), _p(env),
                            _p(w_rad), p1, p2, _p(coef), _p(y), _p(saved), _p(ws), ws.numel(), _stream()),
          "so2mole_fwd")
    return y, saved


def so2mole_bwd(cfg: SO2Config, g: Graph, mix: Mixture, x, pos, rbf, w_rad, w1e, w2e, coef, saved, gy,
                need=GRAD_KEYS + ("coef",), ws=None, chunk_edges=None, env=None, saved_bwd=None):
    """Returns dict gx, gpos, grbf, gw_rad, gw1e, gw2e, gcoef, gedge, genv (requested ones);
    saved_bwd as in so2conv_bwd (out["saved_bwd"])."""
    _common(cfg, g, x, pos, rbf, w_rad, env)
    dt = cfg.torch_dtype
    _dev(gy, "gy", dtype=dt, shape=x.shape)
    _dev(coef, "coef", shape=(mix.n_systems, mix.n_experts))
    p1, p2, keep = _experts(cfg, mix, w1e, w2e)
    s1, s2 = expert_shapes(cfg, mix.n_experts)
    dev = x.device
    out = {}
    out["gx"] = torch.empty_like(x) if "x" in need else None
    out["gpos"] = torch.empty_like(pos) if "pos" in need else None
    out["grbf"] = torch.empty_like(rbf) if "rbf" in need else None
    out["gw_rad"] = torch.empty_like(w_rad) if "w_rad" in need else None
    out["gw1e"] = [torch.empty(s, dtype=dt, device=dev) for s in s1] if "w1" in need else None
    out["gw2e"] = [torch.empty(s, dtype=dt, device=dev) for s in s2] if "w2" in need else None
    out["gcoef"] = torch.empty_like(coef) if "coef" in need else None
    out["gedge"] = torch.empty(g.n_edges, 3, device=dev) if "edge" in need else None
    out["genv"] = torch.empty_like(env) if ("env" in need and env is not None) else None
    q1, q2, keep2 = _experts(cfg, mix, out["gw1e"], out["gw2e"], "gw1e", "gw2e")
    out["saved_bwd"] = saved_bwd = _saved_bwd(cfg, g, saved_bwd, dev, allocate=True)
    ws = _ws_for(cfg, mix, g, 1, saved, ws, chunk_edges, dev)
    c, gc, m = cfg.c(), g.c(), mix.c()
    check(lib().so2mole_bwd(ctypes.byref(c), ctypes.byref(gc), ctypes.byref(m), _p(x), _p(pos), _p(rbf), _p(env),
                            _p(w_rad), p1, p2, _p(coef), _p(saved), _p(gy), _p(out["gx"]), _p(out["gpos"]),
                            _p(out["grbf"]), _p(out["genv"]), _p(out["gw_rad"]), q1, q2, _p(out["gcoef"]),
                            _p(out["gedge"]), _p(saved_bwd), _p(ws), ws.numel(), _stream()), "so2mole_bwd")
    return out


def so2mole_dbwd(cfg: SO2Config, g: Graph, mix: Mixture, x, pos, rbf, w_rad, w1e, w2e, coef, saved, gy, px=None,
                 ppos=None, pedge=None, prbf=None, pw_rad=None, pw1e=None, pw2e=None, pcoef=None,
                 need=DBWD_KEYS + ("coef",), ws=None, chunk_edges=None, env=None, penv=None, saved_bwd=None):
    """Returns dict ggy, gx2, gpos2, grbf2, genv2, gw_rad2, gw1e_2, gw2e_2, gcoef2 (requested ones);
    saved_bwd: out["saved_bwd"] of so2mole_bwd on the same inputs and gy, or None."""
    _common(cfg, g, x, pos, rbf, w_rad, env)
    dt = cfg.torch_dtype
    for t, n, shp, tdt in ((gy, "gy", x.shape, dt), (px, "px", x.shape, dt), (ppos, "ppos", pos.shape, torch.float32),
                           (pedge, "pedge", (g.n_edges, 3), torch.float32), (prbf, "prbf", rbf.shape, torch.float32),
                           (pw_rad, "pw_rad", w_rad.shape, dt), (penv, "penv", cfg.env_shape(g.n_edges), torch.float32),
                           (coef, "coef", (mix.n_systems, mix.n_experts), torch.float32),
                           (pcoef, "pcoef", (mix.n_systems, mix.n_experts), torch.float32)):
        _dev(t, n, dtype=tdt, shape=shp)
    p1, p2, keep = _experts(cfg, mix, w1e, w2e)
    pp1, pp2, keep2 = _experts(cfg, mix, pw1e, pw2e, "pw1e", "pw2e")
    s1, s2 = expert_shapes(cfg, mix.n_experts)
    dev = x.device
    out = {}
    out["ggy"] = torch.empty_like(x) if "gy" in need else None
    out["gx2"] = torch.empty_like(x) if "x" in need else None
    out["gpos2"] = torch.empty_like(pos) if "pos" in need else None
    out["genv2"] = torch.empty_like(env) if ("env" in need and env is not None) else None
    out["grbf2"] = torch.empty_like(rbf) if "rbf" in need else None
    out["gw_rad2"] = torch.empty_like(w_rad) if "w_rad" in need else None
    out["gw1e_2"] = [torch.empty(s, dtype=dt, device=dev) for s in s1] if "w1" in need else None
    out["gw2e_2"] = [torch.empty(s, dtype=dt, device=dev) for s in s2] if "w2" in need else None
    out["gcoef2"] = torch.empty_like(coef) if "coef" in need else None
    q1, q2, keep3 = _experts(cfg, mix, out["gw1e_2"], out["gw2e_2"], "gw1e_2", "gw2e_2")
    saved_bwd = _saved_bwd(cfg, g, saved_bwd, dev, allocate=False)
    ws = _ws_for(cfg, mix, g, 2, saved, ws, chunk_edges, dev)
    c, gc, m = cfg.c(), g.c(), mix.c()
    check(lib().so2mole_dbwd(ctypes.byref(c), ctypes.byref(gc), ctypes.byref(m), _p(x), _p(pos), _p(rbf), _p(env),
                             _p(w_rad), p1, p2, _p(coef), _p(saved), _p(gy), _p(px), _p(ppos), _p(pedge), _p(prbf),
                             _p(penv), _p(pw_rad), pp1, pp2, _p(pcoef), _p(out["ggy"]), _p(out["gx2"]),
                             _p(out["gpos2"]), _p(out["grbf2"]), _p(out["genv2"]), _p(out["gw_rad2"]), q1, q2,
                             _p(out["gcoef2"]), _p(saved_bwd), _p(ws), ws.numel(), _stream()), "so2mole_dbwd")
    return out
