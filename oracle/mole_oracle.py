"""Oracle (test infrastructure only) of the SO(2) convolution with a
system-dependent mixture of linear experts: TrimSO(2) page, Appendix C.1
(Implementation: UMA's edge projections use system-dependent mixtures of
linear experts) and Table 2 (64 linear experts for UMA).

Reading of the page (it names the mixture but gives no formula): a batch
holds S systems; system s owns the contiguous edge range
[sys_edge_ptr[s], sys_edge_ptr[s+1]) of the receiver-sorted edge list (a
structure occupies a contiguous node range, so its incoming edges are
contiguous) and a coefficient vector coef[s] of length K. Every edge of system
s uses, for both SO(2) linears and every order m,

    W_m(s) = sum_k coef[s, k] W_m^(k)

in place of the single weight W_m of the plain operator; the radial weights
are shared by all systems. Everything else is the plain operator of
oracle.so2conv_oracle, evaluated system by system and summed.

Derivatives come from torch.autograd through that definition (the merged
weights are built inside the graph), with respect to x, pos, rbf, W_rad, the
experts W^(k), coef and the envelope. Shares nothing with the HIP path; pinned
in tests/ against the plain operator (one-hot and shared coefficients) and
finite differences.
"""
from __future__ import annotations

import torch

from oracle import so2conv_oracle as O

DT = torch.float64


def merge(experts, coef_s):
    """W(s) = sum_k coef_s[k] W^(k) per block: experts [K, r, c] each, coef_s [K]."""
    return [torch.einsum("k,krc->rc", coef_s, w) for w in experts]


def _system_inputs(base: O.OracleInputs, w1, w2, x=None, pos=None, rbf=None, w_rad=None, env=None, shift=None):
    """The plain operator's inputs with one system's merged weights (optionally replacing leaves)."""
    return O.OracleInputs(base.L, base.M, base.C, base.pos if pos is None else pos, base.x if x is None else x,
                          base.src, base.dst, base.shift if shift is None else shift,
                          base.rbf if rbf is None else rbf, base.w_rad if w_rad is None else w_rad,
                          w1, w2, base.env if env is None else env)


def _pieces(sys_edge_ptr, chunk, edges=None):
    """(system, edge indices) pieces: every system's edges in chunks; `edges`
    (sorted indices) restricts the sum to a subset (exact for nodes all of
    whose incoming edges are in it)."""
    sub = None if edges is None else torch.as_tensor(edges, dtype=torch.int64)
    for s in range(len(sys_edge_ptr) - 1):
        a, b = int(sys_edge_ptr[s]), int(sys_edge_ptr[s + 1])
        idx = torch.arange(a, b) if sub is None else sub[(sub >= a) & (sub < b)]
        for c0 in range(0, idx.shape[0], chunk):
            yield s, idx[c0:c0 + chunk]


def forward(base: O.OracleInputs, w1e, w2e, coef, sys_edge_ptr, chunk=4096, edges=None):
    """y [N, d, C]. base: the plain operator's inputs (its w1/w2 are ignored);
    w1e/w2e: lists over orders of expert stacks [K, rows, cols]; coef [S, K]."""
    N = base.x.shape[0]
    y = torch.zeros(N, (base.L + 1) ** 2, base.C, dtype=DT)
    for s, e_idx in _pieces(sys_edge_ptr, chunk, edges):
        inp = _system_inputs(base, merge(w1e, coef[s]), merge(w2e, coef[s]))
        y = y + O._scatter(inp, e_idx, O.edge_messages(inp, e_idx), N)
    return y


def _leaf(t, on=True):
    return t.detach().clone().requires_grad_(on)


def _setup(base, w1e, w2e, coef, with_shift=False, weights_grad=True):
    """Leaves of the autograd graph; with weights_grad=False the experts and
    coefficients are constants (no gradients for them)."""
    lv = dict(x=_leaf(base.x), pos=_leaf(base.pos), rbf=_leaf(base.rbf), w_rad=_leaf(base.w_rad),
              coef=_leaf(coef, weights_grad))
    lv["w1e"] = [_leaf(w, weights_grad) for w in w1e]
    lv["w2e"] = [_leaf(w, weights_grad) for w in w2e]
    if base.env is not None:
        lv["env"] = _leaf(base.env)
    shift = _leaf(base.shift, with_shift)
    order = ["x", "pos", "rbf", "w_rad"] + (["coef"] if weights_grad else []) + \
        (["env"] if base.env is not None else [])
    flat = [lv[k] for k in order] + ((lv["w1e"] + lv["w2e"]) if weights_grad else [])
    return lv, shift, order, flat


def _y_piece(base, lv, shift, s, e_idx, N):
    inp = _system_inputs(base, merge(lv["w1e"], lv["coef"][s]), merge(lv["w2e"], lv["coef"][s]), x=lv["x"],
                         pos=lv["pos"], rbf=lv["rbf"], w_rad=lv["w_rad"], env=lv.get("env"), shift=shift)
    return O._scatter(inp, e_idx, O.edge_messages(inp, e_idx), N)


def _unflatten(vals, order, nw):
    out = {"g" + k: v for k, v in zip(order, vals)}
    rest = vals[len(order):]
    if rest:
        out["gw1e"], out["gw2e"] = list(rest[:nw]), list(rest[nw:2 * nw])
    return out


def backward(base, w1e, w2e, coef, sys_edge_ptr, gy, chunk=4096, with_edge_grad=False, edges=None,
             weights_grad=True):
    """VJP of `forward` with cotangent gy: dict gx, gpos, grbf, gw_rad, gcoef,
    gw1e, gw2e (lists of [K, r, c]; not with weights_grad=False), genv (with an
    envelope), gedge (if asked)."""
    lv, shift, order, flat = _setup(base, w1e, w2e, coef, with_edge_grad, weights_grad)
    N = base.x.shape[0]
    acc = [torch.zeros_like(t) for t in flat]
    gedge = torch.zeros_like(base.shift) if with_edge_grad else None
    for s, e_idx in _pieces(sys_edge_ptr, chunk, edges):
        y = _y_piece(base, lv, shift, s, e_idx, N)
        g = O._grads(y, flat + ([shift] if with_edge_grad else []), gy)
        for k in range(len(flat)):
            acc[k] += g[k]
        if with_edge_grad:
            gedge += g[-1]
    out = _unflatten(acc, order, len(w1e))
    if with_edge_grad:
        out["gedge"] = gedge
    return out


def double_backward(base, w1e, w2e, coef, sys_edge_ptr, gy, px=None, ppos=None, prbf=None, pw_rad=None,
                    pcoef=None, pw1e=None, pw2e=None, pedge=None, penv=None, chunk=2048, edges=None,
                    weights_grad=True):
    """Derivatives of L = <px, gx> + <ppos, gpos> + <prbf, grbf> + <pw_rad, gw_rad>
    + <pcoef, gcoef> + <pWe, gWe> (+ <pedge, gedge>) (+ <penv, genv>) with respect to
    gy (-> ggy) and every input (x, pos, rbf, w_rad, coef, experts, env). With
    weights_grad=False the experts and coefficients are constants (directions
    on them must be None)."""
    lv, shift, order, flat = _setup(base, w1e, w2e, coef, pedge is not None, weights_grad)
    gyl = _leaf(gy)
    nw = len(w1e)
    dmap = dict(x=px, pos=ppos, rbf=prbf, w_rad=pw_rad, coef=pcoef, env=penv)
    dirs = [dmap[k] for k in order] + ((list(pw1e or [None] * nw) + list(pw2e or [None] * nw)) if weights_grad
                                       else [])
    N = base.x.shape[0]
    acc = [torch.zeros_like(t) for t in flat]
    accgy = torch.zeros_like(gy)
    for s, e_idx in _pieces(sys_edge_ptr, chunk, edges):
        y = _y_piece(base, lv, shift, s, e_idx, N)
        wrt = flat + ([shift] if pedge is not None else [])
        g = O._grads(y, wrt, gyl, create_graph=True)
        Lval = torch.zeros((), dtype=DT)
        for gi, p in zip(g, dirs + ([pedge] if pedge is not None else [])):
            if p is not None:
                Lval = Lval + (gi * p).sum()
        if not Lval.requires_grad:
            continue
        h = O._grads(Lval, flat + [gyl], None)
        for k in range(len(flat)):
            acc[k] += h[k]
        accgy += h[-1]
    out = _unflatten(acc, order, nw)
    out["ggy"] = accgy
    return out
