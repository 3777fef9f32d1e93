"""Shared helpers of the GPU parity tests: seeded workloads, device copies,
oracle evaluation and the comparison metric.

Metrics: per output tensor, max |gpu - oracle| / max |oracle| (max-norm
relative error, `relerr`), and the element-wise relative error with a floor,
max |gpu - oracle| / (|oracle| + floor * max |oracle|) (`elemerr`), which
also sees small elements of a tensor whose maximum is large. The bar is 1e-4
for float32 and 2e-2 for bfloat16 features and weights (the oracle then
receives the same bf16-representable values in float64, so the error measures
only the GPU's own rounding). The element-wise error is held to ten times
that bar (1e-3 and 2e-1) above a floor of 1e-2 (float32) or 1e-1 (bfloat16)
of the tensor's maximum: a float32 sum over ~10^6 edges carries absolute
rounding of ~1e-6 of its largest element, which is ~1e-4 of an element at the
floor.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import so2_synth
from oracle import so2conv_oracle as O

TOL_F32 = 1e-4
TOL_BF16 = 2e-2
FLOOR_F32 = 1e-2
FLOOR_BF16 = 1e-1
TOL_ELEM_F32 = 1e-3
TOL_ELEM_BF16 = 2e-1
BF16_KEYS = ("x", "gy", "px", "w_rad", "w1", "w2")   # arrays of the call's dtype


def workload(base="T", **over):
    cfg = so2_synth.make_config(base, **over)
    return so2_synth.make_inputs(cfg)


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(d, dtype="f32", validate_graph=True):
    """Device copies; with dtype "bf16" the node features, cotangents and
    weights are passed as bfloat16 (exact for bf16-representable inputs)."""
    import so_graph_convolution_amd as K
    cfg = d["cfg"]
    dev = torch.device("cuda:0")
    if dtype == "bf16":
        for k in (k for k in BF16_KEYS if k in d):
            vals = d[k] if isinstance(d[k], list) else [d[k]]
            for a in vals:
                assert np.array_equal(so2_synth.round_bf16(a), a), f"{k} is not bf16-representable"

    def t(a, dt=torch.float32):
        return torch.tensor(np.ascontiguousarray(a), dtype=dt, device=dev)

    ft = torch.bfloat16 if dtype == "bf16" else torch.float32
    grid = None
    if d.get("grid_G") is not None:   # spherical-grid SwiGLU activation
        grid = (t(d["grid_G"]), t(d["grid_P"]))
    kc = K.SO2Config(cfg.lmax, cfg.mmax, cfg.channels, cfg.n_rbf, dtype,
                     act="swiglu_s2" if grid is not None else "gate", grid=grid)
    g = K.so2conv_graph_prepare(cfg.n_atoms, t(d["src"], torch.int32), t(d["dst"], torch.int32), t(d["shift"]),
                                validate=validate_graph)
    out = dict(kcfg=kc, g=g, x=t(d["x"], ft), pos=t(d["pos"]), rbf=t(d["rbf"]), w_rad=t(d["w_rad"], ft),
               w1=[t(w, ft) for w in d["w1"]], w2=[t(w, ft) for w in d["w2"]])
    for k in ("gy", "px", "ppos", "prbf"):
        if k in d:
            out[k] = t(d[k], ft if k in BF16_KEYS else torch.float32)
    return out


def relerr(gpu, ref):
    if isinstance(gpu, (list, tuple)):
        return max(relerr(a, b) for a, b in zip(gpu, ref))
    g = gpu.detach().double().cpu() if isinstance(gpu, torch.Tensor) else torch.as_tensor(gpu, dtype=torch.float64)
    r = ref.detach().double().cpu() if isinstance(ref, torch.Tensor) else torch.as_tensor(ref, dtype=torch.float64)
    den = float(r.abs().max())
    if den == 0.0:
        return float((g - r).abs().max())
    return float((g - r).abs().max()) / den


def elemerr(gpu, ref, floor=FLOOR_F32):
    """max |g - r| / (|r| + floor * max |r|) over the elements of one tensor (or the max over a list)."""
    if isinstance(gpu, (list, tuple)):
        return max(elemerr(a, b, floor) for a, b in zip(gpu, ref))
    g = gpu.detach().double().cpu() if isinstance(gpu, torch.Tensor) else torch.as_tensor(gpu, dtype=torch.float64)
    r = ref.detach().double().cpu() if isinstance(ref, torch.Tensor) else torch.as_tensor(ref, dtype=torch.float64)
    if r.numel() == 0:
        return 0.0
    den = r.abs() + floor * float(r.abs().max())
    if float(den.max()) == 0.0:
        return float((g - r).abs().max())
    return float(((g - r).abs() / den.clamp_min(1e-300)).max())


def errs_both(gpu, ref, dtype="f32"):
    """(max-norm error, floored element-wise error) of one output."""
    return relerr(gpu, ref), elemerr(gpu, ref, FLOOR_BF16 if dtype == "bf16" else FLOOR_F32)


def oracle_inputs(d):
    return O.to_oracle_inputs(d)


def m_major(T_by_l, L, M, W):
    """Assemble oracle per-degree rows [E, 2l+1, W] into the documented m-major layout."""
    E = T_by_l[0].shape[0]
    cols = []
    cols.append(torch.cat([T_by_l[l][:, l, :] for l in range(L + 1)], -1))
    for m in range(1, M + 1):
        cols.append(torch.cat([T_by_l[l][:, l + m, :] for l in range(m, L + 1)]
                              + [T_by_l[l][:, l - m, :] for l in range(m, L + 1)], -1))
    return torch.cat(cols, -1) if E else torch.zeros(0, sum(c.shape[1] for c in cols))


def subgraph(d, edges):
    """Inputs restricted to the given edges and the nodes they touch (renumbered).
    Returns (sub_inputs, nodes) with nodes[k] = original id of sub-node k. Node
    outputs of nodes whose incident edges are all included, and per-edge outputs,
    equal those of the full problem."""
    edges = np.asarray(edges)
    src, dst = d["src"][edges], d["dst"][edges]
    nodes = np.unique(np.concatenate([src, dst]))
    remap = {int(n): k for k, n in enumerate(nodes)}
    sub = dict(d)
    sub["src"] = np.array([remap[int(v)] for v in src], dtype=np.int32)
    sub["dst"] = np.array([remap[int(v)] for v in dst], dtype=np.int32)
    for k in ("shift", "rbf", "prbf"):
        if k in d:
            sub[k] = d[k][edges]
    for k in ("x", "pos", "gy", "px", "ppos"):
        if k in d:
            sub[k] = d[k][nodes]
    import dataclasses
    sub["cfg"] = dataclasses.replace(d["cfg"], n_atoms=len(nodes))
    return sub, nodes


def incident(d, nodes):
    return np.nonzero(np.isin(d["dst"], nodes) | np.isin(d["src"], nodes))[0]


def incoming(d, nodes):
    return np.nonzero(np.isin(d["dst"], nodes))[0]
