"""Parity of the widened rows at their benchmark sizes, in the launch
configurations bench.py times (--op mole, the per-head weights at the medium
workload, --op grid).

Node outputs are sums over a node's incident edges and per-edge outputs
depend on their own edge only, so the oracles evaluate them exactly on the
incident-edge subsets of a few sampled nodes and edges. Outputs that sum over
every edge or node are checked through properties that hold at any size:
y is linear in the second linear's experts (<gW2e, W2e> = <gy, y>), the
expert and coefficient gradients follow from the plain operator's weight
gradients on each system's edges, and U is linear in each channel map
(<gW, W> = <gA, A> = <gU, U>) with node-additive map gradients.
"""
import numpy as np
import pytest
import torch

import so2_synth
from oracle import grid_oracle as GO
from oracle import mole_oracle as MO
from oracle import so2conv_oracle as O
from tests import _cases as H

pytestmark = pytest.mark.gpu
DT = torch.float64


def _incident(d, nodes):
    return np.nonzero(np.isin(d["dst"], nodes) | np.isin(d["src"], nodes))[0]


def _incoming(d, nodes):
    return np.nonzero(np.isin(d["dst"], nodes))[0]


def _t(a):
    return torch.tensor(np.asarray(a), dtype=DT)


def _cpu(v):
    if v is None:
        return None
    return v.cpu() if isinstance(v, torch.Tensor) else [w.cpu() for w in v]


# ---------------------------------------------------------------- mixture of linear experts
@pytest.fixture(scope="module")
def mixture():
    import so_graph_convolution_amd as K
    cfg = so2_synth.CONFIGS["M"]
    d = so2_synth.make_inputs(cfg)
    m = so2_synth.mixture_inputs(d, 16, 64, seed=0)
    E, N = len(d["src"]), cfg.n_atoms
    H.note(f"[full size] mixture N={N} E={E} systems=16 experts=64")
    dd = H.to_dev(d)
    dev = "cuda"
    w1e = [torch.tensor(w, device=dev) for w in m["w1e"]]
    w2e = [torch.tensor(w, device=dev) for w in m["w2e"]]
    coef = torch.tensor(m["coef"], device=dev)
    mix = K.Mixture(64, m["sys_edge_ptr"])
    kc = dd["kcfg"]
    args = (kc, dd["g"], mix, dd["x"], dd["pos"], dd["rbf"], dd["w_rad"], w1e, w2e, coef)
    saved = torch.empty(K.so2conv_saved_bytes(kc, E), dtype=torch.uint8, device=dev)
    ws = torch.empty(max(K.so2mole_workspace_bytes(kc, mix, N, E, s, 0) for s in (0, 1, 2)), dtype=torch.uint8,
                     device=dev)
    y, _ = K.so2mole_fwd(*args, saved=saved, ws=ws)
    bw = K.so2mole_bwd(*args, saved, dd["gy"], ws=ws)
    db = K.so2mole_dbwd(*args, saved, dd["gy"], px=dd["px"], ppos=dd["ppos"], prbf=dd["prbf"], ws=ws)
    torch.cuda.synchronize()
    out = dict(y=y.cpu(), **{k: _cpu(v) for k, v in {**bw, **db}.items() if v is not None})
    del saved, ws, y, bw, db
    torch.cuda.empty_cache()
    rng = np.random.default_rng(321)
    nodes = np.sort(rng.choice(N, 3, replace=False))
    edges = np.sort(rng.choice(E, 48, replace=False))
    return d, m, dd, (w1e, w2e, coef), out, nodes, edges


def test_mixture_full_size_sampled(mixture):
    d, m, dd, _, out, nodes, edges = mixture
    base = H.oracle_inputs(d)
    w1e, w2e, coef = [_t(w) for w in m["w1e"]], [_t(w) for w in m["w2e"]], _t(m["coef"])
    sp, gy = m["sys_edge_ptr"].tolist(), _t(d["gy"])
    kw = dict(weights_grad=False)
    ry = MO.forward(base, w1e, w2e, coef, sp, edges=_incoming(d, nodes))
    rb = MO.backward(base, w1e, w2e, coef, sp, gy, edges=_incident(d, nodes), **kw)
    re = MO.backward(base, w1e, w2e, coef, sp, gy, edges=edges, with_edge_grad=True, **kw)
    dirs = dict(px=_t(d["px"]), ppos=_t(d["ppos"]), prbf=_t(d["prbf"]))
    rdi = MO.double_backward(base, w1e, w2e, coef, sp, gy, edges=_incoming(d, nodes), **dirs, **kw)
    rdn = MO.double_backward(base, w1e, w2e, coef, sp, gy, edges=_incident(d, nodes), **dirs, **kw)
    rde = MO.double_backward(base, w1e, w2e, coef, sp, gy, edges=edges, **dirs, **kw)
    errs = {"y": H.relerr(out["y"][nodes], ry[nodes]),
            "gx": H.relerr(out["gx"][nodes], rb["gx"][nodes]), "gpos": H.relerr(out["gpos"][nodes], rb["gpos"][nodes]),
            "grbf": H.relerr(out["grbf"][edges], re["grbf"][edges]),
            "gedge": H.relerr(out["gedge"][edges], re["gedge"][edges]),
            "ggy": H.relerr(out["ggy"][nodes], rdi["ggy"][nodes]),
            "gx2": H.relerr(out["gx2"][nodes], rdn["gx"][nodes]),
            "grbf2": H.relerr(out["grbf2"][edges], rde["grbf"][edges])}
    H.note("  " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    assert all(v <= H.TOL_F32 for v in errs.values()), errs


def test_mixture_full_size_expert_identity(mixture):
    """y is linear in the second linear's experts jointly: <gW2e, W2e> = <gy, y>."""
    d, m, _, _, out, _, _ = mixture
    lhs = sum(float((g.double() * _t(w)).sum()) for g, w in zip(out["gw2e"], m["w2e"]))
    rhs = float((out["y"].double() * _t(d["gy"])).sum())
    H.note(f"  <gW2e,W2e>={lhs:.6e} <gy,y>={rhs:.6e}")
    assert abs(lhs - rhs) <= 1e-4 * abs(rhs)


def test_mixture_full_size_gradients_follow_the_plain_operator(mixture):
    """gWe^(k) = sum_s coef[s,k] gW(s) and gcoef[s,k] = sum_m <W_m^(k), gW_m(s)>, with
    gW(s) the plain operator's weight gradients on system s's edges at its merged
    weights (the plain path is itself checked against the oracle)."""
    import so_graph_convolution_amd as K
    d, m, dd, (w1e, w2e, coef), out, _, _ = mixture
    N = d["cfg"].n_atoms
    sp = m["sys_edge_ptr"]
    gw1e = [torch.zeros_like(w, dtype=torch.float64) for w in w1e]
    gw2e = [torch.zeros_like(w, dtype=torch.float64) for w in w2e]
    gcoef = torch.zeros(coef.shape, dtype=torch.float64, device="cuda")
    for s in range(len(sp) - 1):
        sl = slice(int(sp[s]), int(sp[s + 1]))
        g = K.so2conv_graph_prepare(N, torch.tensor(d["src"][sl], device="cuda"),
                                    torch.tensor(d["dst"][sl], device="cuda"),
                                    torch.tensor(d["shift"][sl], device="cuda"))
        w1 = [torch.einsum("k,krc->rc", coef[s], w).contiguous() for w in w1e]
        w2 = [torch.einsum("k,krc->rc", coef[s], w).contiguous() for w in w2e]
        args = (dd["kcfg"], g, dd["x"], dd["pos"], torch.tensor(d["rbf"][sl], device="cuda"), dd["w_rad"], w1, w2)
        _, saved = K.so2conv_fwd(*args, saved=True)
        b = K.so2conv_bwd(*args, saved, dd["gy"], need=("w1", "w2"))
        for lst, gl, we in ((gw1e, b["gw1"], w1e), (gw2e, b["gw2"], w2e)):
            for a in range(len(lst)):
                lst[a] += coef[s].double()[:, None, None] * gl[a].double()[None]
                gcoef[s] += (we[a].double() * gl[a].double()[None]).sum((1, 2))
        del saved, b
    torch.cuda.synchronize()
    errs = {"gw1e": H.relerr(out["gw1e"], [x.cpu() for x in gw1e]),
            "gw2e": H.relerr(out["gw2e"], [x.cpu() for x in gw2e]),
            "gcoef": H.relerr(out["gcoef"], gcoef.cpu())}
    H.note("  " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    assert all(v <= H.TOL_F32 for v in errs.values()), errs


# ---------------------------------------------------------------- per-head message weights
def test_heads_full_size_sampled():
    """Medium workload with 8 heads of 16 channels (attention weights times the
    cutoff envelope): sampled fwd, bwd (incl. genv per head) and dbwd with a
    direction on the weights against the oracle."""
    import dataclasses

    import so_graph_convolution_amd as K
    cfg = so2_synth.CONFIGS["M"]
    d = dict(so2_synth.make_inputs(cfg))
    heads = 8
    d["env"] = so2_synth.attention_weights(d, heads, seed=1) * so2_synth.cosine_envelope(d)[:, None]
    E, N = len(d["src"]), cfg.n_atoms
    penv = np.random.default_rng(8).normal(size=(E, heads)).astype(np.float32)
    H.note(f"[full size] heads={heads} N={N} E={E}")
    dd = H.to_dev(d)
    kc = dataclasses.replace(dd["kcfg"], heads=heads)
    env, penv_d = torch.tensor(d["env"], device="cuda"), torch.tensor(penv, device="cuda")
    args = (kc, dd["g"], dd["x"], dd["pos"], dd["rbf"], dd["w_rad"], dd["w1"], dd["w2"])
    saved = torch.empty(K.so2conv_saved_bytes(kc, E), dtype=torch.uint8, device="cuda")
    ws = torch.empty(max(K.so2conv_workspace_bytes(kc, N, E, s) for s in (0, 1, 2)), dtype=torch.uint8, device="cuda")
    y, _ = K.so2conv_fwd(*args, saved=saved, ws=ws, env=env)
    bw = K.so2conv_bwd(*args, saved, dd["gy"], ws=ws, env=env)
    db = K.so2conv_dbwd(*args, saved, dd["gy"], px=dd["px"], ppos=dd["ppos"], prbf=dd["prbf"], penv=penv_d, env=env,
                        ws=ws, need=("gy", "x", "rbf", "env", "w_rad", "w1", "w2"))
    torch.cuda.synchronize()
    out = dict(y=y.cpu(), **{k: _cpu(v) for k, v in {**bw, **db}.items() if v is not None})
    del saved, ws, y, bw, db
    torch.cuda.empty_cache()
    rng = np.random.default_rng(77)
    nodes = np.sort(rng.choice(N, 3, replace=False))
    edges = np.sort(rng.choice(E, 48, replace=False))
    inp = H.oracle_inputs(d)
    gy = _t(d["gy"])
    dirs = dict(px=_t(d["px"]), ppos=_t(d["ppos"]), prbf=_t(d["prbf"]), penv=_t(penv))
    ry = O.forward(inp, edges=_incoming(d, nodes))
    rb = O.backward(inp, gy, edges=_incident(d, nodes))
    re = O.backward(inp, gy, edges=edges, with_edge_grad=True)
    rdi = O.double_backward(inp, gy, edges=_incoming(d, nodes), **dirs)
    rdn = O.double_backward(inp, gy, edges=_incident(d, nodes), **dirs)
    rde = O.double_backward(inp, gy, edges=edges, **dirs)
    errs = {"y": H.relerr(out["y"][nodes], ry[nodes]),
            "gx": H.relerr(out["gx"][nodes], rb["gx"][nodes]), "gpos": H.relerr(out["gpos"][nodes], rb["gpos"][nodes]),
            "genv": H.relerr(out["genv"][edges], re["genv"][edges]),
            "gedge": H.relerr(out["gedge"][edges], re["gedge"][edges]),
            "ggy": H.relerr(out["ggy"][nodes], rdi["ggy"][nodes]),
            "gx2": H.relerr(out["gx2"][nodes], rdn["gx"][nodes]),
            "genv2": H.relerr(out["genv2"][edges], rde["genv"][edges]),
            "grbf2": H.relerr(out["grbf2"][edges], rde["grbf"][edges])}
    H.note("  " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    assert all(v <= H.TOL_F32 for v in errs.values()), errs


# ---------------------------------------------------------------- spherical projection
def test_grid_full_size():
    """The projection benchmark's shapes (10,000 nodes, lmax 4, 128 -> 512 -> 512,
    100 grid points): sampled nodes of U, gx, ggU, gx2 against the oracle; the map
    gradients through linearity and node additivity."""
    import so_graph_convolution_amd as K
    L, ci, ch, co, ng, N = 4, 128, 512, 512, 100, 10000
    dg = (L + 1) ** 2
    rng = np.random.default_rng(7)
    host = dict(x=rng.normal(size=(N, dg, ci)), G=rng.normal(size=(ng, dg)) / np.sqrt(dg),
                W=rng.normal(size=(L + 1, ci, ch)) / np.sqrt(ci), A=rng.normal(size=(ch, co)) / np.sqrt(ch),
                gU=rng.normal(size=(N, ng, co)), px=rng.normal(size=(N, dg, ci)),
                pW=rng.normal(size=(L + 1, ci, ch)) / np.sqrt(ci), pA=rng.normal(size=(ch, co)) / np.sqrt(ch))
    host = {k: v.astype(np.float32) for k, v in host.items()}
    g = {k: torch.tensor(v, device="cuda") for k, v in host.items()}
    cfg = K.GridConfig(L, ci, ch, co, ng)
    H.note(f"[full size] grid N={N} L={L} {ci}/{ch}/{co} n_grid={ng}")
    U = K.so2grid_fwd(cfg, g["x"], g["G"], g["W"], g["A"])
    b = K.so2grid_bwd(cfg, g["x"], g["G"], g["W"], g["A"], g["gU"])
    db = K.so2grid_dbwd(cfg, g["x"], g["G"], g["W"], g["A"], g["gU"], px=g["px"], pW=g["pW"], pA=g["pA"])
    half = []
    for sl in (slice(0, N // 2), slice(N // 2, N)):
        hb = K.so2grid_bwd(cfg, g["x"][sl].contiguous(), g["G"], g["W"], g["A"], g["gU"][sl].contiguous())
        hd = K.so2grid_dbwd(cfg, g["x"][sl].contiguous(), g["G"], g["W"], g["A"], g["gU"][sl].contiguous(),
                            px=g["px"][sl].contiguous(), pW=g["pW"], pA=g["pA"])
        half.append({k: hb.get(k, hd.get(k)).cpu() for k in ("gW", "gA", "gW2", "gA2")})
    uu = float((U.double() * g["gU"].double()).sum())
    gww = float((b["gW"].double() * g["W"].double()).sum())
    gaa = float((b["gA"].double() * g["A"].double()).sum())
    nodes = np.sort(rng.choice(N, 16, replace=False))
    idx = torch.tensor(nodes, device="cuda")
    out = {"U": U[idx].cpu(), "gx": b["gx"][idx].cpu(), "ggU": db["ggU"][idx].cpu(), "gx2": db["gx2"][idx].cpu(),
           "gW": b["gW"].cpu(), "gA": b["gA"].cpu(), "gW2": db["gW2"].cpu(), "gA2": db["gA2"].cpu()}
    torch.cuda.synchronize()
    r = {k: _t(host[k]) for k in ("G", "W", "A", "pW", "pA")}
    xs, gus, pxs = _t(host["x"][nodes]), _t(host["gU"][nodes]), _t(host["px"][nodes])
    ru = GO.forward(xs, r["G"], r["W"], r["A"])
    rb = GO.backward(xs, r["G"], r["W"], r["A"], gus)
    rd = GO.double_backward(xs, r["G"], r["W"], r["A"], gus, px=pxs, pW=r["pW"], pA=r["pA"])
    errs = {"U": H.relerr(out["U"], ru), "gx": H.relerr(out["gx"], rb["gx"]),
            "ggU": H.relerr(out["ggU"], rd["ggU"]), "gx2": H.relerr(out["gx2"], rd["gx"]),
            "<gW,W>": abs(gww - uu) / abs(uu), "<gA,A>": abs(gaa - uu) / abs(uu)}
    for k in ("gW", "gA", "gW2", "gA2"):
        errs[k + " additive"] = H.relerr(out[k], half[0][k] + half[1][k])
    H.note("  " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    assert all(v <= H.TOL_F32 for v in errs.values()), errs
