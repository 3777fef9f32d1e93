"""Parity at the benchmark's full sizes, in the launch configuration bench.py times
(the medium system with forward, backward and double backward; the eSEN-like
small system with forward and backward).

Node outputs are sums over a node's incident edges and per-edge outputs
depend on their own edge only, so the oracle evaluates them exactly on the
incident-edge subset of a few sampled nodes and edges. Weight gradients sum
over every edge; they are checked through properties that hold at any size:
y is linear in W2, so <gW2, W2> = <gy, y>; and a gradient over all edges
equals the sum of the gradients over two disjoint edge sets.
"""
import numpy as np
import pytest
import torch

import so2_synth
from oracle import so2conv_oracle as O
from tests import _cases as H

pytestmark = pytest.mark.gpu
DT = torch.float64


def _incident(d, nodes):
    src, dst = d["src"], d["dst"]
    return np.nonzero(np.isin(dst, nodes) | np.isin(src, nodes))[0]


def _incoming(d, nodes):
    return np.nonzero(np.isin(d["dst"], nodes))[0]


@pytest.fixture(scope="module")
def medium():
    import so_graph_convolution_amd as K
    cfg = so2_synth.CONFIGS["M"]
    d = so2_synth.make_inputs(cfg)
    H.note(f"[full size] medium workload N={cfg.n_atoms} E={len(d['src'])}")
    dd = H.to_dev(d)
    args = (dd["kcfg"], dd["g"], dd["x"], dd["pos"], dd["rbf"], dd["w_rad"], dd["w1"], dd["w2"])
    E, N = len(d["src"]), cfg.n_atoms
    kc = dd["kcfg"]
    saved = torch.empty(K.so2conv_saved_bytes(kc, E), dtype=torch.uint8, device="cuda")
    ws = torch.empty(max(K.so2conv_workspace_bytes(kc, N, E, s) for s in (0, 1, 2)), dtype=torch.uint8, device="cuda")
    # as bench.py runs it: the backward keeps its cotangents for the double backward
    kept = torch.empty(K.so2conv_saved_bwd_bytes(kc, E), dtype=torch.uint8, device="cuda")
    y, _ = K.so2conv_fwd(*args, saved=saved, ws=ws)
    bw = K.so2conv_bwd(*args, saved, dd["gy"], ws=ws, saved_bwd=kept)
    db = K.so2conv_dbwd(*args, saved, dd["gy"], px=dd["px"], ppos=dd["ppos"], prbf=dd["prbf"], ws=ws,
                        saved_bwd=kept)
    torch.cuda.synchronize()
    out = dict(y=y.cpu(), **{k: (v.cpu() if isinstance(v, torch.Tensor) else [w.cpu() for w in v])
                             for k, v in {**bw, **db}.items() if v is not None and k != "saved_bwd"})
    del saved, ws, kept, bw, db
    torch.cuda.empty_cache()
    rng = np.random.default_rng(123)
    nodes = np.sort(rng.choice(N, 4, replace=False))
    edges = np.sort(rng.choice(E, 64, replace=False))
    return d, dd, out, nodes, edges


def test_full_size_forward_sampled(medium):
    d, dd, out, nodes, _ = medium
    inp = H.oracle_inputs(d)
    ref = O.forward(inp, edges=_incoming(d, nodes))[nodes]
    err = H.relerr(out["y"][nodes], ref)
    H.note(f"  y rel err {err:.2e}")
    assert err <= H.TOL_F32


def test_full_size_backward_sampled(medium):
    d, dd, out, nodes, edges = medium
    inp = H.oracle_inputs(d)
    gy = torch.tensor(d["gy"], dtype=DT)
    rn = O.backward(inp, gy, edges=_incident(d, nodes))
    re = O.backward(inp, gy, edges=edges, with_edge_grad=True)
    errs = {"gx": H.relerr(out["gx"][nodes], rn["gx"][nodes]),
            "gpos": H.relerr(out["gpos"][nodes], rn["gpos"][nodes]),
            "grbf": H.relerr(out["grbf"][edges], re["grbf"][edges]),
            "gedge": H.relerr(out["gedge"][edges], re["gedge"][edges])}
    H.note("  " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    assert all(v <= H.TOL_F32 for v in errs.values()), errs


def test_full_size_double_backward_sampled(medium):
    d, dd, out, nodes, edges = medium
    inp = H.oracle_inputs(d)
    t = lambda a: torch.tensor(a, dtype=DT)  # noqa: E731
    kw = dict(px=t(d["px"]), ppos=t(d["ppos"]), prbf=t(d["prbf"]))
    gy = t(d["gy"])
    r_in = O.double_backward(inp, gy, edges=_incoming(d, nodes), **kw)
    r_inc = O.double_backward(inp, gy, edges=_incident(d, nodes), **kw)
    r_e = O.double_backward(inp, gy, edges=edges, **kw)
    errs = {"ggy": H.relerr(out["ggy"][nodes], r_in["ggy"][nodes]),
            "gx2": H.relerr(out["gx2"][nodes], r_inc["gx"][nodes]),
            "grbf2": H.relerr(out["grbf2"][edges], r_e["grbf"][edges])}
    H.note("  " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    assert all(v <= H.TOL_F32 for v in errs.values()), errs


def test_full_size_weight_gradient_identity(medium):
    """y is linear in W2: <gW2, W2> = <gy, y> (Euler's identity for degree-1 functions)."""
    d, dd, out, _, _ = medium
    lhs = sum(float((g.double() * torch.tensor(w, dtype=DT)).sum()) for g, w in zip(out["gw2"], d["w2"]))
    rhs = float((out["y"].double() * torch.tensor(d["gy"], dtype=DT)).sum())
    H.note(f"  <gW2,W2>={lhs:.6e} <gy,y>={rhs:.6e}")
    assert abs(lhs - rhs) <= 1e-4 * abs(rhs)


def test_full_size_weight_gradients_additive(medium):
    """Weight gradients over all edges equal the sum over two halves of the receivers."""
    import so_graph_convolution_amd as K
    d, dd, out, _, _ = medium
    N = d["cfg"].n_atoms
    cut = int(np.searchsorted(d["dst"], N // 2))
    parts = []
    for sl in (slice(0, cut), slice(cut, len(d["src"]))):
        src = torch.tensor(d["src"][sl], device="cuda")
        dst = torch.tensor(d["dst"][sl], device="cuda")
        g = K.so2conv_graph_prepare(N, src, dst, torch.tensor(d["shift"][sl], device="cuda"))
        rbf = torch.tensor(d["rbf"][sl], device="cuda")
        args = (dd["kcfg"], g, dd["x"], dd["pos"], rbf, dd["w_rad"], dd["w1"], dd["w2"])
        _, saved = K.so2conv_fwd(*args, saved=True)
        b = K.so2conv_bwd(*args, saved, dd["gy"], need=("w1", "w2", "w_rad"))
        prbf = torch.tensor(d["prbf"][sl], device="cuda")
        c = K.so2conv_dbwd(*args, saved, dd["gy"], px=dd["px"], ppos=dd["ppos"], prbf=prbf,
                           need=("w1", "w2", "w_rad"))
        torch.cuda.synchronize()
        parts.append((b, c))
        del saved
        torch.cuda.empty_cache()
    errs = {}
    for key, src_key, k2 in (("gw1", 0, "gw1"), ("gw2", 0, "gw2"), ("gw_rad", 0, "gw_rad"),
                             ("gw1_2", 1, "gw1_2"), ("gw2_2", 1, "gw2_2"), ("gw_rad2", 1, "gw_rad2")):
        a, b = parts[0][src_key][k2], parts[1][src_key][k2]
        full = out[key]
        if isinstance(full, list):
            errs[key] = H.relerr(full, [(x + y).cpu() for x, y in zip(a, b)])
        else:
            errs[key] = H.relerr(full, (a + b).cpu())
    H.note("  " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    assert all(v <= H.TOL_F32 for v in errs.values()), errs


@pytest.fixture(scope="module")
def small():
    """eSEN-like small system: 2,000 atoms at 0.1 atoms/A^3, 6 A cutoff (~181k
    edges), lmax 2, mmax 2, C 128, float32; forward and backward with respect
    to features, weights and positions, with the saved forward state."""
    import so_graph_convolution_amd as K
    cfg = so2_synth.CONFIGS["S"]
    d = so2_synth.make_inputs(cfg)
    E, N = len(d["src"]), cfg.n_atoms
    H.note(f"[full size] small workload N={N} E={E}")
    dd = H.to_dev(d)
    args = (dd["kcfg"], dd["g"], dd["x"], dd["pos"], dd["rbf"], dd["w_rad"], dd["w1"], dd["w2"])
    y, saved = K.so2conv_fwd(*args, saved=True)
    bw = K.so2conv_bwd(*args, saved, dd["gy"])
    torch.cuda.synchronize()
    out = dict(y=y.cpu(), **{k: (v.cpu() if isinstance(v, torch.Tensor) else [w.cpu() for w in v])
                             for k, v in bw.items() if v is not None and k != "saved_bwd"})
    del saved, bw
    torch.cuda.empty_cache()
    rng = np.random.default_rng(321)
    nodes = np.sort(rng.choice(N, 6, replace=False))
    edges = np.sort(rng.choice(E, 64, replace=False))
    return d, dd, out, nodes, edges


def test_small_full_size_forward_backward_sampled(small):
    d, dd, out, nodes, edges = small
    inp = H.oracle_inputs(d)
    gy = torch.tensor(d["gy"], dtype=DT)
    ry = O.forward(inp, edges=_incoming(d, nodes))[nodes]
    rn = O.backward(inp, gy, edges=_incident(d, nodes))
    re = O.backward(inp, gy, edges=edges, with_edge_grad=True)
    errs = {"y": H.relerr(out["y"][nodes], ry),
            "gx": H.relerr(out["gx"][nodes], rn["gx"][nodes]),
            "gpos": H.relerr(out["gpos"][nodes], rn["gpos"][nodes]),
            "grbf": H.relerr(out["grbf"][edges], re["grbf"][edges]),
            "gedge": H.relerr(out["gedge"][edges], re["gedge"][edges])}
    H.note("  " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    assert all(v <= H.TOL_F32 for v in errs.values()), errs


def test_small_full_size_weight_gradients(small):
    """<gW2, W2> = <gy, y> (y is linear in W2), and every weight gradient over
    all edges equals the sum over two halves of the receivers."""
    import so_graph_convolution_amd as K
    d, dd, out, _, _ = small
    lhs = sum(float((g.double() * torch.tensor(w, dtype=DT)).sum()) for g, w in zip(out["gw2"], d["w2"]))
    rhs = float((out["y"].double() * torch.tensor(d["gy"], dtype=DT)).sum())
    H.note(f"  <gW2,W2>={lhs:.6e} <gy,y>={rhs:.6e}")
    assert abs(lhs - rhs) <= 1e-4 * abs(rhs)
    N = d["cfg"].n_atoms
    cut = int(np.searchsorted(d["dst"], N // 2))
    parts = []
    for sl in (slice(0, cut), slice(cut, len(d["src"]))):
        g = K.so2conv_graph_prepare(N, torch.tensor(d["src"][sl], device="cuda"),
                                    torch.tensor(d["dst"][sl], device="cuda"),
                                    torch.tensor(d["shift"][sl], device="cuda"))
        args = (dd["kcfg"], g, dd["x"], dd["pos"], torch.tensor(d["rbf"][sl], device="cuda"), dd["w_rad"],
                dd["w1"], dd["w2"])
        _, saved = K.so2conv_fwd(*args, saved=True)
        parts.append(K.so2conv_bwd(*args, saved, dd["gy"], need=("w1", "w2", "w_rad")))
        torch.cuda.synchronize()
    errs = {}
    for key in ("gw1", "gw2", "gw_rad"):
        a, b = parts[0][key], parts[1][key]
        full = out[key]
        errs[key] = H.relerr(full, [(x + y).cpu() for x, y in zip(a, b)]) if isinstance(full, list) \
            else H.relerr(full, (a + b).cpu())
    H.note("  " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    assert all(v <= H.TOL_F32 for v in errs.values()), errs
