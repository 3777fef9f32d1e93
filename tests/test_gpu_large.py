"""Full-size runs of the high-degree (lmax 6, ~1.05M edges) and the large
(100k atoms, ~10M edges, C 256, clustered degrees) workloads through the
memory-bounded chunked path, with sampled outputs checked against the oracle
on extracted subgraphs. Inputs of both hold bf16-representable values (the
pages' bf16 features and weights). The high-degree workload runs with
bfloat16 arrays (bar 2e-2) and in float32 (bar 1e-4); the large one with
bfloat16 arrays, its stated precision."""
import functools

import numpy as np
import pytest
import torch

import so2_synth
from oracle import so2conv_oracle as O
from tests import _cases as H

pytestmark = pytest.mark.gpu
DT = torch.float64


def _oracle_nodes(d, nodes, fn, key, edges_of):
    sub, ids = H.subgraph(d, edges_of(d, nodes))
    pos = np.searchsorted(ids, nodes)
    return fn(sub)[key][pos]


@functools.lru_cache(maxsize=2)
def _inputs(name, directions):
    H.note(f"[{name}] generating inputs")
    return so2_synth.make_inputs(so2_synth.CONFIGS[name], with_directions=directions)


_ORACLE = {}


def _cached(key, fn):
    if key not in _ORACLE:
        _ORACLE[key] = fn()
    return _ORACLE[key]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_high_degree_full_size_chunked(dtype):
    """Recompute chunks of 256k edges (no per-edge state across calls)."""
    import so_graph_convolution_amd as K
    cfg = so2_synth.CONFIGS["H"]
    d = _inputs("H", True)
    E, N = len(d["src"]), cfg.n_atoms
    H.note(f"[high degree {dtype}] N={N} E={E} L={cfg.lmax} C={cfg.channels}")
    dd = H.to_dev(d, dtype)
    args = (dd["kcfg"], dd["g"], dd["x"], dd["pos"], dd["rbf"], dd["w_rad"], dd["w1"], dd["w2"])
    torch.cuda.reset_peak_memory_stats()
    ce = 262144
    y, _ = K.so2conv_fwd(*args, saved=None, chunk_edges=ce)
    bw = K.so2conv_bwd(*args, None, dd["gy"], chunk_edges=ce)
    db = K.so2conv_dbwd(*args, None, dd["gy"], px=dd["px"], ppos=dd["ppos"], prbf=dd["prbf"], chunk_edges=ce)
    torch.cuda.synchronize()
    H.note(f"  peak device memory {torch.cuda.max_memory_allocated() / 2**30:.1f} GiB")
    _check_high_degree(d, dtype, y, bw, db)


@pytest.mark.timeout(900)
def test_high_degree_full_size_bench_configuration():
    """bf16 as bench.py --config H runs it: the saved forward state, one
    workspace sized for 256k-edge chunks, and the backward's cotangents kept
    for the double backward."""
    import so_graph_convolution_amd as K
    cfg = so2_synth.CONFIGS["H"]
    d = _inputs("H", True)
    E, N = len(d["src"]), cfg.n_atoms
    H.note(f"[high degree bench configuration] N={N} E={E} L={cfg.lmax} C={cfg.channels}")
    dd = H.to_dev(d, "bf16")
    kc = dd["kcfg"]
    args = (kc, dd["g"], dd["x"], dd["pos"], dd["rbf"], dd["w_rad"], dd["w1"], dd["w2"])
    saved = torch.empty(K.so2conv_saved_bytes(kc, E), dtype=torch.uint8, device="cuda")
    ws = torch.empty(max(K.so2conv_chunked_workspace_bytes(kc, N, E, s, 262144) for s in (0, 1, 2)),
                     dtype=torch.uint8, device="cuda")
    kept = torch.empty(K.so2conv_saved_bwd_bytes(kc, E), dtype=torch.uint8, device="cuda")
    y, _ = K.so2conv_fwd(*args, saved=saved, ws=ws)
    bw = K.so2conv_bwd(*args, saved, dd["gy"], ws=ws, saved_bwd=kept)
    db = K.so2conv_dbwd(*args, saved, dd["gy"], px=dd["px"], ppos=dd["ppos"], prbf=dd["prbf"], ws=ws, saved_bwd=kept)
    torch.cuda.synchronize()
    del saved, ws, kept
    torch.cuda.empty_cache()
    _check_high_degree(d, "bf16", y, bw, db)


def _check_high_degree(d, dtype, y, bw, db):
    cfg = so2_synth.CONFIGS["H"]
    E, N = len(d["src"]), cfg.n_atoms
    rng = np.random.default_rng(7)
    nodes = np.sort(rng.choice(N, 3, replace=False))
    edges = np.sort(rng.choice(E, 32, replace=False))
    t = lambda a: torch.tensor(a, dtype=DT)  # noqa: E731

    def fwd(sub):
        return {"y": O.forward(H.oracle_inputs(sub))}

    def bwd(sub):
        return O.backward(H.oracle_inputs(sub), t(sub["gy"]), with_edge_grad=True)

    def dbwd(sub):
        return O.double_backward(H.oracle_inputs(sub), t(sub["gy"]), px=t(sub["px"]), ppos=t(sub["ppos"]),
                                 prbf=t(sub["prbf"]))
    ref = _cached("H", lambda: {
        "y": _oracle_nodes(d, nodes, fwd, "y", H.incoming),
        "gx": _oracle_nodes(d, nodes, bwd, "gx", H.incident),
        "gpos": _oracle_nodes(d, nodes, bwd, "gpos", H.incident),
        "ggy": _oracle_nodes(d, nodes, dbwd, "ggy", H.incoming),
        "gx2": _oracle_nodes(d, nodes, dbwd, "gx", H.incident),
        "edges": (bwd(H.subgraph(d, edges)[0]), dbwd(H.subgraph(d, edges)[0]))})
    errs = {
        "y": H.relerr(y.cpu()[nodes], ref["y"]),
        "gx": H.relerr(bw["gx"].cpu()[nodes], ref["gx"]),
        "gpos": H.relerr(bw["gpos"].cpu()[nodes], ref["gpos"]),
        "ggy": H.relerr(db["ggy"].cpu()[nodes], ref["ggy"]),
        "gx2": H.relerr(db["gx2"].cpu()[nodes], ref["gx2"]),
    }
    re_b, re_d = ref["edges"]
    errs["grbf"] = H.relerr(bw["grbf"].cpu()[edges], re_b["grbf"])
    errs["gedge"] = H.relerr(bw["gedge"].cpu()[edges], re_b["gedge"])
    errs["grbf2"] = H.relerr(db["grbf2"].cpu()[edges], re_d["grbf"])
    # weight gradients over all ~1.05M edges: y is linear in W2, so <gW2, W2> = <y, gy>;
    # T = s * (D a) is linear in x, rbf and W_rad and T W1 is bilinear, so
    # <gW1, W1> = <gW_rad, W_rad> = <grbf, rbf> = <gx, x>
    dot = lambda a, b: float((a.double().cpu() * t(np.asarray(b))).sum())  # noqa: E731
    rhs = dot(y, d["gy"])
    errs["<gW2,W2>"] = abs(sum(dot(g, w) for g, w in zip(bw["gw2"], d["w2"])) - rhs) / abs(rhs)
    ref = dot(bw["gx"], d["x"])
    errs["<gW1,W1>"] = abs(sum(dot(g, w) for g, w in zip(bw["gw1"], d["w1"])) - ref) / abs(ref)
    errs["<gWrad,Wrad>"] = abs(dot(bw["gw_rad"], d["w_rad"]) - ref) / abs(ref)
    errs["<grbf,rbf>"] = abs(dot(bw["grbf"], d["rbf"]) - ref) / abs(ref)
    H.note("  " + " ".join(f"{k}={v:.1e}" for k, v in errs.items()))
    tol = H.TOL_BF16 if dtype == "bf16" else H.TOL_F32
    assert all(v <= tol for v in errs.values()), errs


@pytest.mark.timeout(1100)
def test_large_system_full_size_chunked():
    """Forward + backward of the 100k-atom clustered system with bfloat16
    features and weights; peak device memory is reported next to the bytes a
    schedule keeping every per-edge intermediate would need."""
    import so_graph_convolution_amd as K
    cfg = so2_synth.CONFIGS["X"]
    d = _inputs("X", ("gy",))
    E, N = len(d["src"]), cfg.n_atoms
    H.note(f"[large bf16] N={N} E={E} L={cfg.lmax} C={cfg.channels} max in-degree "
           f"{int(np.bincount(d['dst'], minlength=N).max())}")
    dd = H.to_dev(d, "bf16")
    args = (dd["kcfg"], dd["g"], dd["x"], dd["pos"], dd["rbf"], dd["w_rad"], dd["w1"], dd["w2"])
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    ce = 262144
    y, _ = K.so2conv_fwd(*args, saved=None, chunk_edges=ce)
    bw = K.so2conv_bwd(*args, None, dd["gy"], need=("x", "pos", "rbf", "w_rad", "w1", "w2", "edge"), chunk_edges=ce)
    torch.cuda.synchronize()
    peak = torch.cuda.max_memory_allocated()
    kc = dd["kcfg"]
    state = K.so2conv_saved_bytes(kc, E)
    H.note(f"  peak device memory {peak / 2**30:.1f} GiB; keeping the per-edge forward state alone would take "
           f"{state / 2**30:.0f} GiB (GEMM inputs and outputs only)")
    assert peak < 120 * 2**30
    deg = np.bincount(d["dst"], minlength=N)
    rng = np.random.default_rng(8)
    nodes = np.sort(np.concatenate([[int(np.argmax(deg))], rng.choice(N, 2, replace=False)]))
    t = lambda a: torch.tensor(a, dtype=DT)  # noqa: E731

    def fwd(sub):
        return {"y": O.forward(H.oracle_inputs(sub))}

    def bwd(sub):
        return O.backward(H.oracle_inputs(sub), t(sub["gy"]), with_edge_grad=True)
    errs = {
        "y": H.relerr(y.cpu()[nodes], _oracle_nodes(d, nodes, fwd, "y", H.incoming)),
        "gx": H.relerr(bw["gx"].cpu()[nodes], _oracle_nodes(d, nodes, bwd, "gx", H.incident)),
        "gpos": H.relerr(bw["gpos"].cpu()[nodes], _oracle_nodes(d, nodes, bwd, "gpos", H.incident)),
    }
    edges = np.sort(rng.choice(E, 32, replace=False))
    sub, _ = H.subgraph(d, edges)
    re_b = bwd(sub)
    errs["grbf"] = H.relerr(bw["grbf"].cpu()[edges], re_b["grbf"])
    errs["gedge"] = H.relerr(bw["gedge"].cpu()[edges], re_b["gedge"])
    # weight gradients over all ~10M edges: T = s * (D a) is linear in x, rbf and W_rad and
    # T W1 is bilinear, so <gW1, W1> = <gW_rad, W_rad> = <grbf, rbf> = <gx, x>; y is linear
    # in W2, so <gW2, W2> = <gy, y> (gx and grbf are checked element-wise above)
    dot = lambda a, b: float((a.double().cpu() * torch.as_tensor(np.asarray(b), dtype=DT)).sum())  # noqa: E731
    ref = dot(bw["gx"], d["x"])
    for key, val in (("<gW1,W1>", sum(dot(g, w) for g, w in zip(bw["gw1"], d["w1"]))),
                     ("<gWrad,Wrad>", dot(bw["gw_rad"], d["w_rad"])), ("<grbf,rbf>", dot(bw["grbf"], d["rbf"]))):
        errs[key] = abs(val - ref) / abs(ref)
    yy = dot(y, d["gy"])
    errs["<gW2,W2>"] = abs(sum(dot(g, w) for g, w in zip(bw["gw2"], d["w2"])) - yy) / abs(yy)
    H.note("  " + " ".join(f"{k}={v:.1e}" for k, v in errs.items()))
    assert all(v <= H.TOL_BF16 for v in errs.values()), errs
