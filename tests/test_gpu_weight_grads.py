"""Weight gradients at the full sizes, element by element against the oracle.

A weight gradient sums over every edge, and the GPU reduces those sums in
split-K trees whose depth grows with the edge count (725k rows at the medium
system, 2E rows for the complex orders). The oracle's gradients over the same
edges come from tests/golden/make_weight_grad_fixtures.py (oracle only) as
sampled fixtures: a seeded sample of elements, the tensor's maximum and
Frobenius norm, and four projections on seeded normal arrays. Each GPU
gradient is compared on the sampled elements (max-norm and floored
element-wise errors) and through the projections (error / Frobenius norm).

Cases, each in the launch configuration bench.py times for its workload:
  * small system (2,000 atoms, lmax 2, C 128), backward over all 180,658 edges;
  * medium system (10,000 atoms, lmax 4, C 128), backward over all 725,020 edges;
  * medium system, double backward (force pattern) on a block of receivers
    with >= 100,000 incoming edges;
  * high-degree system (lmax 6, bf16), backward and double backward on a
    >= 100,000-edge receiver block;
  * large clustered system (C 256, bf16), backward on a >= 65,536-edge block;
  * the mixture of 64 linear experts on the medium system split into 16
    systems, backward on the first two systems' edges: expert, radial and
    coefficient gradients.
"""
import functools
import os

import numpy as np
import pytest
import torch

import so2_synth
from tests import _cases as H
from tests.golden import make_weight_grad_fixtures as FX

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _fixture(name):
    path = os.path.join(GOLDEN, f"weight_grads_{name}.npz")
    if not os.path.exists(path):
        pytest.skip(f"fixture {path} not written (tests/golden/make_weight_grad_fixtures.py {name})")
    return dict(np.load(path, allow_pickle=False))


@functools.lru_cache(maxsize=1)
def _inputs(cfg_name):
    return so2_synth.make_inputs(so2_synth.CONFIGS[cfg_name])


def _block(d, e_end):
    """The workload restricted to its first e_end edges (whole receivers; every node kept)."""
    if e_end == len(d["src"]):
        return d
    sub = dict(d)
    for k in ("src", "dst", "shift", "rbf", "prbf"):
        sub[k] = d[k][:e_end]
    return sub


def _run(cfg_name, stage, e_end):
    """Weight gradients of the GPU path as bench.py runs the workload: saved forward
    state, one workspace, the backward's cotangents kept for the double backward
    (the large system: recompute chunks of 256k edges, no state)."""
    import so_graph_convolution_amd as K
    cfg = so2_synth.CONFIGS[cfg_name]
    d = _block(_inputs(cfg_name), e_end)
    dtype = cfg.dtype
    dd = H.to_dev(d, dtype)
    kc = dd["kcfg"]
    N, E = cfg.n_atoms, e_end
    H.note(f"[weight grads] {cfg_name} {stage} {dtype} over {E} edges")
    args = (kc, dd["g"], dd["x"], dd["pos"], dd["rbf"], dd["w_rad"], dd["w1"], dd["w2"])
    if cfg_name == "X":
        ce = 262144
        K.so2conv_fwd(*args, saved=None, chunk_edges=ce)
        out = K.so2conv_bwd(*args, None, dd["gy"], need=("w1", "w2", "w_rad"), chunk_edges=ce)
        torch.cuda.synchronize()
        return {k: (out[k].cpu() if isinstance(out[k], torch.Tensor) else [w.cpu() for w in out[k]])
                for k in ("gw1", "gw2", "gw_rad")}
    chunk = 262144 if cfg_name == "H" else None
    if chunk:
        wsb = max(K.so2conv_chunked_workspace_bytes(kc, N, E, s, chunk) for s in (0, 1, 2))
    else:
        wsb = max(K.so2conv_workspace_bytes(kc, N, E, s) for s in (0, 1, 2))
    saved = torch.empty(K.so2conv_saved_bytes(kc, E), dtype=torch.uint8, device="cuda")
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    kept = torch.empty(K.so2conv_saved_bwd_bytes(kc, E), dtype=torch.uint8, device="cuda")
    K.so2conv_fwd(*args, saved=saved, ws=ws)
    bw = K.so2conv_bwd(*args, saved, dd["gy"], ws=ws, saved_bwd=kept)
    if stage == "bwd":
        res = {k: bw[k] for k in ("gw1", "gw2", "gw_rad")}
    else:
        db = K.so2conv_dbwd(*args, saved, dd["gy"], px=dd["px"], ppos=dd["ppos"], prbf=dd["prbf"], ws=ws,
                            saved_bwd=kept)
        res = {"gw1": db["gw1_2"], "gw2": db["gw2_2"], "gw_rad": db["gw_rad2"]}
    torch.cuda.synchronize()
    res = {k: (v.cpu() if isinstance(v, torch.Tensor) else [w.cpu() for w in v]) for k, v in res.items()}
    del saved, ws, kept, bw
    torch.cuda.empty_cache()
    return res


def _run_mole(cfg_name, e_end, n_sys):
    """Expert, radial and coefficient gradients of the mixture as bench.py --op
    mole runs it (saved forward state, one workspace), on the first n_sys
    systems' edges."""
    import so_graph_convolution_amd as K
    d = _block(_inputs(cfg_name), e_end)
    _, mb = FX.mole_block(_inputs(cfg_name), n_sys)
    dd = H.to_dev(d)
    kc, N, E = dd["kcfg"], so2_synth.CONFIGS[cfg_name].n_atoms, e_end
    H.note(f"[weight grads] {cfg_name} mixture bwd over {E} edges, {n_sys} systems, {FX.MOLE_EXPERTS} experts")
    w1e = [torch.tensor(w, device="cuda") for w in mb["w1e"]]
    w2e = [torch.tensor(w, device="cuda") for w in mb["w2e"]]
    coef = torch.tensor(mb["coef"], device="cuda")
    mix = K.Mixture(FX.MOLE_EXPERTS, mb["sys_edge_ptr"])
    args = (kc, dd["g"], mix, dd["x"], dd["pos"], dd["rbf"], dd["w_rad"], w1e, w2e, coef)
    saved = torch.empty(K.so2conv_saved_bytes(kc, E), dtype=torch.uint8, device="cuda")
    ws = torch.empty(max(K.so2mole_workspace_bytes(kc, mix, N, E, s, 0) for s in (0, 1)), dtype=torch.uint8,
                     device="cuda")
    K.so2mole_fwd(*args, saved=saved, ws=ws)
    bw = K.so2mole_bwd(*args, saved, dd["gy"], ws=ws)
    torch.cuda.synchronize()
    res = {"gw1e": [w.cpu() for w in bw["gw1e"]], "gw2e": [w.cpu() for w in bw["gw2e"]],
           "gw_rad": bw["gw_rad"].cpu(), "gcoef": bw["gcoef"].cpu()}
    del saved, ws, bw
    torch.cuda.empty_cache()
    return res


def _compare(name):
    fx = _fixture(name)
    cfg_name, stage = str(fx["config"]), str(fx["stage"])
    e_end = int(fx["edge_end"])
    if stage == "mole_bwd":
        got = _run_mole(cfg_name, e_end, FX.FIXTURES[name][2])
    else:
        got = _run(cfg_name, stage, e_end)
    dtype = so2_synth.CONFIGS[cfg_name].dtype
    tol = H.TOL_BF16 if dtype == "bf16" else H.TOL_F32
    tol_elem = H.TOL_ELEM_BF16 if dtype == "bf16" else H.TOL_ELEM_F32
    floor = H.FLOOR_BF16 if dtype == "bf16" else H.FLOOR_F32
    worst = {}
    for k_tensor, (key, g) in enumerate(FX.tensor_list(got)):
        a = g.double().numpy()
        idx, val = fx[f"{key}/idx"], fx[f"{key}/val"]
        mx, fro = float(fx[f"{key}/maxabs"]), float(fx[f"{key}/fro"])
        s = a.reshape(-1)[idx]
        proj = np.array([(a * FX.projection_direction(k_tensor, k, a.shape)).sum() for k in range(FX.N_PROJ)])
        worst[key] = {"max": float(np.abs(s - val).max() / mx),
                      "elem": float((np.abs(s - val) / (np.abs(val) + floor * mx)).max()),
                      "proj": float(np.abs(proj - fx[f"{key}/proj"]).max() / fro),
                      "maxabs": abs(float(np.abs(a).max()) - mx) / mx}
    for key, e in worst.items():
        H.note(f"  {key}: " + " ".join(f"{k}={v:.2e}" for k, v in e.items()))
    bad = {key: e for key, e in worst.items()
           if not all(v <= (tol_elem if k == "elem" else tol) for k, v in e.items())}
    assert not bad, bad


@pytest.mark.timeout(300)
def test_small_backward_all_edges():
    _compare("S_bwd_all")


@pytest.mark.timeout(300)
def test_medium_backward_all_edges():
    _compare("M_bwd_all")


@pytest.mark.timeout(300)
def test_medium_double_backward_receiver_block():
    _compare("M_dbwd_block")


@pytest.mark.timeout(300)
def test_high_degree_backward_receiver_block():
    _compare("H_bwd_block")


@pytest.mark.timeout(300)
def test_high_degree_double_backward_receiver_block():
    _compare("H_dbwd_block")


@pytest.mark.timeout(600)
def test_large_backward_receiver_block():
    _compare("X_bwd_block")


@pytest.mark.timeout(300)
def test_mixture_backward_two_systems():
    _compare("M_mole_bwd_block")
