"""GPU parity of the backward and double backward against the float64 oracle
(autograd derivatives of the plain definition)."""
import numpy as np
import pytest
import torch

from oracle import so2conv_oracle as O
from tests import _cases as H
from tests.test_gpu_fwd import FWD_CASES

pytestmark = pytest.mark.gpu

DT = torch.float64


def _run_fwd(dd):
    import so_graph_convolution_amd as K
    args = (dd["kcfg"], dd["g"], dd["x"], dd["pos"], dd["rbf"], dd["w_rad"], dd["w1"], dd["w2"])
    y, saved = K.so2conv_fwd(*args, saved=True)
    return args, y, saved


@pytest.mark.parametrize("name,base,over", FWD_CASES, ids=[c[0] for c in FWD_CASES])
def test_backward_matches_oracle(name, base, over):
    import so_graph_convolution_amd as K
    d = H.workload(base, **over)
    cfg = d["cfg"]
    H.note(f"[backward] {name} L={cfg.lmax} M={cfg.mmax} C={cfg.channels} E={len(d['src'])}")
    dd = H.to_dev(d)
    args, y, saved = _run_fwd(dd)
    out = K.so2conv_bwd(*args, saved, dd["gy"])
    torch.cuda.synchronize()
    ref = O.backward(H.oracle_inputs(d), torch.tensor(d["gy"], dtype=DT), with_edge_grad=True)
    errs = {k: H.relerr(out[k], ref[k]) for k in ("gx", "gpos", "grbf", "gw_rad", "gw1", "gw2", "gedge")}
    H.note("  " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    assert all(v <= H.TOL_F32 for v in errs.values()), errs


DBWD_CASES = [c for c in FWD_CASES if c[0] in ("tiny_T", "l4m2_c48_ragged", "l3m1_c32", "l6m2_c16", "l0m0_c16",
                                                  "l4m4_c16")]


@pytest.mark.parametrize("name,base,over", DBWD_CASES, ids=[c[0] for c in DBWD_CASES])
def test_double_backward_force_pattern(name, base, over):
    """Directions on (x, pos, rbf) only: the force-training pattern (p_W = 0)."""
    import so_graph_convolution_amd as K
    d = H.workload(base, **over)
    cfg = d["cfg"]
    H.note(f"[double_backward] {name} L={cfg.lmax} M={cfg.mmax} C={cfg.channels} E={len(d['src'])}")
    dd = H.to_dev(d)
    args, y, saved = _run_fwd(dd)
    out = K.so2conv_dbwd(*args, saved, dd["gy"], px=dd["px"], ppos=dd["ppos"], prbf=dd["prbf"])
    torch.cuda.synchronize()
    t = lambda a: torch.tensor(a, dtype=DT)  # noqa: E731
    ref = O.double_backward(H.oracle_inputs(d), t(d["gy"]), px=t(d["px"]), ppos=t(d["ppos"]), prbf=t(d["prbf"]))
    pairs = {"ggy": "ggy", "gx2": "gx", "grbf2": "grbf", "gw_rad2": "gw_rad", "gw1_2": "gw1", "gw2_2": "gw2"}
    errs = {k: H.relerr(out[k], ref[v]) for k, v in pairs.items()}
    H.note("  " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    assert all(v <= H.TOL_F32 for v in errs.values()), errs


def test_double_backward_all_directions():
    """Every direction nonzero, including weight and edge-vector directions."""
    import so_graph_convolution_amd as K
    d = H.workload("T", n_atoms=40, box=8.0, rc=3.5, lmax=3, mmax=2, channels=16, n_rbf=8, seed=12, min_dist=0.0)
    H.note(f"[double_backward all] E={len(d['src'])}")
    dd = H.to_dev(d)
    args, y, saved = _run_fwd(dd)
    g = np.random.default_rng(99)
    pw_rad = g.normal(size=d["w_rad"].shape).astype(np.float32)
    pw1 = [g.normal(size=w.shape).astype(np.float32) * 0.1 for w in d["w1"]]
    pw2 = [g.normal(size=w.shape).astype(np.float32) * 0.1 for w in d["w2"]]
    pedge = g.normal(size=(len(d["src"]), 3)).astype(np.float32)
    dv = lambda a: torch.tensor(a, device="cuda")  # noqa: E731
    out = K.so2conv_dbwd(*args, saved, dd["gy"], px=dd["px"], ppos=dd["ppos"], pedge=dv(pedge), prbf=dd["prbf"],
                         pw_rad=dv(pw_rad), pw1=[dv(w) for w in pw1], pw2=[dv(w) for w in pw2])
    torch.cuda.synchronize()
    t = lambda a: torch.tensor(a, dtype=DT)  # noqa: E731
    ref = O.double_backward(H.oracle_inputs(d), t(d["gy"]), px=t(d["px"]), ppos=t(d["ppos"]), prbf=t(d["prbf"]),
                            pw_rad=t(pw_rad), pw1=[t(w) for w in pw1], pw2=[t(w) for w in pw2], pedge=t(pedge))
    pairs = {"ggy": "ggy", "gx2": "gx", "grbf2": "grbf", "gw_rad2": "gw_rad", "gw1_2": "gw1", "gw2_2": "gw2"}
    errs = {k: H.relerr(out[k], ref[v]) for k, v in pairs.items()}
    H.note("  " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    assert all(v <= H.TOL_F32 for v in errs.values()), errs


def test_backward_deterministic():
    import so_graph_convolution_amd as K
    d = H.workload("T", n_atoms=150, box=12.0, rc=4.0, lmax=4, mmax=2, channels=48, n_rbf=16, seed=5, min_dist=0.0)
    dd = H.to_dev(d)
    args, y, saved = _run_fwd(dd)
    a = K.so2conv_bwd(*args, saved, dd["gy"])
    b = K.so2conv_bwd(*args, saved, dd["gy"])
    c = K.so2conv_dbwd(*args, saved, dd["gy"], px=dd["px"], ppos=dd["ppos"], prbf=dd["prbf"])
    e = K.so2conv_dbwd(*args, saved, dd["gy"], px=dd["px"], ppos=dd["ppos"], prbf=dd["prbf"])
    torch.cuda.synchronize()
    for k in ("gx", "gpos", "grbf", "gw_rad", "gedge"):
        assert torch.equal(a[k], b[k]), k
    for k in ("gw1", "gw2"):
        assert all(torch.equal(u, v) for u, v in zip(a[k], b[k])), k
    for k in ("ggy", "gx2", "grbf2", "gw_rad2"):
        assert torch.equal(c[k], e[k]), k


def test_torque_has_no_roll_component():
    """The operator is invariant to the frame's roll about each edge, so the
    per-edge torque has no component along the edge: the edge gradient
    gedge = rhat x tau / rho is orthogonal to the edge, and sum_i gpos_i = 0."""
    import so_graph_convolution_amd as K
    d = H.workload("T", seed=4)
    dd = H.to_dev(d)
    args, y, saved = _run_fwd(dd)
    out = K.so2conv_bwd(*args, saved, dd["gy"])
    torch.cuda.synchronize()
    v = (torch.tensor(d["pos"][d["src"]].astype(np.float64) - d["pos"][d["dst"]] + d["shift"]))
    ge = out["gedge"].double().cpu()
    assert float((ge * v).sum(1).abs().max()) <= 1e-5 * float(ge.abs().max() * v.abs().max())
    gp = out["gpos"].double().cpu()
    assert float(gp.sum(0).abs().max()) <= 1e-4 * float(gp.abs().max())
