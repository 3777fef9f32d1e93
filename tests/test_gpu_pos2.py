"""Position derivatives of the double backward (gpos2): d/dpos of
L = <px, gx> + <ppos, gpos> + <pedge, gedge> + <prbf, grbf> + <pW, gW>,
through the edge frames and the tangent's rotation rates, against the
oracle's autograd value (pinned on the CPU by finite differences of the
backward)."""
import numpy as np
import pytest
import torch

from oracle import so2conv_oracle as O
from tests import _cases as H
from tests.test_gpu_bwd import DBWD_CASES

pytestmark = pytest.mark.gpu
DT = torch.float64
ALL = ("gy", "x", "pos", "rbf", "w_rad", "w1", "w2")
OTHERS = ("ggy", "gx2", "grbf2", "gw_rad2", "gw1_2", "gw2_2")


def _args(dd):
    return (dd["kcfg"], dd["g"], dd["x"], dd["pos"], dd["rbf"], dd["w_rad"], dd["w1"], dd["w2"])


def _t(a):
    return None if a is None else torch.tensor(a, dtype=DT)


@pytest.mark.parametrize("name,base,over", DBWD_CASES, ids=[c[0] for c in DBWD_CASES])
def test_gpos2_force_pattern(name, base, over):
    import so_graph_convolution_amd as K
    d = H.workload(base, **over)
    cfg = d["cfg"]
    H.note(f"[gpos2] {name} L={cfg.lmax} M={cfg.mmax} C={cfg.channels} E={len(d['src'])}")
    dd = H.to_dev(d)
    args = _args(dd)
    y, saved = K.so2conv_fwd(*args, saved=True)
    dirs = dict(px=dd["px"], ppos=dd["ppos"], prbf=dd["prbf"])
    out = K.so2conv_dbwd(*args, saved, dd["gy"], need=ALL, **dirs)
    base_out = K.so2conv_dbwd(*args, saved, dd["gy"], **dirs)
    torch.cuda.synchronize()
    # requesting gpos2 leaves every other output bitwise unchanged
    for k in OTHERS:
        a, b = out[k], base_out[k]
        assert all(torch.equal(u, v) for u, v in zip(a, b)) if isinstance(a, list) else torch.equal(a, b), k
    ref = O.double_backward(H.oracle_inputs(d), _t(d["gy"]), px=_t(d["px"]), ppos=_t(d["ppos"]), prbf=_t(d["prbf"]))
    err = H.relerr(out["gpos2"], ref["gpos"])
    H.note(f"  gpos2={err:.2e}  |sum| {float(out['gpos2'].double().sum(0).abs().max()):.1e}")
    assert err <= H.TOL_F32
    # translation invariance: the node sums cancel
    assert float(out["gpos2"].double().sum(0).abs().max()) <= 1e-4 * float(out["gpos2"].abs().max()) + 1e-6


@pytest.mark.parametrize("only", ["ppos", "px", "pedge", "prbf", "pw"])
def test_gpos2_single_direction(only):
    """Each direction alone: rotation-rate terms (ppos, pedge) and the terms with
    a zero rate (px, prbf, weights) separately."""
    import so_graph_convolution_amd as K
    d = H.workload("T", n_atoms=40, box=8.0, rc=3.5, lmax=3, mmax=2, channels=16, n_rbf=8, seed=12, min_dist=0.0)
    dd = H.to_dev(d)
    args = _args(dd)
    g = np.random.default_rng(5)
    dv = lambda a: torch.tensor(a, device="cuda")  # noqa: E731
    host = {}
    if only == "ppos":
        host["ppos"] = d["ppos"]
    elif only == "px":
        host["px"] = d["px"]
    elif only == "prbf":
        host["prbf"] = d["prbf"]
    elif only == "pedge":
        host["pedge"] = g.normal(size=(len(d["src"]), 3)).astype(np.float32)
    else:
        host["pw_rad"] = g.normal(size=d["w_rad"].shape).astype(np.float32)
        host["pw1"] = [(g.normal(size=w.shape) * 0.1).astype(np.float32) for w in d["w1"]]
        host["pw2"] = [(g.normal(size=w.shape) * 0.1).astype(np.float32) for w in d["w2"]]
    dev = {k: ([dv(w) for w in v] if isinstance(v, list) else dv(v)) for k, v in host.items()}
    y, saved = K.so2conv_fwd(*args, saved=True)
    out = K.so2conv_dbwd(*args, saved, dd["gy"], need=("pos",), **dev)
    torch.cuda.synchronize()
    ref = O.double_backward(H.oracle_inputs(d), _t(d["gy"]),
                            **{k: ([_t(w) for w in v] if isinstance(v, list) else _t(v)) for k, v in host.items()})
    err = H.relerr(out["gpos2"], ref["gpos"])
    H.note(f"[gpos2 {only}] {err:.2e}")
    assert err <= H.TOL_F32


def test_gpos2_all_directions_chunked():
    import so_graph_convolution_amd as K
    d = H.workload("T", n_atoms=150, box=12.0, rc=4.0, lmax=4, mmax=2, channels=48, n_rbf=16, seed=5, min_dist=0.0)
    E = len(d["src"])
    assert E > 1024
    dd = H.to_dev(d)
    args = _args(dd)
    g = np.random.default_rng(17)
    pw_rad = g.normal(size=d["w_rad"].shape).astype(np.float32)
    pw1 = [(g.normal(size=w.shape) * 0.1).astype(np.float32) for w in d["w1"]]
    pw2 = [(g.normal(size=w.shape) * 0.1).astype(np.float32) for w in d["w2"]]
    pedge = g.normal(size=(E, 3)).astype(np.float32)
    dv = lambda a: torch.tensor(a, device="cuda")  # noqa: E731
    kw = dict(px=dd["px"], ppos=dd["ppos"], pedge=dv(pedge), prbf=dd["prbf"], pw_rad=dv(pw_rad),
              pw1=[dv(w) for w in pw1], pw2=[dv(w) for w in pw2])
    y, _ = K.so2conv_fwd(*args, saved=None, chunk_edges=1024)
    out = K.so2conv_dbwd(*args, None, dd["gy"], need=ALL, chunk_edges=1024, **kw)
    torch.cuda.synchronize()
    ref = O.double_backward(H.oracle_inputs(d), _t(d["gy"]), px=_t(d["px"]), ppos=_t(d["ppos"]), prbf=_t(d["prbf"]),
                            pw_rad=_t(pw_rad), pw1=[_t(w) for w in pw1], pw2=[_t(w) for w in pw2], pedge=_t(pedge))
    pairs = {"gpos2": "gpos", "ggy": "ggy", "gx2": "gx", "grbf2": "grbf", "gw_rad2": "gw_rad", "gw1_2": "gw1",
             "gw2_2": "gw2"}
    errs = {k: H.relerr(out[k], ref[v]) for k, v in pairs.items()}
    H.note("[gpos2 all directions, 1024-edge chunks] " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    assert all(v <= H.TOL_F32 for v in errs.values()), errs


def test_gpos2_bf16_and_empty():
    import so_graph_convolution_amd as K
    d = H.workload("T", dtype="bf16", n_atoms=48, box=9.0, rc=4.5, lmax=6, mmax=2, channels=16, n_rbf=8, seed=11)
    dd = H.to_dev(d, "bf16")
    args = _args(dd)
    y, saved = K.so2conv_fwd(*args, saved=True)
    out = K.so2conv_dbwd(*args, saved, dd["gy"], need=ALL, px=dd["px"], ppos=dd["ppos"], prbf=dd["prbf"])
    torch.cuda.synchronize()
    assert out["gpos2"].dtype == torch.float32
    ref = O.double_backward(H.oracle_inputs(d), _t(d["gy"]), px=_t(d["px"]), ppos=_t(d["ppos"]), prbf=_t(d["prbf"]))
    err = H.relerr(out["gpos2"], ref["gpos"])
    H.note(f"[gpos2 bf16 lmax 6] {err:.2e}")
    assert err <= H.TOL_BF16
    kc = dd["kcfg"]
    e = torch.zeros(0, dtype=torch.int32, device="cuda")
    g0 = K.so2conv_graph_prepare(d["cfg"].n_atoms, e, e, torch.zeros(0, 3, device="cuda"))
    rbf0 = torch.zeros(0, kc.n_rbf, device="cuda")
    a0 = (kc, g0, dd["x"], dd["pos"], rbf0, dd["w_rad"], dd["w1"], dd["w2"])
    y0, s0 = K.so2conv_fwd(*a0, saved=True)
    o0 = K.so2conv_dbwd(*a0, s0, dd["gy"], need=ALL, px=dd["px"], ppos=dd["ppos"])
    torch.cuda.synchronize()
    assert not bool(o0["gpos2"].any())
