"""Node-to-node spherical projection with fused channel maps (TrimSO(2) page,
Appendix B.4) through the C ABI, against the float64 oracle (the
unreassociated definition, autograd derivatives). Bar: 1e-4 max-norm
relative error per output."""
import numpy as np
import pytest
import torch

from oracle import grid_oracle as GO
from tests import _cases as H

pytestmark = pytest.mark.gpu
DT = torch.float64

CASES = [  # (name, lmax, c_in, c_h, c_out, n_grid, n_nodes)
    ("l2_small_ragged", 2, 16, 32, 16, 18, 37),
    ("l4_eqv3_widths", 4, 128, 256, 128, 100, 301),
    ("l6_ragged", 6, 32, 64, 48, 200, 75),
    ("l0_tiny", 0, 4, 8, 4, 1, 5),
    ("l3_grid_tiles", 3, 64, 32, 96, 65, 130),
]


def _inputs(L, ci, ch, co, ng, N, seed):
    rng = np.random.default_rng(seed)
    d = (L + 1) ** 2
    a = dict(x=rng.normal(size=(N, d, ci)), G=rng.normal(size=(ng, d)) / np.sqrt(d),
             W=rng.normal(size=(L + 1, ci, ch)) / np.sqrt(ci), A=rng.normal(size=(ch, co)) / np.sqrt(ch),
             gU=rng.normal(size=(N, ng, co)), px=rng.normal(size=(N, d, ci)),
             pW=rng.normal(size=(L + 1, ci, ch)) / np.sqrt(ci), pA=rng.normal(size=(ch, co)) / np.sqrt(ch))
    return {k: v.astype(np.float32) for k, v in a.items()}


def _dev(a):
    return {k: torch.tensor(v, device="cuda") for k, v in a.items()}


def _ref(a):
    return {k: torch.tensor(v, dtype=DT) for k, v in a.items()}


@pytest.mark.parametrize("name,L,ci,ch,co,ng,N", CASES, ids=[c[0] for c in CASES])
def test_grid_projection_matches_oracle(name, L, ci, ch, co, ng, N):
    import so_graph_convolution_amd as K
    cfg = K.GridConfig(L, ci, ch, co, ng)
    a = _inputs(L, ci, ch, co, ng, N, seed=L + ng)
    g, r = _dev(a), _ref(a)
    H.note(f"[grid] {name} L={L} c={ci}/{ch}/{co} n_grid={ng} N={N}")
    U = K.so2grid_fwd(cfg, g["x"], g["G"], g["W"], g["A"])
    bw = K.so2grid_bwd(cfg, g["x"], g["G"], g["W"], g["A"], g["gU"])
    db = K.so2grid_dbwd(cfg, g["x"], g["G"], g["W"], g["A"], g["gU"], px=g["px"], pW=g["pW"], pA=g["pA"])
    torch.cuda.synchronize()
    rU = GO.forward(r["x"], r["G"], r["W"], r["A"])
    rb = GO.backward(r["x"], r["G"], r["W"], r["A"], r["gU"])
    rd = GO.double_backward(r["x"], r["G"], r["W"], r["A"], r["gU"], px=r["px"], pW=r["pW"], pA=r["pA"])
    errs = {"U": H.relerr(U, rU)}
    errs.update({k: H.relerr(bw[k], rb[k]) for k in ("gx", "gW", "gA")})
    errs.update({k: H.relerr(db[k], rd[v]) for k, v in (("ggU", "ggU"), ("gx2", "gx"), ("gW2", "gW"), ("gA2", "gA"))})
    H.note("  " + " ".join(f"{k}={v:.1e}" for k, v in errs.items()))
    assert all(v <= H.TOL_F32 for v in errs.values()), errs


@pytest.mark.parametrize("only", ["px", "pW", "pA"])
def test_grid_double_backward_single_direction(only):
    import so_graph_convolution_amd as K
    L, ci, ch, co, ng, N = 3, 32, 48, 16, 40, 57
    cfg = K.GridConfig(L, ci, ch, co, ng)
    a = _inputs(L, ci, ch, co, ng, N, seed=99)
    g, r = _dev(a), _ref(a)
    db = K.so2grid_dbwd(cfg, g["x"], g["G"], g["W"], g["A"], g["gU"], **{only: g[only]})
    torch.cuda.synchronize()
    rd = GO.double_backward(r["x"], r["G"], r["W"], r["A"], r["gU"], **{only: r[only]})
    errs = {k: H.relerr(db[k], rd[v]) for k, v in (("ggU", "ggU"), ("gx2", "gx"), ("gW2", "gW"), ("gA2", "gA"))}
    H.note(f"[grid dbwd {only}] " + " ".join(f"{k}={v:.1e}" for k, v in errs.items()))
    assert all(v <= H.TOL_F32 for v in errs.values()), errs


def test_grid_no_nodes():
    import so_graph_convolution_amd as K
    cfg = K.GridConfig(2, 8, 8, 8, 10)
    a = _inputs(2, 8, 8, 8, 10, 0, seed=1)
    g = _dev(a)
    U = K.so2grid_fwd(cfg, g["x"], g["G"], g["W"], g["A"])
    bw = K.so2grid_bwd(cfg, g["x"], g["G"], g["W"], g["A"], g["gU"])
    torch.cuda.synchronize()
    assert U.shape == (0, 10, 8)
    assert not bool(bw["gW"].any()) and not bool(bw["gA"].any())


BACK_CASES = [  # (name, lmax, c_h, c_out, n_grid, n_nodes)
    ("back_l2_small_ragged", 2, 32, 16, 18, 37),
    ("back_l4_eqv3_widths", 4, 512, 128, 100, 301),
    ("back_l6_ragged", 6, 64, 48, 200, 75),
    ("back_l0_tiny", 0, 8, 4, 1, 5),
]


@pytest.mark.parametrize("name,L,ch,co,ng,N", BACK_CASES, ids=[c[0] for c in BACK_CASES])
def test_grid_back_projection_matches_oracle(name, L, ch, co, ng, N):
    """Z^(l) = H_l (Y A) (Appendix B.4, the second identity), its backward and
    double backward through the C ABI against the oracle's definition order."""
    import so_graph_convolution_amd as K
    cfg = K.GridConfig(L, 4, ch, co, ng)
    rng = np.random.default_rng(100 + L + ng)
    d = (L + 1) ** 2
    a = {k: v.astype(np.float32) for k, v in dict(
        Y=rng.normal(size=(N, ng, ch)), H=rng.normal(size=(d, ng)) / np.sqrt(ng),
        A=rng.normal(size=(ch, co)) / np.sqrt(ch), gZ=rng.normal(size=(N, d, co)), pY=rng.normal(size=(N, ng, ch)),
        pA=rng.normal(size=(ch, co)) / np.sqrt(ch)).items()}
    g, r = _dev(a), _ref(a)
    H.note(f"[grid back] {name} L={L} c={ch}/{co} n_grid={ng} N={N}")
    Z = K.so2grid_back_fwd(cfg, g["Y"], g["H"], g["A"])
    bw = K.so2grid_back_bwd(cfg, g["Y"], g["H"], g["A"], g["gZ"])
    db = K.so2grid_back_dbwd(cfg, g["Y"], g["H"], g["A"], g["gZ"], pY=g["pY"], pA=g["pA"])
    d1 = K.so2grid_back_dbwd(cfg, g["Y"], g["H"], g["A"], g["gZ"], pY=g["pY"])     # one direction only
    torch.cuda.synchronize()
    rZ = GO.back_forward(r["Y"], r["H"], r["A"])
    rb = GO.back_backward(r["Y"], r["H"], r["A"], r["gZ"])
    rd = GO.back_double_backward(r["Y"], r["H"], r["A"], r["gZ"], pY=r["pY"], pA=r["pA"])
    r1 = GO.back_double_backward(r["Y"], r["H"], r["A"], r["gZ"], pY=r["pY"])
    errs = {"Z": H.relerr(Z, rZ), "gY": H.relerr(bw["gY"], rb["gY"]), "gA": H.relerr(bw["gA"], rb["gA"]),
            "ggZ": H.relerr(db["ggZ"], rd["ggZ"]), "gY2": H.relerr(db["gY2"], rd["gY"]),
            "gA2": H.relerr(db["gA2"], rd["gA"]), "ggZ(pY)": H.relerr(d1["ggZ"], r1["ggZ"]),
            "gA2(pY)": H.relerr(d1["gA2"], r1["gA"])}
    assert float(d1["gY2"].abs().max()) == 0.0          # no pA: dL/dY is zero
    H.note("  " + " ".join(f"{k}={v:.1e}" for k, v in errs.items()))
    assert all(v <= H.TOL_F32 for v in errs.values()), errs
