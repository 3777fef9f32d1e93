"""GPU parity of the spherical-grid SwiGLU activation on edges (so2s2_*;
TrimSO(2) page, Table 2, Appendix C.1 and Appendix B.4; the reading is stated in
oracle/s2act_oracle.py) against the float64 oracle: forward, backward and
double backward at small and ragged shapes (column counts that leave a partial
16-column block, both row-tile variants and their boundary at 16 rows, the
largest row count and grid), an empty edge set, and the full high-degree size
on sampled edges."""
import numpy as np
import pytest
import torch

from oracle import s2act_oracle as SO
from tests import _cases as H

pytestmark = pytest.mark.gpu
DT = torch.float64

CASES = [  # (name, E, rows, C, n_grid)
    ("tiny", 5, 3, 16, 7),
    ("lmax4_rows", 37, 19, 128, 100),
    ("lmax6_rows", 50, 29, 64, 60),
    ("ragged_channels", 13, 8, 24, 33),
    ("max_rows_channels", 7, 32, 256, 40),
    ("rows16_boundary", 11, 16, 20, 17),
    ("rows17_wide_channels", 3, 17, 300, 48),
    ("one_row_max_grid", 9, 1, 40, 256),
    ("max_grid_two_row_tiles", 5, 20, 32, 256),
]


def _inputs(E, q, C, ng, seed):
    rng = np.random.default_rng(seed)
    a = dict(U=rng.normal(size=(E, q, 2 * C)), G=rng.normal(size=(ng, q)) / np.sqrt(q),
             P=rng.normal(size=(q, ng)) / np.sqrt(ng), gZ=rng.normal(size=(E, q, C)), pU=rng.normal(size=(E, q, 2 * C)))
    return {k: v.astype(np.float32) for k, v in a.items()}


@pytest.mark.parametrize("name,E,q,C,ng", CASES, ids=[c[0] for c in CASES])
def test_grid_activation_matches_oracle(name, E, q, C, ng):
    import so_graph_convolution_amd as K
    a = _inputs(E, q, C, ng, seed=q + C)
    g = {k: torch.tensor(v, device="cuda") for k, v in a.items()}
    r = {k: torch.tensor(v, dtype=DT) for k, v in a.items()}
    cfg = K.S2Config(q, C, ng)
    H.note(f"[s2act] {name} E={E} rows={q} C={C} n_grid={ng}")
    Z = K.so2s2_fwd(cfg, g["U"], g["G"], g["P"])
    gU = K.so2s2_bwd(cfg, g["U"], g["G"], g["P"], g["gZ"])
    dd = K.so2s2_dbwd(cfg, g["U"], g["G"], g["P"], g["gZ"], g["pU"])
    torch.cuda.synchronize()
    rd = SO.double_backward(r["U"], r["G"], r["P"], r["gZ"], r["pU"])
    errs = {"Z": H.relerr(Z, SO.forward(r["U"], r["G"], r["P"])),
            "gU": H.relerr(gU, SO.backward(r["U"], r["G"], r["P"], r["gZ"])),
            "ggZ": H.relerr(dd["ggZ"], rd["ggZ"]), "gU2": H.relerr(dd["gU2"], rd["gU2"])}
    H.note("  " + " ".join(f"{k}={v:.1e}" for k, v in errs.items()))
    assert all(v <= H.TOL_F32 for v in errs.values()), errs


def test_grid_activation_single_outputs_and_no_edges():
    import so_graph_convolution_amd as K
    a = _inputs(9, 19, 32, 20, seed=3)
    g = {k: torch.tensor(v, device="cuda") for k, v in a.items()}
    cfg = K.S2Config(19, 32, 20)
    both = K.so2s2_dbwd(cfg, g["U"], g["G"], g["P"], g["gZ"], g["pU"])
    only_z = K.so2s2_dbwd(cfg, g["U"], g["G"], g["P"], g["gZ"], g["pU"], need=("gZ",))
    only_u = K.so2s2_dbwd(cfg, g["U"], g["G"], g["P"], g["gZ"], g["pU"], need=("U",))
    torch.cuda.synchronize()
    assert only_z["gU2"] is None and only_u["ggZ"] is None
    assert torch.equal(only_z["ggZ"], both["ggZ"]) and torch.equal(only_u["gU2"], both["gU2"])
    e0 = torch.zeros(0, 19, 64, device="cuda")
    Z0 = K.so2s2_fwd(cfg, e0, g["G"], g["P"])
    torch.cuda.synchronize()
    assert Z0.shape == (0, 19, 32)


def test_grid_activation_full_size_sampled():
    """High-degree size (1,045,678 edges, 29 rows of lmax 6 / mmax 2, C = 128,
    100 grid points) as the benchmark runs it: forward, backward and both
    double-backward outputs on 48 sampled edges against the oracle."""
    import so_graph_convolution_amd as K
    E, q, C, ng = 1045678, 29, 128, 100
    gen = torch.Generator(device="cuda").manual_seed(0)
    U = torch.randn(E, q, 2 * C, device="cuda", generator=gen)
    gZ = torch.randn(E, q, C, device="cuda", generator=gen)
    G = torch.randn(ng, q, device="cuda", generator=gen) / q ** 0.5
    P = torch.randn(q, ng, device="cuda", generator=gen) / ng ** 0.5
    cfg = K.S2Config(q, C, ng)
    H.note(f"[s2act full] E={E} rows={q} C={C} n_grid={ng}")
    idx = torch.tensor(np.random.default_rng(1).choice(E, 48, replace=False)).cuda()
    Us, gZs = U[idx].double().cpu(), gZ[idx].double().cpu()
    Gd, Pd = G.double().cpu(), P.double().cpu()
    Z = K.so2s2_fwd(cfg, U, G, P)
    torch.cuda.synchronize()
    errs = {"Z": H.relerr(Z[idx], SO.forward(Us, Gd, Pd))}
    del Z
    gU = K.so2s2_bwd(cfg, U, G, P, gZ)
    torch.cuda.synchronize()
    errs["gU"] = H.relerr(gU[idx], SO.backward(Us, Gd, Pd, gZs))
    del gU
    pU = torch.randn(E, q, 2 * C, device="cuda", generator=gen)
    dd = K.so2s2_dbwd(cfg, U, G, P, gZ, pU)
    torch.cuda.synchronize()
    rd = SO.double_backward(Us, Gd, Pd, gZs, pU[idx].double().cpu())
    errs["ggZ"] = H.relerr(dd["ggZ"][idx], rd["ggZ"])
    errs["gU2"] = H.relerr(dd["gU2"][idx], rd["gU2"])
    H.note("  " + " ".join(f"{k}={v:.1e}" for k, v in errs.items()))
    assert all(v <= H.TOL_F32 for v in errs.values()), errs
