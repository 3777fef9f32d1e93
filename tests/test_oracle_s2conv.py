"""Pins for the oracle's convolution with the spherical-grid SwiGLU activation
(TrimSO(2) page, Appendix C.1 "Implementation": EquiformerV3's Edge -> Edge
activation; Table 2 names it SwiGLU-S2; Appendix B.4: the basis evaluated at
grid points, the nonlinearity on grid values).

The activation's reading (oracle/s2act_oracle.py) is pinned on its own in
test_oracle_s2act.py; these pins fix how the convolution feeds it:
  * lmax = 0, written with numpy only: the value half is the first C output
    channels of the first linear, the gate half the next C, and the second
    linear reads z;
  * the grid values are the rotated input function at the grid points: with
    a first linear that passes degree-1 inputs through, G u_v equals
    Y_{1,+1}(R_e^T g) evaluated directly, which fixes the degree-major row
    order (l, then m ascending) and the sign of every order;
  * a frame roll by one longitude step of a uniform grid permutes the grid
    points, so it leaves the output unchanged exactly, while a generic roll
    does not;
  * central finite differences for the backward and the double backward.
"""
import math

import numpy as np
import pytest
import torch

import so2_synth
from oracle import so2conv_oracle as O

DT = torch.float64


def _inputs(L=2, M=2, C=4, n_grid=9, n_atoms=12, box=6.0, rc=3.6, n_rbf=6, seed=0, edges_max=None):
    cfg = so2_synth.make_config("T", n_atoms=n_atoms, box=box, rc=rc, lmax=L, mmax=M, channels=C,
                                n_rbf=n_rbf, seed=seed, min_dist=0.6, act="swiglu_s2", n_grid=n_grid)
    d = so2_synth.make_inputs(cfg)
    if edges_max is not None and len(d["src"]) > edges_max:
        keep = np.sort(np.random.default_rng(seed).choice(len(d["src"]), edges_max, replace=False))
        for k in ("src", "dst", "shift", "rbf", "prbf"):
            d[k] = d[k][keep]
    return d


def _silu(a):
    return a / (1 + np.exp(-a))


def test_lmax0_closed_form():
    """L = 0: u = (s * [x_j | x_i]) W1[0], v = u[:C], a = u[C:],
    z = sum_g P[0, g] SiLU(G[g, 0] a) G[g, 0] v, y_i = sum_{j->i} z W2[0]."""
    C = 5
    d = _inputs(L=0, M=0, C=C, n_grid=6, seed=3)
    x = d["x"][:, 0, :].astype(np.float64)
    s = d["rbf"].astype(np.float64) @ d["w_rad"].astype(np.float64)
    T = np.concatenate([x[d["src"]], x[d["dst"]]], 1) * s
    u = T @ d["w1"][0].astype(np.float64)
    v, a = u[:, :C], u[:, C:]
    G = d["grid_G"].astype(np.float64)[:, 0]
    P = d["grid_P"].astype(np.float64)[0]
    z = sum(P[g] * _silu(G[g] * a) * G[g] * v for g in range(len(G)))
    t = z @ d["w2"][0].astype(np.float64)
    ref = np.zeros_like(x)
    np.add.at(ref, d["dst"], t)
    y = O.forward(O.to_oracle_inputs(d))[:, 0, :].numpy()
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_grid_values_are_the_rotated_function():
    """x holds only Y_{1,+1} (channel 0) on every node and the first linear passes
    source channel 0 of each degree to value channel 0 of that degree, so the
    edge-frame value rows are the rotated function's coefficients: G u_v at
    edge-frame points g must equal s_{e,1,0} Y_{1,+1}(R_e^T g), with
    Y_{1,+1}(u) = sqrt(3 / 4 pi) u_x."""
    L, M, C = 2, 1, 4
    d = _inputs(L=L, M=M, C=C, seed=5, edges_max=30)
    d["x"] = np.zeros_like(d["x"])
    d["x"][:, 1 * 1 + 1 + 1, 0] = 1.0                     # node row (l=1, m=+1)
    w1 = [np.zeros_like(w) for w in d["w1"]]
    for l in range(L + 1):                                 # order 0: degree l, channel 0 -> value channel 0
        w1[0][l * 2 * C, l * 2 * C] = 1.0
    for m in range(1, M + 1):                              # order m: W_m0 passes channel 0, W_m1 = 0
        for k in range(L - m + 1):
            w1[m][k * 2 * C, k * 2 * C] = 1.0
    d["w1"] = w1
    inp = O.to_oracle_inputs(d)
    U = O.activation_input(inp)                            # [E, q, 2C], rows degree-major
    rows = O.grid_rows(L, M)
    assert rows == [(l, m) for l in range(L + 1) for m in range(-min(l, M), min(l, M) + 1)]
    rng = np.random.default_rng(0)
    g = rng.normal(size=(11, 3))
    g /= np.linalg.norm(g, axis=1, keepdims=True)
    G = torch.cat([O.real_sh(l, torch.tensor(g, dtype=DT))[:, [mm + l for mm in range(-min(l, M), min(l, M) + 1)]]
                   for l in range(L + 1)], 1)               # [n_g, q]
    vals = torch.einsum("gr,er->eg", G, U[:, :, 0]).numpy()
    E = len(d["src"])
    s = (d["rbf"].astype(np.float64) @ d["w_rad"].astype(np.float64)).reshape(E, L + 1, 2 * C)[:, 1, 0]
    v = d["pos"][d["src"]].astype(np.float64) - d["pos"][d["dst"]] + d["shift"]
    R = O.edge_frame(torch.tensor(v / np.linalg.norm(v, axis=1, keepdims=True), dtype=DT)).numpy()
    back = np.einsum("eba,gb->ega", R, g)                 # R_e^T g
    ref = s[:, None] * math.sqrt(3 / (4 * math.pi)) * back[:, :, 0]
    np.testing.assert_allclose(vals, ref, rtol=1e-11, atol=1e-12)
    assert np.abs(ref).max() > 0.1


def _uniform_grid(L, M, n_theta, n_phi):
    """Gauss-Legendre latitudes x n_phi uniform longitudes: G [n_g, q] (O.real_sh
    at the points, rows degree-major) and P = w G^T with the quadrature weights."""
    xs, ws = np.polynomial.legendre.leggauss(n_theta)
    pts, wts = [], []
    for ct, wt in zip(xs, ws):
        st = math.sqrt(1 - ct * ct)
        for j in range(n_phi):
            ph = 2 * math.pi * j / n_phi
            pts.append((st * math.cos(ph), st * math.sin(ph), ct))
            wts.append(wt * 2 * math.pi / n_phi)
    u = torch.tensor(np.array(pts), dtype=DT)
    G = torch.cat([O.real_sh(l, u)[:, [m + l for m in O.retained_orders(l, M)]] for l in range(L + 1)], 1)
    P = (torch.tensor(wts, dtype=DT)[:, None] * G).T.contiguous()
    return G, P


def test_uniform_grid_is_a_quadrature():
    """P G = identity on the retained rows (Gauss-Legendre with L + 1 nodes, 2M + 1 or
    more longitudes): the grid resolves every retained row exactly."""
    G, P = _uniform_grid(4, 2, 5, 7)
    assert torch.allclose(P @ G, torch.eye(G.shape[1], dtype=DT), atol=1e-12)


def test_roll_by_one_grid_step_is_exact():
    L, M, n_phi = 3, 2, 7
    d = _inputs(L=L, M=M, C=3, seed=8, edges_max=40)
    G, P = _uniform_grid(L, M, L + 2, n_phi)
    inp = O.to_oracle_inputs(d)
    inp.grid = (G, P)
    E = len(d["src"])
    y0 = O.forward(inp)
    step = torch.full((E,), 2 * math.pi / n_phi, dtype=DT) * torch.tensor(
        np.random.default_rng(1).integers(-3, 4, size=E), dtype=DT)
    y1 = O.forward(inp, roll=step)
    assert torch.allclose(y1, y0, atol=1e-11 * y0.abs().max())
    y2 = O.forward(inp, roll=torch.full((E,), 0.37, dtype=DT))
    assert (y2 - y0).abs().max() > 1e-4 * y0.abs().max()


# ----------------------------------------------------------------------------- derivatives
def _perturbed(inp, which, p, eps):
    new = O.OracleInputs(inp.L, inp.M, inp.C, inp.pos, inp.x, inp.src, inp.dst, inp.shift,
                         inp.rbf, inp.w_rad, list(inp.w1), list(inp.w2), inp.env, inp.grid)
    if which in ("w1", "w2"):
        setattr(new, which, [w + eps * q for w, q in zip(getattr(inp, which), p)])
    else:
        setattr(new, which, getattr(inp, which) + eps * p)
    return new


def _dirs(inp, seed):
    g = torch.Generator().manual_seed(seed)

    def r(t):
        return torch.randn(t.shape, generator=g, dtype=DT)
    return dict(x=r(inp.x), pos=r(inp.pos), rbf=r(inp.rbf), w_rad=r(inp.w_rad),
                w1=[r(w) for w in inp.w1], w2=[r(w) for w in inp.w2])


def _dot(a, b):
    if isinstance(a, list):
        return sum((x * y).sum() for x, y in zip(a, b))
    return (a * b).sum()


@pytest.fixture(scope="module")
def small():
    d = _inputs(L=2, M=1, C=3, n_grid=8, n_atoms=10, box=6.0, rc=3.4, seed=11, edges_max=30)
    inp = O.to_oracle_inputs(d)
    gy = torch.tensor(d["gy"], dtype=DT)
    return inp, gy


@pytest.mark.parametrize("which", ["x", "pos", "rbf", "w_rad", "w1", "w2"])
def test_backward_matches_finite_differences(small, which):
    inp, gy = small
    g = O.backward(inp, gy)
    key = {"x": "gx", "pos": "gpos", "rbf": "grbf", "w_rad": "gw_rad", "w1": "gw1", "w2": "gw2"}[which]
    p = _dirs(inp, 21)[which]
    eps = 1e-5
    fd = ((O.forward(_perturbed(inp, which, p, eps)) * gy).sum()
          - (O.forward(_perturbed(inp, which, p, -eps)) * gy).sum()) / (2 * eps)
    an = _dot(g[key], p)
    assert abs(float(an - fd)) <= 1e-7 * max(1.0, abs(float(fd)))


@pytest.mark.parametrize("which", ["x", "pos", "w1"])
def test_double_backward_matches_fd_of_backward(small, which):
    inp, gy = small
    p = _dirs(inp, 23)
    q = _dirs(inp, 24)[which]
    dd = O.double_backward(inp, gy, px=p["x"], ppos=p["pos"], prbf=p["rbf"], pw_rad=p["w_rad"],
                           pw1=p["w1"], pw2=p["w2"])
    key = {"x": "gx", "pos": "gpos", "w1": "gw1"}[which]
    eps = 1e-5

    def L(e):
        g = O.backward(_perturbed(inp, which, q, e), gy)
        return (_dot(g["gx"], p["x"]) + _dot(g["gpos"], p["pos"]) + _dot(g["grbf"], p["rbf"])
                + _dot(g["gw_rad"], p["w_rad"]) + _dot(g["gw1"], p["w1"]) + _dot(g["gw2"], p["w2"]))
    fd = (L(eps) - L(-eps)) / (2 * eps)
    an = _dot(dd[key], q)
    assert abs(float(an - fd)) <= 1e-6 * max(1.0, abs(float(fd)))


def test_double_backward_ggy_is_forward_jvp(small):
    inp, gy = small
    p = _dirs(inp, 22)
    dd = O.double_backward(inp, gy, px=p["x"], pw1=p["w1"])
    eps = 1e-5
    jvp = (O.forward(_perturbed(_perturbed(inp, "x", p["x"], eps), "w1", p["w1"], eps))
           - O.forward(_perturbed(_perturbed(inp, "x", p["x"], -eps), "w1", p["w1"], -eps))) / (2 * eps)
    assert torch.allclose(dd["ggy"], jvp, atol=1e-7 * jvp.abs().max())
