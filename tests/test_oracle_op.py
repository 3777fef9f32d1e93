"""Pins for the oracle's operator, backward and double backward.

The pages print no operator values, so the oracle is pinned by:
  * a library routine: the SO(2) linear equals a complex matrix product;
  * invariants: rotation equivariance, invariance to the frame's roll about
    the edge axis, translation and edge-order invariance, chunk additivity;
  * special cases written independently here: lmax = 0 (scalar message
    passing) and mmax = 0 (needs only spherical harmonics, taken from scipy);
  * central finite differences for every first derivative and for the
    double backward, plus Hessian symmetry.
"""
import math

import numpy as np
import pytest
import scipy.special
import torch

import so2_synth
from oracle import so2conv_oracle as O

DT = torch.float64


def _inputs(L=2, M=2, C=4, n_atoms=12, box=6.0, rc=3.6, n_rbf=6, seed=0, edges_max=None):
    cfg = so2_synth.make_config("T", n_atoms=n_atoms, box=box, rc=rc, lmax=L, mmax=M, channels=C,
                                n_rbf=n_rbf, seed=seed, min_dist=0.6)
    d = so2_synth.make_inputs(cfg)
    if edges_max is not None and len(d["src"]) > edges_max:
        keep = np.sort(np.random.default_rng(seed).choice(len(d["src"]), edges_max, replace=False))
        for k in ("src", "dst", "shift", "rbf", "prbf"):
            d[k] = d[k][keep]
    return d


def _rand_rot(seed):
    g = np.random.default_rng(seed)
    A = g.normal(size=(3, 3))
    Q, R = np.linalg.qr(A)
    Q = Q * np.sign(np.diag(R))
    if np.linalg.det(Q) < 0:
        Q[:, 0] = -Q[:, 0]
    return torch.tensor(Q, dtype=DT)


def test_so2_linear_is_complex_product():
    g = np.random.default_rng(0)
    Tp, Tm = g.normal(size=(7, 6)), g.normal(size=(7, 6))
    W = g.normal(size=(6, 10))
    up, um = O._so2_linear(torch.tensor(Tp), torch.tensor(Tm), torch.tensor(W))
    ref = (Tp + 1j * Tm) @ (W[:, :5] + 1j * W[:, 5:])
    np.testing.assert_allclose(up.numpy(), ref.real, atol=1e-13)
    np.testing.assert_allclose(um.numpy(), ref.imag, atol=1e-13)


@pytest.mark.parametrize("L,M", [(2, 2), (4, 2), (3, 1)])
def test_equivariance(L, M):
    d = _inputs(L=L, M=M, C=3, seed=1)
    inp = O.to_oracle_inputs(d)
    y = O.forward(inp)
    Q = _rand_rot(2)
    inp2 = O.to_oracle_inputs(d)
    inp2.pos = inp.pos @ Q.T
    inp2.shift = inp.shift @ Q.T
    xr = torch.empty_like(inp.x)
    yr = torch.empty_like(y)
    for l in range(L + 1):
        blk = slice(l * l, (l + 1) ** 2)
        Dq = O.wigner_d(l, Q)
        xr[:, blk] = torch.einsum("mn,knc->kmc", Dq, inp.x[:, blk])
        yr[:, blk] = torch.einsum("mn,knc->kmc", Dq, y[:, blk])
    inp2.x = xr
    y2 = O.forward(inp2)
    assert torch.allclose(y2, yr, atol=1e-11 * y.abs().max())


def test_roll_invariance_translation_and_order():
    d = _inputs(L=4, M=2, C=3, seed=3)
    inp = O.to_oracle_inputs(d)
    y = O.forward(inp)
    E = inp.src.shape[0]
    roll = torch.tensor(np.random.default_rng(4).uniform(0, 2 * np.pi, E), dtype=DT)
    assert torch.allclose(O.forward(inp, roll=roll), y, atol=1e-12 * y.abs().max())
    inp.pos = inp.pos + torch.tensor([0.3, -1.1, 2.0], dtype=DT)
    assert torch.allclose(O.forward(inp), y, atol=1e-11 * y.abs().max())
    perm = torch.tensor(np.random.default_rng(5).permutation(E))
    inp.src, inp.dst, inp.shift, inp.rbf = inp.src[perm], inp.dst[perm], inp.shift[perm], inp.rbf[perm]
    assert torch.allclose(O.forward(inp, chunk=7), y, atol=1e-11 * y.abs().max())


def test_lmax0_is_scalar_message_passing():
    """L = 0: y_i = sum_{j->i} SiLU((rbf W_rad) * [x_j | x_i]) W1) W2, written with numpy only."""
    d = _inputs(L=0, M=0, C=5, seed=6)
    x = d["x"][:, 0, :].astype(np.float64)
    s = d["rbf"].astype(np.float64) @ d["w_rad"].astype(np.float64)
    a = np.concatenate([x[d["src"]], x[d["dst"]]], 1) * s
    h = a @ d["w1"][0].astype(np.float64)
    h = h / (1 + np.exp(-h))
    t = h @ d["w2"][0].astype(np.float64)
    ref = np.zeros_like(x)
    np.add.at(ref, d["dst"], t)
    y = O.forward(O.to_oracle_inputs(d))[:, 0, :].numpy()
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


def _scipy_real_sh(l, u):
    polar = np.arccos(np.clip(u[:, 2], -1, 1))
    azim = np.arctan2(u[:, 1], u[:, 0])
    out = np.zeros((len(u), 2 * l + 1))
    for m in range(0, l + 1):
        c = scipy.special.sph_harm_y(l, m, polar, azim)
        if m == 0:
            out[:, l] = c.real
        else:
            out[:, l + m] = math.sqrt(2) * (-1) ** m * c.real
            out[:, l - m] = math.sqrt(2) * (-1) ** m * c.imag
    return out


def test_mmax0_needs_only_harmonics():
    """M = 0: the rotated m = 0 component is c_l Y_l(rhat) . a^(l) and the message is
    c_l Y_l(rhat) t^(l), c_l = sqrt(4 pi/(2l+1)); written with numpy + scipy harmonics."""
    L, C = 3, 4
    d = _inputs(L=L, M=0, C=C, seed=7)
    src, dst = d["src"], d["dst"]
    v = d["pos"][src].astype(np.float64) - d["pos"][dst] + d["shift"]
    rh = v / np.linalg.norm(v, axis=1, keepdims=True)
    E = len(src)
    s = (d["rbf"].astype(np.float64) @ d["w_rad"].astype(np.float64)).reshape(E, L + 1, 2 * C)
    x = d["x"].astype(np.float64)
    T0 = []
    Ys = []
    for l in range(L + 1):
        Y = math.sqrt(4 * math.pi / (2 * l + 1)) * _scipy_real_sh(l, rh)
        Ys.append(Y)
        blk = slice(l * l, (l + 1) ** 2)
        a = np.concatenate([x[src, blk], x[dst, blk]], 2)
        T0.append(s[:, l] * np.einsum("em,emc->ec", Y, a))
    o = np.concatenate(T0, 1) @ d["w1"][0].astype(np.float64)
    u = o[:, :(L + 1) * C].reshape(E, L + 1, C)
    g = o[:, (L + 1) * C:].reshape(E, L, C)
    z = np.empty_like(u)
    z[:, 0] = u[:, 0] / (1 + np.exp(-u[:, 0]))
    z[:, 1:] = u[:, 1:] / (1 + np.exp(-g))
    t = (z.reshape(E, -1) @ d["w2"][0].astype(np.float64)).reshape(E, L + 1, C)
    ref = np.zeros_like(x)
    for l in range(L + 1):
        np.add.at(ref[:, l * l:(l + 1) ** 2], dst, Ys[l][:, :, None] * t[:, l, None, :])
    y = O.forward(O.to_oracle_inputs(d)).numpy()
    np.testing.assert_allclose(y, ref, rtol=1e-11, atol=1e-11 * np.abs(ref).max())


# ----------------------------------------------------------------------------- derivatives
def _perturbed(inp, which, p, eps):
    new = O.OracleInputs(inp.L, inp.M, inp.C, inp.pos, inp.x, inp.src, inp.dst, inp.shift,
                         inp.rbf, inp.w_rad, list(inp.w1), list(inp.w2), inp.env)
    if which == "w1":
        new.w1 = [w + eps * q for w, q in zip(inp.w1, p)]
    elif which == "w2":
        new.w2 = [w + eps * q for w, q in zip(inp.w2, p)]
    else:
        setattr(new, which, getattr(inp, which) + eps * p)
    return new


def _dirs(inp, seed):
    g = torch.Generator().manual_seed(seed)

    def r(t):
        return torch.randn(t.shape, generator=g, dtype=DT)
    return dict(x=r(inp.x), pos=r(inp.pos), rbf=r(inp.rbf), w_rad=r(inp.w_rad), shift=r(inp.shift),
                w1=[r(w) for w in inp.w1], w2=[r(w) for w in inp.w2])


def _dot(a, b):
    if isinstance(a, list):
        return sum((x * y).sum() for x, y in zip(a, b))
    return (a * b).sum()


@pytest.fixture(scope="module")
def small():
    d = _inputs(L=3, M=2, C=3, n_atoms=10, box=6.0, rc=3.4, seed=11, edges_max=40)
    inp = O.to_oracle_inputs(d)
    gy = torch.tensor(d["gy"], dtype=DT)
    return d, inp, gy


@pytest.mark.parametrize("which", ["x", "pos", "rbf", "w_rad", "w1", "w2", "shift"])
def test_backward_matches_finite_differences(small, which):
    d, inp, gy = small
    g = O.backward(inp, gy, with_edge_grad=True)
    key = {"x": "gx", "pos": "gpos", "rbf": "grbf", "w_rad": "gw_rad", "w1": "gw1", "w2": "gw2",
           "shift": "gedge"}[which]
    p = _dirs(inp, 21)[which]
    eps = 1e-5
    fp = (O.forward(_perturbed(inp, which, p, eps)) * gy).sum()
    fm = (O.forward(_perturbed(inp, which, p, -eps)) * gy).sum()
    fd = (fp - fm) / (2 * eps)
    an = _dot(g[key], p)
    assert abs(float(an - fd)) <= 1e-7 * max(1.0, abs(float(fd)))


def test_backward_translation_sum_zero(small):
    _, inp, gy = small
    g = O.backward(inp, gy)
    assert torch.allclose(g["gpos"].sum(0), torch.zeros(3, dtype=DT), atol=1e-11 * g["gpos"].abs().max())


def test_double_backward_ggy_is_forward_jvp(small):
    """d L / d gy = J p (the forward's directional derivative along p), cf. Eq.(5)."""
    _, inp, gy = small
    p = _dirs(inp, 22)
    dd = O.double_backward(inp, gy, px=p["x"], ppos=p["pos"], prbf=p["rbf"], pw_rad=p["w_rad"],
                           pw1=p["w1"], pw2=p["w2"])
    eps = 1e-5

    def shifted(e):
        new = _perturbed(inp, "x", p["x"], e)
        new = _perturbed(new, "pos", p["pos"], e)
        new = _perturbed(new, "rbf", p["rbf"], e)
        new = _perturbed(new, "w_rad", p["w_rad"], e)
        new = _perturbed(new, "w1", p["w1"], e)
        return _perturbed(new, "w2", p["w2"], e)
    jvp = (O.forward(shifted(eps)) - O.forward(shifted(-eps))) / (2 * eps)
    assert torch.allclose(dd["ggy"], jvp, atol=1e-7 * jvp.abs().max())


@pytest.mark.parametrize("which", ["x", "pos", "rbf", "w_rad", "w1", "w2"])
def test_double_backward_matches_fd_of_backward(small, which):
    _, inp, gy = small
    p = _dirs(inp, 23)
    q = _dirs(inp, 24)[which]
    dd = O.double_backward(inp, gy, px=p["x"], ppos=p["pos"], prbf=p["rbf"], pw_rad=p["w_rad"],
                           pw1=p["w1"], pw2=p["w2"], pedge=p["shift"])
    key = {"x": "gx", "pos": "gpos", "rbf": "grbf", "w_rad": "gw_rad", "w1": "gw1", "w2": "gw2"}[which]
    eps = 1e-5

    def L(e):
        g = O.backward(_perturbed(inp, which, q, e), gy, with_edge_grad=True)
        return (_dot(g["gx"], p["x"]) + _dot(g["gpos"], p["pos"]) + _dot(g["grbf"], p["rbf"])
                + _dot(g["gw_rad"], p["w_rad"]) + _dot(g["gw1"], p["w1"]) + _dot(g["gw2"], p["w2"])
                + _dot(g["gedge"], p["shift"]))
    fd = (L(eps) - L(-eps)) / (2 * eps)
    an = _dot(dd[key], q)
    assert abs(float(an - fd)) <= 1e-6 * max(1.0, abs(float(fd)))


def test_double_backward_hessian_symmetry(small):
    _, inp, gy = small
    p1, p2 = _dirs(inp, 31)["x"], _dirs(inp, 32)["x"]
    h1 = O.double_backward(inp, gy, px=p1)["gx"]
    h2 = O.double_backward(inp, gy, px=p2)["gx"]
    a, b = float((p2 * h1).sum()), float((p1 * h2).sum())
    assert abs(a - b) <= 1e-10 * max(1.0, abs(a))


def test_backward_scaling_identities(small):
    """The first linear's input T = s * (D a) is linear in x, in rbf and in W_rad
    (s = rbf W_rad), and T W1 is bilinear, so scaling any one of x, rbf, W_rad,
    W1 by (1 + t) changes every first-linear output the same way: the four
    directional derivatives agree, <gx, x> = <grbf, rbf> = <gW_rad, W_rad> =
    <gW1, W1>. y is linear in W2: <gW2, W2> = <gy, y>. (These hold at any size
    and tie the weight gradients to per-node and per-edge outputs.)"""
    _, inp, gy = small
    g = O.backward(inp, gy)
    y = O.forward(inp)
    vals = [float(_dot(g["gx"], inp.x)), float(_dot(g["grbf"], inp.rbf)), float(_dot(g["gw_rad"], inp.w_rad)),
            float(_dot(g["gw1"], inp.w1))]
    ref = vals[0]
    assert abs(ref) > 1e-6
    assert all(abs(v - ref) <= 1e-11 * abs(ref) for v in vals), vals
    a, b = float(_dot(g["gw2"], inp.w2)), float((gy * y).sum())
    assert abs(a - b) <= 1e-11 * abs(b)
