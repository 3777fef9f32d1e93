"""Pins for the spherical-projection oracle (TrimSO(2) page, Appendix B.4):
a brute-force loop over every index of the definition on a tiny case, the
page's reassociation B_l = W_l A, linearity in x and in each channel map,
and central finite differences for the backward and the double backward."""
import itertools

import pytest
import torch

from oracle import grid_oracle as GO

DT = torch.float64


def _case(L=2, C_in=3, C_h=4, C_out=2, n_g=5, N=3, seed=0):
    g = torch.Generator().manual_seed(seed)
    r = lambda *s: torch.randn(*s, generator=g, dtype=DT)  # noqa: E731
    d = (L + 1) ** 2
    return r(N, d, C_in), r(n_g, d), r(L + 1, C_in, C_h), r(C_h, C_out)


def test_brute_force_definition():
    x, G, W, A = _case()
    N, d, C_in = x.shape
    n_g, C_h, C_out, L = G.shape[0], W.shape[2], A.shape[1], W.shape[0] - 1
    U = GO.forward(x, G, W, A)
    for i, gp, c in itertools.product(range(N), range(n_g), range(C_out)):
        s = 0.0
        for l in range(L + 1):
            for m in range(2 * l + 1):
                j = l * l + m
                for k in range(C_in):
                    for h in range(C_h):
                        s += float(G[gp, j]) * float(x[i, j, k]) * float(W[l, k, h]) * float(A[h, c])
        assert abs(float(U[i, gp, c]) - s) <= 1e-12 * max(1.0, abs(s))


def test_reassociation_with_B():
    """sum_l G_l (X^(l) B_l) with B_l = W_l A equals the definition."""
    x, G, W, A = _case(L=3, C_in=4, C_h=6, C_out=3, n_g=7, N=4, seed=1)
    B = W @ A
    U2 = sum(torch.einsum("gm,nmc->ngc", G[:, l * l:(l + 1) ** 2], x[:, l * l:(l + 1) ** 2, :] @ B[l])
             for l in range(W.shape[0]))
    assert torch.allclose(GO.forward(x, G, W, A), U2, atol=1e-12)


def test_linear_in_each_argument():
    x, G, W, A = _case(seed=2)
    x2, _, W2, A2 = _case(seed=3)
    f = GO.forward
    assert torch.allclose(f(x + 2 * x2, G, W, A), f(x, G, W, A) + 2 * f(x2, G, W, A), atol=1e-12)
    assert torch.allclose(f(x, G, W + W2, A), f(x, G, W, A) + f(x, G, W2, A), atol=1e-12)
    assert torch.allclose(f(x, G, W, A - A2), f(x, G, W, A) - f(x, G, W, A2), atol=1e-12)


def _dot(a, b):
    return float((a * b).sum())


@pytest.mark.parametrize("which", ["x", "W", "A"])
def test_backward_matches_fd(which):
    x, G, W, A = _case(L=3, C_in=3, C_h=5, C_out=4, n_g=9, N=3, seed=4)
    gU = torch.randn(x.shape[0], G.shape[0], A.shape[1], generator=torch.Generator().manual_seed(5), dtype=DT)
    g = GO.backward(x, G, W, A, gU)
    q = torch.randn_like({"x": x, "W": W, "A": A}[which])
    eps = 1e-6

    def f(e):
        args = dict(x=x, W=W, A=A)
        args[which] = args[which] + e * q
        return _dot(GO.forward(args["x"], G, args["W"], args["A"]), gU)
    fd = (f(eps) - f(-eps)) / (2 * eps)
    assert abs(_dot(g["g" + which], q) - fd) <= 1e-7 * max(1.0, abs(fd))


@pytest.mark.parametrize("which", ["gU", "x", "W", "A"])
def test_double_backward_matches_fd(which):
    x, G, W, A = _case(L=2, C_in=3, C_h=4, C_out=3, n_g=8, N=3, seed=6)
    gen = torch.Generator().manual_seed(7)
    r = lambda t: torch.randn(t.shape, generator=gen, dtype=DT)  # noqa: E731
    gU = torch.randn(x.shape[0], G.shape[0], A.shape[1], generator=gen, dtype=DT)
    px, pW, pA = r(x), r(W), r(A)
    dd = GO.double_backward(x, G, W, A, gU, px=px, pW=pW, pA=pA)
    base = dict(x=x, W=W, A=A, gU=gU)
    q = r(base[which])
    eps = 1e-6

    def L(e):
        a = dict(base)
        a[which] = a[which] + e * q
        g = GO.backward(a["x"], G, a["W"], a["A"], a["gU"])
        return _dot(g["gx"], px) + _dot(g["gW"], pW) + _dot(g["gA"], pA)
    fd = (L(eps) - L(-eps)) / (2 * eps)
    key = {"gU": "ggU", "x": "gx", "W": "gW", "A": "gA"}[which]
    assert abs(_dot(dd[key], q) - fd) <= 1e-7 * max(1.0, abs(fd))


def _basis(L, u):
    """[n_g, (L+1)^2] real orthonormal harmonics at the unit vectors u."""
    from oracle.so2conv_oracle import real_sh
    return torch.cat([real_sh(l, u) for l in range(L + 1)], dim=-1)


def _unit(n, g):
    v = torch.randn(n, 3, generator=g, dtype=DT)
    return v / v.norm(dim=-1, keepdim=True)


def test_addition_theorem_closed_form():
    """With G the harmonics at grid points u_g, identity channel maps and the
    coefficients of Y(u0) as the node's features, the projection is the
    zonal kernel sum_l (2l+1)/(4 pi) P_l(u_g . u0) (addition theorem)."""
    from scipy.special import eval_legendre
    L, n_g = 4, 23
    g = torch.Generator().manual_seed(5)
    u, u0 = _unit(n_g, g), _unit(1, g)
    G = _basis(L, u)
    x = _basis(L, u0).reshape(1, -1, 1)                       # one node, one channel
    W = torch.ones(L + 1, 1, 1, dtype=DT)
    U = GO.forward(x, G, W, torch.ones(1, 1, dtype=DT))[0, :, 0]
    t = (u @ u0[0]).numpy()
    ref = sum((2 * l + 1) / (4 * torch.pi) * eval_legendre(l, t) for l in range(L + 1))
    assert torch.allclose(U, torch.as_tensor(ref), atol=1e-12, rtol=0)


def test_rotating_features_rotates_the_grid():
    """Features rotated by D(Q) read on the grid u equal the unrotated features
    read on the grid Q^T u (Y(Q^T u) = D(Q)^T Y(u))."""
    from oracle.so2conv_oracle import wigner_d
    L, n_g = 3, 11
    g = torch.Generator().manual_seed(6)
    x, _, W, A = _case(L=L, C_in=3, C_h=4, C_out=2, n_g=n_g, N=2, seed=7)
    Q, _ = torch.linalg.qr(torch.randn(3, 3, generator=g, dtype=DT))
    if torch.det(Q) < 0:
        Q = -Q
    u = _unit(n_g, g)
    xr = torch.cat([torch.einsum("mk,nkc->nmc", wigner_d(l, Q), x[:, l * l:(l + 1) ** 2])
                    for l in range(L + 1)], dim=1)
    lhs = GO.forward(xr, _basis(L, u), W, A)
    rhs = GO.forward(x, _basis(L, u @ Q), W, A)
    assert torch.allclose(lhs, rhs, atol=1e-11, rtol=0)


# ----------------------------------------------------------------------------- back-projection
def _back_case(L=2, C_h=4, C_out=3, n_g=6, N=3, seed=10):
    g = torch.Generator().manual_seed(seed)
    r = lambda *s: torch.randn(*s, generator=g, dtype=DT)  # noqa: E731
    return r(N, n_g, C_h), r((L + 1) ** 2, n_g), r(C_h, C_out)


def test_back_brute_force_definition():
    Y, H, A = _back_case()
    N, n_g, C_h = Y.shape
    d, C_out = H.shape[0], A.shape[1]
    Z = GO.back_forward(Y, H, A)
    for i, j, c in itertools.product(range(N), range(d), range(C_out)):
        s = sum(float(H[j, gp]) * float(Y[i, gp, h]) * float(A[h, c]) for gp in range(n_g) for h in range(C_h))
        assert abs(float(Z[i, j, c]) - s) <= 1e-12 * max(1.0, abs(s))


def _scipy_basis(L, u):
    """[n, (L+1)^2] real orthonormal harmonics from scipy (no Condon-Shortley
    phase, orders -l..l, Y_1 = sqrt(3/4pi) (y, z, x))."""
    import math

    import numpy as np
    import scipy.special
    u = u.numpy()
    polar = np.arccos(np.clip(u[:, 2], -1, 1))
    azim = np.arctan2(u[:, 1], u[:, 0])
    cols = []
    for l in range(L + 1):
        out = np.zeros((len(u), 2 * l + 1))
        for m in range(l + 1):
            c = scipy.special.sph_harm_y(l, m, polar, azim)
            if m == 0:
                out[:, l] = c.real
            else:
                out[:, l + m] = math.sqrt(2) * (-1) ** m * c.real
                out[:, l - m] = math.sqrt(2) * (-1) ** m * c.imag
        cols.append(out)
    return torch.tensor(np.concatenate(cols, 1), dtype=DT)


def test_back_projection_inverts_an_exact_quadrature_grid():
    """G = harmonics at a Gauss-Legendre x uniform grid exact to degree 2L and
    H = G^T diag(w): H_l G_l' = delta_ll' I, so back-projecting the grid values
    of band-limited coefficients with an identity channel map returns them
    (and a channel map A maps them by A)."""
    import numpy as np
    L = 3
    zs, wz = np.polynomial.legendre.leggauss(L + 1)
    nphi = 2 * L + 1
    phi = 2 * np.pi * np.arange(nphi) / nphi
    Zg, Pg = np.meshgrid(zs, phi, indexing="ij")
    st = np.sqrt(1 - Zg * Zg)
    u = torch.tensor(np.stack([st * np.cos(Pg), st * np.sin(Pg), Zg], -1).reshape(-1, 3), dtype=DT)
    w = torch.tensor((np.repeat(wz[:, None], nphi, 1) * 2 * np.pi / nphi).reshape(-1), dtype=DT)
    G = _scipy_basis(L, u)                                   # [n_g, d]
    H = G.T * w                                              # [d, n_g]
    g = torch.Generator().manual_seed(11)
    X = torch.randn(2, (L + 1) ** 2, 5, generator=g, dtype=DT)
    Y = torch.einsum("gj,njc->ngc", G, X)                    # grid values
    assert torch.allclose(GO.back_forward(Y, H, torch.eye(5, dtype=DT)), X, atol=1e-12)
    A = torch.randn(5, 3, generator=g, dtype=DT)
    assert torch.allclose(GO.back_forward(Y, H, A), X @ A, atol=1e-12)


def test_back_reordering_and_linearity():
    """(H_l Y) A_out equals the definition H_l (Y A_out); Z is linear in Y and in A."""
    Y, H, A = _back_case(L=3, C_h=5, C_out=4, n_g=9, N=2, seed=12)
    Y2, _, A2 = _back_case(L=3, C_h=5, C_out=4, n_g=9, N=2, seed=13)
    Z = GO.back_forward(Y, H, A)
    assert torch.allclose(torch.einsum("jg,ngh->njh", H, Y) @ A, Z, atol=1e-12)
    f = GO.back_forward
    assert torch.allclose(f(Y + 3 * Y2, H, A), Z + 3 * f(Y2, H, A), atol=1e-12)
    assert torch.allclose(f(Y, H, A - A2), Z - f(Y, H, A2), atol=1e-12)


@pytest.mark.parametrize("which", ["Y", "A"])
def test_back_backward_matches_fd(which):
    Y, H, A = _back_case(L=2, C_h=4, C_out=3, n_g=7, N=3, seed=14)
    gZ = torch.randn(Y.shape[0], H.shape[0], A.shape[1], generator=torch.Generator().manual_seed(15), dtype=DT)
    g = GO.back_backward(Y, H, A, gZ)
    q = torch.randn_like({"Y": Y, "A": A}[which])
    eps = 1e-6

    def f(e):
        a = dict(Y=Y, A=A)
        a[which] = a[which] + e * q
        return _dot(GO.back_forward(a["Y"], H, a["A"]), gZ)
    fd = (f(eps) - f(-eps)) / (2 * eps)
    assert abs(_dot(g["g" + which], q) - fd) <= 1e-7 * max(1.0, abs(fd))


@pytest.mark.parametrize("which", ["gZ", "Y", "A"])
def test_back_double_backward_matches_fd(which):
    Y, H, A = _back_case(L=2, C_h=4, C_out=3, n_g=7, N=3, seed=16)
    gen = torch.Generator().manual_seed(17)
    r = lambda t: torch.randn(t.shape, generator=gen, dtype=DT)  # noqa: E731
    gZ = torch.randn(Y.shape[0], H.shape[0], A.shape[1], generator=gen, dtype=DT)
    pY, pA = r(Y), r(A)
    dd = GO.back_double_backward(Y, H, A, gZ, pY=pY, pA=pA)
    base = dict(Y=Y, A=A, gZ=gZ)
    q = r(base[which])
    eps = 1e-6

    def L(e):
        a = dict(base)
        a[which] = a[which] + e * q
        g = GO.back_backward(a["Y"], H, a["A"], a["gZ"])
        return _dot(g["gY"], pY) + _dot(g["gA"], pA)
    fd = (L(eps) - L(-eps)) / (2 * eps)
    key = {"gZ": "ggZ", "Y": "gY", "A": "gA"}[which]
    assert abs(_dot(dd[key], q) - fd) <= 1e-7 * max(1.0, abs(fd))
