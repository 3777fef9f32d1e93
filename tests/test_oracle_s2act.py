"""Pins for the SwiGLU-S2 oracle (TrimSO(2) page, Table 2, Appendix C.1 and Appendix B.4; the
reading is stated in the oracle's header): a brute-force loop over the
definition, the identity grid (where it is plain SwiGLU on the coefficients),
linearity in the value half, a zero gate, a constant gate on an exact
quadrature grid of real harmonics (where the round trip is exact), and central
finite differences for the backward and the double backward."""
import itertools
import math

import numpy as np
import torch

from oracle import s2act_oracle as SO

DT = torch.float64


def _case(E=3, q=4, C=2, n_g=5, seed=0):
    g = torch.Generator().manual_seed(seed)
    r = lambda *s: torch.randn(*s, generator=g, dtype=DT)  # noqa: E731
    return r(E, q, 2 * C), r(n_g, q), r(q, n_g)


def test_brute_force_definition():
    U, G, P = _case()
    E, q, C2 = U.shape
    C, n_g = C2 // 2, G.shape[0]
    Z = SO.forward(U, G, P)
    for e, r, c in itertools.product(range(E), range(q), range(C)):
        s = 0.0
        for gp in range(n_g):
            v = sum(float(G[gp, j]) * float(U[e, j, c]) for j in range(q))
            a = sum(float(G[gp, j]) * float(U[e, j, C + c]) for j in range(q))
            s += float(P[r, gp]) * (a / (1.0 + math.exp(-a))) * v
        assert abs(float(Z[e, r, c]) - s) <= 1e-12 * max(1.0, abs(s))


def test_identity_grid_is_plain_swiglu():
    U, _, _ = _case(E=4, q=6, C=3, seed=1)
    eye = torch.eye(6, dtype=DT)
    Z = SO.forward(U, eye, eye)
    ug, uv = U[:, :, 3:], U[:, :, :3]
    ref = ug / (1.0 + torch.exp(-ug)) * uv
    assert torch.allclose(Z, ref, rtol=0, atol=1e-14)


def test_linear_in_the_value_half_and_zero_gate():
    U, G, P = _case(seed=2)
    C = U.shape[2] // 2
    Z = SO.forward(U, G, P)
    U2 = U.clone()
    U2[:, :, :C] *= -2.5
    assert torch.allclose(SO.forward(U2, G, P), -2.5 * Z, rtol=0, atol=1e-12)
    U3 = U.clone()
    U3[:, :, C:] = 0.0
    assert float(SO.forward(U3, G, P).abs().max()) == 0.0


def _dot(a, b):
    return float((a * b).sum())


def test_backward_matches_finite_differences():
    U, G, P = _case(seed=3)
    gZ = torch.randn(U.shape[0], U.shape[1], U.shape[2] // 2, generator=torch.Generator().manual_seed(9), dtype=DT)
    d = torch.randn(U.shape, generator=torch.Generator().manual_seed(10), dtype=DT)
    eps = 1e-6
    fd = (_dot(SO.forward(U + eps * d, G, P), gZ) - _dot(SO.forward(U - eps * d, G, P), gZ)) / (2 * eps)
    an = _dot(SO.backward(U, G, P, gZ), d)
    assert abs(an - fd) <= 1e-8 * max(1.0, abs(fd))


def test_double_backward_matches_finite_differences():
    U, G, P = _case(seed=4)
    gen = torch.Generator().manual_seed(11)
    gZ = torch.randn(U.shape[0], U.shape[1], U.shape[2] // 2, generator=gen, dtype=DT)
    pU = torch.randn(U.shape, generator=gen, dtype=DT)
    dd = SO.double_backward(U, G, P, gZ, pU)
    eps = 1e-6
    # d/dgZ of <pU, gU(gZ)> is the forward's directional derivative along pU
    jvp = (SO.forward(U + eps * pU, G, P) - SO.forward(U - eps * pU, G, P)) / (2 * eps)
    assert torch.allclose(dd["ggZ"], jvp, rtol=0, atol=1e-8 * float(jvp.abs().max()))
    # d/dU of <pU, gU(U)> along a direction q
    qd = torch.randn(U.shape, generator=gen, dtype=DT)
    L = lambda X: _dot(SO.backward(X, G, P, gZ), pU)  # noqa: E731
    fd = (L(U + eps * qd) - L(U - eps * qd)) / (2 * eps)
    assert abs(_dot(dd["gU2"], qd) - fd) <= 1e-7 * max(1.0, abs(fd))


def test_constant_gate_on_an_exact_sphere_grid():
    """G = the retained real harmonics (lmax 4, mmax 2: 19 rows) at the nodes of
    a product grid exact to degree 8 (Gauss-Legendre in cos(theta) x uniform
    phi), P = G^T times the quadrature weights. A gate half that is nonzero
    only on the (0, 0) row makes SiLU(G u_g) constant over the sphere, so the
    grid round trip returns SiLU(g / sqrt(4 pi)) times the value half exactly
    (orthonormality of the harmonics under an exact quadrature)."""
    from oracle import so2conv_oracle as O
    L, M = 4, 2
    zs, wz = np.polynomial.legendre.leggauss(L + 1)
    nphi = 2 * L + 1
    phi = 2 * math.pi * np.arange(nphi) / nphi
    Zg, Pg = np.meshgrid(zs, phi, indexing="ij")
    st = np.sqrt(1 - Zg * Zg)
    u = torch.tensor(np.stack([st * np.cos(Pg), st * np.sin(Pg), Zg], -1).reshape(-1, 3), dtype=DT)
    w = torch.tensor((np.repeat(wz[:, None], nphi, axis=1) * (2 * math.pi / nphi)).reshape(-1), dtype=DT)
    cols = []
    for l in range(L + 1):
        Y = O.real_sh(l, u)                       # [n_g, 2l+1], m = -l..l
        q = min(l, M)
        cols.append(Y[:, l - q:l + q + 1])
    G = torch.cat(cols, dim=1)                    # [n_g, 19]
    P = (G * w[:, None]).T.contiguous()           # [19, n_g]
    gen = torch.Generator().manual_seed(5)
    E, C = 3, 4
    U = torch.zeros(E, G.shape[1], 2 * C, dtype=DT)
    U[:, :, :C] = torch.randn(E, G.shape[1], C, generator=gen, dtype=DT)
    g0 = torch.randn(E, 1, C, generator=gen, dtype=DT) * 3
    U[:, 0:1, C:] = g0
    a = g0 / math.sqrt(4 * math.pi)
    ref = a / (1 + torch.exp(-a)) * U[:, :, :C]
    assert torch.allclose(SO.forward(U, G, P), ref, rtol=0, atol=1e-12)
