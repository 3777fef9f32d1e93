"""Pins for the oracle's real spherical harmonics, Wigner-D blocks and edge frame.

Each check ties the oracle to something other than itself: closed forms,
scipy's complex spherical harmonics (an independent library routine),
group-homomorphism and orthogonality invariants, and the addition theorem.
"""
import math

import numpy as np
import pytest
import scipy.special
import torch

from oracle import so2conv_oracle as O

DT = torch.float64


def _rand_unit(n, seed):
    g = np.random.default_rng(seed)
    v = g.normal(size=(n, 3))
    return torch.tensor(v / np.linalg.norm(v, axis=1, keepdims=True), dtype=DT)


def _rand_rot(n, seed):
    g = np.random.default_rng(seed)
    q = g.normal(size=(n, 4))
    q /= np.linalg.norm(q, axis=1, keepdims=True)
    w, x, y, z = q.T
    R = np.stack([
        np.stack([1 - 2 * (y * y + z * z), 2 * (x * y - z * w), 2 * (x * z + y * w)], -1),
        np.stack([2 * (x * y + z * w), 1 - 2 * (x * x + z * z), 2 * (y * z - x * w)], -1),
        np.stack([2 * (x * z - y * w), 2 * (y * z + x * w), 1 - 2 * (x * x + y * y)], -1)], -2)
    return torch.tensor(R, dtype=DT)


def test_y1_closed_form():
    u = _rand_unit(50, 1)
    Y = O.real_sh(1, u)
    ref = math.sqrt(3 / (4 * math.pi)) * torch.stack([u[:, 1], u[:, 2], u[:, 0]], -1)
    assert torch.allclose(Y, ref, atol=1e-14)


@pytest.mark.parametrize("l", range(0, 7))
def test_y_l0_at_pole(l):
    Y = O.real_sh(l, torch.tensor([[0.0, 0.0, 1.0]], dtype=DT))[0]
    expect = torch.zeros(2 * l + 1, dtype=DT)
    expect[l] = math.sqrt((2 * l + 1) / (4 * math.pi))
    assert torch.allclose(Y, expect, atol=1e-13)


@pytest.mark.parametrize("l", range(0, 7))
def test_against_scipy_complex_harmonics(l):
    """Real SH without Condon-Shortley phase from scipy's complex Y_l^m (which has it):
    Y_{l,m} = sqrt2 (-1)^m Re Y_l^m, Y_{l,-m} = sqrt2 (-1)^m Im Y_l^m (m > 0)."""
    u = _rand_unit(64, 10 + l).numpy()
    polar = np.arccos(np.clip(u[:, 2], -1, 1))
    azim = np.arctan2(u[:, 1], u[:, 0])
    ref = np.zeros((64, 2 * l + 1))
    for m in range(0, l + 1):
        c = scipy.special.sph_harm_y(l, m, polar, azim)
        if m == 0:
            ref[:, l] = c.real
        else:
            ref[:, l + m] = math.sqrt(2) * (-1) ** m * c.real
            ref[:, l - m] = math.sqrt(2) * (-1) ** m * c.imag
    ours = O.real_sh(l, torch.tensor(u, dtype=DT)).numpy()
    np.testing.assert_allclose(ours, ref, atol=1e-12)


@pytest.mark.parametrize("l", range(0, 7))
def test_orthonormal_dense_grid(l):
    # a much denser product grid than the one the oracle's Wigner-D uses
    zs, wz = np.polynomial.legendre.leggauss(24)
    nphi = 48
    phi = 2 * np.pi * np.arange(nphi) / nphi
    Z, P = np.meshgrid(zs, phi, indexing="ij")
    st = np.sqrt(1 - Z * Z)
    u = torch.tensor(np.stack([st * np.cos(P), st * np.sin(P), Z], -1).reshape(-1, 3), dtype=DT)
    w = torch.tensor((np.repeat(wz[:, None], nphi, 1) * 2 * np.pi / nphi).reshape(-1), dtype=DT)
    Y = O.real_sh(l, u)
    G = torch.einsum("gm,gn,g->mn", Y, Y, w)
    assert torch.allclose(G, torch.eye(2 * l + 1, dtype=DT), atol=1e-12)


@pytest.mark.parametrize("l", range(0, 7))
def test_wigner_orthogonal_and_homomorphism(l):
    R1, R2 = _rand_rot(8, 3), _rand_rot(8, 4)
    D1, D2, D12 = O.wigner_d(l, R1), O.wigner_d(l, R2), O.wigner_d(l, R1 @ R2)
    eye = torch.eye(2 * l + 1, dtype=DT).expand(8, -1, -1)
    assert torch.allclose(D1 @ D1.transpose(1, 2), eye, atol=1e-12)
    assert torch.allclose(D12, D1 @ D2, atol=1e-12)
    assert torch.allclose(torch.linalg.det(D1), torch.ones(8, dtype=DT), atol=1e-10)


@pytest.mark.parametrize("l", range(0, 7))
def test_wigner_rotates_harmonics(l):
    """Defining property Y(R u) = D(R) Y(u) at points the quadrature never visits."""
    R = _rand_rot(6, 5)
    u = _rand_unit(20, 6)
    D = O.wigner_d(l, R)
    lhs = O.real_sh(l, torch.einsum("rab,gb->rga", R, u))
    rhs = torch.einsum("rmn,gn->rgm", D, O.real_sh(l, u))
    assert torch.allclose(lhs, rhs, atol=1e-12)


def test_wigner_l1_is_permuted_rotation():
    R = _rand_rot(10, 7)
    P = torch.tensor([[0, 1, 0], [0, 0, 1], [1, 0, 0]], dtype=DT)   # (x,y,z) -> (y,z,x)
    assert torch.allclose(O.wigner_d(1, R), P @ R @ P.T, atol=1e-13)


@pytest.mark.parametrize("l", range(1, 7))
def test_wigner_z_rotation_block_form(l):
    """Rotation about z by alpha maps (Y_{+m}, Y_{-m}) by
    [[cos m a, -sin m a], [sin m a, cos m a]] and fixes Y_{l0}."""
    a = 0.7
    R = torch.tensor([[math.cos(a), -math.sin(a), 0], [math.sin(a), math.cos(a), 0], [0, 0, 1]], dtype=DT)
    D = O.wigner_d(l, R)
    ref = torch.zeros(2 * l + 1, 2 * l + 1, dtype=DT)
    ref[l, l] = 1
    for m in range(1, l + 1):
        c, s = math.cos(m * a), math.sin(m * a)
        ref[l + m, l + m] = c
        ref[l + m, l - m] = -s
        ref[l - m, l + m] = s
        ref[l - m, l - m] = c
    assert torch.allclose(D, ref, atol=1e-13)


def test_edge_frame_properties():
    u = _rand_unit(200, 8)
    u[0] = torch.tensor([0.0, 0.0, 1.0])
    u[1] = torch.tensor([0.0, 0.0, -1.0])
    u[2] = torch.tensor([1.0, 0.0, 0.0])
    R = O.edge_frame(u)
    eye = torch.eye(3, dtype=DT).expand(200, -1, -1)
    assert torch.allclose(R @ R.transpose(1, 2), eye, atol=1e-13)
    assert torch.allclose(torch.linalg.det(R), torch.ones(200, dtype=DT), atol=1e-13)
    z = torch.tensor([0.0, 0.0, 1.0], dtype=DT)
    assert torch.allclose(torch.einsum("eab,eb->ea", R, u), z.expand(200, -1), atol=1e-13)


@pytest.mark.parametrize("l", range(0, 7))
def test_edge_frame_alignment_and_addition_theorem(l):
    """In the edge frame the edge's harmonics vanish except at m = 0 (A.2), and the
    m = 0 row of D equals sqrt(4 pi/(2l+1)) Y_l(rhat) (addition theorem)."""
    u = _rand_unit(30, 9)
    D = O.wigner_d(l, O.edge_frame(u))
    Yr = O.real_sh(l, u)
    aligned = torch.einsum("emn,en->em", D, Yr)
    expect = torch.zeros_like(aligned)
    expect[:, l] = math.sqrt((2 * l + 1) / (4 * math.pi))
    assert torch.allclose(aligned, expect, atol=1e-12)
    assert torch.allclose(D[:, l, :], math.sqrt(4 * math.pi / (2 * l + 1)) * Yr, atol=1e-12)


@pytest.mark.parametrize("L,M", [(0, 0), (2, 2), (4, 2), (6, 2), (4, 4), (3, 1)])
def test_counts_closed_forms(L, M):
    q = O.q_count(L, M)
    assert q == (L + 1) * (2 * M + 1) - M * (M + 1)
    K = O.k_count(L, M)
    brute = sum(1 for l in range(L + 1) for m in range(-l, l + 1) if abs(m) <= M for _ in range(2 * l + 1))
    assert K == brute
