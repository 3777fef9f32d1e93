"""The so(3) generator table compiled into the library (the literal operands
of the kernels' torque and rotation-rate products), read on the CPU through
the C ABI and pinned to the oracle: each block G_k^(l) = d/dt D^(l)(exp(t [e_k]_x))
at t = 0 (TrimSO(2) page, Section 2's frame rotation, differentiated for the
position derivatives of Appendix B.1) against a central difference of the
oracle's quadrature Wigner-D blocks in float64, plus the so(3) identities the
generators of any representation satisfy."""
import math

import numpy as np
import pytest
import torch

from oracle import so2conv_oracle as O

LMAX = 6


def _blocks(table):
    """[k][l] -> (2l+1) x (2l+1) float64 blocks of the library's table."""
    out, off = [], 0
    for l in range(LMAX + 1):
        n = 2 * l + 1
        out.append(off)
        off += n * n
    assert off == table.shape[1]
    return [[table[k, out[l]:out[l] + (2 * l + 1) ** 2].double().view(2 * l + 1, 2 * l + 1) for l in range(LMAX + 1)]
            for k in range(3)]


@pytest.fixture(scope="module")
def table():
    import so_graph_convolution_amd as K
    return _blocks(K.so2conv_generator_table())


def _rot(k, t):
    """exp(t [e_k]_x): rotation by t about axis k (float64)."""
    c, s = math.cos(t), math.sin(t)
    R = torch.eye(3, dtype=torch.float64)
    i, j = [(1, 2), (2, 0), (0, 1)][k]
    R[i, i], R[i, j], R[j, i], R[j, j] = c, -s, s, c
    return R


@pytest.mark.parametrize("l", range(LMAX + 1))
def test_blocks_match_oracle_derivative(table, l):
    h = 1e-5
    for k in range(3):
        fd = (O.wigner_d(l, _rot(k, h)) - O.wigner_d(l, _rot(k, -h))) / (2 * h)
        err = (table[k][l] - fd).abs().max().item()
        assert err < 2e-6, (k, l, err)


@pytest.mark.parametrize("l", range(1, LMAX + 1))
def test_so3_identities(table, l):
    Gx, Gy, Gz = (table[k][l] for k in range(3))
    for G in (Gx, Gy, Gz):
        assert torch.allclose(G, -G.T, atol=1e-6)                      # antisymmetric
    assert torch.allclose(Gx @ Gy - Gy @ Gx, Gz, atol=1e-5)            # [G_x, G_y] = G_z, cyclic
    assert torch.allclose(Gy @ Gz - Gz @ Gy, Gx, atol=1e-5)
    assert torch.allclose(Gz @ Gx - Gx @ Gz, Gy, atol=1e-5)
    cas = Gx @ Gx + Gy @ Gy + Gz @ Gz                                   # Casimir: -l(l+1) I
    assert torch.allclose(cas, -l * (l + 1) * torch.eye(2 * l + 1, dtype=torch.float64), atol=1e-4)


def test_query_rejects_short_buffer():
    import ctypes

    import so_graph_convolution_amd as K
    n = K.lib().so2conv_generator_table(None, 0)
    buf = (ctypes.c_float * 4)()
    assert K.lib().so2conv_generator_table(buf, 4) < 0
    assert n == 3 * sum((2 * l + 1) ** 2 for l in range(LMAX + 1))
