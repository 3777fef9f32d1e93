"""Oracle (test infrastructure only) of the spherical-grid SwiGLU activation on
edges (SwiGLU-S2): TrimSO(2) page, Table 2 (EquiformerV3's activation is
SwiGLU-S2), Appendix C.1 "Implementation" (EquiformerV3 uses its spherical-grid activation for
Edge -> Edge) and Appendix B.4 (G_l evaluates the degree-l basis at n_g grid
points; the nonlinearity acts on grid values).

Reading of the pages (they name the activation but give no formula): every
edge carries q retained coefficient rows (the (l, m) rows of the edge frame)
of 2C channels, a value half (channels 0..C-1) and a gate half (C..2C-1). Per
edge and channel c

    v = G u_v,   a = G u_g            (grid values, n_g of each)
    s = SiLU(a) * v                   (SwiGLU at every grid point)
    z = P s                           (back to the q rows)

with G [n_g, q] (the retained basis at the grid points) and P [q, n_g] (the
projection back, e.g. quadrature weights times G^T) supplied by the caller.
G and P are fixed; derivatives are taken with respect to the features:

  backward(gZ)            -> gU                      (vector-Jacobian product)
  double_backward(gZ, pU) -> dL/dgZ, dL/dU  for L = <pU, gU>

This module evaluates exactly that expression in float64 and differentiates
it with torch.autograd. It shares nothing with the HIP path; tests/ pins it
against a brute-force loop, the identity grid (plain SwiGLU), linearity in
the value half and finite differences.
"""
from __future__ import annotations

import torch

DT = torch.float64


def forward(U: torch.Tensor, G: torch.Tensor, P: torch.Tensor) -> torch.Tensor:
    """U [E, q, 2C], G [n_g, q], P [q, n_g] -> Z [E, q, C]."""
    C = U.shape[2] // 2
    v = torch.einsum("gr,erc->egc", G, U[:, :, :C])
    a = torch.einsum("gr,erc->egc", G, U[:, :, C:])
    s = torch.nn.functional.silu(a) * v
    return torch.einsum("rg,egc->erc", P, s)


def _leaf(t):
    return t.detach().clone().requires_grad_(True)


def backward(U, G, P, gZ):
    """gU of <gZ, Z>."""
    Ul = _leaf(U)
    (gU,) = torch.autograd.grad(forward(Ul, G, P), [Ul], gZ)
    return gU


def double_backward(U, G, P, gZ, pU):
    """dict ggZ, gU2: derivatives of L = <pU, gU> with respect to gZ and U."""
    Ul, gZl = _leaf(U), _leaf(gZ)
    (gU,) = torch.autograd.grad(forward(Ul, G, P), [Ul], gZl, create_graph=True)
    ggZ, gU2 = torch.autograd.grad((gU * pU).sum(), [gZl, Ul])
    return dict(ggZ=ggZ, gU2=gU2)
