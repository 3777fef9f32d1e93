"""Oracle (test infrastructure only) of the node-to-node spherical projection
with its channel maps, and of the back-projection from the grid: TrimSO(2)
page, Appendix B.4 (Spherical activations).

For one atom with features X^(l) (n_l x C_in, degree-major rows of the node
array), the grid values before the nonlinearity are

    U = [ sum_l G_l (X^(l) W_l) ] A                      (definition)

with G_l the degree-l basis evaluated at n_g grid points (a caller-supplied
n_g x (L+1)^2 matrix, column block l), W_l (C_in x C_h) and A (C_h x C_out).
This module computes exactly that expression, in float64, for every node,
and its derivatives with torch.autograd:

  backward(gU)                 -> gX, gW, gA      (vector-Jacobian product)
  double_backward(gU, pX, pW, pA)
      L = <pX, gX> + <pW, gW> + <pA, gA>  ->  dL/dgU, dL/dX, dL/dW, dL/dA

It shares nothing with the HIP path (which uses the reassociated form
B_l = W_l A); tests/ pins it against a brute-force loop and finite
differences. Only tests/, the smoke check and the benchmark's CPU leg use it.
"""
from __future__ import annotations

import torch

DT = torch.float64


def forward(x: torch.Tensor, G: torch.Tensor, W: torch.Tensor, A: torch.Tensor) -> torch.Tensor:
    """x [N, (L+1)^2, C_in], G [n_g, (L+1)^2], W [L+1, C_in, C_h], A [C_h, C_out] -> U [N, n_g, C_out]."""
    L = W.shape[0] - 1
    N, n_g = x.shape[0], G.shape[0]
    acc = torch.zeros(N, n_g, W.shape[2], dtype=x.dtype)
    for l in range(L + 1):
        rows = slice(l * l, (l + 1) * (l + 1))
        xw = x[:, rows, :] @ W[l]                                  # [N, n_l, C_h]
        acc = acc + torch.einsum("gm,nmh->ngh", G[:, rows], xw)    # G_l (X^(l) W_l)
    return acc @ A


def _leaves(*ts):
    return [t.detach().clone().requires_grad_(True) for t in ts]


def backward(x, G, W, A, gU):
    """dict gx, gW, gA of <gU, U>."""
    xl, Wl, Al = _leaves(x, W, A)
    U = forward(xl, G, Wl, Al)
    gx, gW, gA = torch.autograd.grad(U, [xl, Wl, Al], gU)
    return dict(gx=gx, gW=gW, gA=gA)


def double_backward(x, G, W, A, gU, px=None, pW=None, pA=None):
    """Derivatives of L = <px, gx> + <pW, gW> + <pA, gA> (the backward's outputs
    paired with directions; None = zero) with respect to gU, x, W and A."""
    xl, Wl, Al = _leaves(x, W, A)
    gUl = gU.detach().clone().requires_grad_(True)
    U = forward(xl, G, Wl, Al)
    g = torch.autograd.grad(U, [xl, Wl, Al], gUl, create_graph=True)
    Lval = torch.zeros((), dtype=DT)
    for gi, p in zip(g, (px, pW, pA)):
        if p is not None:
            Lval = Lval + (gi * p).sum()
    out = torch.autograd.grad(Lval, [gUl, xl, Wl, Al], allow_unused=True)
    z = [torch.zeros_like(t) if o is None else o for o, t in zip(out, (gUl, xl, Wl, Al))]
    return dict(ggU=z[0], gx=z[1], gW=z[2], gA=z[3])


# ----------------------------------------------------------------------------- back-projection
# TrimSO(2) page, Appendix B.4 (Forward computation, the second identity):
# after the nonlinearity on the grid, the values Y (n_g x C_h per atom) return
# to coefficients through H_l (n_l x n_g, the degree-l rows of a caller-
# supplied (L+1)^2 x n_g matrix) and an output channel map A_out (C_h x C_out):
#     Z^(l) = H_l (Y A_out)                                  (definition)
# The page's reordering (H_l Y) A_out is what the HIP path computes; the
# oracle keeps the definition's order.

def back_forward(Y: torch.Tensor, H: torch.Tensor, A: torch.Tensor) -> torch.Tensor:
    """Y [N, n_g, C_h], H [(L+1)^2, n_g], A [C_h, C_out] -> Z [N, (L+1)^2, C_out]."""
    YA = Y @ A                                                   # [N, n_g, C_out]
    return torch.einsum("jg,ngc->njc", H, YA)


def back_backward(Y, H, A, gZ):
    """dict gY, gA of <gZ, Z> (H is a fixed basis, not differentiated)."""
    Yl, Al = _leaves(Y, A)
    Z = back_forward(Yl, H, Al)
    gY, gA = torch.autograd.grad(Z, [Yl, Al], gZ)
    return dict(gY=gY, gA=gA)


def back_double_backward(Y, H, A, gZ, pY=None, pA=None):
    """Derivatives of L = <pY, gY> + <pA, gA> (None = zero) with respect to gZ, Y and A."""
    Yl, Al = _leaves(Y, A)
    gZl = gZ.detach().clone().requires_grad_(True)
    Z = back_forward(Yl, H, Al)
    g = torch.autograd.grad(Z, [Yl, Al], gZl, create_graph=True)
    Lval = torch.zeros((), dtype=DT)
    for gi, p in zip(g, (pY, pA)):
        if p is not None:
            Lval = Lval + (gi * p).sum()
    out = torch.autograd.grad(Lval, [gZl, Yl, Al], allow_unused=True)
    z = [torch.zeros_like(t) if o is None else o for o, t in zip(out, (gZl, Yl, Al))]
    return dict(ggZ=z[0], gY=z[1], gA=z[2])
