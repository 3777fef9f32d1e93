"""Pins for the mixture-of-linear-experts oracle (TrimSO(2) page, Appendix C.1:
UMA's system-dependent mixtures of linear experts; Table 2: 64 experts).

  * one-hot coefficients: each system's output is the plain operator (itself
    pinned) with that system's single expert on that system's edges;
  * shared coefficients: the whole batch is the plain operator with the
    expert mixture merged independently in numpy;
  * chain rule through the plain operator: gW^(k) = sum_s coef[s,k] gW(s) and
    gcoef[s,k] = sum_m <W_m^(k), gW_m(s)>, with gW(s) the plain backward's
    weight gradient on system s's edges at its merged weights;
  * central finite differences of the forward (backward outputs) and of the
    backward (double-backward outputs) along coefficient and expert directions.
An empty system (no edges) is part of every case."""
import numpy as np
import pytest
import torch

from oracle import mole_oracle as MO
from oracle import so2conv_oracle as O
from tests.test_oracle_op import DT, _inputs

K_EXPERTS = 3


def _randn(shape, g):
    return torch.randn(shape, generator=g, dtype=DT)


@pytest.fixture(scope="module")
def case():
    d = _inputs(L=2, M=2, C=3, n_atoms=10, box=6.0, rc=3.4, seed=5, edges_max=48)
    base = O.to_oracle_inputs(d)
    g = torch.Generator().manual_seed(9)
    w1e = [_randn((K_EXPERTS,) + tuple(w.shape), g) * 0.5 for w in base.w1]
    w2e = [_randn((K_EXPERTS,) + tuple(w.shape), g) * 0.5 for w in base.w2]
    b = np.searchsorted(d["dst"], [4, 7])
    sys_edge_ptr = [0, int(b[0]), int(b[0]), int(b[1]), len(d["src"])]     # system 1 is empty
    S = len(sys_edge_ptr) - 1
    coef = torch.rand(S, K_EXPERTS, generator=g, dtype=DT) + 0.1
    gy = torch.tensor(d["gy"], dtype=DT)
    return d, base, w1e, w2e, coef, sys_edge_ptr, gy


def _plain_with(base, w1, w2):
    return O.OracleInputs(base.L, base.M, base.C, base.pos, base.x, base.src, base.dst, base.shift, base.rbf,
                          base.w_rad, w1, w2, base.env)


def test_one_hot_coefficients_select_an_expert(case):
    d, base, w1e, w2e, _, sp, _ = case
    S = len(sp) - 1
    pick = [2, 0, 1, 0][:S]
    coef = torch.zeros(S, K_EXPERTS, dtype=DT)
    for s, k in enumerate(pick):
        coef[s, k] = 1.0
    y = MO.forward(base, w1e, w2e, coef, sp)
    ref = torch.zeros_like(y)
    for s, k in enumerate(pick):
        edges = np.arange(sp[s], sp[s + 1])
        if len(edges):
            ref += O.forward(_plain_with(base, [w[k] for w in w1e], [w[k] for w in w2e]), edges=edges)
    assert torch.allclose(y, ref, atol=1e-12, rtol=0)


def test_shared_coefficients_are_the_merged_plain_operator(case):
    d, base, w1e, w2e, _, sp, _ = case
    a = np.array([0.3, -1.2, 0.7])
    coef = torch.tensor(np.tile(a, (len(sp) - 1, 1)), dtype=DT)
    merged1 = [torch.tensor(np.tensordot(a, w.numpy(), axes=1), dtype=DT) for w in w1e]
    merged2 = [torch.tensor(np.tensordot(a, w.numpy(), axes=1), dtype=DT) for w in w2e]
    y = MO.forward(base, w1e, w2e, coef, sp)
    assert torch.allclose(y, O.forward(_plain_with(base, merged1, merged2)), atol=1e-11, rtol=0)


def test_gradients_follow_the_plain_backward(case):
    d, base, w1e, w2e, coef, sp, gy = case
    g = MO.backward(base, w1e, w2e, coef, sp, gy)
    gw1e = [torch.zeros_like(w) for w in w1e]
    gw2e = [torch.zeros_like(w) for w in w2e]
    gcoef = torch.zeros_like(coef)
    for s in range(len(sp) - 1):
        edges = np.arange(sp[s], sp[s + 1])
        if not len(edges):
            continue
        w1s = [torch.einsum("k,krc->rc", coef[s], w) for w in w1e]
        w2s = [torch.einsum("k,krc->rc", coef[s], w) for w in w2e]
        b = O.backward(_plain_with(base, w1s, w2s), gy, edges=edges)
        for m in range(len(w1e)):
            gw1e[m] += coef[s][:, None, None] * b["gw1"][m][None]
            gw2e[m] += coef[s][:, None, None] * b["gw2"][m][None]
            gcoef[s] += (w1e[m] * b["gw1"][m][None]).sum((1, 2)) + (w2e[m] * b["gw2"][m][None]).sum((1, 2))
    assert torch.allclose(g["gcoef"], gcoef, atol=1e-10, rtol=0)
    for m in range(len(w1e)):
        assert torch.allclose(g["gw1e"][m], gw1e[m], atol=1e-10, rtol=0)
        assert torch.allclose(g["gw2e"][m], gw2e[m], atol=1e-10, rtol=0)
    assert torch.all(g["gcoef"][1] == 0)                                 # the empty system


def _fd(f, eps=1e-5):
    return (f(eps) - f(-eps)) / (2 * eps)


@pytest.mark.parametrize("which", ["coef", "w1e", "w2e"])
def test_backward_matches_finite_differences(case, which):
    d, base, w1e, w2e, coef, sp, gy = case
    g = torch.Generator().manual_seed(31)
    p = {"coef": _randn(coef.shape, g), "w1e": [_randn(w.shape, g) for w in w1e],
         "w2e": [_randn(w.shape, g) for w in w2e]}[which]

    def val(eps):
        c = coef + eps * p if which == "coef" else coef
        a = [w + eps * q for w, q in zip(w1e, p)] if which == "w1e" else w1e
        b = [w + eps * q for w, q in zip(w2e, p)] if which == "w2e" else w2e
        return (MO.forward(base, a, b, c, sp) * gy).sum()
    gr = MO.backward(base, w1e, w2e, coef, sp, gy)["g" + which]
    pred = (gr * p).sum() if which == "coef" else sum((x * y).sum() for x, y in zip(gr, p))
    fd = _fd(val)
    assert abs(float(pred - fd)) <= 1e-6 * max(1.0, abs(float(fd)))


def test_double_backward_matches_finite_differences(case):
    """Directions on coef, experts and x together; every output against the FD
    of <p, backward> along a random direction of its argument, and ggy against
    the forward's directional derivative."""
    d, base, w1e, w2e, coef, sp, gy = case
    g = torch.Generator().manual_seed(41)
    pcoef = _randn(coef.shape, g)
    pw1e = [_randn(w.shape, g) for w in w1e]
    pw2e = [_randn(w.shape, g) for w in w2e]
    px = _randn(base.x.shape, g)
    h = MO.double_backward(base, w1e, w2e, coef, sp, gy, px=px, pcoef=pcoef, pw1e=pw1e, pw2e=pw2e)

    def Lfun(coef_, w1e_, w2e_, gy_, x_=None):
        b2 = base if x_ is None else O.OracleInputs(base.L, base.M, base.C, base.pos, x_, base.src, base.dst,
                                                    base.shift, base.rbf, base.w_rad, base.w1, base.w2, base.env)
        r = MO.backward(b2, w1e_, w2e_, coef_, sp, gy_)
        return ((r["gx"] * px).sum() + (r["gcoef"] * pcoef).sum()
                + sum((a * b).sum() for a, b in zip(r["gw1e"], pw1e))
                + sum((a * b).sum() for a, b in zip(r["gw2e"], pw2e)))
    qc = _randn(coef.shape, g)
    q1 = [_randn(w.shape, g) for w in w1e]
    q2 = [_randn(w.shape, g) for w in w2e]
    qg = _randn(gy.shape, g)
    qx = _randn(base.x.shape, g)
    checks = [
        ((h["gcoef"] * qc).sum(), _fd(lambda e: Lfun(coef + e * qc, w1e, w2e, gy))),
        (sum((a * b).sum() for a, b in zip(h["gw1e"], q1)),
         _fd(lambda e: Lfun(coef, [w + e * q for w, q in zip(w1e, q1)], w2e, gy))),
        (sum((a * b).sum() for a, b in zip(h["gw2e"], q2)),
         _fd(lambda e: Lfun(coef, w1e, [w + e * q for w, q in zip(w2e, q2)], gy))),
        ((h["ggy"] * qg).sum(), _fd(lambda e: Lfun(coef, w1e, w2e, gy + e * qg))),
        ((h["gx"] * qx).sum(), _fd(lambda e: Lfun(coef, w1e, w2e, gy, base.x + e * qx))),
    ]
    for pred, fd in checks:
        assert abs(float(pred - fd)) <= 1e-6 * max(1.0, abs(float(fd))), (float(pred), float(fd))
