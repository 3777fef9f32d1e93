"""Pins for per-head message weights in the oracle (TrimSO(2) page, Appendix
C.1: EquiformerV3 applies attention weights before aggregation; Table 2: 8
heads of 16 value channels). Weights env [E, H], head h covering channels
[h C/H, (h+1) C/H):

  * heads that all carry the same weight are the per-edge envelope;
  * the channels of head h are exactly the per-edge-envelope operator with
    env = env[:, h] on those channels (channels do not mix after the second
    linear, so each head's weights act on its channel group alone);
  * genv [E, H] and the double backward with a direction on the weights agree
    with central finite differences."""
import numpy as np
import pytest
import torch

from oracle import so2conv_oracle as O
from tests.test_oracle_op import DT, _dirs, _dot, _inputs, _perturbed

H = 2


@pytest.fixture(scope="module")
def head_case():
    d = dict(_inputs(L=3, M=2, C=4, n_atoms=10, box=6.0, rc=3.4, seed=13, edges_max=36))
    d["env"] = np.random.default_rng(5).uniform(0.2, 1.0, (len(d["src"]), H))
    return d, O.to_oracle_inputs(d), torch.tensor(d["gy"], dtype=DT)


def _with(d, env):
    d2 = dict(d)
    d2["env"] = env
    return O.to_oracle_inputs(d2)


def test_equal_heads_are_the_edge_envelope(head_case):
    d, _, _ = head_case
    e1 = d["env"][:, 0]
    y_heads = O.forward(_with(d, np.stack([e1] * H, 1)))
    assert torch.allclose(y_heads, O.forward(_with(d, e1)), rtol=0, atol=1e-14)


def test_each_head_is_the_envelope_on_its_channels(head_case):
    d, inp, _ = head_case
    y = O.forward(inp)
    hs = inp.C // H
    for h in range(H):
        ref = O.forward(_with(d, d["env"][:, h]))
        sl = slice(h * hs, (h + 1) * hs)
        assert torch.allclose(y[:, :, sl], ref[:, :, sl], rtol=0, atol=1e-14)


def _randn(shape, seed):
    return torch.randn(shape, generator=torch.Generator().manual_seed(seed), dtype=DT)


def test_genv_per_head_matches_finite_differences(head_case):
    d, inp, gy = head_case
    q = _randn((len(d["src"]), H), 7)
    g = O.backward(inp, gy)
    assert g["genv"].shape == q.shape
    eps = 1e-6
    fd = (_dot(O.forward(_perturbed(inp, "env", q, eps)), gy)
          - _dot(O.forward(_perturbed(inp, "env", q, -eps)), gy)) / (2 * eps)
    assert abs(float(_dot(g["genv"], q) - fd)) <= 1e-7 * max(1.0, abs(float(fd)))


@pytest.mark.parametrize("which", ["gy", "env", "x"])
def test_double_backward_with_head_direction(head_case, which):
    d, inp, gy = head_case
    p = _dirs(inp, 43)
    penv = _randn((len(d["src"]), H), 47)
    dd = O.double_backward(inp, gy, px=p["x"], ppos=p["pos"], penv=penv)
    eps = 1e-5
    if which == "gy":
        def shifted(e):
            s = _perturbed(inp, "x", p["x"], e)
            s = _perturbed(s, "pos", p["pos"], e)
            return _perturbed(s, "env", penv, e)
        jvp = (O.forward(shifted(eps)) - O.forward(shifted(-eps))) / (2 * eps)
        assert torch.allclose(dd["ggy"], jvp, atol=1e-7 * float(jvp.abs().max()))
        return
    q = {"x": _dirs(inp, 44)["x"], "env": _randn((len(d["src"]), H), 53)}[which]

    def L(e):
        g = O.backward(_perturbed(inp, which, q, e), gy)
        return _dot(g["gx"], p["x"]) + _dot(g["gpos"], p["pos"]) + _dot(g["genv"], penv)
    fd = (L(eps) - L(-eps)) / (2 * eps)
    an = _dot(dd[{"x": "gx", "env": "genv"}[which]], q)
    assert abs(float(an - fd)) <= 1e-6 * max(1.0, abs(float(fd)))
