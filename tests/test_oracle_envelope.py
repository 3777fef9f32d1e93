"""Pins for the oracle's optional per-edge cutoff envelope: each message is
scaled by env[e] before the receiver sum (TrimSO(2) page, Appendix C.1
Implementation: eSEN and UMA sum messages with their cutoff envelopes).

  * env = 1 is the operator without an envelope;
  * the output is the env-weighted sum of the single-edge outputs computed
    without an envelope (so the envelope multiplies the final message, after
    the gate and the second linear);
  * genv and the double backward with a direction on env agree with central
    finite differences of the forward and of the backward."""
import numpy as np
import pytest
import torch

from oracle import so2conv_oracle as O
from tests.test_oracle_op import DT, _dirs, _dot, _inputs, _perturbed


@pytest.fixture(scope="module")
def env_case():
    d = dict(_inputs(L=3, M=2, C=3, n_atoms=10, box=6.0, rc=3.4, seed=11, edges_max=40))
    d["env"] = np.random.default_rng(3).uniform(0.2, 1.0, len(d["src"]))
    return d, O.to_oracle_inputs(d), torch.tensor(d["gy"], dtype=DT)


def _without(d, env):
    d2 = dict(d)
    d2["env"] = env
    return O.to_oracle_inputs(d2)


def _randn(n, seed):
    return torch.randn(n, generator=torch.Generator().manual_seed(seed), dtype=DT)


def test_unit_envelope_is_no_envelope(env_case):
    d, _, _ = env_case
    assert torch.equal(O.forward(_without(d, np.ones(len(d["src"])))), O.forward(_without(d, None)))


def test_envelope_scales_each_final_message(env_case):
    d, inp, _ = env_case
    inp0 = _without(d, None)
    ref = sum(float(d["env"][e]) * O.forward(inp0, edges=np.array([e])) for e in range(len(d["src"])))
    y = O.forward(inp)
    assert torch.allclose(y, ref, rtol=0, atol=1e-12 * float(ref.abs().max()))


def test_genv_matches_finite_differences(env_case):
    d, inp, gy = env_case
    q = _randn(len(d["src"]), 5)
    g = O.backward(inp, gy)
    eps = 1e-6
    fd = (_dot(O.forward(_perturbed(inp, "env", q, eps)), gy)
          - _dot(O.forward(_perturbed(inp, "env", q, -eps)), gy)) / (2 * eps)
    assert abs(float(_dot(g["genv"], q) - fd)) <= 1e-7 * max(1.0, abs(float(fd)))


@pytest.mark.parametrize("which", ["gy", "x", "pos", "env"])
def test_double_backward_with_envelope_direction(env_case, which):
    d, inp, gy = env_case
    p = _dirs(inp, 23)
    penv = _randn(len(d["src"]), 29)
    dd = O.double_backward(inp, gy, px=p["x"], ppos=p["pos"], prbf=p["rbf"], penv=penv)
    eps = 1e-5
    if which == "gy":
        # ggy is the forward's derivative along (px, ppos, prbf, penv)
        def shifted(e):
            s = _perturbed(inp, "x", p["x"], e)
            s = _perturbed(s, "pos", p["pos"], e)
            s = _perturbed(s, "rbf", p["rbf"], e)
            return _perturbed(s, "env", penv, e)
        jvp = (O.forward(shifted(eps)) - O.forward(shifted(-eps))) / (2 * eps)
        assert torch.allclose(dd["ggy"], jvp, atol=1e-7 * float(jvp.abs().max()))
        return
    q = {"x": _dirs(inp, 24)["x"], "pos": _dirs(inp, 24)["pos"], "env": _randn(len(d["src"]), 31)}[which]

    def L(e):
        g = O.backward(_perturbed(inp, which, q, e), gy)
        return (_dot(g["gx"], p["x"]) + _dot(g["gpos"], p["pos"]) + _dot(g["grbf"], p["rbf"])
                + _dot(g["genv"], penv))
    fd = (L(eps) - L(-eps)) / (2 * eps)
    an = _dot(dd[{"x": "gx", "pos": "gpos", "env": "genv"}[which]], q)
    assert abs(float(an - fd)) <= 1e-6 * max(1.0, abs(float(fd)))
