"""Per-edge cutoff envelope on the messages (y_i = sum env_e R_e^T t_e) and
per-head attention weights (env [E, H], channel c weighted by its head's
weight): forward, backward (incl. genv, gpos, gedge) and double backward
(incl. a direction penv on the weights, genv2 and gpos2) through the C ABI
against the oracle; float32 and bf16, one chunk and 1024-edge chunks; heads
of 16 and 32 channels (summed inside a wave) and of one and two waves."""
import dataclasses

import numpy as np
import pytest
import torch

import so2_synth
from oracle import so2conv_oracle as O
from tests import _cases as H

pytestmark = pytest.mark.gpu
DT = torch.float64
CASES = [
    ("l4m2_c48_ragged", dict(n_atoms=150, box=12.0, rc=4.0, lmax=4, mmax=2, channels=48, n_rbf=16, seed=5,
                             min_dist=0.0), "f32", None),
    ("l2m2_c16_tiny", dict(), "f32", None),
    ("l6m2_c16", dict(n_atoms=48, box=9.0, rc=4.5, lmax=6, mmax=2, channels=16, n_rbf=8, seed=11), "f32", None),
    ("l4m2_c48_chunked", dict(n_atoms=150, box=12.0, rc=4.0, lmax=4, mmax=2, channels=48, n_rbf=16, seed=5,
                              min_dist=0.0), "f32", 1024),
    ("l3m2_c32_bf16", dict(n_atoms=40, box=8.0, rc=4.0, lmax=3, mmax=2, channels=32, n_rbf=8, seed=14), "bf16", None),
]
HEAD_CASES = [
    # name, workload overrides, dtype, chunk_edges, heads
    ("l4m2_c128_h8", dict(n_atoms=100, box=11.0, rc=4.0, lmax=4, mmax=2, channels=128, n_rbf=16, seed=6,
                          min_dist=0.0), "f32", None, 8),
    ("l4m2_c128_h2_chunked", dict(n_atoms=100, box=11.0, rc=4.0, lmax=4, mmax=2, channels=128, n_rbf=16, seed=7,
                                  min_dist=0.0), "f32", 1024, 2),
    ("l2m2_c256_h2", dict(n_atoms=40, box=8.0, rc=4.0, lmax=2, mmax=2, channels=256, n_rbf=8, seed=15), "f32",
     None, 2),
    ("l3m2_c64_h2_bf16", dict(n_atoms=40, box=8.0, rc=4.0, lmax=3, mmax=2, channels=64, n_rbf=8, seed=14), "bf16",
     None, 2),
    ("l6m2_c96_h3", dict(n_atoms=48, box=9.0, rc=4.5, lmax=6, mmax=2, channels=96, n_rbf=8, seed=11), "f32", None, 3),
]
BW = {"gx": "gx", "gpos": "gpos", "grbf": "grbf", "genv": "genv", "gw_rad": "gw_rad", "gw1": "gw1", "gw2": "gw2",
      "gedge": "gedge"}
DB = {"ggy": "ggy", "gx2": "gx", "gpos2": "gpos", "grbf2": "grbf", "genv2": "genv", "gw_rad2": "gw_rad",
      "gw1_2": "gw1", "gw2_2": "gw2"}


@pytest.mark.parametrize("name,over,dtype,chunk,heads", [c + (1,) for c in CASES] + HEAD_CASES,
                         ids=[c[0] for c in CASES] + [c[0] for c in HEAD_CASES])
def test_envelope_matches_oracle(name, over, dtype, chunk, heads):
    import so_graph_convolution_amd as K
    d = dict(H.workload("T", dtype=dtype, **over))
    E = len(d["src"])
    if heads == 1:
        d["env"] = so2_synth.cosine_envelope(d)
        penv = np.random.default_rng(41).normal(size=E).astype(np.float32)
    else:
        d["env"] = (so2_synth.attention_weights(d, heads, seed=3) * so2_synth.cosine_envelope(d)[:, None])
        penv = np.random.default_rng(41).normal(size=(E, heads)).astype(np.float32)
    H.note(f"[envelope] {name} E={E} dtype={dtype} chunks={chunk} heads={heads}")
    dd = H.to_dev(d, dtype)
    dd["kcfg"] = dataclasses.replace(dd["kcfg"], heads=heads)
    env = torch.tensor(d["env"], device="cuda")
    args = (dd["kcfg"], dd["g"], dd["x"], dd["pos"], dd["rbf"], dd["w_rad"], dd["w1"], dd["w2"])
    keep = chunk is None
    y, saved = K.so2conv_fwd(*args, saved=True if keep else None, chunk_edges=chunk, env=env)
    bw = K.so2conv_bwd(*args, saved, dd["gy"], chunk_edges=chunk, env=env)
    db = K.so2conv_dbwd(*args, saved, dd["gy"], px=dd["px"], ppos=dd["ppos"], prbf=dd["prbf"],
                        penv=torch.tensor(penv, device="cuda"), env=env, chunk_edges=chunk,
                        need=("gy", "x", "pos", "rbf", "env", "w_rad", "w1", "w2"))
    torch.cuda.synchronize()
    inp = H.oracle_inputs(d)
    t = lambda a: torch.tensor(a, dtype=DT)  # noqa: E731
    gy = t(d["gy"])
    ry = O.forward(inp)
    rb = O.backward(inp, gy, with_edge_grad=True)
    rd = O.double_backward(inp, gy, px=t(d["px"]), ppos=t(d["ppos"]), prbf=t(d["prbf"]), penv=t(penv))
    errs = {"y": H.relerr(y, ry)}
    errs.update({k: H.relerr(bw[k], rb[v]) for k, v in BW.items()})
    errs.update({k: H.relerr(db[k], rd[v]) for k, v in DB.items()})
    H.note("  " + " ".join(f"{k}={v:.1e}" for k, v in errs.items()))
    tol = H.TOL_BF16 if dtype == "bf16" else H.TOL_F32
    assert all(v <= tol for v in errs.values()), errs


def test_envelope_of_ones_is_bitwise_no_envelope():
    import so_graph_convolution_amd as K
    d = H.workload("T", n_atoms=40, box=8.0, rc=4.0, lmax=3, mmax=2, channels=32, n_rbf=8, seed=14)
    dd = H.to_dev(d)
    args = (dd["kcfg"], dd["g"], dd["x"], dd["pos"], dd["rbf"], dd["w_rad"], dd["w1"], dd["w2"])
    ones = torch.ones(len(d["src"]), device="cuda")
    y0, s0 = K.so2conv_fwd(*args, saved=True)
    y1, s1 = K.so2conv_fwd(*args, saved=True, env=ones)
    b0 = K.so2conv_bwd(*args, s0, dd["gy"])
    b1 = K.so2conv_bwd(*args, s1, dd["gy"], env=ones)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)
    for k in ("gx", "gpos", "grbf", "gedge"):
        assert torch.equal(b0[k], b1[k]), k


def test_envelope_derivatives_need_an_envelope():
    import so_graph_convolution_amd as K
    d = H.workload("T", seed=2)
    dd = H.to_dev(d)
    args = (dd["kcfg"], dd["g"], dd["x"], dd["pos"], dd["rbf"], dd["w_rad"], dd["w1"], dd["w2"])
    y, saved = K.so2conv_fwd(*args, saved=True)
    with pytest.raises(K.So2Error) as ei:
        K.so2conv_dbwd(*args, saved, dd["gy"], penv=torch.ones(len(d["src"]), device="cuda"))
    assert ei.value.code == -1
