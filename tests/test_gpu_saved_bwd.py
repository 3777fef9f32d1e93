"""Double backward that reuses the backward's cotangents (saved_bwd): the
backward writes Zbar, Ubar and Tbar, the double backward takes them for the
cotangents of its tangent chain and forms only the primal chain's. Every
output against the float64 oracle, and against the same call without the
saved cotangents; the backward's own outputs are bitwise unchanged by keeping
them. Float32 and bf16, one chunk and different chunkings in the two calls,
lmax 0..6, every direction (weights, edge vectors, positions), envelope and
per-head weights."""
import dataclasses

import numpy as np
import pytest
import torch

import so2_synth
from oracle import so2conv_oracle as O
from tests import _cases as H

pytestmark = pytest.mark.gpu
DT = torch.float64
BIG = dict(n_atoms=150, box=12.0, rc=4.0, lmax=4, mmax=2, channels=48, n_rbf=16, seed=5, min_dist=0.0)
CASES = [
    # name, workload overrides, dtype, (bwd chunk, dbwd chunk), heads (0: none), every direction
    ("l4m2_c48_ragged", BIG, "f32", (None, None), 0, False),
    ("tiny_T_all_directions", dict(), "f32", (None, None), 0, True),
    ("l6m2_c16", dict(n_atoms=48, box=9.0, rc=4.5, lmax=6, mmax=2, channels=16, n_rbf=8, seed=11), "f32",
     (None, None), 0, False),
    ("l0m0_c16", dict(lmax=0, mmax=0, channels=16, seed=3), "f32", (None, None), 0, False),
    ("l3m1_c32_all_directions", dict(n_atoms=40, box=8.0, rc=3.5, lmax=3, mmax=1, channels=32, n_rbf=8, seed=12,
                                     min_dist=0.0), "f32", (None, None), 0, True),
    ("l4m2_c48_chunks_1024_2048", BIG, "f32", (1024, 2048), 0, False),
    ("l3m2_c32_bf16", dict(n_atoms=40, box=8.0, rc=4.0, lmax=3, mmax=2, channels=32, n_rbf=8, seed=14), "bf16",
     (None, None), 0, True),
    ("l4m2_c128_h8_envelope", dict(n_atoms=100, box=11.0, rc=4.0, lmax=4, mmax=2, channels=128, n_rbf=16, seed=6,
                                   min_dist=0.0), "f32", (None, None), 8, False),
    ("l4m2_c48_envelope_chunked", BIG, "f32", (2048, 1024), 1, False),
]
BW = ("gx", "gpos", "grbf", "gw_rad", "gw1", "gw2", "gedge", "genv")
DB = {"ggy": "ggy", "gx2": "gx", "gpos2": "gpos", "grbf2": "grbf", "genv2": "genv", "gw_rad2": "gw_rad",
      "gw1_2": "gw1", "gw2_2": "gw2"}


def _same(a, b):
    if a is None or b is None:
        return a is None and b is None
    if isinstance(a, list):
        return all(torch.equal(x, y) for x, y in zip(a, b))
    return torch.equal(a, b)


def _rel(a, b):
    if isinstance(a, list):
        return max(_rel(x, y) for x, y in zip(a, b))
    a, b = a.double(), b.double()
    return float((a - b).abs().max() / b.abs().max().clamp_min(1e-30))


@pytest.mark.parametrize("name,over,dtype,chunks,heads,every", CASES, ids=[c[0] for c in CASES])
def test_saved_backward_state_matches_oracle(name, over, dtype, chunks, heads, every):
    import so_graph_convolution_amd as K
    d = dict(H.workload("T", dtype=dtype, **over))
    E = len(d["src"])
    cb, cd = chunks
    if cb or cd:
        assert E > 2048   # both calls run several chunks, cut at different edges
    rng = np.random.default_rng(77)
    penv = None
    if heads == 1:
        d["env"] = so2_synth.cosine_envelope(d)
        penv = rng.normal(size=E).astype(np.float32)
    elif heads > 1:
        d["env"] = so2_synth.attention_weights(d, heads, seed=3) * so2_synth.cosine_envelope(d)[:, None]
        penv = rng.normal(size=(E, heads)).astype(np.float32)
    H.note(f"[saved_bwd] {name} L={over.get('lmax', 2)} E={E} dtype={dtype} chunks={chunks} heads={heads}")
    dd = H.to_dev(d, dtype)
    if heads > 1:
        dd["kcfg"] = dataclasses.replace(dd["kcfg"], heads=heads)
    env = torch.tensor(d["env"], device="cuda") if heads else None
    dv = lambda a: torch.tensor(a, device="cuda")  # noqa: E731
    wt = lambda a: dv(a).to(dd["x"].dtype)  # noqa: E731
    dirs = dict(px=dd["px"], ppos=dd["ppos"], prbf=dd["prbf"])
    host = {}
    # weight directions in the call's dtype; the oracle sees the same (rounded) values
    rw = (lambda a: torch.tensor(a).to(torch.bfloat16).float().numpy()) if dtype == "bf16" else (lambda a: a)
    if every:
        host = dict(pw_rad=rw(rng.normal(size=d["w_rad"].shape).astype(np.float32)),
                    pw1=[rw((rng.normal(size=w.shape) * 0.1).astype(np.float32)) for w in d["w1"]],
                    pw2=[rw((rng.normal(size=w.shape) * 0.1).astype(np.float32)) for w in d["w2"]],
                    pedge=rng.normal(size=(E, 3)).astype(np.float32))
        dirs.update(pw_rad=wt(host["pw_rad"]), pw1=[wt(w) for w in host["pw1"]], pw2=[wt(w) for w in host["pw2"]],
                    pedge=dv(host["pedge"]))
    if penv is not None:
        dirs["penv"] = dv(penv)
    need = ("gy", "x", "pos", "rbf", "w_rad", "w1", "w2") + (("env",) if heads else ())
    args = (dd["kcfg"], dd["g"], dd["x"], dd["pos"], dd["rbf"], dd["w_rad"], dd["w1"], dd["w2"])
    keep = cb is None and cd is None
    y, saved = K.so2conv_fwd(*args, saved=True if keep else None, env=env)
    plain = K.so2conv_bwd(*args, saved, dd["gy"], chunk_edges=cb, env=env)
    bw = K.so2conv_bwd(*args, saved, dd["gy"], chunk_edges=cb, env=env, saved_bwd=True)
    db = K.so2conv_dbwd(*args, saved, dd["gy"], chunk_edges=cd, env=env, need=need, saved_bwd=bw["saved_bwd"],
                        **dirs)
    db0 = K.so2conv_dbwd(*args, saved, dd["gy"], chunk_edges=cd, env=env, need=need, **dirs)
    torch.cuda.synchronize()
    for k in BW:
        assert _same(bw[k], plain[k]), k      # keeping the cotangents changes nothing in the backward
    inp = H.oracle_inputs(d)
    t = lambda a: torch.tensor(a, dtype=DT)  # noqa: E731
    ref = O.double_backward(inp, t(d["gy"]), px=t(d["px"]), ppos=t(d["ppos"]), prbf=t(d["prbf"]),
                            penv=None if penv is None else t(penv),
                            **({} if not every else dict(pw_rad=t(host["pw_rad"]), pw1=[t(w) for w in host["pw1"]],
                                                         pw2=[t(w) for w in host["pw2"]], pedge=t(host["pedge"]))))
    keys = [k for k in DB if db.get(k) is not None]
    errs = {k: H.relerr(db[k], ref[DB[k]]) for k in keys}
    diff = {k: _rel(db[k], db0[k]) for k in keys}
    H.note("  oracle " + " ".join(f"{k}={v:.1e}" for k, v in errs.items()))
    H.note("  vs recomputed cotangents " + " ".join(f"{k}={v:.1e}" for k, v in diff.items()))
    tol = H.TOL_BF16 if dtype == "bf16" else H.TOL_F32
    assert all(v <= tol for v in errs.values()), errs
    # the same values up to the rounding of the stacked and unstacked products
    assert all(v <= (1e-2 if dtype == "bf16" else 1e-5) for v in diff.values()), diff
