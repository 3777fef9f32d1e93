"""Both float32 product paths against the float64 oracle: the default (every
float32 operand as the exact sum of three bfloat16 pieces, piece products on
the bfloat16 matrix cores, float32 accumulation) and SO2_F32_NATIVE (the
float32 matrix cores, complex products of orders >= 1 with three real
products). Forward, backward and the force-pattern double backward; the
float32 bar for the max-norm error and the element-wise bar above its floor.
"""
import dataclasses

import pytest
import torch

from oracle import so2conv_oracle as O
from tests import _cases as H

pytestmark = pytest.mark.gpu
DT = torch.float64

CASES = [
    ("l4m2_c48_ragged", "T", dict(n_atoms=40, box=8.0, rc=4.5, lmax=4, mmax=2, channels=48, seed=21)),
    ("l2m2_c128", "T", dict(n_atoms=48, box=8.0, rc=4.0, lmax=2, mmax=2, channels=128, n_rbf=16, seed=22)),
    ("l6m2_c32", "T", dict(n_atoms=24, box=8.0, rc=4.0, lmax=6, mmax=2, channels=32, seed=23)),
]


@pytest.mark.parametrize("native", [False, True], ids=["pieces", "native"])
@pytest.mark.parametrize("name,base,over", CASES, ids=[c[0] for c in CASES])
def test_f32_paths_match_oracle(name, base, over, native):
    import so_graph_convolution_amd as K
    d = H.workload(base, **over)
    cfg = d["cfg"]
    H.note(f"[f32 path {'native' if native else 'pieces'}] {name} L={cfg.lmax} C={cfg.channels} E={len(d['src'])}")
    dd = H.to_dev(d)
    kc = dataclasses.replace(dd["kcfg"], f32_native=native)
    args = (kc, dd["g"], dd["x"], dd["pos"], dd["rbf"], dd["w_rad"], dd["w1"], dd["w2"])
    y, saved = K.so2conv_fwd(*args, saved=True)
    bw = K.so2conv_bwd(*args, saved, dd["gy"])
    db = K.so2conv_dbwd(*args, saved, dd["gy"], px=dd["px"], ppos=dd["ppos"], prbf=dd["prbf"])
    torch.cuda.synchronize()
    t = lambda a: torch.tensor(a, dtype=DT)  # noqa: E731
    inp = H.oracle_inputs(d)
    ry = O.forward(inp)
    rb = O.backward(inp, t(d["gy"]))
    rd = O.double_backward(inp, t(d["gy"]), px=t(d["px"]), ppos=t(d["ppos"]), prbf=t(d["prbf"]))
    pairs = [("y", y, ry)] + [(k, bw[k], rb[k]) for k in ("gx", "gpos", "grbf", "gw_rad", "gw1", "gw2")] + \
        [("ggy", db["ggy"], rd["ggy"]), ("gx2", db["gx2"], rd["gx"]), ("gw1_2", db["gw1_2"], rd["gw1"]),
         ("gw2_2", db["gw2_2"], rd["gw2"]), ("gw_rad2", db["gw_rad2"], rd["gw_rad"])]
    errs = {k: H.errs_both(g, r) for k, g, r in pairs}
    H.note("  " + " ".join(f"{k}={e[0]:.1e}/{e[1]:.1e}" for k, e in errs.items()))
    bad = {k: e for k, e in errs.items() if not (e[0] <= H.TOL_F32 and e[1] <= H.TOL_ELEM_F32)}
    assert not bad, bad
