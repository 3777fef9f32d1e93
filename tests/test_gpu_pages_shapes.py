"""Parity at the pages' captured-batch size (399 atoms, 17,880 edges, lmax 4,
mmax 2, C 128, float32) in bench.py's launch configuration: forward state kept,
the backward keeping its cotangents for the double backward. Every output of
the three stages, the weight gradients included, is compared element by
element with the float64 oracle over all edges. At this size the weight
gradients are split over the edges in 512-row chunks (35 splits per product),
so the test also pins the fixed-order split reduction at depth."""
import numpy as np
import pytest
import torch

from oracle import so2conv_oracle as O
from tests import _cases as H

pytestmark = pytest.mark.gpu
DT = torch.float64
BW = {"gx": "gx", "gpos": "gpos", "grbf": "grbf", "gw_rad": "gw_rad", "gw1": "gw1", "gw2": "gw2"}
DB = {"ggy": "ggy", "gx2": "gx", "grbf2": "grbf", "gw_rad2": "gw_rad", "gw1_2": "gw1", "gw2_2": "gw2"}


def test_captured_batch_size_matches_oracle():
    import so_graph_convolution_amd as K
    d = H.workload("P1")
    E, N = len(d["src"]), d["cfg"].n_atoms
    H.note(f"[pages shapes] P1 N={N} E={E}")
    dd = H.to_dev(d)
    kc = dd["kcfg"]
    args = (kc, dd["g"], dd["x"], dd["pos"], dd["rbf"], dd["w_rad"], dd["w1"], dd["w2"])
    saved = torch.empty(K.so2conv_saved_bytes(kc, E), dtype=torch.uint8, device="cuda")
    ws = torch.empty(max(K.so2conv_workspace_bytes(kc, N, E, s) for s in (0, 1, 2)), dtype=torch.uint8, device="cuda")
    kept = torch.empty(K.so2conv_saved_bwd_bytes(kc, E), dtype=torch.uint8, device="cuda")
    y, _ = K.so2conv_fwd(*args, saved=saved, ws=ws)
    bw = K.so2conv_bwd(*args, saved, dd["gy"], ws=ws, saved_bwd=kept)
    db = K.so2conv_dbwd(*args, saved, dd["gy"], px=dd["px"], ppos=dd["ppos"], prbf=dd["prbf"], ws=ws,
                        saved_bwd=kept)
    torch.cuda.synchronize()
    inp = H.oracle_inputs(d)
    t = lambda a: torch.tensor(np.asarray(a), dtype=DT)  # noqa: E731
    gy = t(d["gy"])
    ry = O.forward(inp)
    rb = O.backward(inp, gy)
    rd = O.double_backward(inp, gy, px=t(d["px"]), ppos=t(d["ppos"]), prbf=t(d["prbf"]))
    errs = {"y": H.errs_both(y, ry)}
    errs.update({k: H.errs_both(bw[k], rb[v]) for k, v in BW.items()})
    errs.update({k: H.errs_both(db[k], rd[v]) for k, v in DB.items()})
    H.note("  " + " ".join(f"{k}={v[0]:.1e}/{v[1]:.1e}" for k, v in errs.items()))
    bad = {k: v for k, v in errs.items() if v[0] > H.TOL_F32 or v[1] > H.TOL_ELEM_F32}
    assert not bad, bad
