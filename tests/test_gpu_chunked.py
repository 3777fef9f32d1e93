"""Chunked, memory-bounded execution: edges processed in chunks of 1024 (node
ranges split across chunks, sender segments cut by chunk), with and without
the saved forward state, against the oracle."""
import pytest
import torch

from oracle import so2conv_oracle as O
from tests import _cases as H

pytestmark = pytest.mark.gpu
DT = torch.float64

CASES = [
    ("l4m2_c48_ragged", dict(n_atoms=150, box=12.0, rc=4.0, lmax=4, mmax=2, channels=48, n_rbf=16, seed=5,
                             min_dist=0.0)),
    ("l2m2_c32_multi_image", dict(n_atoms=32, box=8.0, rc=5.0, lmax=2, mmax=2, channels=32, n_rbf=8, seed=21)),
]


@pytest.mark.parametrize("name,over", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("keep_state", [False, True], ids=["recompute", "saved"])
def test_chunked_matches_oracle(name, over, keep_state):
    import so_graph_convolution_amd as K
    d = H.workload("T", **over)
    E = len(d["src"])
    H.note(f"[chunked {'saved' if keep_state else 'recompute'}] {name} E={E} chunks of 1024")
    assert E > 1024   # at least two chunks
    dd = H.to_dev(d)
    args = (dd["kcfg"], dd["g"], dd["x"], dd["pos"], dd["rbf"], dd["w_rad"], dd["w1"], dd["w2"])
    y, saved = K.so2conv_fwd(*args, saved=True if keep_state else None, chunk_edges=1024)
    bw = K.so2conv_bwd(*args, saved, dd["gy"], chunk_edges=1024)
    db = K.so2conv_dbwd(*args, saved, dd["gy"], px=dd["px"], ppos=dd["ppos"], prbf=dd["prbf"], chunk_edges=1024)
    torch.cuda.synchronize()
    inp = H.oracle_inputs(d)
    t = lambda a: torch.tensor(a, dtype=DT)  # noqa: E731
    gy = t(d["gy"])
    ry = O.forward(inp)
    rb = O.backward(inp, gy, with_edge_grad=True)
    rd = O.double_backward(inp, gy, px=t(d["px"]), ppos=t(d["ppos"]), prbf=t(d["prbf"]))
    errs = {"y": H.relerr(y, ry)}
    errs.update({k: H.relerr(bw[k], rb[k]) for k in ("gx", "gpos", "grbf", "gw_rad", "gw1", "gw2", "gedge")})
    pairs = {"ggy": "ggy", "gx2": "gx", "grbf2": "grbf", "gw_rad2": "gw_rad", "gw1_2": "gw1", "gw2_2": "gw2"}
    errs.update({k: H.relerr(db[k], rd[v]) for k, v in pairs.items()})
    H.note("  " + " ".join(f"{k}={v:.1e}" for k, v in errs.items()))
    assert all(v <= H.TOL_F32 for v in errs.values()), errs


def test_workspace_too_small_is_an_error():
    import so_graph_convolution_amd as K
    d = H.workload("T", seed=2)
    dd = H.to_dev(d)
    args = (dd["kcfg"], dd["g"], dd["x"], dd["pos"], dd["rbf"], dd["w_rad"], dd["w1"], dd["w2"])
    tiny = torch.empty(1024, dtype=torch.uint8, device="cuda")
    with pytest.raises(K.So2Error) as ei:
        K.so2conv_fwd(*args, saved=None, ws=tiny)
    assert ei.value.code == -3
