"""The forward gate in the first linear's epilogue (SO2_FUSED_GATE) gives
bitwise the results of the separate gate pass: every output of fwd, bwd and
dbwd, float32 through bfloat16 pieces and bfloat16, one chunk (saved state)
and 1024-edge recompute chunks, and the mixture of experts (one launch holds
several systems' products)."""
import dataclasses

import pytest
import torch

import so2_synth
from tests import _cases as H

pytestmark = pytest.mark.gpu

CASES = [
    ("l4m2_c48_f32", dict(n_atoms=60, box=9.0, rc=4.0, lmax=4, mmax=2, channels=48, n_rbf=8, seed=31), "f32", None),
    ("l6m2_c32_bf16", dict(n_atoms=48, box=9.0, rc=4.5, lmax=6, mmax=2, channels=32, n_rbf=8, seed=32), "bf16", None),
    ("l2m2_c128_f32_chunked", dict(n_atoms=60, box=9.0, rc=4.0, lmax=2, mmax=2, channels=128, n_rbf=8, seed=33),
     "f32", 1024),
    ("l0m0_c16_f32", dict(n_atoms=40, box=8.0, rc=4.0, lmax=0, mmax=0, channels=16, n_rbf=8, seed=34), "f32", None),
]


def _flat(out):
    for k in sorted(out):
        v = out[k]
        if v is None or k == "saved_bwd":
            continue
        for i, t in enumerate(v if isinstance(v, list) else [v]):
            yield f"{k}[{i}]", t


def _run(K, kc, dd, chunk):
    args = (kc, dd["g"], dd["x"], dd["pos"], dd["rbf"], dd["w_rad"], dd["w1"], dd["w2"])
    y, saved = K.so2conv_fwd(*args, saved=True if chunk is None else None, chunk_edges=chunk)
    bw = K.so2conv_bwd(*args, saved, dd["gy"], chunk_edges=chunk)
    db = K.so2conv_dbwd(*args, saved, dd["gy"], px=dd["px"], ppos=dd["ppos"], prbf=dd["prbf"], chunk_edges=chunk,
                        need=("gy", "x", "pos", "rbf", "w_rad", "w1", "w2"))
    torch.cuda.synchronize()
    return dict(y=y, **{f"b_{k}": v for k, v in bw.items()}, **{f"d_{k}": v for k, v in db.items()})


@pytest.mark.parametrize("name,over,dtype,chunk", CASES, ids=[c[0] for c in CASES])
def test_fused_gate_is_bitwise_the_gate_pass(name, over, dtype, chunk):
    import so_graph_convolution_amd as K
    d = H.workload("T", dtype=dtype, **over)
    H.note(f"[fused gate] {name} E={len(d['src'])} dtype={dtype} chunks={chunk}")
    dd = H.to_dev(d, dtype)
    a = _run(K, dd["kcfg"], dd, chunk)
    b = _run(K, dataclasses.replace(dd["kcfg"], fused_gate=True), dd, chunk)
    diff = [k for (k, x), (_, y) in zip(_flat(a), _flat(b)) if not torch.equal(x, y)]
    assert not diff, diff


def test_fused_gate_mixture_is_bitwise():
    import so_graph_convolution_amd as K
    d = H.workload("T", n_atoms=50, box=9.0, rc=4.0, lmax=3, mmax=2, channels=32, n_rbf=8, seed=35)
    m = so2_synth.mixture_inputs(d, 3, 4, seed=1)
    dd = H.to_dev(d)
    mix = K.Mixture(4, m["sys_edge_ptr"])
    w1e = [torch.tensor(w, device="cuda") for w in m["w1e"]]
    w2e = [torch.tensor(w, device="cuda") for w in m["w2e"]]
    coef = torch.tensor(m["coef"], device="cuda")
    res = []
    for kc in (dd["kcfg"], dataclasses.replace(dd["kcfg"], fused_gate=True)):
        args = (kc, dd["g"], mix, dd["x"], dd["pos"], dd["rbf"], dd["w_rad"], w1e, w2e, coef)
        y, saved = K.so2mole_fwd(*args, saved=True)
        bw = K.so2mole_bwd(*args, saved, dd["gy"])
        torch.cuda.synchronize()
        res.append(dict(y=y, **bw))
    diff = [k for (k, x), (_, y) in zip(_flat(res[0]), _flat(res[1])) if not torch.equal(x, y)]
    assert not diff, diff
