"""bfloat16 features and weights with float32 accumulation (the pages' bf16
configurations): forward, backward and double backward through the C ABI
against the float64 oracle on the same bf16-representable inputs. Bar: 2e-2
max-norm relative error per output; the stored GEMM operand of the rotation
on gather is checked to one bf16 rounding."""
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
                             min_dist=0.0)),
    ("l6m2_c16", dict(n_atoms=48, box=9.0, rc=4.5, lmax=6, mmax=2, channels=16, n_rbf=8, seed=11)),
    ("l2m2_c128", dict(n_atoms=40, box=8.0, rc=4.0, lmax=2, mmax=2, channels=128, n_rbf=8, seed=12)),
    ("l4m2_c256", dict(n_atoms=24, box=8.0, rc=4.0, lmax=4, mmax=2, channels=256, n_rbf=8, seed=13)),
    ("l1m1_c32", dict(n_atoms=32, box=8.0, rc=4.0, lmax=1, mmax=1, channels=32, n_rbf=8, seed=14)),
]


def _workload(over):
    return H.workload("T", dtype="bf16", **over)


def _args(dd):
    return (dd["kcfg"], dd["g"], dd["x"], dd["pos"], dd["rbf"], dd["w_rad"], dd["w1"], dd["w2"])


def _oracle_all(d):
    inp = H.oracle_inputs(d)
    t = lambda a: torch.tensor(a, dtype=DT)  # noqa: E731
    gy = t(d["gy"])
    return (O.forward(inp), O.backward(inp, gy, with_edge_grad=True),
            O.double_backward(inp, gy, px=t(d["px"]), ppos=t(d["ppos"]), prbf=t(d["prbf"])))


DB_PAIRS = {"ggy": "ggy", "gx2": "gx", "grbf2": "grbf", "gw_rad2": "gw_rad", "gw1_2": "gw1", "gw2_2": "gw2"}
BW_KEYS = ("gx", "gpos", "grbf", "gw_rad", "gw1", "gw2", "gedge")


def _errors(y, bw, db, ref):
    ry, rb, rd = ref
    errs = {"y": H.relerr(y, ry)}
    errs.update({k: H.relerr(bw[k], rb[k]) for k in BW_KEYS})
    errs.update({k: H.relerr(db[k], rd[v]) for k, v in DB_PAIRS.items()})
    return errs


def _dtypes_ok(dd, y, bw, db):
    bf = torch.bfloat16
    assert y.dtype == bf and bw["gx"].dtype == bf and bw["gw_rad"].dtype == bf
    assert all(w.dtype == bf for w in bw["gw1"] + bw["gw2"] + db["gw1_2"] + db["gw2_2"])
    assert db["ggy"].dtype == bf and db["gx2"].dtype == bf
    assert bw["gpos"].dtype == torch.float32 and bw["grbf"].dtype == torch.float32


@pytest.mark.parametrize("name,over", CASES, ids=[c[0] for c in CASES])
def test_bf16_matches_oracle(name, over):
    import so_graph_convolution_amd as K
    d = _workload(over)
    cfg = d["cfg"]
    H.note(f"[bf16] {name} L={cfg.lmax} M={cfg.mmax} C={cfg.channels} E={len(d['src'])}")
    dd = H.to_dev(d, "bf16")
    args = _args(dd)
    y, saved = K.so2conv_fwd(*args, saved=True)
    bw = K.so2conv_bwd(*args, saved, dd["gy"])
    db = K.so2conv_dbwd(*args, saved, dd["gy"], px=dd["px"], ppos=dd["ppos"], prbf=dd["prbf"])
    torch.cuda.synchronize()
    _dtypes_ok(dd, y, bw, db)
    errs = _errors(y, bw, db, _oracle_all(d))
    H.note("  " + " ".join(f"{k}={v:.1e}" for k, v in errs.items()))
    assert all(v <= H.TOL_BF16 for v in errs.values()), errs


def test_bf16_rotate_gather_is_one_rounding():
    import so_graph_convolution_amd as K
    d = _workload(CASES[0][1])
    cfg = d["cfg"]
    dd = H.to_dev(d, "bf16")
    T = K.so2conv_debug_rotate_gather(dd["kcfg"], dd["g"], dd["x"], dd["pos"], dd["rbf"], dd["w_rad"])
    torch.cuda.synchronize()
    assert T.dtype == torch.bfloat16
    rows = O.rotated_inputs(H.oracle_inputs(d))
    ref = H.m_major(rows, cfg.lmax, cfg.mmax, 2 * cfg.channels)
    # one round-to-nearest of a float32 value (8-bit significand): |err| <= 2^-8 |ref| (+ float32 noise)
    g = T.double().cpu()
    bound = 2.0 ** -8 * ref.abs() + 1e-5 * float(ref.abs().max())
    assert bool(((g - ref).abs() <= bound).all()), float(((g - ref).abs() - bound).max())


@pytest.mark.parametrize("keep_state", [False, True], ids=["recompute", "saved"])
def test_bf16_chunked(keep_state):
    import so_graph_convolution_amd as K
    d = _workload(CASES[0][1])
    E = len(d["src"])
    assert E > 1024
    H.note(f"[bf16 chunked {'saved' if keep_state else 'recompute'}] E={E} chunks of 1024")
    dd = H.to_dev(d, "bf16")
    args = _args(dd)
    y, saved = K.so2conv_fwd(*args, saved=True if keep_state else None, chunk_edges=1024)
    bw = K.so2conv_bwd(*args, saved, dd["gy"], chunk_edges=1024)
    db = K.so2conv_dbwd(*args, saved, dd["gy"], px=dd["px"], ppos=dd["ppos"], prbf=dd["prbf"], chunk_edges=1024)
    torch.cuda.synchronize()
    errs = _errors(y, bw, db, _oracle_all(d))
    H.note("  " + " ".join(f"{k}={v:.1e}" for k, v in errs.items()))
    assert all(v <= H.TOL_BF16 for v in errs.values()), errs


def test_bf16_all_directions():
    import so_graph_convolution_amd as K
    d = _workload(CASES[4][1])
    dd = H.to_dev(d, "bf16")
    args = _args(dd)
    g = np.random.default_rng(3)
    rb = so2_synth.round_bf16
    pw_rad = rb(g.normal(size=d["w_rad"].shape).astype(np.float32))
    pw1 = [rb((g.normal(size=w.shape) * 0.1).astype(np.float32)) for w in d["w1"]]
    pw2 = [rb((g.normal(size=w.shape) * 0.1).astype(np.float32)) for w in d["w2"]]
    pedge = g.normal(size=(len(d["src"]), 3)).astype(np.float32)
    bf = lambda a: torch.tensor(a, dtype=torch.bfloat16, device="cuda")  # noqa: E731
    y, saved = K.so2conv_fwd(*args, saved=True)
    out = K.so2conv_dbwd(*args, saved, dd["gy"], px=dd["px"], ppos=dd["ppos"],
                         pedge=torch.tensor(pedge, device="cuda"), prbf=dd["prbf"], pw_rad=bf(pw_rad),
                         pw1=[bf(w) for w in pw1], pw2=[bf(w) for w in pw2])
    torch.cuda.synchronize()
    t = lambda a: torch.tensor(a, dtype=DT)  # noqa: E731
    ref = O.double_backward(H.oracle_inputs(d), t(d["gy"]), px=t(d["px"]), ppos=t(d["ppos"]), prbf=t(d["prbf"]),
                            pw_rad=t(pw_rad), pw1=[t(w) for w in pw1], pw2=[t(w) for w in pw2], pedge=t(pedge))
    errs = {k: H.relerr(out[k], ref[v]) for k, v in DB_PAIRS.items()}
    H.note("  " + " ".join(f"{k}={v:.1e}" for k, v in errs.items()))
    assert all(v <= H.TOL_BF16 for v in errs.values()), errs


def test_bf16_deterministic_and_empty_graph():
    import so_graph_convolution_amd as K
    d = _workload(CASES[1][1])
    dd = H.to_dev(d, "bf16")
    args = _args(dd)
    y1, s1 = K.so2conv_fwd(*args, saved=True)
    b1 = K.so2conv_bwd(*args, s1, dd["gy"])
    y2, s2 = K.so2conv_fwd(*args, saved=True)
    b2 = K.so2conv_bwd(*args, s2, dd["gy"])
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    assert all(torch.equal(a, b) for a, b in zip(b1["gw1"] + [b1["gx"], b1["gpos"]], b2["gw1"] + [b2["gx"], b2["gpos"]]))
    # no edges: zero outputs in the call's dtype
    kc = dd["kcfg"]
    e = torch.zeros(0, dtype=torch.int32, device="cuda")
    g0 = K.so2conv_graph_prepare(d["cfg"].n_atoms, e, e, torch.zeros(0, 3, device="cuda"))
    rbf0 = torch.zeros(0, kc.n_rbf, device="cuda")
    y0, sv0 = K.so2conv_fwd(kc, g0, dd["x"], dd["pos"], rbf0, dd["w_rad"], dd["w1"], dd["w2"], saved=True)
    bw0 = K.so2conv_bwd(kc, g0, dd["x"], dd["pos"], rbf0, dd["w_rad"], dd["w1"], dd["w2"], sv0, dd["gy"])
    torch.cuda.synchronize()
    assert y0.dtype == torch.bfloat16 and not bool(y0.any())
    assert not bool(bw0["gx"].any()) and not any(bool(w.any()) for w in bw0["gw1"])
