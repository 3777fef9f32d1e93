"""Mixture of linear experts (so2mole_*: system s uses sum_k coef[s,k] W^(k) in
both SO(2) linears) through the C ABI against the mixture oracle: forward,
backward (incl. expert and coefficient gradients) and double backward with
directions on x, positions, rbf, coefficients and experts, also reusing the
backward's kept cotangents (saved_bwd); float32 and bf16,
one chunk and 1024-edge chunks whose borders cut systems, an empty system in
every case. A single system with a one-hot coefficient is bitwise the plain
operator with that expert."""
import numpy as np
import pytest
import torch

import so2_synth
from oracle import mole_oracle as MO
from tests import _cases as H

pytestmark = pytest.mark.gpu
DT = torch.float64
BIG = dict(n_atoms=150, box=12.0, rc=4.0, lmax=4, mmax=2, channels=48, n_rbf=16, seed=5, min_dist=0.0)
CASES = [
    # name, workload overrides, dtype, chunk_edges, systems, experts, envelope
    ("l2m2_c16_S3_K4", dict(), "f32", None, 3, 4, False),
    ("l4m2_c48_S5_K8", BIG, "f32", None, 5, 8, True),
    ("l4m2_c48_S5_K8_chunked", BIG, "f32", 1024, 5, 8, False),
    ("l3m2_c32_bf16_S3_K4", dict(n_atoms=40, box=8.0, rc=4.0, lmax=3, mmax=2, channels=32, n_rbf=8, seed=14),
     "bf16", None, 3, 4, False),
]


def _dev_mix(m, dtype):
    ft = torch.bfloat16 if dtype == "bf16" else torch.float32

    def t(a, dt=torch.float32):
        return torch.tensor(np.ascontiguousarray(a), dtype=dt, device="cuda")
    return dict(w1e=[t(w, ft) for w in m["w1e"]], w2e=[t(w, ft) for w in m["w2e"]], coef=t(m["coef"]),
                pcoef=t(m["pcoef"]), pw1e=[t(w, ft) for w in m["pw1e"]], pw2e=[t(w, ft) for w in m["pw2e"]])


def _t(a):
    return torch.tensor(np.asarray(a, dtype=np.float64), dtype=DT)


@pytest.mark.parametrize("name,over,dtype,chunk,S,K,use_env", CASES, ids=[c[0] for c in CASES])
def test_mixture_matches_oracle(name, over, dtype, chunk, S, K, use_env):
    import so_graph_convolution_amd as Kx
    d = dict(H.workload("T", dtype=dtype, **over))
    if use_env:
        d["env"] = so2_synth.cosine_envelope(d)
    m = so2_synth.mixture_inputs(d, S, K, seed=1, empty_system=True, bf16=dtype == "bf16")
    H.note(f"[mixture] {name} E={len(d['src'])} systems={m['sys_edge_ptr'].tolist()} dtype={dtype} chunks={chunk}")
    dd = H.to_dev(d, dtype)
    mx = _dev_mix(m, dtype)
    mix = Kx.Mixture(K, m["sys_edge_ptr"])
    env = torch.tensor(d["env"], device="cuda") if use_env else None
    args = (dd["kcfg"], dd["g"], mix, dd["x"], dd["pos"], dd["rbf"], dd["w_rad"], mx["w1e"], mx["w2e"], mx["coef"])
    keep = chunk is None
    y, saved = Kx.so2mole_fwd(*args, saved=True if keep else None, chunk_edges=chunk, env=env)
    bw = Kx.so2mole_bwd(*args, saved, dd["gy"], chunk_edges=chunk, env=env)
    dirs = dict(px=dd["px"], ppos=dd["ppos"], prbf=dd["prbf"], pcoef=mx["pcoef"], pw1e=mx["pw1e"], pw2e=mx["pw2e"],
                chunk_edges=chunk, env=env, need=("gy", "x", "pos", "rbf", "w_rad", "w1", "w2", "coef"))
    db = Kx.so2mole_dbwd(*args, saved, dd["gy"], **dirs)
    # the double backward again, reusing the backward's kept cotangents
    bw_k = Kx.so2mole_bwd(*args, saved, dd["gy"], chunk_edges=chunk, env=env, saved_bwd=True)
    db_k = Kx.so2mole_dbwd(*args, saved, dd["gy"], saved_bwd=bw_k["saved_bwd"], **dirs)
    torch.cuda.synchronize()
    for k in ("gx", "gpos", "grbf", "gw_rad", "gcoef", "gedge"):
        assert torch.equal(bw_k[k], bw[k]), k
    base = H.oracle_inputs(d)
    w1e, w2e = [_t(w) for w in m["w1e"]], [_t(w) for w in m["w2e"]]
    coef, sp, gy = _t(m["coef"]), m["sys_edge_ptr"].tolist(), _t(d["gy"])
    ry = MO.forward(base, w1e, w2e, coef, sp)
    rb = MO.backward(base, w1e, w2e, coef, sp, gy, with_edge_grad=True)
    rd = MO.double_backward(base, w1e, w2e, coef, sp, gy, px=_t(d["px"]), ppos=_t(d["ppos"]), prbf=_t(d["prbf"]),
                            pcoef=_t(m["pcoef"]), pw1e=[_t(w) for w in m["pw1e"]], pw2e=[_t(w) for w in m["pw2e"]])
    errs = {"y": H.relerr(y, ry)}
    for k in ("gx", "gpos", "grbf", "gw_rad", "gw1e", "gw2e", "gcoef", "gedge"):
        errs[k] = H.relerr(bw[k], rb[k])
    if use_env:
        errs["genv"] = H.relerr(bw["genv"], rb["genv"])
    for k, v in (("ggy", "ggy"), ("gx2", "gx"), ("gpos2", "gpos"), ("grbf2", "grbf"), ("gw_rad2", "gw_rad"),
                 ("gw1e_2", "gw1e"), ("gw2e_2", "gw2e"), ("gcoef2", "gcoef")):
        errs[k] = H.relerr(db[k], rd[v])
        errs[k + " kept"] = H.relerr(db_k[k], rd[v])
    H.note("  " + " ".join(f"{k}={v:.1e}" for k, v in errs.items()))
    tol = H.TOL_BF16 if dtype == "bf16" else H.TOL_F32
    assert all(v <= tol for v in errs.values()), errs
    # the empty system's coefficients get no gradient
    assert float(bw["gcoef"][1].abs().max()) == 0.0


def test_one_hot_single_system_is_the_plain_operator():
    """S = 1 with coef = e_2: every output bitwise equal to so2conv_* with
    expert 2's weights (the merge multiplies by 1 and adds zeros)."""
    import so_graph_convolution_amd as Kx
    d = H.workload("T", **BIG)
    K = 4
    m = so2_synth.mixture_inputs(d, 1, K, seed=2)
    dd = H.to_dev(d)
    mx = _dev_mix(m, "f32")
    coef = torch.zeros(1, K, device="cuda")
    coef[0, 2] = 1.0
    mix = Kx.Mixture(K, m["sys_edge_ptr"])
    H.note(f"[mixture] one-hot single system E={len(d['src'])}")
    margs = (dd["kcfg"], dd["g"], mix, dd["x"], dd["pos"], dd["rbf"], dd["w_rad"], mx["w1e"], mx["w2e"], coef)
    w1 = [w[2].contiguous() for w in mx["w1e"]]
    w2 = [w[2].contiguous() for w in mx["w2e"]]
    pargs = (dd["kcfg"], dd["g"], dd["x"], dd["pos"], dd["rbf"], dd["w_rad"], w1, w2)
    y0, s0 = Kx.so2conv_fwd(*pargs, saved=True)
    y1, s1 = Kx.so2mole_fwd(*margs, saved=True)
    b0 = Kx.so2conv_bwd(*pargs, s0, dd["gy"])
    b1 = Kx.so2mole_bwd(*margs, s1, dd["gy"])
    d0 = Kx.so2conv_dbwd(*pargs, s0, dd["gy"], px=dd["px"], ppos=dd["ppos"], prbf=dd["prbf"])
    d1 = Kx.so2mole_dbwd(*margs, s1, dd["gy"], px=dd["px"], ppos=dd["ppos"], prbf=dd["prbf"])
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)
    for k in ("gx", "gpos", "grbf", "gw_rad", "gedge"):
        assert torch.equal(b0[k], b1[k]), k
    for a, b in zip(b0["gw1"], b1["gw1e"]):
        assert torch.equal(a, b[2])
        assert float(b[[0, 1, 3]].abs().max()) == 0.0
    for a, b in zip(b0["gw2"], b1["gw2e"]):
        assert torch.equal(a, b[2])
    for k in ("ggy", "gx2", "grbf2", "gw_rad2"):
        assert torch.equal(d0[k], d1[k]), k
    for a, b in zip(d0["gw1_2"], d1["gw1e_2"]):
        assert torch.equal(a, b[2])


def test_mixture_without_edges():
    import so_graph_convolution_amd as Kx
    d = dict(H.workload("T", seed=3))
    for k in ("src", "dst"):
        d[k] = d[k][:0]
    for k in ("shift", "rbf", "prbf"):
        d[k] = d[k][:0]
    m = so2_synth.mixture_inputs(d, 2, 4, seed=3)
    dd = H.to_dev(d)
    mx = _dev_mix(m, "f32")
    mix = Kx.Mixture(4, m["sys_edge_ptr"])
    H.note("[mixture] no edges")
    args = (dd["kcfg"], dd["g"], mix, dd["x"], dd["pos"], dd["rbf"], dd["w_rad"], mx["w1e"], mx["w2e"], mx["coef"])
    y, saved = Kx.so2mole_fwd(*args, saved=True)
    bw = Kx.so2mole_bwd(*args, saved, dd["gy"])
    db = Kx.so2mole_dbwd(*args, saved, dd["gy"], px=dd["px"], pcoef=mx["pcoef"])
    torch.cuda.synchronize()
    assert float(y.abs().max()) == 0.0
    for v in (bw["gx"], bw["gcoef"], db["ggy"], db["gx2"], db["gcoef2"]):
        assert float(v.abs().max()) == 0.0
    assert max(float(w.abs().max()) for w in bw["gw1e"] + db["gw2e_2"]) == 0.0
