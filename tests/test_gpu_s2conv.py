"""GPU parity of the convolution with the spherical-grid SwiGLU activation
(EquiformerV3's Edge -> Edge activation: TrimSO(2) page, Appendix C.1
"Implementation" and Table 2; per-head attention weights before the receiver
sum) through the C ABI against the float64 oracle: forward, backward and
double backward with weight directions, float32 (both product paths) and
bfloat16, one chunk and 1024-edge chunks, one and two 16-row tiles of the
grid kernels (q = 9, 13 and q = 19, 25, 29), the backward's kept cotangents, an
empty edge set and the argument checks."""
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
    # name, workload overrides, dtype, chunk_edges, heads, weight directions
    ("l2m2_c16_tiny", dict(n_grid=9), "f32", None, 1, True),
    ("l4m2_c32_native", dict(n_atoms=60, box=9.0, rc=4.0, lmax=4, mmax=2, channels=32, n_rbf=8, seed=5, n_grid=70),
     "f32_native", None, 1, True),
    ("l4m2_c48_chunked", dict(n_atoms=150, box=12.0, rc=4.0, lmax=4, mmax=2, channels=48, n_rbf=16, seed=5,
                              min_dist=0.0, n_grid=70), "f32", 1024, 1, False),
    ("l4m1_c32_rows13", dict(n_atoms=40, box=8.0, rc=4.0, lmax=4, mmax=1, channels=32, n_rbf=8, seed=14, n_grid=40),
     "f32", None, 1, True),
    ("l4m4_c16_rows25", dict(n_atoms=30, box=7.0, rc=4.0, lmax=4, mmax=4, channels=16, n_rbf=8, seed=15, n_grid=81),
     "f32", None, 1, False),
    ("l6m2_c32_bf16", dict(n_atoms=48, box=9.0, rc=4.5, lmax=6, mmax=2, channels=32, n_rbf=8, seed=11, n_grid=98),
     "bf16", None, 1, True),
    ("l4m2_c128_h8_bf16", dict(n_atoms=80, box=10.0, rc=4.0, lmax=4, mmax=2, channels=128, n_rbf=16, seed=6,
                               min_dist=0.0, n_grid=70), "bf16", None, 8, False),
    ("l6m2_c128_h8", dict(n_atoms=48, box=9.0, rc=4.5, lmax=6, mmax=2, channels=128, n_rbf=8, seed=12, n_grid=98),
     "f32", None, 8, False),
]
BW = {"gx": "gx", "gpos": "gpos", "grbf": "grbf", "gw_rad": "gw_rad", "gw1": "gw1", "gw2": "gw2", "gedge": "gedge"}
DB = {"ggy": "ggy", "gx2": "gx", "gpos2": "gpos", "grbf2": "grbf", "gw_rad2": "gw_rad", "gw1_2": "gw1",
      "gw2_2": "gw2"}


def _case(over, dtype, heads):
    d = dict(H.workload("T", dtype="bf16" if dtype == "bf16" else "f32", act="swiglu_s2", **over))
    if heads > 1:
        d["env"] = so2_synth.attention_weights(d, heads, seed=3)
    return d


def _weight_dirs(d, bf16):
    rng = np.random.default_rng(77)
    r = (lambda a: so2_synth.round_bf16(a)) if bf16 else (lambda a: a)
    pw1 = [r(rng.normal(size=w.shape).astype(np.float32) * 0.1) for w in d["w1"]]
    pw2 = [r(rng.normal(size=w.shape).astype(np.float32) * 0.1) for w in d["w2"]]
    pwr = r(rng.normal(size=d["w_rad"].shape).astype(np.float32) * 0.1)
    return pwr, pw1, pw2


@pytest.mark.parametrize("name,over,dtype,chunk,heads,wdirs", CASES, ids=[c[0] for c in CASES])
def test_s2conv_matches_oracle(name, over, dtype, chunk, heads, wdirs):
    import so_graph_convolution_amd as K
    d = _case(over, dtype, heads)
    E = len(d["src"])
    H.note(f"[s2conv] {name} E={E} dtype={dtype} chunks={chunk} heads={heads} n_grid={d['cfg'].n_grid}")
    dd = H.to_dev(d, "bf16" if dtype == "bf16" else "f32")
    dd["kcfg"] = dataclasses.replace(dd["kcfg"], heads=heads, f32_native=dtype == "f32_native")
    ft = dd["x"].dtype
    env = torch.tensor(d["env"], device="cuda") if heads > 1 else None
    pwr, pw1, pw2 = _weight_dirs(d, dtype == "bf16") if wdirs else (None, None, None)
    dev = lambda a: torch.tensor(a, dtype=ft, device="cuda")  # noqa: E731
    args = (dd["kcfg"], dd["g"], dd["x"], dd["pos"], dd["rbf"], dd["w_rad"], dd["w1"], dd["w2"])
    keep = chunk is None
    y, saved = K.so2conv_fwd(*args, saved=True if keep else None, chunk_edges=chunk, env=env)
    bw = K.so2conv_bwd(*args, saved, dd["gy"], chunk_edges=chunk, env=env)
    db = K.so2conv_dbwd(*args, saved, dd["gy"], px=dd["px"], ppos=dd["ppos"], prbf=dd["prbf"],
                        pw_rad=None if pwr is None else dev(pwr), pw1=None if pw1 is None else [dev(w) for w in pw1],
                        pw2=None if pw2 is None else [dev(w) for w in pw2], env=env, chunk_edges=chunk,
                        need=("gy", "x", "pos", "rbf", "w_rad", "w1", "w2"))
    torch.cuda.synchronize()
    inp = H.oracle_inputs(d)
    t = lambda a: torch.tensor(a, dtype=DT)  # noqa: E731
    gy = t(d["gy"])
    ry = O.forward(inp)
    rb = O.backward(inp, gy, with_edge_grad=True)
    rd = O.double_backward(inp, gy, px=t(d["px"]), ppos=t(d["ppos"]), prbf=t(d["prbf"]),
                           pw_rad=None if pwr is None else t(pwr), pw1=None if pw1 is None else [t(w) for w in pw1],
                           pw2=None if pw2 is None else [t(w) for w in pw2])
    errs = {"y": H.errs_both(y, ry, dtype)}
    errs.update({k: H.errs_both(bw[k], rb[v], dtype) for k, v in BW.items()})
    errs.update({k: H.errs_both(db[k], rd[v], dtype) for k, v in DB.items()})
    H.note("  " + " ".join(f"{k}={v[0]:.1e}/{v[1]:.1e}" for k, v in errs.items()))
    tol, tol_e = (H.TOL_BF16, H.TOL_ELEM_BF16) if dtype == "bf16" else (H.TOL_F32, H.TOL_ELEM_F32)
    bad = {k: v for k, v in errs.items() if v[0] > tol or v[1] > tol_e}
    assert not bad, bad


def test_s2conv_kept_cotangents_and_no_edges():
    """The double backward reusing the backward's kept cotangents equals the one
    that forms them itself; a graph without edges gives zero outputs."""
    import so_graph_convolution_amd as K
    d = _case(dict(n_atoms=40, box=8.0, rc=4.0, lmax=4, mmax=2, channels=32, n_rbf=8, seed=9, n_grid=50), "f32", 1)
    dd = H.to_dev(d)
    args = (dd["kcfg"], dd["g"], dd["x"], dd["pos"], dd["rbf"], dd["w_rad"], dd["w1"], dd["w2"])
    y, saved = K.so2conv_fwd(*args, saved=True)
    bw = K.so2conv_bwd(*args, saved, dd["gy"], saved_bwd=True)
    need = ("gy", "x", "rbf", "w_rad", "w1", "w2")
    a = K.so2conv_dbwd(*args, saved, dd["gy"], px=dd["px"], need=need, saved_bwd=bw["saved_bwd"])
    b = K.so2conv_dbwd(*args, saved, dd["gy"], px=dd["px"], need=need)
    torch.cuda.synchronize()
    for k in ("ggy", "gx2", "grbf2", "gw_rad2", "gw1_2", "gw2_2"):
        assert H.relerr(a[k], b[k]) <= 1e-5, k
    # no edges
    e = torch.zeros(0, dtype=torch.int32, device="cuda")
    g0 = K.so2conv_graph_prepare(d["cfg"].n_atoms, e, e, torch.zeros(0, 3, device="cuda"))
    args0 = (dd["kcfg"], g0, dd["x"], dd["pos"], torch.zeros(0, d["cfg"].n_rbf, device="cuda"), dd["w_rad"],
             dd["w1"], dd["w2"])
    y0, s0 = K.so2conv_fwd(*args0, saved=True)
    b0 = K.so2conv_bwd(*args0, s0, dd["gy"], need=("x", "pos", "w_rad", "w1", "w2"))
    torch.cuda.synchronize()
    assert float(y0.abs().max()) == 0.0
    assert float(b0["gx"].abs().max()) == 0.0
    assert all(float(w.abs().max()) == 0.0 for w in b0["gw1"])


def test_s2conv_argument_checks():
    import so_graph_convolution_amd as K
    d = _case(dict(n_grid=9), "f32", 1)
    dd = H.to_dev(d)
    args = (dd["g"], dd["x"], dd["pos"], dd["rbf"], dd["w_rad"], dd["w1"], dd["w2"])
    G, P = dd["kcfg"].grid
    bad = K.SO2Config(2, 2, 16, d["cfg"].n_rbf, "f32", act="swiglu_s2", grid=(G, P))
    c = bad.c()
    c.grid_basis = None                                    # NULL table -> SO2_EINVAL before any work
    ws = torch.empty(K.so2conv_workspace_bytes(bad, dd["g"].n_nodes, dd["g"].n_edges, 0), dtype=torch.uint8,
                     device="cuda")
    y = torch.empty_like(dd["x"])
    import ctypes
    from so_graph_convolution_amd._binding import lib
    s1, s2 = K.weight_shapes(bad)
    arr1 = (ctypes.c_void_p * len(dd["w1"]))(*[w.data_ptr() for w in dd["w1"]])
    arr2 = (ctypes.c_void_p * len(dd["w2"]))(*[w.data_ptr() for w in dd["w2"]])
    gc = dd["g"].c()
    r = lib().so2conv_fwd(ctypes.byref(c), ctypes.byref(gc), ctypes.c_void_p(dd["x"].data_ptr()),
                          ctypes.c_void_p(dd["pos"].data_ptr()), ctypes.c_void_p(dd["rbf"].data_ptr()), None,
                          ctypes.c_void_p(dd["w_rad"].data_ptr()), ctypes.cast(arr1, ctypes.c_void_p),
                          ctypes.cast(arr2, ctypes.c_void_p), ctypes.c_void_p(y.data_ptr()), None,
                          ctypes.c_void_p(ws.data_ptr()), ws.numel(), None)
    assert r == -1 and "grid" in lib().so2conv_last_error().decode()
    # the mixture takes the gate only
    mix = K.Mixture(4, [0, len(d["src"])])
    e1, e2 = K.expert_shapes(dd["kcfg"], 4)
    with pytest.raises(K.So2Error):
        K.so2mole_fwd(dd["kcfg"], dd["g"], mix, dd["x"], dd["pos"], dd["rbf"], dd["w_rad"],
                      [torch.zeros(s, device="cuda") for s in e1], [torch.zeros(s, device="cuda") for s in e2],
                      torch.full((1, 4), 0.25, device="cuda"))
    del args
