"""GPU parity of graph preparation, rotation on gather and the forward pass
against numpy (integer arrays, bit-exact) and the float64 CPU oracle."""
import numpy as np
import pytest
import torch

from oracle import so2conv_oracle as O
from tests import _cases as H

pytestmark = pytest.mark.gpu

FWD_CASES = [
    # (name, base config, overrides)
    ("tiny_T", "T", {}),
    ("l4m2_c48_ragged", "T", dict(n_atoms=150, box=12.0, rc=4.0, lmax=4, mmax=2, channels=48, n_rbf=16, seed=5,
                                  min_dist=0.0)),
    ("l3m1_c32", "T", dict(n_atoms=80, box=10.0, rc=4.0, lmax=3, mmax=1, channels=32, n_rbf=8, seed=6, min_dist=0.0)),
    ("l6m2_c16", "T", dict(n_atoms=60, box=9.0, rc=3.5, lmax=6, mmax=2, channels=16, n_rbf=8, seed=7, min_dist=0.0)),
    ("l0m0_c16", "T", dict(lmax=0, mmax=0, seed=8)),
    ("l4m4_c16", "T", dict(n_atoms=40, box=8.0, rc=3.5, lmax=4, mmax=4, channels=16, n_rbf=8, seed=9, min_dist=0.0)),
    ("l2m2_c128", "T", dict(n_atoms=120, box=12.0, rc=4.5, lmax=2, mmax=2, channels=128, n_rbf=64, seed=10,
                            min_dist=0.0)),
]


@pytest.mark.parametrize("name,base,over", FWD_CASES, ids=[c[0] for c in FWD_CASES])
def test_graph_prepare_bit_exact(name, base, over):
    d = H.workload(base, **over)
    H.note(f"[graph_prepare] {name} N={d['cfg'].n_atoms} E={len(d['src'])}")
    dd = H.to_dev(d)
    g = dd["g"]
    N = d["cfg"].n_atoms
    src, dst = d["src"].astype(np.int64), d["dst"].astype(np.int64)
    ref_dst_ptr = np.searchsorted(dst, np.arange(N + 1), side="left")
    ref_perm = np.argsort(src, kind="stable")
    ref_src_ptr = np.searchsorted(src[ref_perm], np.arange(N + 1), side="left")
    assert np.array_equal(g.dst_ptr.cpu().numpy(), ref_dst_ptr)
    assert np.array_equal(g.src_perm.cpu().numpy()[:len(src)], ref_perm)
    assert np.array_equal(g.src_ptr.cpu().numpy(), ref_src_ptr)


def test_graph_prepare_rejects_unsorted():
    import so_graph_convolution_amd as K
    src = torch.tensor([0, 1, 2], dtype=torch.int32, device="cuda")
    dst = torch.tensor([2, 0, 1], dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError):
        K.so2conv_graph_prepare(3, src, dst)


@pytest.mark.parametrize("name,base,over", FWD_CASES, ids=[c[0] for c in FWD_CASES])
def test_rotate_gather_matches_oracle(name, base, over):
    import so_graph_convolution_amd as K
    d = H.workload(base, **over)
    cfg = d["cfg"]
    H.note(f"[rotate_gather] {name} L={cfg.lmax} M={cfg.mmax} C={cfg.channels} E={len(d['src'])}")
    dd = H.to_dev(d)
    T = K.so2conv_debug_rotate_gather(dd["kcfg"], dd["g"], dd["x"], dd["pos"], dd["rbf"], dd["w_rad"])
    torch.cuda.synchronize()
    inp = H.oracle_inputs(d)
    ref = H.m_major(O.rotated_inputs(inp), cfg.lmax, cfg.mmax, 2 * cfg.channels)
    err = H.relerr(T, ref)
    H.note(f"  rel err {err:.3e}")
    assert err <= H.TOL_F32


@pytest.mark.parametrize("name,base,over", FWD_CASES, ids=[c[0] for c in FWD_CASES])
def test_forward_matches_oracle(name, base, over):
    import so_graph_convolution_amd as K
    d = H.workload(base, **over)
    cfg = d["cfg"]
    H.note(f"[forward] {name} L={cfg.lmax} M={cfg.mmax} C={cfg.channels} E={len(d['src'])}")
    dd = H.to_dev(d)
    y, _ = K.so2conv_fwd(dd["kcfg"], dd["g"], dd["x"], dd["pos"], dd["rbf"], dd["w_rad"], dd["w1"], dd["w2"])
    torch.cuda.synchronize()
    ref = O.forward(H.oracle_inputs(d))
    err = H.relerr(y, ref)
    H.note(f"  rel err {err:.3e}")
    assert err <= H.TOL_F32


def test_forward_deterministic():
    import so_graph_convolution_amd as K
    d = H.workload("T", n_atoms=150, box=12.0, rc=4.0, lmax=4, mmax=2, channels=48, n_rbf=16, seed=5, min_dist=0.0)
    dd = H.to_dev(d)
    args = (dd["kcfg"], dd["g"], dd["x"], dd["pos"], dd["rbf"], dd["w_rad"], dd["w1"], dd["w2"])
    y1, _ = K.so2conv_fwd(*args)
    y2, _ = K.so2conv_fwd(*args)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


def test_forward_isolated_nodes_and_no_edges():
    import so_graph_convolution_amd as K
    d = H.workload("T", seed=3)
    dd = H.to_dev(d)
    # a graph with no edges: the output is exactly zero
    e = torch.zeros(0, dtype=torch.int32, device="cuda")
    g0 = K.so2conv_graph_prepare(d["cfg"].n_atoms, e, e, torch.zeros(0, 3, device="cuda"))
    y, _ = K.so2conv_fwd(dd["kcfg"], g0, dd["x"], dd["pos"], dd["rbf"][:0].contiguous(), dd["w_rad"], dd["w1"],
                         dd["w2"])
    torch.cuda.synchronize()
    assert float(y.abs().max()) == 0.0
