"""The per-order products (and the projection's) run on direct-to-LDS kernels
when every operand is 16-byte aligned, and on register-staged kernels when one
is not (here: a user tensor that starts 4 bytes into its allocation, which the
float32 weights of orders >= 1 and the projection's input are read in place
as). Both kernel families give each MFMA step the same k values in the same
tile order, so the two runs must agree bit for bit; the aligned run is pinned
to the oracle by the other parity tests."""
import pytest
import torch

from tests import _cases as H

pytestmark = pytest.mark.gpu


def _misaligned(t):
    buf = torch.empty(t.numel() + 1, dtype=t.dtype, device=t.device)
    v = buf[1:].view(t.shape)
    v.copy_(t)
    assert v.data_ptr() % 16 != 0 and v.is_contiguous()
    return v


def _same(a, b, name):
    if a is None or b is None:
        assert a is None and b is None, name
        return
    if isinstance(a, (list, tuple)):
        for i, (u, w) in enumerate(zip(a, b)):
            _same(u, w, f"{name}[{i}]")
        return
    assert torch.equal(a, b), f"{name} differs: max |diff| {float((a - b).abs().max()):.3e}"


def test_conv_misaligned_weights_bitwise():
    import so_graph_convolution_amd as K
    d = H.workload("T", n_atoms=150, box=12.0, rc=4.0, lmax=4, mmax=2, channels=48, n_rbf=16, seed=5,
                   min_dist=0.0)
    dd = H.to_dev(d)
    H.note(f"[gemm paths] conv L=4 M=2 C=48 E={len(d['src'])}")

    def run(w1, w2):
        args = (dd["kcfg"], dd["g"], dd["x"], dd["pos"], dd["rbf"], dd["w_rad"], w1, w2)
        y, saved = K.so2conv_fwd(*args, saved=True)
        b = K.so2conv_bwd(*args, saved, dd["gy"])
        db = K.so2conv_dbwd(*args, saved, dd["gy"], px=dd["px"], ppos=dd["ppos"], prbf=dd["prbf"])
        torch.cuda.synchronize()
        return y, b, db

    ref = run(dd["w1"], dd["w2"])
    mis = run([_misaligned(w) for w in dd["w1"]], [_misaligned(w) for w in dd["w2"]])
    _same(ref[0], mis[0], "y")
    for stage in (1, 2):
        assert ref[stage].keys() == mis[stage].keys()
        for k in ref[stage]:
            _same(ref[stage][k], mis[stage][k], k)


def test_grid_misaligned_input_bitwise():
    import so_graph_convolution_amd as K
    from tests.test_gpu_grid import _dev, _inputs
    L, ci, ch, co, ng, N = 4, 128, 256, 128, 100, 301
    cfg = K.GridConfig(L, ci, ch, co, ng)
    g = _dev(_inputs(L, ci, ch, co, ng, N, seed=3))
    H.note(f"[gemm paths] grid L={L} c={ci}/{ch}/{co} n_grid={ng} N={N}")

    def run(x):
        U = K.so2grid_fwd(cfg, x, g["G"], g["W"], g["A"])
        bw = K.so2grid_bwd(cfg, x, g["G"], g["W"], g["A"], g["gU"])
        torch.cuda.synchronize()
        return U, bw

    ref, mis = run(g["x"]), run(_misaligned(g["x"]))
    _same(ref[0], mis[0], "U")
    for k in ref[1]:
        _same(ref[1][k], mis[1][k], k)
