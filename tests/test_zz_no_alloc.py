"""so2conv_fwd_noalloc (the forward through the library's fixed device scratch)
against so2conv_fwd, through the C ABI: two calls in a row, the second on a
smaller input, so the second runs on whatever the first left in the scratch;
and the host-side refusal of a configuration whose smallest chunk does not fit.
"""
import numpy as np
import pytest
import torch

import so2_synth
from tests import _cases as H

pytestmark = pytest.mark.gpu


def _fwd_pair(d, dtype="f32"):
    import so_graph_convolution_amd as K
    dd = H.to_dev(d, dtype)
    args = (dd["kcfg"], dd["g"], dd["x"], dd["pos"], dd["rbf"], dd["w_rad"], dd["w1"], dd["w2"])
    y_ref, _ = K.so2conv_fwd(*args, saved=True)
    y = K.so2conv_fwd_noalloc(*args)
    torch.cuda.synchronize()
    return y, y_ref


def test_noalloc_matches_fwd_two_calls():
    big = so2_synth.make_inputs(so2_synth.CONFIGS["S"], with_directions=False)
    small = so2_synth.make_inputs(so2_synth.make_config("T", n_atoms=24, box=8.0, rc=4.0, seed=5),
                                  with_directions=False)
    errs = []
    for name, d in (("eSEN-like small, 180k edges (scratch in edge chunks)", big), ("tiny, 24 atoms", small)):
        H.note(f"[noalloc] {name}: N={d['cfg'].n_atoms} E={len(d['src'])}")
        y, y_ref = _fwd_pair(d)
        e = H.errs_both(y, y_ref)
        H.note(f"  max-norm {e[0]:.2e} element-wise {e[1]:.2e}")
        errs.append(e)
    assert all(e[0] <= H.TOL_F32 and e[1] <= H.TOL_ELEM_F32 for e in errs), errs


def test_noalloc_refuses_oversized_configuration():
    """bfloat16 at 20,000 nodes keeps 1 GiB of float32 node copies in the
    workspace: more than the scratch holds, refused before any launch."""
    import so_graph_convolution_amd as K
    cfg = K.SO2Config(6, 2, 128, 64, "bf16")
    N, E = 20000, 2048
    dev = torch.device("cuda:0")
    src = torch.zeros(E, dtype=torch.int32, device=dev)
    dst = torch.zeros(E, dtype=torch.int32, device=dev)
    g = K.so2conv_graph_prepare(N, src, dst, torch.zeros(E, 3, device=dev), validate=False)
    s1, s2 = K.weight_shapes(cfg)
    bf = torch.bfloat16
    x = torch.zeros(N, cfg.d, 128, dtype=bf, device=dev)
    with pytest.raises(K.So2Error) as ei:
        K.so2conv_fwd_noalloc(cfg, g, x, torch.zeros(N, 3, device=dev), torch.zeros(E, 64, device=dev),
                              torch.zeros(64, 7 * 256, dtype=bf, device=dev),
                              [torch.zeros(s, dtype=bf, device=dev) for s in s1],
                              [torch.zeros(s, dtype=bf, device=dev) for s in s2])
    assert ei.value.code == -3 and "fixed scratch" in str(ei.value), str(ei.value)
