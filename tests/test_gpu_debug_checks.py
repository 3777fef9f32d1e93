"""Device-side input validation (cfg flag SO2_DEBUG_CHECKS): bad inputs are
reported as SO2_EDEVICE before any compute kernel runs, and the word of
failed checks is readable through so2conv_debug_status. Every input here
keeps its indices in range, so nothing reads out of bounds either way."""
import dataclasses

import numpy as np
import pytest
import torch

from tests import _cases as H

pytestmark = pytest.mark.gpu


def _setup(d, validate_graph=True):
    dd = H.to_dev(d, validate_graph=validate_graph)
    return dataclasses.replace(dd["kcfg"], debug_checks=True), dd


def _fwd(kc, dd):
    import so_graph_convolution_amd as K
    return K.so2conv_fwd(kc, dd["g"], dd["x"], dd["pos"], dd["rbf"], dd["w_rad"], dd["w1"], dd["w2"], saved=True)


def test_valid_inputs_pass_the_checks():
    import so_graph_convolution_amd as K
    d = H.workload("T", seed=3)
    kc, dd = _setup(d)
    y, saved = _fwd(kc, dd)
    K.so2conv_bwd(kc, dd["g"], dd["x"], dd["pos"], dd["rbf"], dd["w_rad"], dd["w1"], dd["w2"], saved, dd["gy"])
    K.so2conv_debug_status()
    assert bool(torch.isfinite(y).all())


@pytest.mark.parametrize("fault", ["zero_length_edge", "nan_rbf", "dst_decreasing"])
def test_bad_inputs_are_reported(fault):
    import so_graph_convolution_amd as K
    d = dict(H.workload("T", seed=3))
    if fault == "zero_length_edge":
        e = int(np.nonzero(~d["shift"].any(1))[0][0])           # an edge with no periodic shift
        pos = d["pos"].copy()
        pos[d["src"][e]] = pos[d["dst"][e]]                      # v_e = 0 exactly
        d["pos"] = pos
        bit = "zero-length edge"
    elif fault == "nan_rbf":
        rbf = d["rbf"].copy()
        rbf[5, 1] = np.nan
        d["rbf"] = rbf
        bit = "non-finite input"
    else:
        d["dst"] = d["dst"][::-1].copy()        # indices stay in range
        d["src"] = d["src"][::-1].copy()
        d["shift"] = d["shift"][::-1].copy()
        d["rbf"] = d["rbf"][::-1].copy()
        bit = "dst decreasing"
    kc, dd = _setup(d, validate_graph=(fault != "dst_decreasing"))
    H.note(f"[debug checks] {fault}")
    with pytest.raises(K.So2Error) as ei:
        _fwd(kc, dd)
    assert ei.value.code == -5 and bit in str(ei.value)
    with pytest.raises(K.So2Error) as ei:
        K.so2conv_debug_status()
    assert ei.value.code == -5
    K.so2conv_debug_status()    # reported once, then clear
