"""The C-ABI library loads on the CPU and exports every entry point that
include/so2conv.h declares (no compute call is made without a GPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "so2conv.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(so2(?:conv|grid|mole|s2)_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_entry_points():
    names = declared_functions()
    for must in ("so2conv_fwd", "so2conv_bwd", "so2conv_dbwd", "so2conv_graph_prepare", "so2conv_last_error"):
        assert must in names


def test_library_exports_every_declared_symbol():
    from so_graph_convolution_amd import _binding
    if not os.path.exists(_binding.LIB_PATH):
        pytest.fail("libso2conv.so is not built (run __graft_entry__.build())")
    lib = ctypes.CDLL(_binding.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(declared_functions()) == set(_binding.EXPORTS)


def test_host_side_argument_checks():
    """Configuration queries run on the host only."""
    import so_graph_convolution_amd as K
    lib = K.lib()
    assert lib.so2conv_supported(4, 2) == 1
    assert lib.so2conv_supported(7, 2) == 0
    good = K.SO2Config(4, 2, 128, 64)
    assert K.so2conv_saved_bytes(good, 1000) > 0
    assert K.so2conv_workspace_bytes(good, 100, 1000, 2) > K.so2conv_workspace_bytes(good, 100, 1000, 0)
    assert K.so2conv_saved_bytes(K.SO2Config(4, 2, 100, 64), 10) == 0       # C not a multiple of 16
    assert K.so2conv_saved_bytes(K.SO2Config(4, 5, 128, 64), 10) == 0       # mmax > lmax
    assert K.so2conv_saved_bytes(K.SO2Config(4, 2, 128, 6), 10) == 0        # n_rbf not a multiple of 4


def test_host_side_dtype_and_flag_checks():
    """bf16 halves the stored GEMM operands; unknown cfg flags are rejected."""
    import ctypes

    import so_graph_convolution_amd as K
    from so_graph_convolution_amd._binding import Cfg
    f32, bf16 = K.SO2Config(4, 2, 128, 64), K.SO2Config(4, 2, 128, 64, "bf16")
    # per edge at lmax 4, C 128: S, U, V float32 and T, Z bfloat16 -> 41,216 bytes (55,808 in float32)
    assert K.so2conv_saved_bytes(f32, 1024) == 1024 * 55808
    assert K.so2conv_saved_bytes(bf16, 1024) == 1024 * 41216
    assert K.so2conv_saved_bytes(K.SO2Config(4, 2, 128, 64, debug_checks=True), 8) > 0
    assert K.so2conv_saved_bytes(K.SO2Config(4, 2, 128, 64, f32_native=True), 8) > 0
    assert K.so2conv_saved_bytes(K.SO2Config(4, 2, 128, 64, fused_gate=True), 8) > 0
    bad = Cfg(4, 2, 128, 64, 0, 16)      # unknown flag bit
    assert K.lib().so2conv_saved_bytes(ctypes.byref(bad), 8) == 0
    odd = Cfg(4, 2, 128, 64, 7, 0)       # unknown dtype
    assert K.lib().so2conv_saved_bytes(ctypes.byref(odd), 8) == 0


def test_mixture_host_checks():
    """Mixture arguments are checked on the host before any device work: the
    workspace query returns 0 and the entry points return SO2_EINVAL /
    SO2_EUNSUPPORTED with a message (graph pointers are never dereferenced)."""
    import ctypes

    import numpy as np

    import so_graph_convolution_amd as K
    from so_graph_convolution_amd._binding import GraphC, MoleCfg
    cfg = K.SO2Config(4, 2, 128, 64)
    good = K.Mixture(64, [0, 400, 400, 1000])
    plain = K.so2conv_workspace_bytes(cfg, 100, 1000, 1)
    assert K.so2mole_workspace_bytes(cfg, good, 100, 1000, 1) > plain
    assert K.so2mole_workspace_bytes(cfg, good, 100, 1000, 1, 256) < K.so2mole_workspace_bytes(cfg, good, 100, 1000, 1,
                                                                                              1000)
    assert K.so2mole_workspace_bytes(cfg, K.Mixture(64, [0, 500, 400, 1000]), 100, 1000, 1) == 0   # decreasing
    assert K.so2mole_workspace_bytes(cfg, K.Mixture(64, [0, 400, 999]), 100, 1000, 1) == 0        # wrong end
    assert K.so2mole_workspace_bytes(cfg, K.Mixture(6, [0, 1000]), 100, 1000, 1) == 0             # K % 4
    c = cfg.c()
    fake = 0x1000
    g = GraphC(100, 1000, fake, fake, None, fake, fake, fake)
    bad_ptr = np.array([0, 700, 600, 1000], dtype=np.int64)
    m = MoleCfg(3, 64, bad_ptr.ctypes.data)
    r = K.lib().so2mole_fwd(ctypes.byref(c), ctypes.byref(g), ctypes.byref(m), *([None] * 11), 0, None)
    assert r == -1 and b"non-decreasing" in K.lib().so2conv_last_error()
    m = MoleCfg(3, 10, np.array([0, 100, 200, 1000], dtype=np.int64).ctypes.data)
    r = K.lib().so2mole_bwd(ctypes.byref(c), ctypes.byref(g), ctypes.byref(m), *([None] * 21), 0, None)
    assert r == -2 and b"n_experts" in K.lib().so2conv_last_error()


def test_grid_activation_host_checks():
    """so2s2_*: every size check runs on the host before any GPU call."""
    from so_graph_convolution_amd import _binding
    from so_graph_convolution_amd._binding import S2Cfg
    lib = _binding.lib()
    E_UNSUP, E_INVAL = -2, -1
    cases = [((0, 16, 10, 0, 0), E_UNSUP), ((33, 16, 10, 0, 0), E_UNSUP), ((8, 0, 10, 0, 0), E_UNSUP),
             ((8, 65537, 10, 0, 0), E_UNSUP), ((8, 16, 0, 0, 0), E_UNSUP), ((32, 16, 257, 0, 0), E_UNSUP),
             ((8, 16, 10, 1, 0), E_UNSUP), ((8, 16, 10, 0, 4), E_INVAL)]
    for fields, code in cases:
        c = S2Cfg(*fields)
        assert lib.so2s2_fwd(ctypes.byref(c), 5, None, None, None, None, None) == code, fields
    c = S2Cfg(8, 16, 10, 0, 0)
    assert lib.so2s2_fwd(ctypes.byref(c), 0, None, None, None, None, None) == 0          # no edges: no-op
    assert lib.so2s2_fwd(ctypes.byref(c), -1, None, None, None, None, None) == E_INVAL
    assert lib.so2s2_bwd(ctypes.byref(c), 4, None, None, None, None, None, None) == E_INVAL
    assert lib.so2s2_dbwd(ctypes.byref(c), 4, None, None, None, None, None, None, None, None) == E_INVAL


def test_saved_backward_state_bytes():
    """The backward's kept cotangents: Zbar and Tbar float32, Ubar in the
    operand type."""
    import so_graph_convolution_amd as K
    f32, bf16 = K.SO2Config(4, 2, 128, 64), K.SO2Config(4, 2, 128, 64, "bf16")
    # per edge at lmax 4, C 128: Zbar 2432 + Tbar 4864 floats, Ubar 2944 elements
    assert K.so2conv_saved_bwd_bytes(f32, 1024) == 1024 * 40960
    assert K.so2conv_saved_bwd_bytes(bf16, 1024) == 1024 * 35072
    assert K.so2conv_saved_bwd_bytes(K.SO2Config(4, 5, 128, 64), 10) == 0   # mmax > lmax


def test_swiglu_s2_config_host_checks():
    """The spherical-grid SwiGLU activation widens the first linear's output to
    2C per retained row; at most 32 retained rows and 1..256 grid points."""
    import ctypes

    import so_graph_convolution_amd as K
    from so_graph_convolution_amd._binding import SO2_ACT_SWIGLU_S2, Cfg

    def saved(*fields):
        return K.lib().so2conv_saved_bytes(ctypes.byref(Cfg(*fields)), 1024)
    # per edge at lmax 4, C 128 (q = 19): S 5,120 + T 19,456 + U 19,456 + Z 9,728 + V 9,728 bytes
    assert saved(4, 2, 128, 64, 0, 0, 1, SO2_ACT_SWIGLU_S2, 70) == 1024 * 63488
    assert saved(4, 2, 128, 64, 0, 0, 1, 0, 0) == 1024 * 55808          # the gate ignores n_grid
    assert saved(6, 2, 128, 64, 1, 0, 8, SO2_ACT_SWIGLU_S2, 98) > 0      # q = 29, bfloat16, 8 heads
    assert saved(6, 3, 128, 64, 0, 0, 1, SO2_ACT_SWIGLU_S2, 98) == 0     # q = 37 > 32
    assert saved(4, 2, 128, 64, 0, 0, 1, SO2_ACT_SWIGLU_S2, 0) == 0      # no grid points
    assert saved(4, 2, 128, 64, 0, 0, 1, SO2_ACT_SWIGLU_S2, 257) == 0
    assert saved(4, 2, 128, 64, 0, 0, 1, 2, 70) == 0                     # unknown activation
    with pytest.raises(ValueError):
        K.SO2Config(4, 2, 128, 64, act="swiglu_s2")                      # tables missing
    with pytest.raises(ValueError):
        K.SO2Config(4, 2, 128, 64, act="relu")
