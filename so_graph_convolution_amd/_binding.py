"""ctypes binding of libso2conv.so (argument marshalling only).

Every step of the convolution runs in the library's HIP kernels; this module
only passes tensor storage pointers, sizes and the current HIP stream. There
is no fallback: if the library is missing, importing it raises.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libso2conv.so")

SO2_OK, SO2_EINVAL, SO2_EUNSUPPORTED, SO2_EWORKSPACE, SO2_EHIP, SO2_EDEVICE = 0, -1, -2, -3, -4, -5
SO2_DEBUG_CHECKS = 2
SO2_F32_NATIVE = 4
SO2_FUSED_GATE = 8
SO2_ACT_GATE = 0
SO2_ACT_SWIGLU_S2 = 1

c_vp = ctypes.c_void_p
c_sz = ctypes.c_size_t
c_i32 = ctypes.c_int32
c_i64 = ctypes.c_int64


class Cfg(ctypes.Structure):
    _fields_ = [("lmax", c_i32), ("mmax", c_i32), ("channels", c_i32), ("n_rbf", c_i32), ("dtype", c_i32),
                ("flags", c_i32), ("heads", c_i32), ("act", c_i32), ("n_grid", c_i32), ("grid_basis", c_vp),
                ("grid_proj", c_vp)]


class GridCfg(ctypes.Structure):
    _fields_ = [("lmax", c_i32), ("c_in", c_i32), ("c_h", c_i32), ("c_out", c_i32), ("n_grid", c_i32),
                ("dtype", c_i32), ("flags", c_i32)]


class S2Cfg(ctypes.Structure):
    _fields_ = [("rows", c_i32), ("channels", c_i32), ("n_grid", c_i32), ("dtype", c_i32), ("flags", c_i32)]


class MoleCfg(ctypes.Structure):
    _fields_ = [("n_systems", c_i32), ("n_experts", c_i32), ("sys_edge_ptr", c_vp)]


class GraphC(ctypes.Structure):
    _fields_ = [("n_nodes", c_i32), ("n_edges", c_i64), ("src", c_vp), ("dst", c_vp), ("shift", c_vp),
                ("dst_ptr", c_vp), ("src_perm", c_vp), ("src_ptr", c_vp)]


EXPORTS = {
    "so2conv_graph_workspace_bytes": (c_sz, [c_i32, c_i64]),
    "so2conv_graph_prepare": (ctypes.c_int, [c_i32, c_i64, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_sz, c_vp]),
    "so2conv_workspace_bytes": (c_sz, [ctypes.POINTER(Cfg), c_i32, c_i64, ctypes.c_int]),
    "so2conv_saved_bytes": (c_sz, [ctypes.POINTER(Cfg), c_i64]),
    "so2conv_saved_bwd_bytes": (c_sz, [ctypes.POINTER(Cfg), c_i64]),
    "so2conv_chunked_workspace_bytes": (c_sz, [ctypes.POINTER(Cfg), c_i32, c_i64, ctypes.c_int, c_i64]),
    # (cfg, g, x, pos, rbf, env, w_rad, w1, w2, y, saved, ws, ws_bytes, stream)
    "so2conv_fwd": (ctypes.c_int, [ctypes.POINTER(Cfg), ctypes.POINTER(GraphC)] + [c_vp] * 10 + [c_sz, c_vp]),
    # (cfg, g, x, pos, rbf, env, w_rad, w1, w2, y, stream)
    "so2conv_fwd_noalloc": (ctypes.c_int, [ctypes.POINTER(Cfg), ctypes.POINTER(GraphC)] + [c_vp] * 9),
    # (cfg, g, x, pos, rbf, env, w_rad, w1, w2, saved, gy, gx, gpos, grbf, genv, gw_rad, gw1, gw2, gedge,
    #  ws, ws_bytes, stream)
    "so2conv_bwd": (ctypes.c_int, [ctypes.POINTER(Cfg), ctypes.POINTER(GraphC)] + [c_vp] * 19 + [c_sz, c_vp]),
    # (cfg, g, x, pos, rbf, env, w_rad, w1, w2, saved, gy, px, ppos, pedge, prbf, penv, pw_rad, pw1, pw2,
    #  ggy, gx2, gpos2, grbf2, genv2, gw_rad2, gw1_2, gw2_2, ws, ws_bytes, stream)
    "so2conv_dbwd": (ctypes.c_int, [ctypes.POINTER(Cfg), ctypes.POINTER(GraphC)] + [c_vp] * 27 + [c_sz, c_vp]),
    "so2conv_debug_rotate_gather": (ctypes.c_int, [ctypes.POINTER(Cfg), ctypes.POINTER(GraphC), c_vp, c_vp, c_vp,
                                                   c_vp, c_vp, c_vp, c_sz, c_vp]),
    "so2conv_last_error": (ctypes.c_char_p, []),
    "so2conv_profile_enable": (ctypes.c_int, [ctypes.c_int]),
    "so2conv_profile_reset": (ctypes.c_int, []),
    "so2conv_profile_read": (ctypes.c_int, [ctypes.c_int, ctypes.POINTER(c_i64), ctypes.POINTER(ctypes.c_double),
                                            ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double)]),
    "so2conv_supported": (ctypes.c_int, [c_i32, c_i32]),
    "so2conv_generator_table": (ctypes.c_int, [c_vp, c_i64]),
    "so2conv_debug_status": (ctypes.c_int, [c_vp]),
    "so2mole_workspace_bytes": (c_sz, [ctypes.POINTER(Cfg), ctypes.POINTER(MoleCfg), c_i32, c_i64, ctypes.c_int,
                                       c_i64]),
    "so2mole_fwd": (ctypes.c_int, [ctypes.POINTER(Cfg), ctypes.POINTER(GraphC), ctypes.POINTER(MoleCfg)] + [c_vp] * 11
                    + [c_sz, c_vp]),
    "so2mole_bwd": (ctypes.c_int, [ctypes.POINTER(Cfg), ctypes.POINTER(GraphC), ctypes.POINTER(MoleCfg)] + [c_vp] * 21
                    + [c_sz, c_vp]),
    "so2mole_dbwd": (ctypes.c_int, [ctypes.POINTER(Cfg), ctypes.POINTER(GraphC), ctypes.POINTER(MoleCfg)]
                     + [c_vp] * 30 + [c_sz, c_vp]),
    "so2grid_workspace_bytes": (c_sz, [ctypes.POINTER(GridCfg), c_i32, ctypes.c_int]),
    # (cfg, N, x, G, W, A, U, ws, ws_bytes, stream)
    "so2grid_fwd": (ctypes.c_int, [ctypes.POINTER(GridCfg), c_i32] + [c_vp] * 6 + [c_sz, c_vp]),
    # (cfg, N, x, G, W, A, gU, gx, gW, gA, ws, ws_bytes, stream)
    "so2grid_bwd": (ctypes.c_int, [ctypes.POINTER(GridCfg), c_i32] + [c_vp] * 9 + [c_sz, c_vp]),
    # (cfg, N, x, G, W, A, gU, px, pW, pA, ggU, gx2, gW2, gA2, ws, ws_bytes, stream)
    "so2grid_dbwd": (ctypes.c_int, [ctypes.POINTER(GridCfg), c_i32] + [c_vp] * 13 + [c_sz, c_vp]),
    "so2grid_back_workspace_bytes": (c_sz, [ctypes.POINTER(GridCfg), c_i32, ctypes.c_int]),
    # (cfg, N, Y, H, A, Z, ws, ws_bytes, stream)
    "so2grid_back_fwd": (ctypes.c_int, [ctypes.POINTER(GridCfg), c_i32] + [c_vp] * 5 + [c_sz, c_vp]),
    # (cfg, N, Y, H, A, gZ, gY, gA, ws, ws_bytes, stream)
    "so2grid_back_bwd": (ctypes.c_int, [ctypes.POINTER(GridCfg), c_i32] + [c_vp] * 7 + [c_sz, c_vp]),
    # (cfg, N, Y, H, A, gZ, pY, pA, ggZ, gY2, gA2, ws, ws_bytes, stream)
    "so2grid_back_dbwd": (ctypes.c_int, [ctypes.POINTER(GridCfg), c_i32] + [c_vp] * 10 + [c_sz, c_vp]),
    # (cfg, E, U, G, P, Z, stream)
    "so2s2_fwd": (ctypes.c_int, [ctypes.POINTER(S2Cfg), c_i64] + [c_vp] * 5),
    # (cfg, E, U, G, P, gZ, gU, stream)
    "so2s2_bwd": (ctypes.c_int, [ctypes.POINTER(S2Cfg), c_i64] + [c_vp] * 6),
    # (cfg, E, U, G, P, gZ, pU, ggZ, gU2, stream)
    "so2s2_dbwd": (ctypes.c_int, [ctypes.POINTER(S2Cfg), c_i64] + [c_vp] * 8),
}

_lib = None


def lib():
    """Load the library (once). Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with so_graph_convolution_amd/build.py "
                              "(or __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in EXPORTS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


class So2Error(RuntimeError):
    def __init__(self, code, where):
        msg = lib().so2conv_last_error().decode()
        super().__init__(f"{where} failed with status {code}: {msg}")
        self.code = code


def check(code, where):
    if code != SO2_OK:
        raise So2Error(code, where)
