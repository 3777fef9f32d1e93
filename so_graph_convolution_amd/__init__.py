"""MI355X-native fused edgewise SO(2) convolution (forward, backward, double backward).

The computation lives in the HIP library libso2conv.so (C ABI declared in
include/so2conv.h); this package is its thin PyTorch binding.
"""
from ._binding import EXPORTS, LIB_PATH, So2Error, lib  # noqa: F401
from .ops import (DBWD_KEYS, GRAD_KEYS, Graph, SO2Config, so2conv_bwd, so2conv_dbwd, so2conv_generator_table,  # noqa: F401
                  so2conv_debug_rotate_gather, so2conv_fwd, so2conv_fwd_noalloc, so2conv_graph_prepare, so2conv_saved_bytes,
                  so2conv_saved_bwd_bytes,
                  so2conv_workspace_bytes, weight_shapes, so2conv_profile_enable, so2conv_profile_read,
                  so2conv_profile_reset, so2conv_chunked_workspace_bytes, so2conv_debug_status)
from .grid_ops import (GridConfig, so2grid_back_bwd, so2grid_back_dbwd, so2grid_back_fwd,  # noqa: F401
                       so2grid_back_workspace_bytes, so2grid_bwd, so2grid_dbwd, so2grid_fwd, so2grid_workspace_bytes)
from .mole_ops import (Mixture, expert_shapes, so2mole_bwd, so2mole_dbwd, so2mole_fwd,  # noqa: F401
                       so2mole_workspace_bytes)
from .s2_ops import S2Config, so2s2_bwd, so2s2_dbwd, so2s2_fwd  # noqa: F401
