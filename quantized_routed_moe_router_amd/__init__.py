"""ds4moe: routed 2-bit (or 4-bit) MoE FFN layer for AMD MI355X (gfx950).

The layer runs in libds4moe.so (hand-written HIP kernels behind a C ABI,
include/ds4moe.h).  `binding` exposes the same entry points to Python;
`layer.DeviceLayer` keeps packed weights resident in HBM.  Importing this
package loads the library and fails if it has not been built.
"""
from . import binding
from .binding import (DS4MOE_BF16, DS4MOE_F32, MODE_DECODE, MODE_PREFILL, MODE_ROUTE, Ds4MoeError,
                      ds4moe_dequant, ds4moe_dequant_q2k, ds4moe_forward_decode, ds4moe_forward_prefill,
                      ds4moe_forward_timed, ds4moe_pack, ds4moe_pack_q2k, ds4moe_packed_bytes,
                      ds4moe_packed_bytes_bits, ds4moe_route, ds4moe_workspace_bytes, make_dims, make_routing,
                      make_weights)
from .layer import DeviceLayer, ExpertCache, from_layer_inputs

binding.lib()  # load now: a missing build is an error, never a silent fallback

__all__ = ["binding", "DeviceLayer", "ExpertCache", "from_layer_inputs", "Ds4MoeError", "ds4moe_dequant", "ds4moe_dequant_q2k",
           "ds4moe_forward_decode", "ds4moe_forward_prefill", "ds4moe_forward_timed", "ds4moe_pack", "ds4moe_pack_q2k",
           "ds4moe_packed_bytes", "ds4moe_packed_bytes_bits",
           "ds4moe_route", "ds4moe_workspace_bytes", "make_dims", "make_routing", "make_weights",
           "DS4MOE_BF16", "DS4MOE_F32", "MODE_DECODE", "MODE_PREFILL", "MODE_ROUTE"]
