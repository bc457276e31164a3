"""MI355X (gfx950) MoE expert layer: route, dispatch, grouped SwiGLU FFN,
combine, and their backward passes, as hand-written HIP kernels behind the
C ABI of libmoe.so (include/moe.h). This package is the Python binding:
argument marshalling and buffer allocation with torch, nothing else.
"""
from . import _lib  # noqa: F401
from ._lib import (  # noqa: F401
    MoeShape, MoeError, load, moe_route, moe_dispatch, moe_dispatch_noalloc, moe_read_device_status, moe_grouped_ffn_fwd,
    moe_combine, moe_combine_bwd, moe_grouped_ffn_bwd, moe_route_bwd, moe_dispatch_bwd, mxfp8_quantize,
    workspace_size, save_size, mx_image_size, mx_dout_image_size, mx_xp_image_size, moe_load_stats, LOAD_STATS,
    mxfp8_quantize_grouped, moe_kernel_timer, moe_kernel_timer_count, GEMM_MODES,
)
from .layer import MoELayer  # noqa: F401
