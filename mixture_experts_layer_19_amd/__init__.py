"""Dropless top-k mixture-of-experts FFN layer forward for AMD MI355X (gfx950).

The compute path is the HIP library libmoe_mi355x.so (C ABI in include/moe.h); `binding`
wraps it with the same names. Importing this package loads nothing: the library is loaded
on the first call, and a call raises if it has not been built.
"""
from .binding import (  # noqa: F401
    LayerConfig,
    MoeError,
    Op,
    moe_combine,
    moe_dispatch,
    moe_dispatch_capacity,
    moe_expert_capacity,
    moe_expert_ffn,
    moe_forward,
    moe_get_device_error,
    moe_route,
    moe_shared_ffn,
    moe_update_bias,
    moe_workspace_size,
    workspace,
)
