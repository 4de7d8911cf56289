"""MoE token layout, dispatch and combine for MI355X (gfx950).

The hot path is hand-written HIP in ``csrc/`` behind the C ABI of
``include/moe_layout.h``; this package is its thin Python binding.
"""
from .api import (  # noqa: F401
    FIELDS,
    CuBudgetStream,
    Handle,
    MoeError,
    moe_bench_copy,
    moe_time_next_kernel,
    moe_combine,
    moe_combine_bwd,
    moe_dispatch,
    moe_dispatch_bwd,
    moe_layout,
    moe_layout_noalloc,
    moe_workspace_size,
    moe_send_capacity,
    moe_recv_capacity,
    moe_send,
    moe_expand,
    moe_reduce_partitions,
    moe_combine_partitions,
)
from . import autograd  # noqa: F401

__version__ = "0.1.0"
