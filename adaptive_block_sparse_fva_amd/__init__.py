"""Adaptive block-sparse self-attention for video DiTs on AMD Instinct MI355X.

The hot path lives in libfva.so (hand-written HIP for gfx950, C ABI in
include/fva.h); `adaptive_block_sparse_fva_amd.fva` is its ctypes binding.
"""

from .fva import (  # noqa: F401
    BalanceInfo,
    BalanceParams,
    Buffers,
    FvaError,
    GsrsSchedule,
    Problem,
    attn_workgroups,
    compute_units,
    balance,
    balance_params,
    block_importance,
    gsrs_action,
    gsrs_schedule,
    kv_layout,
    load_library,
    make_problem,
    mfma_probe,
    plan,
    reselect,
    route,
    route_noalloc,
    schedule,
    sasa_refill,
    sizes,
    sparse_attn_fwd,
)

__version__ = "0.4.0"
