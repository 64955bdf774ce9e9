"""MI355X-native fused variable-length attention forward.

The compute runs in ``libvarlen_attn.so`` (hand-written HIP for gfx950, C
interface in ``include/varlen_attn.h``); this package is a thin ctypes
binding plus the seeded synthetic workloads used by tests and the bench.
"""
from ._binding import (  # noqa: F401
    EXPORTED_SYMBOLS,
    LIB_PATH,
    VaTensor,
    VarlenAttnError,
    auto_num_splits,
    library,
    plan,
    raw_fwd,
    raw_fwd_fp8,
    raw_fwd_splitkv,
    raw_fwd_splitkv_noalloc,
    scratch_bytes,
    splitkv_counts,
    splitkv_workspace_bytes,
    status_string,
    tile_range,
    varlen_attn_fwd,
    varlen_attn_fwd_fp8,
    varlen_attn_fwd_noalloc,
    varlen_attn_merge,
    work_unit,
)

__all__ = [
    "varlen_attn_fwd",
    "varlen_attn_fwd_fp8",
    "raw_fwd_fp8",
    "varlen_attn_merge",
    "status_string",
    "tile_range",
    "work_unit",
    "plan",
    "library",
    "raw_fwd",
    "raw_fwd_splitkv",
    "raw_fwd_splitkv_noalloc",
    "varlen_attn_fwd_noalloc",
    "scratch_bytes",
    "splitkv_workspace_bytes",
    "splitkv_counts",
    "auto_num_splits",
    "VaTensor",
    "VarlenAttnError",
    "EXPORTED_SYMBOLS",
    "LIB_PATH",
]
