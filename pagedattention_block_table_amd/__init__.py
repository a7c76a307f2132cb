"""Paged-attention decode over a block table for AMD Instinct MI355X (gfx950).

The compute lives in the HIP library ``libpa.so`` (C interface in include/pa.h);
this package holds its ctypes binding (``_lib``), the seeded synthetic workloads
(``workloads``) and the build script (``build``). Importing the package does not load
the library; the first call does, and raises if it has not been built.
"""
from ._lib import (PA_BF16, PA_F16, PA_F32, PA_FP8_E4M3, BlockManager, DecodePlan,  # noqa: F401
                   PagedAttentionError,
                   balanced_workspace, pa_append_kv, pa_balanced_workspace_bytes, pa_copy_blocks, pa_check_tables,
                   pa_debug_fp8_to_f32, pa_debug_fp8_to_16bit, pa_debug_trace, pa_decode, pa_decode_balanced,
                   grouped_workspace, pa_debug_trace_grouped, pa_decode_grouped, pa_grouped_workspace_bytes,
                   pa_decode_ordered, pa_decode_partitioned, pa_decode_partitioned_noalloc, pa_extend, ordered_workspace,
                   pa_ordered_workspace_bytes, pa_partitioned_workspace_bytes, pa_status_str,
                   pa_version)

__all__ = ["pa_decode", "pa_decode_partitioned", "pa_partitioned_workspace_bytes",
           "pa_decode_partitioned_noalloc",
           "pa_decode_balanced", "pa_balanced_workspace_bytes", "balanced_workspace",
           "pa_decode_ordered", "pa_ordered_workspace_bytes", "ordered_workspace",
           "pa_decode_grouped", "pa_grouped_workspace_bytes", "grouped_workspace", "pa_debug_trace_grouped",
           "pa_extend", "pa_append_kv", "pa_copy_blocks", "pa_debug_trace", "pa_check_tables", "pa_debug_fp8_to_f32",
           "pa_debug_fp8_to_16bit", "pa_status_str",
           "pa_version", "PagedAttentionError", "DecodePlan", "BlockManager"]
