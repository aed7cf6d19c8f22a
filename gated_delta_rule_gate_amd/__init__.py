"""MI355X (gfx950) Kimi Delta Attention: chunked prefill, its backward, and the fused recurrence.

The computation lives in the HIP library ``_build/libkda.so`` (C ABI in
``include/kda.h``); this package only marshals arguments to it.
"""
from ._binding import (KdaError, chunk_kda, chunk_kda_bwd, chunk_kda_noalloc, gate_cumsum, lib, recurrent_kda,  # noqa: F401
                       resolved_schedule, resolved_segment, workspace_bytes, check_offsets)

__all__ = ["chunk_kda", "chunk_kda_bwd", "chunk_kda_noalloc", "recurrent_kda", "gate_cumsum", "KdaError", "lib", "resolved_schedule", "resolved_segment", "check_offsets",
           "workspace_bytes"]
