"""MI355X (gfx950) Kimi Delta Attention forward: chunked prefill and fused recurrence.

The computation lives in the HIP library ``_build/libkda.so`` (C ABI in
``include/kda.h``); this package only marshals arguments to it.
"""
from ._binding import (KdaError, chunk_kda, gate_cumsum, lib, recurrent_kda, workspace_bytes)  # noqa: F401

__all__ = ["chunk_kda", "recurrent_kda", "gate_cumsum", "KdaError", "lib", "workspace_bytes"]
