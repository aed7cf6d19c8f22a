"""Shared helpers of the GPU parity tests: input staging and the parity bounds.

Bounds (per tensor, over valid rows only):
  fp32 inputs:                   max-abs <= 1e-4
  bf16 inputs, fp32 accumulation: rel-RMS <= 5e-3 and max-abs <= 2e-2
  pass-through states:           bit-exact
rel-RMS is ||x - y||_2 / ||y||_2 over all compared elements.
"""
import math
import os

import numpy as np
import pytest
import torch

import kda_synth

FP32_MAX_ABS = 1e-4
BF16_REL_RMS = 5e-3
BF16_MAX_ABS = 2e-2


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def to_dev(d):
    return {k: (None if v is None else v.to("cuda")) for k, v in d.items()}


def f64(t):
    return kda_synth.to_f64(t)


def parity(got, want, dtype, what=""):
    """Asserts the parity bound for ``dtype`` ('bf16' or 'fp32'); returns (max_abs, rel_rms)."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    assert np.isfinite(got).all(), "%s: non-finite values in GPU output" % what
    diff = got - want
    max_abs = float(np.abs(diff).max()) if diff.size else 0.0
    den = float(np.sqrt(np.sum(want * want)))
    rel = float(np.sqrt(np.sum(diff * diff)) / den) if den > 0 else float(np.sqrt(np.sum(diff * diff)))
    log = os.environ.get("KDA_PARITY_LOG")
    if log:
        with open(log, "a") as f:
            f.write("%s | %s | %s | max-abs %.3e | rel-RMS %.3e\n" % (
                os.environ.get("PYTEST_CURRENT_TEST", "?").split(" ")[0], what, dtype, max_abs, rel))
    if dtype == "fp32":
        assert max_abs <= FP32_MAX_ABS, "%s: max-abs %.3e > %.1e" % (what, max_abs, FP32_MAX_ABS)
    else:
        assert rel <= BF16_REL_RMS, "%s: rel-RMS %.3e > %.1e (max-abs %.3e)" % (what, rel, BF16_REL_RMS, max_abs)
        assert max_abs <= BF16_MAX_ABS, "%s: max-abs %.3e > %.1e (rel-RMS %.3e)" % (what, max_abs, BF16_MAX_ABS, rel)
    return max_abs, rel


def valid_rows(cu, T):
    """Boolean mask over the packed token axis of the rows inside the contract."""
    m = np.zeros(T, dtype=bool)
    m[: int(cu[-1])] = True
    return m


def dtype_name(t):
    return "bf16" if t == torch.bfloat16 else "fp32"


def log2e():
    return 1.0 / math.log(2.0)


def tile_width(K, V=None):
    """The chunk kernels' tile width: 64, 128 or 256, the smallest covering max(K, V)."""
    m = max(K, V if V is not None else K)
    return 64 if m <= 64 else (128 if m <= 128 else 256)


def pipe_refuses(schedule, gate="safe", C=64, K=128, V=None, dtype=torch.bfloat16):
    """Whether the named schedule is the pipelined kernel and these arguments are outside
    what it takes (bf16, chunk 64, tile width 128, safe gate)."""
    return schedule == "pipe" and not (gate == "safe" and C == 64 and tile_width(K, V) == 128 and
                                       dtype == torch.bfloat16)


def expect_unsupported(fn):
    """Asserts that fn() raises the library's KDA_ERR_UNSUPPORTED."""
    from gated_delta_rule_gate_amd import KdaError

    with pytest.raises(KdaError, match="UNSUPPORTED"):
        fn()
