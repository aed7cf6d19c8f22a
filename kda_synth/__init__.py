"""Seeded synthetic inputs for the KDA forward pass.

This module only draws random numbers and rounds them to the storage dtype.
It holds none of the method's arithmetic: no gate activation the library
computes, no cumsum, no recurrence. Both the HIP path and the oracle consume
the exact tensors it returns (the oracle after an exact upcast to float64).

Recipe (per tensor, from one numpy PCG64 stream seeded with ``seed``):

* q, k   N(0,1) fp32, l2-normalised per row (x / sqrt(sum x^2 + 1e-6)) in fp32,
         then rounded once to the storage dtype (bf16: round-to-nearest-even).
         The caller normalises; the library does not ("Add fused recurrent_kda
         for decode and inference prefill", PR #345 text: k keeps an explicit
         l2norm before the op).
* v      N(0,1), rounded to the storage dtype.
* beta   sigmoid(N(0,1)), fp32 [B, T, H] (post-sigmoid beta).
* x      raw gate input N(0,1) fp32 [B, T, H, K].
* A_log  log U[1, 16] fp32 [H];  dt_bias N(0,1) fp32 [H, K].
* h0     0.1 * N(0,1) fp32 [N, H, K, V].
* log2 decode gate: lower_bound * sigmoid(exp(A_log) (x + dt_bias)) / ln 2,
         which lies in [lower_bound/ln2, 0) -- the distribution of a bounded
         per-token gate expressed in log2 units, as the decode workload
         specifies it.
"""
import math

import numpy as np
import torch

L2_EPS = 1e-6


def _rng(seed):
    return np.random.Generator(np.random.PCG64(int(seed)))


def _randn(rng, shape):
    return rng.standard_normal(size=shape, dtype=np.float32)


def _sigmoid32(x):
    return (1.0 / (1.0 + np.exp(-x.astype(np.float64)))).astype(np.float32)


def _l2norm32(x):
    ss = np.sum(x * x, axis=-1, keepdims=True, dtype=np.float32)
    return (x / np.sqrt(ss + np.float32(L2_EPS))).astype(np.float32)


def to_dtype(a32, dtype):
    """fp32 numpy -> torch CPU tensor of ``dtype`` (bf16 rounding is RNE)."""
    t = torch.from_numpy(np.ascontiguousarray(a32))
    return t.to(dtype) if dtype != torch.float32 else t


def varlen_offsets(seed, n_slots=10, n_empty=2, total=15872, max_len=4096, empty_at=None):
    """int32 offsets [n_slots+1]: ``n_slots - n_empty`` non-empty lengths in [1, max_len]
    that sum to ``total``, and ``n_empty`` empty slots (repeated offsets) at seeded
    positions, or at ``empty_at`` when given."""
    rng = _rng(seed)
    m = n_slots - n_empty
    while True:
        cuts = np.sort(rng.choice(np.arange(1, total), size=m - 1, replace=False))
        lens = np.diff(np.concatenate([[0], cuts, [total]]))
        if lens.min() >= 1 and lens.max() <= max_len:
            break
    if empty_at is None:
        empty_at = sorted(rng.choice(n_slots, size=n_empty, replace=False).tolist())
    full = []
    it = iter(lens.tolist())
    for s in range(n_slots):
        full.append(0 if s in empty_at else next(it))
    return np.concatenate([[0], np.cumsum(full)]).astype(np.int32)


def chunk_inputs(B, T, H, K, V, dtype=torch.bfloat16, seed=0, with_h0=True, n_slots=None):
    """Inputs for the chunked prefill. Packed batches pass B=1 and ``n_slots``.

    Returns a dict of CPU tensors: q, k [B,T,H,K]; v [B,T,H,V] (storage dtype);
    x [B,T,H,K], beta [B,T,H], A_log [H], dt_bias [H,K], h0 [N,H,K,V] or None (fp32).
    """
    rng = _rng(seed)
    N = B if n_slots is None else n_slots
    q = _l2norm32(_randn(rng, (B, T, H, K)))
    k = _l2norm32(_randn(rng, (B, T, H, K)))
    v = _randn(rng, (B, T, H, V))
    beta = _sigmoid32(_randn(rng, (B, T, H)))
    x = _randn(rng, (B, T, H, K))
    A_log = np.log(rng.uniform(1.0, 16.0, size=(H,))).astype(np.float32)
    dt_bias = _randn(rng, (H, K))
    h0 = (np.float32(0.1) * _randn(rng, (N, H, K, V))).astype(np.float32) if with_h0 else None
    return dict(q=to_dtype(q, dtype), k=to_dtype(k, dtype), v=to_dtype(v, dtype),
                x=torch.from_numpy(x), beta=torch.from_numpy(beta), A_log=torch.from_numpy(A_log),
                dt_bias=torch.from_numpy(dt_bias), h0=None if h0 is None else torch.from_numpy(h0))


def log2_gate(x, A_log, dt_bias, lower_bound=-5.0):
    """Per-token log2 decay drawn from the bounded-gate distribution (see module doc)."""
    x64 = np.asarray(x, dtype=np.float64)
    a = np.exp(np.asarray(A_log, dtype=np.float64))[:, None]
    z = a * (x64 + np.asarray(dt_bias, dtype=np.float64))
    g = lower_bound / (1.0 + np.exp(-z)) / math.log(2.0)
    return torch.from_numpy(g.astype(np.float32))


def to_f64(t):
    """Exact upcast of a CPU/GPU tensor to a float64 numpy array (None passes through)."""
    if t is None:
        return None
    return t.detach().to("cpu").to(torch.float64).numpy()
