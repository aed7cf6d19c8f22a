"""FP64 CPU oracle for the Kimi Delta Attention (KDA) forward pass.

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. It shares no code
with the HIP library (``gated_delta_rule_gate_amd``) and never imports it.

Two independent formulations:

* ``recurrent`` (O1, the primary oracle): the token-by-token recurrence in C,
  FP64, OpenMP over (slot, head) pairs -- ``kda_oracle.c``.
* ``chunked`` (O2): the chunked form in numpy FP64, emitting every
  intermediate (gate cumsum, grams, triangular inverse, WY factors, chunk
  states, corrected values) -- ``chunked.py``. It is pinned against O1.

Gate activations (``gate``) follow "FLA KDA Skill", section "Gate modes".
Every array handed to the oracle is float64; callers upcast the exact bytes
the GPU consumes (bf16 and fp32 upcast to fp64 exactly).

Every function here is pinned by ``tests/test_oracle_pins.py``; none is
"parity unpinned".
"""
import ctypes
import math

import numpy as np

from . import build as _build
from .chunked import chunk_cumsum_log2, chunked_forward  # noqa: F401  (re-exported)

GATE_LOGE = 0
GATE_SAFE = 1
GATE_SOFTPLUS = 2

_LIB = None


def _lib():
    global _LIB
    if _LIB is None:
        path = _build.build(force=False)
        lib = ctypes.CDLL(path)
        dp = ctypes.POINTER(ctypes.c_double)
        ip = ctypes.POINTER(ctypes.c_int32)
        lib.kda_oracle_gate.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                        dp, dp, dp, ctypes.c_double, dp]
        lib.kda_oracle_gate.restype = None
        lib.kda_oracle_recurrent.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                             ip, dp, dp, dp, dp, ctypes.c_int, dp, ctypes.c_double,
                                             dp, dp, dp, ctypes.c_int]
        lib.kda_oracle_recurrent.restype = None
        lib.kda_oracle_recurrent_bwd.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                                 ip, dp, dp, dp, dp, dp, ctypes.c_double, dp, dp, dp,
                                                 dp, dp, dp, dp, dp, dp, ctypes.c_int]
        lib.kda_oracle_recurrent_bwd.restype = None
        _LIB = lib
    return _LIB


def _f64(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def gate(kind, x, A_log=None, dt_bias=None, lower_bound=0.0):
    """Per-token natural-log decay g from the raw gate input.

    kind 0 (pre-gated): g = x.
    kind 1 (safe):      g = lower_bound * sigmoid(exp(A_log) * (x + dt_bias)).
    kind 2 (softplus):  g = -exp(A_log) * softplus(x + dt_bias).
    x has shape [..., H, K]; A_log [H]; dt_bias [H, K] or None.
    """
    x = _f64(x)
    H, K = x.shape[-2], x.shape[-1]
    T = x.size // (H * K)
    out = np.empty_like(x)
    A = _f64(A_log) if A_log is not None else np.zeros(H)
    dt = _f64(dt_bias).reshape(H, K) if dt_bias is not None else None
    _lib().kda_oracle_gate(int(kind), T, H, K, _ptr(x), _ptr(A), _ptr(dt), float(lower_bound), _ptr(out))
    return out


L2NORM_EPS = 1e-6


def l2norm_rows(x, eps=L2NORM_EPS):
    """Each row (last axis) divided by sqrt(sum of its squares + eps), in FP64.

    The explicit normalisation that the kernels' q_l2norm option defers to the
    output ("Add fused recurrent_kda ...", stacked description of the fused
    q-l2norm option: the eps floor is l2norm's default, read as 1e-6).
    """
    x = _f64(x)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def beta_from_logits(x):
    """The logistic sigmoid 1 / (1 + e^-x) in FP64: beta from raw logits ("FLA KDA
    Skill", section "Correctness checklist": raw beta logits and post-sigmoid beta).
    Written as e^x / (1 + e^x) for x < 0 so that neither branch overflows.
    """
    x = _f64(x)
    e = np.exp(-np.abs(x))
    return np.where(x >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def _offsets(B, T, cu_seqlens):
    if cu_seqlens is None:
        return np.arange(B + 1, dtype=np.int32) * T
    assert B == 1, "packed inputs have batch 1"
    return np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))


def recurrent(q, k, v, g, beta, h0=None, cu_seqlens=None, scale=None, g_is_log2=False, nthreads=0):
    """O1: token-by-token FP64 recurrence.

    q, k [B, T, H, K]; v [B, T, H, V]; g [B, T, H, K] (natural log, or log2 when
    ``g_is_log2``); beta [B, T, H]; h0 [N, H, K, V] or None; cu_seqlens [N+1]
    int32 (then B == 1). Returns (o [B, T, H, V] with NaN in rows outside the
    contract, ht [N, H, K, V]).
    """
    q, k, v, g, beta = (_f64(a) for a in (q, k, v, g, beta))
    B, T, H, K = q.shape
    V = v.shape[-1]
    cu = _offsets(B, T, cu_seqlens)
    N = len(cu) - 1
    if scale is None:
        scale = 1.0 / math.sqrt(K)
    h0a = _f64(h0).reshape(N, H, K, V) if h0 is not None else None
    o = np.full((B, T, H, V), np.nan)
    ht = np.empty((N, H, K, V))
    _lib().kda_oracle_recurrent(N, H, K, V, cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                _ptr(q), _ptr(k), _ptr(v), _ptr(g), int(bool(g_is_log2)), _ptr(beta),
                                float(scale), _ptr(h0a), _ptr(o), _ptr(ht), int(nthreads))
    return o, ht


def recurrent_bwd(q, k, v, g, beta, do, dht=None, h0=None, cu_seqlens=None, scale=None, nthreads=0):
    """Gradients of L = sum(do * o) + sum(dht * ht) through O1 (natural-log gate g).

    Reverse mode through the token recurrence, FP64 (``kda_oracle.c``). Shapes as
    in ``recurrent``; do [B, T, H, V]; dht [N, H, K, V] or None. Returns (dq, dk,
    dv, dg, dbeta, dh0), each shaped like its input (dh0 [N, H, K, V]); rows
    outside the packed contract are NaN. dg is the gradient of the per-token
    natural-log decay; ``gate_bwd`` carries it to a raw gate input.
    """
    q, k, v, g, beta, do = (_f64(a) for a in (q, k, v, g, beta, do))
    B, T, H, K = q.shape
    V = v.shape[-1]
    cu = _offsets(B, T, cu_seqlens)
    N = len(cu) - 1
    if scale is None:
        scale = 1.0 / math.sqrt(K)
    h0a = _f64(h0).reshape(N, H, K, V) if h0 is not None else None
    dhta = _f64(dht).reshape(N, H, K, V) if dht is not None else None
    dq = np.full((B, T, H, K), np.nan)
    dk = np.full((B, T, H, K), np.nan)
    dv = np.full((B, T, H, V), np.nan)
    dg = np.full((B, T, H, K), np.nan)
    dbeta = np.full((B, T, H), np.nan)
    dh0 = np.empty((N, H, K, V))
    _lib().kda_oracle_recurrent_bwd(N, H, K, V, cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                    _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), float(scale), _ptr(h0a),
                                    _ptr(do), _ptr(dhta), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg), _ptr(dbeta),
                                    _ptr(dh0), int(nthreads))
    return dq, dk, dv, dg, dbeta, dh0


def gate_bwd(kind, x, dg, A_log=None, dt_bias=None, lower_bound=0.0):
    """Carries dg (gradient of the natural-log decay that ``gate`` returns) back to
    the raw input x [..., H, K], A_log [H] and dt_bias [H, K] ("FLA KDA Skill",
    section "Gate modes", differentiated):

      safe      g = lb s(z), z = e^A (x + dt):  dg/dx = dg/d dt = lb s(z)(1 - s(z)) e^A,
                dg/dA = dg/dx (x + dt)
      softplus  g = -e^A sp(z), z = x + dt:     dg/dx = dg/d dt = -e^A s(z),  dg/dA = g
      pre-gated g = x:                           dg/dx = 1, no parameters

    Returns (dx, dA_log [H] or None, ddt_bias [H, K] or None); the parameter
    gradients sum over every token. Rows of dg that are NaN (outside the packed
    contract) must be masked by the caller.
    """
    x, dg = _f64(x), _f64(dg)
    H, K = x.shape[-2], x.shape[-1]
    if kind == GATE_LOGE:
        return dg.copy(), None, None
    A = _f64(A_log).reshape(H)
    dt = _f64(dt_bias).reshape(H, K) if dt_bias is not None else np.zeros((H, K))
    eA = np.exp(A)[:, None]
    z0 = x + dt
    if kind == GATE_SAFE:
        s = beta_from_logits(eA * z0)
        gx = lower_bound * s * (1.0 - s) * eA
        ga = gx * z0
    else:
        s = beta_from_logits(z0)
        gx = -eA * s
        ga = gate(GATE_SOFTPLUS, x, A_log, dt_bias, lower_bound)
    dx = dg * gx
    lead = tuple(range(x.ndim - 2))
    return dx, np.sum(dg * ga, axis=lead).sum(axis=-1), np.sum(dx, axis=lead)
