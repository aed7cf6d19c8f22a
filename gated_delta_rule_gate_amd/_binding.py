"""ctypes binding of libkda.so (include/kda.h): argument marshalling only.

Every step of the computation runs in the HIP library. PyTorch supplies device
memory and the current stream. When the library has not been built, every
entry point raises: there is no fallback path.
"""
import ctypes
import math
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "_build", "libkda.so")

KDA_BF16, KDA_F32 = 0, 1
GATE_KINDS = {"loge": 0, "safe": 1, "softplus": 2, "log2_cumsum": 3, "log2": 4}
SCHEDULES = {"auto": 0, "staged": 1, "fused": 2, "split": 3, "pipe": 4}

_LIB = None


class KdaError(RuntimeError):
    """A status code other than KDA_OK returned by the library."""


class KdaArgs(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int), ("T", ctypes.c_int), ("H", ctypes.c_int), ("K", ctypes.c_int),
                ("V", ctypes.c_int), ("N", ctypes.c_int), ("chunk_size", ctypes.c_int), ("dtype", ctypes.c_int),
                ("scale", ctypes.c_float), ("gate_kind", ctypes.c_int), ("A_log", ctypes.c_void_p),
                ("dt_bias", ctypes.c_void_p), ("lower_bound", ctypes.c_float), ("schedule", ctypes.c_int),
                ("Hk", ctypes.c_int), ("q_l2norm", ctypes.c_int), ("beta_logits", ctypes.c_int),
                ("segment", ctypes.c_int)]


def lib():
    """Loads libkda.so (raises if it is not built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libkda.so is not built (%s); run __graft_entry__.build()" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        vp, ap = ctypes.c_void_p, ctypes.POINTER(KdaArgs)
        L.kda_status_string.argtypes = [ctypes.c_int]
        L.kda_status_string.restype = ctypes.c_char_p
        L.kda_last_error.argtypes = []
        L.kda_last_error.restype = ctypes.c_char_p
        L.kda_recurrent_fwd.argtypes = [ap] + [vp] * 10
        L.kda_recurrent_fwd.restype = ctypes.c_int
        L.kda_gate_cumsum.argtypes = [ap, vp, vp, ctypes.c_int, vp, vp]
        L.kda_gate_cumsum.restype = ctypes.c_int
        if hasattr(L, "kda_chunk_fwd"):
            L.kda_chunk_workspace_bytes.argtypes = [ap]
            L.kda_chunk_workspace_bytes.restype = ctypes.c_size_t
            L.kda_chunk_schedule.argtypes = [ap]
            L.kda_chunk_schedule.restype = ctypes.c_int
            L.kda_chunk_segment.argtypes = [ap]
            L.kda_chunk_segment.restype = ctypes.c_int
            L.kda_check_offsets.argtypes = [vp, ctypes.c_int, ctypes.c_int, vp, vp]
            L.kda_check_offsets.restype = ctypes.c_int
            L.kda_chunk_fwd.argtypes = [ap] + [vp] * 10 + [ctypes.c_size_t, vp]
            L.kda_chunk_fwd.restype = ctypes.c_int
            L.kda_chunk_states_count.argtypes = [ap, ctypes.c_int]
            L.kda_chunk_states_count.restype = ctypes.c_size_t
            L.kda_chunk_fwd_states.argtypes = [ap] + [vp] * 11 + [ctypes.c_size_t, vp]
            L.kda_chunk_fwd_states.restype = ctypes.c_int
        if hasattr(L, "kda_chunk_fwd_noalloc"):
            L.kda_chunk_fwd_noalloc.argtypes = [ap] + [vp] * 10
            L.kda_chunk_fwd_noalloc.restype = ctypes.c_int
            L.kda_chunk_noalloc_max_bytes.argtypes = []
            L.kda_chunk_noalloc_max_bytes.restype = ctypes.c_size_t
        if hasattr(L, "kda_chunk_bwd"):
            L.kda_chunk_bwd_workspace_bytes.argtypes = [ap]
            L.kda_chunk_bwd_workspace_bytes.restype = ctypes.c_size_t
            L.kda_chunk_bwd.argtypes = [ap] + [vp] * 18 + [ctypes.c_size_t, vp]
            L.kda_chunk_bwd.restype = ctypes.c_int
        if hasattr(L, "kda_chunk_stage"):
            L.kda_chunk_stage.argtypes = [ap, ctypes.c_int] + [vp] * 10 + [ctypes.c_size_t, vp]
            L.kda_chunk_stage.restype = ctypes.c_int
            L.kda_staged_workspace_offset.argtypes = [ap, ctypes.c_int]
            L.kda_staged_workspace_offset.restype = ctypes.c_size_t
        _LIB = L
    return _LIB


def check(status):
    if status != 0:
        L = lib()
        msg = L.kda_status_string(status).decode()
        if status == 9:
            msg += " (" + L.kda_last_error().decode() + ")"
        raise KdaError(msg)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _require(cond, msg):
    if not cond:
        raise ValueError(msg)


def _check_tensors(named, device):
    for name, t in named.items():
        if t is None:
            continue
        _require(t.is_cuda and t.device == device, "%s must be on %s" % (name, device))
        _require(t.is_contiguous(), "%s must be contiguous" % name)
        if t.requires_grad:
            raise RuntimeError("%s requires grad: this forward-only op does not track gradients; "
                               "use a training implementation of chunk_kda for backward" % name)


def make_args(q, v, H, N, gate_kind, chunk_size=64, scale=None, A_log=None, dt_bias=None, lower_bound=-5.0,
              schedule="auto", q_l2norm=False, beta_logits=False, segment=0):
    B, T, Hk, K = q.shape
    V = v.shape[-1]
    a = KdaArgs()
    a.B, a.T, a.H, a.K, a.V, a.N = B, T, H, K, V, N
    a.Hk = Hk if Hk != H else 0
    a.chunk_size = int(chunk_size)
    a.dtype = KDA_BF16 if q.dtype == torch.bfloat16 else KDA_F32
    a.scale = float(scale) if scale is not None else 0.0
    a.gate_kind = GATE_KINDS[gate_kind] if isinstance(gate_kind, str) else int(gate_kind)
    a.A_log = A_log.data_ptr() if A_log is not None else None
    a.dt_bias = dt_bias.data_ptr() if dt_bias is not None else None
    a.lower_bound = float(lower_bound) if lower_bound is not None else 0.0
    a.schedule = SCHEDULES[schedule] if isinstance(schedule, str) else int(schedule)
    a.q_l2norm = 1 if q_l2norm else 0
    a.beta_logits = 1 if beta_logits else 0
    a.segment = int(segment)
    return a


def _common(q, k, v, g, beta, initial_state, cu_seqlens, A_log, dt_bias):
    _require(q.dim() == 4 and k.shape == q.shape, "q, k must be [B, T, Hk, K] of one shape")
    _require(v.dim() == 4 and v.shape[:2] == q.shape[:2] and v.shape[2] % q.shape[2] == 0,
             "v must be [B, T, H, V] with H a multiple of q's heads Hk")
    _require(q.dtype in (torch.bfloat16, torch.float32) and k.dtype == q.dtype and v.dtype == q.dtype,
             "q, k, v must share dtype bf16 or fp32")
    B, T, Hk, K = q.shape
    H, V = v.shape[2], v.shape[3]
    _require(g.shape == (B, T, H, K) and g.dtype == torch.float32, "g must be fp32 [B, T, H, K]")
    _require(beta.shape == (B, T, H) and beta.dtype == torch.float32, "beta must be fp32 [B, T, H]")
    if cu_seqlens is not None:
        _require(B == 1, "packed inputs (cu_seqlens) need batch 1")
        _require(cu_seqlens.dtype == torch.int32 and cu_seqlens.dim() == 1, "cu_seqlens must be int32 [N+1]")
        N = cu_seqlens.numel() - 1
    else:
        N = B
    if initial_state is not None:
        _require(initial_state.shape == (N, H, K, V) and initial_state.dtype == torch.float32,
                 "initial_state must be fp32 [N, H, K, V]")
    _check_tensors(dict(q=q, k=k, v=v, g=g, beta=beta, initial_state=initial_state, cu_seqlens=cu_seqlens,
                        A_log=A_log, dt_bias=dt_bias), q.device)
    return B, T, H, K, V, N


def _check_outputs(out, final_state, B, T, H, K, V, N, dtype, device):
    """Caller-supplied outputs: the kernels write B*T*H*V elements of o and N*H*K*V
    fp32 of the final state through raw pointers, so shape, dtype, layout and
    device are checked here (the C ABI cannot see them)."""
    if out is not None:
        _require(tuple(out.shape) == (B, T, H, V) and out.dtype == dtype,
                 "out must be %s [B, T, H, V] = %s" % (dtype, (B, T, H, V)))
    if final_state is not None:
        _require(tuple(final_state.shape) == (N, H, K, V) and final_state.dtype == torch.float32,
                 "final_state must be fp32 [N, H, K, V] = %s" % ((N, H, K, V),))
    _check_tensors(dict(out=out, final_state=final_state), device)


def recurrent_kda(q, k, v, g, beta, initial_state=None, *, cu_seqlens=None, output_final_state=False,
                  gate_kind="log2", A_log=None, dt_bias=None, lower_bound=-5.0, scale=None, final_state=None,
                  out=None, q_l2norm=False, beta_logits=False):
    """Fused token-sequential KDA forward. Returns (o, ht); ht is None unless requested.

    g is the per-token decay (log2 units by default; ``gate_kind`` "loge", "safe"
    or "softplus" select the other gate contracts). ``final_state`` may be a
    preallocated fp32 [N, H, K, V] output, including ``initial_state`` itself for
    an in-place state update. ``out`` may preallocate o; rows outside the
    packed contract are left as they are. ``q_l2norm=True`` takes raw q and
    normalises it inside (each output row scaled by 1/sqrt(|q|^2 + 1e-6)).
    ``beta_logits=True`` takes beta as logits (the sigmoid runs in the kernel).
    """
    B, T, H, K, V, N = _common(q, k, v, g, beta, initial_state, cu_seqlens, A_log, dt_bias)
    _check_outputs(out, final_state, B, T, H, K, V, N, q.dtype, q.device)
    o = out if out is not None else torch.empty((B, T, H, V), dtype=q.dtype, device=q.device)
    ht = final_state
    if ht is None and output_final_state:
        ht = torch.empty((N, H, K, V), dtype=torch.float32, device=q.device)
    a = make_args(q, v, H, N, gate_kind, scale=scale, A_log=A_log, dt_bias=dt_bias, lower_bound=lower_bound,
                  q_l2norm=q_l2norm, beta_logits=beta_logits)
    check(lib().kda_recurrent_fwd(ctypes.byref(a), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                  _ptr(initial_state), _ptr(cu_seqlens), _ptr(o), _ptr(ht), _stream()))
    return o, ht


def gate_cumsum(g, *, chunk_size=64, gate_kind="safe", A_log=None, dt_bias=None, lower_bound=-5.0,
                cu_seqlens=None, out=None):
    """Step (1) alone: the gate activation and the chunk-local cumsum in log2 units.

    g is fp32 [B, T, H, K]. ``chunk_size`` 1 gives the per-token log2 decay that
    ``recurrent_kda`` takes; 32 or 64 gives the gate that ``chunk_kda`` takes with
    ``gate_kind="log2_cumsum"`` and the same chunk size. Rows outside the packed
    contract are left as they are in ``out``.
    """
    _require(g.dim() == 4 and g.dtype == torch.float32, "g must be fp32 [B, T, H, K]")
    B, T, H, K = g.shape
    if cu_seqlens is not None:
        _require(B == 1, "packed inputs (cu_seqlens) need batch 1")
        _require(cu_seqlens.dtype == torch.int32 and cu_seqlens.dim() == 1, "cu_seqlens must be int32 [N+1]")
        N = cu_seqlens.numel() - 1
    else:
        N = B
    out = out if out is not None else torch.empty_like(g)
    _require(out.shape == g.shape and out.dtype == torch.float32, "out must be fp32 like g")
    _check_tensors(dict(g=g, out=out, cu_seqlens=cu_seqlens, A_log=A_log, dt_bias=dt_bias), g.device)
    a = make_args(g, g, H, N, gate_kind, chunk_size=64, A_log=A_log, dt_bias=dt_bias, lower_bound=lower_bound)
    check(lib().kda_gate_cumsum(ctypes.byref(a), _ptr(g), _ptr(cu_seqlens), int(chunk_size), _ptr(out), _stream()))
    return out


def chunk_kda(q, k, v, g, beta, initial_state=None, *, cu_seqlens=None, output_final_state=False,
              chunk_size=64, gate_kind="safe", A_log=None, dt_bias=None, lower_bound=-5.0, scale=None,
              schedule="auto", final_state=None, out=None, q_l2norm=False, return_intermediate_states=False,
              intermediate_states=None, beta_logits=False, segment=0, workspace=None):
    """Chunked KDA prefill forward. Returns (o, ht); ht is None unless requested.

    g is the raw gate input for ``gate_kind`` "safe" / "softplus" (activation in
    the kernel), the natural-log decay for "loge", or the output of
    ``gate_cumsum`` with the same chunk size for "log2_cumsum". ``out`` may
    preallocate o. ``q_l2norm=True`` takes raw q and normalises it inside: each
    output row is scaled by 1/sqrt(|q|^2 + 1e-6) (o is linear in each q row).
    ``beta_logits=True`` takes beta as logits (the sigmoid runs in the kernels).

    ``return_intermediate_states=True`` returns (o, ht, h_states): the fp32 state
    entering every chunk, [B, ceil(T / C), H, K, V] for a dense batch and
    [1, ceil(T / C) + N, H, K, V] for a packed one, whose chunks are numbered slot
    by slot (slot n starts at the sum of ceil(len_m / C) over m < n; entries past
    the last chunk are left as they are). ``intermediate_states`` may preallocate it.

    ``segment`` (split schedule): chunks per segment of the chain-parallel state
    scan; 0 lets the library choose from the sizes, -1 keeps one serial chain per
    (sequence, head). The states path always runs the serial chain.

    ``workspace`` may pass a uint8 device tensor of at least ``workspace_bytes``
    for these arguments, reused across calls; otherwise each call allocates one.
    """
    B, T, H, K, V, N = _common(q, k, v, g, beta, initial_state, cu_seqlens, A_log, dt_bias)
    _check_outputs(out, final_state, B, T, H, K, V, N, q.dtype, q.device)
    o = out if out is not None else torch.empty((B, T, H, V), dtype=q.dtype, device=q.device)
    ht = final_state
    if ht is None and output_final_state:
        ht = torch.empty((N, H, K, V), dtype=torch.float32, device=q.device)
    a = make_args(q, v, H, N, gate_kind, chunk_size=chunk_size, scale=scale, A_log=A_log, dt_bias=dt_bias,
                  lower_bound=lower_bound, schedule=schedule, q_l2norm=q_l2norm, beta_logits=beta_logits,
                  segment=segment)
    L = lib()
    ws_bytes = L.kda_chunk_workspace_bytes(ctypes.byref(a))
    if workspace is not None:
        _require(workspace.dtype == torch.uint8 and workspace.dim() == 1 and workspace.numel() >= ws_bytes,
                 "workspace must be a 1-D uint8 tensor of at least %d bytes" % ws_bytes)
        _check_tensors(dict(workspace=workspace), q.device)
        ws = workspace
    else:
        ws = torch.empty((max(int(ws_bytes), 256),), dtype=torch.uint8, device=q.device)
    if not (return_intermediate_states or intermediate_states is not None):
        check(L.kda_chunk_fwd(ctypes.byref(a), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                              _ptr(initial_state), _ptr(cu_seqlens), _ptr(o), _ptr(ht), _ptr(ws),
                              ctypes.c_size_t(ws.numel()), _stream()))
        return o, ht
    count = int(L.kda_chunk_states_count(ctypes.byref(a), 1 if cu_seqlens is not None else 0))
    _require(count > 0 or T == 0, "unsupported shape for intermediate states")
    shape = (B, count // B, H, K, V)
    hs = intermediate_states
    if hs is None:
        hs = torch.empty(shape, dtype=torch.float32, device=q.device)
    _require(hs.shape == shape and hs.dtype == torch.float32, "intermediate_states must be fp32 %s" % (shape,))
    _check_tensors(dict(intermediate_states=hs), q.device)
    check(L.kda_chunk_fwd_states(ctypes.byref(a), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                 _ptr(initial_state), _ptr(cu_seqlens), _ptr(o), _ptr(ht), _ptr(hs), _ptr(ws),
                                 ctypes.c_size_t(ws.numel()), _stream()))
    return o, ht, hs


def chunk_kda_noalloc(q, k, v, g, beta, initial_state=None, *, out, final_state=None, cu_seqlens=None,
                      chunk_size=64, gate_kind="safe", A_log=None, dt_bias=None, lower_bound=-5.0, scale=None,
                      schedule="auto", q_l2norm=False, beta_logits=False, segment=0):
    """``chunk_kda`` through kda_chunk_fwd_noalloc, which allocates nothing: the
    intermediates live in the library's static device array. The caller passes the
    output ``out`` (and ``final_state`` to receive the final state); this wrapper
    allocates nothing either. Returns (out, final_state)."""
    B, T, H, K, V, N = _common(q, k, v, g, beta, initial_state, cu_seqlens, A_log, dt_bias)
    _require(out is not None, "out must be preallocated")
    _check_outputs(out, final_state, B, T, H, K, V, N, q.dtype, q.device)
    a = make_args(q, v, H, N, gate_kind, chunk_size=chunk_size, scale=scale, A_log=A_log, dt_bias=dt_bias,
                  lower_bound=lower_bound, schedule=schedule, q_l2norm=q_l2norm, beta_logits=beta_logits,
                  segment=segment)
    check(lib().kda_chunk_fwd_noalloc(ctypes.byref(a), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                      _ptr(initial_state), _ptr(cu_seqlens), _ptr(out), _ptr(final_state),
                                      _stream()))
    return out, final_state


def chunk_kda_bwd(q, k, v, g, beta, do, initial_state=None, *, dht=None, cu_seqlens=None, chunk_size=64,
                  gate_kind="safe", A_log=None, dt_bias=None, lower_bound=-5.0, scale=None, beta_logits=False):
    """Backward of ``chunk_kda``: gradients of sum(do * o) + sum(dht * ht).

    Returns a dict with dq, dk (dtype of q), dv (dtype of v), dg (fp32, of g as
    passed: the raw gate input for "safe" / "softplus"), dbeta (fp32), dh0 (fp32,
    [N, H, K, V]) and, for "safe" / "softplus", dA_log [H] and ddt_bias [H, K].
    The forward is recomputed inside the library.
    """
    B, T, H, K, V, N = _common(q, k, v, g, beta, initial_state, cu_seqlens, A_log, dt_bias)
    _require(do.shape == (B, T, H, V) and do.dtype == q.dtype, "do must be [B, T, H, V] in q's dtype")
    if dht is not None:
        _require(dht.shape == (N, H, K, V) and dht.dtype == torch.float32, "dht must be fp32 [N, H, K, V]")
    _check_tensors(dict(do=do, dht=dht), q.device)
    a = make_args(q, v, H, N, gate_kind, chunk_size=chunk_size, scale=scale, A_log=A_log, dt_bias=dt_bias,
                  lower_bound=lower_bound, schedule="staged", beta_logits=beta_logits)
    L = lib()
    ws_bytes = int(L.kda_chunk_bwd_workspace_bytes(ctypes.byref(a)))
    ws = torch.empty((max(ws_bytes, 256),), dtype=torch.uint8, device=q.device)
    dev = q.device
    out = dict(dq=torch.empty_like(q), dk=torch.empty_like(k), dv=torch.empty_like(v),
               dg=torch.empty(g.shape, dtype=torch.float32, device=dev),
               dbeta=torch.empty(beta.shape, dtype=torch.float32, device=dev),
               dh0=torch.empty((N, H, K, V), dtype=torch.float32, device=dev))
    gated = gate_kind in ("safe", "softplus")
    out["dA_log"] = torch.empty((H,), dtype=torch.float32, device=dev) if gated else None
    out["ddt_bias"] = torch.empty((H, K), dtype=torch.float32, device=dev) if gated and dt_bias is not None else None
    check(L.kda_chunk_bwd(ctypes.byref(a), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state),
                          _ptr(cu_seqlens), _ptr(do), _ptr(dht), _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]),
                          _ptr(out["dg"]), _ptr(out["dbeta"]), _ptr(out["dh0"]), _ptr(out["dA_log"]),
                          _ptr(out["ddt_bias"]), _ptr(ws), ctypes.c_size_t(ws.numel()), _stream()))
    return out


def workspace_bytes(q, v, H, N, chunk_size=64, schedule="auto", segment=0, gate_kind="safe"):
    a = make_args(q, v, H, N, gate_kind, chunk_size=chunk_size, schedule=schedule, segment=segment)
    return int(lib().kda_chunk_workspace_bytes(ctypes.byref(a)))


OFFSET_FLAGS = {1: "offsets decrease", 2: "first offset negative", 4: "last offset past the capacity"}


def check_offsets(cu_seqlens, T):
    """Flag bits of the packed-offset contract for capacity T (0: valid), checked on the
    device by kda_check_offsets; this wrapper synchronises to read the flag."""
    _require(cu_seqlens.is_cuda and cu_seqlens.dtype == torch.int32 and cu_seqlens.dim() == 1,
             "cu_seqlens must be a 1-D int32 device tensor")
    flags = torch.empty((1,), dtype=torch.int32, device=cu_seqlens.device)
    check(lib().kda_check_offsets(_ptr(cu_seqlens), cu_seqlens.numel() - 1, int(T), _ptr(flags), _stream()))
    return int(flags.item())


def resolved_schedule(q, v, H, N, chunk_size=64, schedule="auto"):
    """The schedule kda_chunk_fwd runs for these sizes ("staged", "fused" or "split"), or None."""
    a = make_args(q, v, H, N, "safe", chunk_size=chunk_size, schedule=schedule)
    r = int(lib().kda_chunk_schedule(ctypes.byref(a)))
    return {v_: k for k, v_ in SCHEDULES.items()}.get(r)


def resolved_segment(q, v, H, N, chunk_size=64, schedule="auto", segment=0):
    """Chunks per segment of the split schedule's state scan for these sizes (0: one
    serial chain per (sequence, head), or not the split schedule)."""
    a = make_args(q, v, H, N, "safe", chunk_size=chunk_size, schedule=schedule, segment=segment)
    return int(lib().kda_chunk_segment(ctypes.byref(a)))


STAGES = {"index": 0, "gate": 1, "grams": 2, "solve": 3, "wy": 4, "scan": 5, "output": 6}
WS_FIELDS = {"chunk_off": 0, "b": 1, "Akk": 2, "Aqk": 3, "T": 4, "w": 5, "u": 6, "vnew": 7, "hc": 8}


class StagedRun:
    """Drives the staged schedule one step at a time (include/kda_stages.h) on a
    workspace whose intermediates are exposed as fp32 tensor views."""

    def __init__(self, q, k, v, g, beta, initial_state=None, *, cu_seqlens=None, chunk_size=64,
                 gate_kind="safe", A_log=None, dt_bias=None, lower_bound=-5.0, scale=None, out=None,
                 final_state=None):
        B, T, H, K, V, N = _common(q, k, v, g, beta, initial_state, cu_seqlens, A_log, dt_bias)
        _check_outputs(out, final_state, B, T, H, K, V, N, q.dtype, q.device)
        self.t = dict(q=q, k=k, v=v, g=g, beta=beta, h0=initial_state, cu=cu_seqlens)
        self.o = out if out is not None else torch.empty((B, T, H, V), dtype=q.dtype, device=q.device)
        self.ht = final_state if final_state is not None else \
            torch.empty((N, H, K, V), dtype=torch.float32, device=q.device)
        self.args = make_args(q, v, H, N, gate_kind, chunk_size=chunk_size, scale=scale, A_log=A_log,
                              dt_bias=dt_bias, lower_bound=lower_bound, schedule="staged")
        self._keep = (A_log, dt_bias)
        L = lib()
        nbytes = int(L.kda_chunk_workspace_bytes(ctypes.byref(self.args)))
        self.ws = torch.zeros((nbytes,), dtype=torch.uint8, device=q.device)
        C = int(chunk_size)
        rows = B * T
        nch = max((T + C - 1) // C + N, B * ((T + C - 1) // C))
        D = 64 if max(K, V) <= 64 else (128 if max(K, V) <= 128 else 256)  # the kernels' tile width
        shapes = dict(b=(rows, H, D), Akk=(rows, H, C), Aqk=(rows, H, C), T=(rows, H, C), w=(rows, H, D),
                      u=(rows, H, D), vnew=(rows, H, D), hc=(nch, H, K, V))
        self.views = {}
        for name, shp in shapes.items():
            off = int(L.kda_staged_workspace_offset(ctypes.byref(self.args), WS_FIELDS[name]))
            n = 1
            for x in shp:
                n *= x
            self.views[name] = self.ws[off:off + 4 * n].view(torch.float32).view(shp)

    def run(self, stage):
        t = self.t
        check(lib().kda_chunk_stage(ctypes.byref(self.args), STAGES[stage], _ptr(t["q"]), _ptr(t["k"]), _ptr(t["v"]),
                                    _ptr(t["g"]), _ptr(t["beta"]), _ptr(t["h0"]), _ptr(t["cu"]), _ptr(self.o),
                                    _ptr(self.ht), _ptr(self.ws), ctypes.c_size_t(self.ws.numel()), _stream()))
