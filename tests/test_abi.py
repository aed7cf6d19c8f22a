"""CPU checks of the C ABI: the library loads, exports every declared entry point,
and rejects invalid arguments with the documented status codes before launching."""
import ctypes
import glob
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def kda_lib():
    from gated_delta_rule_gate_amd import _binding, build

    if not os.path.exists(_binding.LIB_PATH):
        build.build()
    return _binding.lib()


def _declared():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^[A-Za-z_][\w \*]*?\b(kda_\w+)\s*\(", text, flags=re.M):
            names.add(m.group(1))
    return sorted(names)


def test_headers_declare_entry_points():
    names = _declared()
    for required in ("kda_chunk_fwd", "kda_recurrent_fwd", "kda_chunk_workspace_bytes", "kda_status_string"):
        assert required in names, required


def test_every_declared_symbol_is_exported(kda_lib):
    missing = [n for n in _declared() if not hasattr(kda_lib, n)]
    assert not missing, missing


def test_status_strings(kda_lib):
    for code in range(10):
        s = kda_lib.kda_status_string(code).decode()
        assert s.startswith("KDA_")


def _args(**kw):
    from gated_delta_rule_gate_amd._binding import KdaArgs

    a = KdaArgs()
    a.B, a.T, a.H, a.K, a.V, a.N = 1, 64, 1, 128, 128, 1
    a.chunk_size, a.dtype, a.scale, a.gate_kind = 64, 0, 0.0, 4
    a.lower_bound, a.schedule = -5.0, 0
    for k, v in kw.items():
        setattr(a, k, v)
    return a


FAKE = ctypes.c_void_p(0x100000)  # aligned, never dereferenced: validation fails before any launch


@pytest.mark.parametrize("kw,code", [
    (dict(), 1),                       # NULL q
    (dict(dtype=7), 3),
    (dict(gate_kind=9), 5),
    (dict(gate_kind=1), 5),            # SAFE without A_log
    (dict(K=44), 8),                   # widths are multiples of 8
    (dict(K=264), 8),                  # ... up to 256
    (dict(V=0), 2),
    (dict(B=2, N=1), 2),               # dense needs N == B
    (dict(H=0), 2),
    (dict(q_l2norm=2), 2),             # the q_l2norm flag is 0 or 1
    (dict(beta_logits=-1), 2),         # so is beta_logits
    (dict(H=3, Hk=2), 2),              # value heads must be a multiple of the q/k heads
    (dict(H=4097), 2),                 # at most 4096 heads per call
])
def test_recurrent_rejects(kda_lib, kw, code):
    a = _args(**kw)
    null_q = not kw
    q = None if null_q else FAKE
    st = kda_lib.kda_recurrent_fwd(ctypes.byref(a), q, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, None, None)
    assert st == code, (kw, st)


def test_misaligned_pointer_rejected(kda_lib):
    a = _args()
    bad = ctypes.c_void_p(0x100002)
    st = kda_lib.kda_recurrent_fwd(ctypes.byref(a), bad, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, None, None)
    assert st == 6


def test_safe_lower_bound_range(kda_lib):
    for lb, code in ((-5.5, 5), (0.0, 5), (0.5, 5)):
        a = _args(gate_kind=1, A_log=0x100000, lower_bound=lb)
        st = kda_lib.kda_recurrent_fwd(ctypes.byref(a), FAKE, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, None, None)
        assert st == code, lb


FAKE2 = ctypes.c_void_p(0x40000000)  # a second aligned address far from FAKE (no overlap)


@pytest.mark.parametrize("kw,chunk,code", [
    (dict(gate_kind=0), 16, 4),                 # chunk size not in {1, 32, 64}
    (dict(gate_kind=3), 64, 5),                 # a pre-cumsummed gate is no input here
    (dict(gate_kind=2), 64, 5),                 # SOFTPLUS without A_log
    (dict(gate_kind=0, K=44), 64, 8),
    (dict(gate_kind=0, B=2, N=1), 64, 2),
    (dict(gate_kind=0, H=4097), 64, 2),        # at most 4096 heads per call
])
def test_gate_cumsum_rejects(kda_lib, kw, chunk, code):
    a = _args(**kw)
    st = kda_lib.kda_gate_cumsum(ctypes.byref(a), FAKE, None, chunk, FAKE2, None)
    assert st == code, (kw, st)


def test_gate_cumsum_rejects_overlap_and_null(kda_lib):
    a = _args(gate_kind=0)
    assert kda_lib.kda_gate_cumsum(ctypes.byref(a), FAKE, None, 64, FAKE, None) == 2
    assert kda_lib.kda_gate_cumsum(ctypes.byref(a), None, None, 64, FAKE2, None) == 1
    assert kda_lib.kda_gate_cumsum(None, FAKE, None, 64, FAKE2, None) == 1


@pytest.mark.parametrize("kw,code", [
    (dict(gate_kind=4), 5),                    # per-token log2 gate is the recurrent contract
    (dict(gate_kind=0, chunk_size=16), 4),
    (dict(gate_kind=0, V=12), 8),              # widths are multiples of 8
    (dict(gate_kind=0, K=52, V=48), 8),
    (dict(gate_kind=0, H=4097), 2),            # at most 4096 heads per call
])
def test_chunk_rejects(kda_lib, kw, code):
    a = _args(**kw)
    st = kda_lib.kda_chunk_fwd(ctypes.byref(a), FAKE, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, None,
                               FAKE2, ctypes.c_size_t(1 << 30), None)
    assert st == code, (kw, st)


def test_recurrent_rejects_precumsummed_gate(kda_lib):
    a = _args(gate_kind=3)
    st = kda_lib.kda_recurrent_fwd(ctypes.byref(a), FAKE, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, None, None)
    assert st == 5


def test_chunk_states_count(kda_lib):
    """Entries of the chunk-start states: B * ceil(T / C) dense, ceil(T / C) + N packed."""
    a = _args(gate_kind=0, B=3, N=3, T=203)
    assert kda_lib.kda_chunk_states_count(ctypes.byref(a), 0) == 3 * 4
    assert kda_lib.kda_chunk_states_count(ctypes.byref(a), 1) == 0  # packed needs B == 1
    a = _args(gate_kind=0, B=1, N=5, T=420, chunk_size=32)
    assert kda_lib.kda_chunk_states_count(ctypes.byref(a), 1) == 14 + 5
    assert kda_lib.kda_chunk_states_count(ctypes.byref(a), 0) == 0  # dense needs N == B
    assert kda_lib.kda_chunk_states_count(ctypes.byref(_args(gate_kind=0, V=68)), 0) == 0  # V % 8 != 0


def test_chunk_states_rejects(kda_lib):
    a = _args(gate_kind=0)
    call = lambda hs: kda_lib.kda_chunk_fwd_states(ctypes.byref(a), FAKE, FAKE, FAKE, FAKE, FAKE, None, None, FAKE,
                                                   None, hs, FAKE2, ctypes.c_size_t(1 << 30), None)
    assert call(None) == 1                          # states wanted but no buffer
    assert call(ctypes.c_void_p(0x100004)) == 6     # misaligned
    a.chunk_size = 16
    assert call(FAKE) == 4                          # the checks of kda_chunk_fwd come first


def _bwd(kda_lib, a, **ptr):
    args = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, h0=None, cu=None, do=FAKE, dht=None, dq=FAKE2, dk=FAKE2,
                dv=FAKE2, dg=FAKE2, dbeta=FAKE2, dh0=None, dA=None, ddt=None, ws=FAKE2)
    args.update(ptr)
    return kda_lib.kda_chunk_bwd(ctypes.byref(a), args["q"], args["k"], args["v"], args["g"], args["beta"],
                                 args["h0"], args["cu"], args["do"], args["dht"], args["dq"], args["dk"], args["dv"],
                                 args["dg"], args["dbeta"], args["dh0"], args["dA"], args["ddt"], args["ws"],
                                 ctypes.c_size_t(1 << 40), None)


def test_chunk_bwd_rejects(kda_lib):
    """The backward's own limits, checked before any launch."""
    ok = dict(gate_kind=0)
    assert _bwd(kda_lib, _args(**ok), do=None) == 1             # d_o required
    assert _bwd(kda_lib, _args(**ok), dg=None) == 1             # gradients required
    assert _bwd(kda_lib, _args(**ok), dq=ctypes.c_void_p(0x40000004)) == 6
    assert _bwd(kda_lib, _args(gate_kind=3)) == 8                # pre-cumsummed gate
    assert _bwd(kda_lib, _args(gate_kind=0, q_l2norm=1)) == 8    # forward-only option
    assert _bwd(kda_lib, _args(gate_kind=0, H=4, Hk=2)) == 8     # grouped value heads
    assert _bwd(kda_lib, _args(gate_kind=0, K=256, V=256)) == 8  # tile wider than 128
    assert _bwd(kda_lib, _args(gate_kind=0, chunk_size=16)) == 4
    assert kda_lib.kda_chunk_bwd_workspace_bytes(ctypes.byref(_args(gate_kind=0, K=256, V=256))) == 0
    assert kda_lib.kda_chunk_bwd_workspace_bytes(ctypes.byref(_args(gate_kind=0))) > 0
    # more heads than one call takes: no workspace size, and the call itself is refused
    assert kda_lib.kda_chunk_bwd_workspace_bytes(ctypes.byref(_args(gate_kind=0, H=4097))) == 0
    assert kda_lib.kda_chunk_workspace_bytes(ctypes.byref(_args(gate_kind=0, H=4097))) == 0
    assert _bwd(kda_lib, _args(gate_kind=0, H=4097)) == 2


def test_split_schedule_limits_and_workspace(kda_lib):
    """The split schedule: bf16 and tiles up to 128 only, a schedule value past
    the enumeration rejected, and a workspace that holds the chunk prefix and, per
    (chunk, head) of the larger of the dense and packed chunk bounds, the bf16
    operands q~, k~, w^T (C*D each) and A_qk (C*C) and the fp32 u (C*D), 2^b_L
    (D) and row scales (C)."""
    call = lambda a: kda_lib.kda_chunk_fwd(ctypes.byref(a), FAKE, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, None,
                                           FAKE2, ctypes.c_size_t(1 << 40), None)
    assert call(_args(gate_kind=0, schedule=3, dtype=1)) == 8            # fp32
    assert call(_args(gate_kind=0, schedule=3, K=256, V=256)) == 8       # tile 256
    assert call(_args(gate_kind=0, schedule=5)) == 2                     # no such schedule
    assert call(_args(gate_kind=0, schedule=4)) == 8                     # the pipelined kernel: safe gate only
    align = lambda x: (x + 255) // 256 * 256
    for B, N, T, H, K, V, C in ((3, 3, 203, 2, 128, 128, 64), (1, 5, 420, 4, 96, 64, 32)):
        D = 64 if max(K, V) <= 64 else 128
        nt = (T + C - 1) // C
        nch = max(B * nt, nt + N)
        per = 2 * (3 * C * D + C * C) + 4 * (C * D + D + C)
        serial = align(4 * (N + 1)) + align(nch * H * per)
        a = _args(gate_kind=0, schedule=3, B=B, N=N, T=T, H=H, K=K, V=V, chunk_size=C, segment=-1)
        assert kda_lib.kda_chunk_workspace_bytes(ctypes.byref(a)) == serial
        assert kda_lib.kda_chunk_segment(ctypes.byref(a)) == 0
        # segments of 3 chunks add the segment prefix, E (bf16) and o_local (fp32) per
        # (chunk, head), and [M | B] (fp32, D x 2D) plus the incoming state (bf16, D x D)
        # per (segment, head) of the larger of the dense and packed segment bounds
        a = _args(gate_kind=0, schedule=3, B=B, N=N, T=T, H=H, K=K, V=V, chunk_size=C, segment=3)
        nseg = max(B * max(1, (nt + 2) // 3), N + (nt + N + 2) // 3)
        seg = align(4 * (N + 1)) + align(nch * H * C * D * 6 + nseg * H * D * D * 10)
        assert kda_lib.kda_chunk_workspace_bytes(ctypes.byref(a)) == serial + seg
        assert kda_lib.kda_chunk_segment(ctypes.byref(a)) == 3
    assert kda_lib.kda_chunk_workspace_bytes(ctypes.byref(_args(gate_kind=0, schedule=3, dtype=1))) == 0
    # the segment length applies to the split schedule only
    assert kda_lib.kda_chunk_segment(ctypes.byref(_args(gate_kind=0, schedule=2, segment=3))) == 0


def test_resolved_schedule(kda_lib):
    """What AUTO runs: fused for one (sequence, head) pair per compute unit, split
    for few pairs with long sequences, staged for fp32 or tiles past 128; a named
    schedule that cannot take the arguments resolves to -1. (Without a device the
    library assumes 256 compute units.)"""
    sched = lambda **kw: kda_lib.kda_chunk_schedule(ctypes.byref(_args(gate_kind=0, **kw)))
    assert sched(B=4, N=4, T=4096, H=64) == 2
    assert sched(B=2, N=2, T=16384, H=16) == 3
    assert sched(B=2, N=2, T=16384, H=16, dtype=1) == 1
    assert sched(B=2, N=2, T=16384, H=16, K=256, V=256) == 2                   # fused at 32-row chunks
    # a gate the caller cumsummed over 64-row chunks cannot switch to 32-row chunks
    assert kda_lib.kda_chunk_schedule(ctypes.byref(_args(gate_kind=3, B=2, N=2, T=16384, H=16, K=256, V=256))) == 1
    assert sched(B=2, N=2, T=16384, H=16, K=256, V=256, dtype=1) == 1          # fp32: staged
    assert sched(B=2, N=2, T=16384, H=16, K=256, V=256, chunk_size=32, schedule=2) == 2
    assert sched(B=2, N=2, T=16384, H=16, K=256, V=256, schedule=2) == -1      # named fused: 32-row chunks only
    assert sched(B=4, N=4, T=4096, H=64, schedule=3) == 3
    assert sched(B=2, N=2, T=16384, H=16, schedule=2) == 2
    assert sched(dtype=1, schedule=2) == -1
    assert sched(K=256, V=256, schedule=3) == -1
    assert sched(chunk_size=16) == -1
    # the pipelined kernel (safe gate, bf16, chunk 64, tile 128): what AUTO runs for more
    # (sequence, head) pairs than half the compute units; named, on any count; a named
    # fused schedule runs the fused kernel
    safe = lambda **kw: kda_lib.kda_chunk_schedule(ctypes.byref(_args(gate_kind=1, **kw)))
    assert safe(B=4, N=4, T=4096, H=64) == 4
    assert safe(B=4, N=4, T=4096, H=64, schedule=2) == 2
    assert safe(B=4, N=4, T=4096, H=64, K=96, V=72) == 4
    assert safe(B=1, N=1, T=300, H=2, schedule=4) == 4
    assert safe(B=1, N=1, T=300, H=2, schedule=2) == 2
    assert safe(B=4, N=4, T=4096, H=64, chunk_size=32) == 2
    assert safe(B=4, N=4, T=4096, H=64, K=64, V=64) == 2
    assert safe(B=2, N=2, T=16384, H=16) == 3
    assert safe(schedule=4, chunk_size=32) == -1
    assert safe(schedule=4, K=64, V=64) == -1
    assert safe(schedule=4, dtype=1) == -1
    assert safe(schedule=5) == -1
    a = _args(gate_kind=0, B=2, N=2, T=16384, H=16)
    b = _args(gate_kind=0, B=2, N=2, T=16384, H=16, schedule=3)
    assert kda_lib.kda_chunk_workspace_bytes(ctypes.byref(a)) == kda_lib.kda_chunk_workspace_bytes(ctypes.byref(b))


def test_check_offsets_rejects(kda_lib):
    """kda_check_offsets: NULL offsets or flags, negative N or T, checked before any launch."""
    assert kda_lib.kda_check_offsets(None, 3, 100, FAKE2, None) == 1
    assert kda_lib.kda_check_offsets(FAKE, 3, 100, None, None) == 1
    assert kda_lib.kda_check_offsets(FAKE, -1, 100, FAKE2, None) == 2
    assert kda_lib.kda_check_offsets(FAKE, 3, -5, FAKE2, None) == 2


def test_binding_rejects_bad_outputs():
    """Caller-supplied o and final-state buffers are checked before any pointer
    reaches the library: wrong shape, dtype, layout or device raise."""
    import torch

    from gated_delta_rule_gate_amd._binding import _check_outputs

    B, T, H, K, V, N = 2, 5, 3, 8, 16, 2
    cpu = torch.device("cpu")
    bad_out = [torch.empty((B, T, H, V + 1), dtype=torch.bfloat16),
               torch.empty((B, T, H, V), dtype=torch.float32),
               torch.empty((B, T, V, H), dtype=torch.bfloat16).transpose(2, 3)]
    for o in bad_out:
        with pytest.raises(ValueError):
            _check_outputs(o, None, B, T, H, K, V, N, torch.bfloat16, cpu)
    bad_ht = [torch.empty((N, H, K, V + 8), dtype=torch.float32),
              torch.empty((N, H, K, V), dtype=torch.bfloat16),
              torch.empty((N, H, V, K), dtype=torch.float32).transpose(2, 3)]
    for ht in bad_ht:
        with pytest.raises(ValueError):
            _check_outputs(None, ht, B, T, H, K, V, N, torch.bfloat16, cpu)
    # right shapes on the wrong device (host memory) are refused too
    with pytest.raises(ValueError):
        _check_outputs(torch.empty((B, T, H, V), dtype=torch.bfloat16), None, B, T, H, K, V, N, torch.bfloat16,
                       torch.device("cuda", 0))
