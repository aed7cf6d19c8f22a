"""kda_chunk_fwd_noalloc (the entry point that allocates nothing) against
kda_chunk_fwd on the same inputs: two calls in a row, the second smaller, on
the split schedule (whose key-side records and chunk prefix live in the static
array), then an AUTO shape whose split records would not fit (runs fused), and
a staged-only shape too large for the array (refused before any launch)."""
import numpy as np
import pytest
import torch

import kda_synth
from kda_testlib import need_gpu, parity

pytestmark = pytest.mark.gpu


def _dev(d):
    return {k: (v.cuda() if v is not None else None) for k, v in d.items()}


def _both(d, cu, schedule):
    from gated_delta_rule_gate_amd import chunk_kda, chunk_kda_noalloc

    dd = _dev(d)
    cu_d = None if cu is None else torch.from_numpy(np.asarray(cu, dtype=np.int32)).cuda()
    kw = dict(cu_seqlens=cu_d, gate_kind="safe", A_log=dd["A_log"], dt_bias=dd["dt_bias"], lower_bound=-5.0,
              schedule=schedule)
    o_ref, ht_ref = chunk_kda(dd["q"], dd["k"], dd["v"], dd["x"], dd["beta"], dd["h0"], output_final_state=True, **kw)
    out = torch.full_like(o_ref, float("nan"))
    ht = torch.full_like(ht_ref, float("nan"))
    chunk_kda_noalloc(dd["q"], dd["k"], dd["v"], dd["x"], dd["beta"], dd["h0"], out=out, final_state=ht, **kw)
    torch.cuda.synchronize()
    return (out.float().cpu().numpy(), ht.cpu().numpy()), (o_ref.float().cpu().numpy(), ht_ref.cpu().numpy())


def _check(got, want, end=None):
    (o, ht), (o_ref, ht_ref) = got, want
    if end is not None:
        o, o_ref = o[:, :end], o_ref[:, :end]
    parity(o, o_ref, "bf16", "o")
    parity(ht, ht_ref, "bf16", "ht")
    assert np.array_equal(o, o_ref) and np.array_equal(ht, ht_ref), "same kernels, same inputs: bit-equal"


def test_noalloc_split_twice_then_smaller():
    need_gpu()
    from gated_delta_rule_gate_amd import lib

    assert lib().kda_chunk_noalloc_max_bytes() == 64 << 20
    lens = [300, 0, 410, 77]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    d = kda_synth.chunk_inputs(1, int(cu[-1]) + 9, 4, 128, 128, dtype=torch.bfloat16, seed=3100, n_slots=len(lens))
    _check(*_both(d, cu, "split"), end=int(cu[-1]))
    # the second call is smaller: fewer slots, heads and tokens; the array keeps the
    # first call's records, which must not leak into this one
    lens2 = [100, 57]
    cu2 = np.concatenate([[0], np.cumsum(lens2)]).astype(np.int32)
    d2 = kda_synth.chunk_inputs(1, int(cu2[-1]), 2, 128, 128, dtype=torch.bfloat16, seed=3101, n_slots=len(lens2))
    _check(*_both(d2, cu2, "split"), end=int(cu2[-1]))
    # and a dense call after the packed ones
    d3 = kda_synth.chunk_inputs(2, 190, 3, 64, 64, dtype=torch.bfloat16, seed=3102)
    _check(*_both(d3, None, "split"))


def test_noalloc_auto_falls_back_to_fused():
    """Few long sequences: AUTO picks split, whose records (745 MB) exceed the
    64 MiB array; the no-allocation call runs the fused schedule instead."""
    need_gpu()
    from gated_delta_rule_gate_amd import resolved_schedule, workspace_bytes

    d = kda_synth.chunk_inputs(2, 16384, 16, 128, 128, dtype=torch.bfloat16, seed=3103)
    assert resolved_schedule(d["q"], d["v"], 16, 2) == "split"
    assert workspace_bytes(d["q"], d["v"], 16, 2) > (64 << 20)
    got, _ = _both(d, None, "fused")
    from gated_delta_rule_gate_amd import chunk_kda_noalloc

    dd = _dev(d)
    out = torch.full((2, 16384, 16, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    ht = torch.full((2, 16, 128, 128), float("nan"), dtype=torch.float32, device="cuda")
    chunk_kda_noalloc(dd["q"], dd["k"], dd["v"], dd["x"], dd["beta"], dd["h0"], out=out, final_state=ht,
                      gate_kind="safe", A_log=dd["A_log"], dt_bias=dd["dt_bias"], lower_bound=-5.0, schedule="auto")
    torch.cuda.synchronize()
    _check((out.float().cpu().numpy(), ht.cpu().numpy()), got)


def test_noalloc_refuses_oversized_workspace():
    """fp32 runs only the staged schedule, whose fp32 intermediates for this size
    exceed the array: refused with KDA_ERR_WORKSPACE before any launch."""
    need_gpu()
    from gated_delta_rule_gate_amd import KdaError, chunk_kda_noalloc, workspace_bytes

    d = kda_synth.chunk_inputs(1, 65536, 8, 64, 64, dtype=torch.float32, seed=3104)
    assert workspace_bytes(d["q"], d["v"], 8, 1) > (64 << 20)
    dd = _dev(d)
    out = torch.zeros((1, 65536, 8, 64), dtype=torch.float32, device="cuda")
    with pytest.raises(KdaError, match="WORKSPACE"):
        chunk_kda_noalloc(dd["q"], dd["k"], dd["v"], dd["x"], dd["beta"], dd["h0"], out=out, gate_kind="safe",
                          A_log=dd["A_log"], dt_bias=dd["dt_bias"], lower_bound=-5.0)
    torch.cuda.synchronize()
    assert float(out.abs().max()) == 0.0  # nothing ran
