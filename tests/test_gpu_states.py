"""GPU parity of the chunk-start states (return_intermediate_states).

"FLA KDA Skill", section "Correctness checklist", names return_intermediate_states
among the forward's axes. The reading here: the fp32 state entering each chunk,
chunks numbered slot by slot. The oracle is the FP64 chunked form with its
intermediates (oracle.chunked.chunked_forward, emit=True), whose chunk-start
states are pinned on the CPU to the token recurrence run over each prefix.
Asking for the states must not change o or ht: both equal a plain call bit for
bit. A slot's first chunk holds h0 bit for bit; entries past the last chunk of a
packed batch keep what the caller put there.
"""
import numpy as np
import pytest
import torch

import kda_synth
import oracle
from oracle.chunked import chunked_forward
from kda_testlib import f64, need_gpu, parity

pytestmark = pytest.mark.gpu


def _oracle(d, C, cu=None):
    g = oracle.gate(oracle.GATE_SAFE, f64(d["x"]), f64(d["A_log"]), f64(d["dt_bias"]), -5.0)
    h0 = None if d["h0"] is None else f64(d["h0"])
    return chunked_forward(f64(d["q"]), f64(d["k"]), f64(d["v"]), g, f64(d["beta"]), h0=h0, cu_seqlens=cu,
                           chunk_size=C, emit=True)


def _run(d, schedule, C, cu=None, states=True, prefill=None):
    from gated_delta_rule_gate_amd import chunk_kda

    dd = {k: (v.cuda() if v is not None else None) for k, v in d.items()}
    cu_d = None if cu is None else torch.from_numpy(np.asarray(cu, dtype=np.int32)).cuda()
    kw = dict(cu_seqlens=cu_d, output_final_state=True, chunk_size=C, gate_kind="safe", A_log=dd["A_log"],
              dt_bias=dd["dt_bias"], lower_bound=-5.0, schedule=schedule)
    if states:
        kw["return_intermediate_states"] = True
        if prefill is not None:
            kw["intermediate_states"] = prefill.cuda()
    res = chunk_kda(dd["q"], dd["k"], dd["v"], dd["x"], dd["beta"], dd["h0"], **kw)
    torch.cuda.synchronize()
    return [None if r is None else r.float().cpu() for r in res]


@pytest.mark.parametrize("schedule,D,C", [(s_, d_, c_) for s_ in ("fused", "split", "staged")
                                          for d_, c_ in ((128, 64), (128, 32), (64, 64))] + [("pipe", 128, 64)])
def test_dense_states(schedule, D, C):
    need_gpu()
    B, T, H = 2, 203, 3
    d = kda_synth.chunk_inputs(B, T, H, D, D, dtype=torch.bfloat16, seed=1100 + D + C)
    o, ht, hs = _run(d, schedule, C)
    NT = (T + C - 1) // C
    assert hs.shape == (B, NT, H, D, D)
    o_ref, ht_ref, it = _oracle(d, C)
    parity(hs.numpy().reshape(B * NT, H, D, D), it["hc"], "bf16", "h_states")
    parity(o.numpy(), o_ref, "bf16", "o")
    parity(ht.numpy(), ht_ref, "bf16", "ht")
    # each sequence's first chunk holds h0 exactly
    assert torch.equal(hs[:, 0], d["h0"].float())
    # the states leave o and ht as a plain call computes them
    o2, ht2 = _run(d, schedule, C, states=False)
    assert torch.equal(o, o2) and torch.equal(ht, ht2)


@pytest.mark.parametrize("schedule", ["fused", "split", "staged", "pipe"])
def test_packed_states_with_empty_slots(schedule):
    """Five slots, one empty, two (sequence, head) pairs per slot: the fused
    kernel also splits the value columns. Entries past the last chunk keep the
    caller's NaN fill."""
    need_gpu()
    C, H, D, SLOTS, CAP = 64, 2, 128, 5, 420
    cu = kda_synth.varlen_offsets(113, n_slots=SLOTS, n_empty=1, total=400, max_len=CAP)
    d = kda_synth.chunk_inputs(1, CAP, H, D, D, dtype=torch.bfloat16, seed=113, n_slots=SLOTS)
    count = (CAP + C - 1) // C + SLOTS
    fill = torch.full((1, count, H, D, D), float("nan"))
    o, ht, hs = _run(d, schedule, C, cu=cu, prefill=fill)
    o_ref, ht_ref, it = _oracle(d, C, cu=cu)
    nch = it["hc"].shape[0]
    assert nch == sum((int(cu[n + 1]) - int(cu[n]) + C - 1) // C for n in range(SLOTS))
    parity(hs[0, :nch].numpy(), it["hc"], "bf16", "h_states")
    assert torch.isnan(hs[0, nch:]).all(), "entries past the last chunk were written"
    n_valid = int(cu[-1])
    parity(o[:, :n_valid].numpy(), o_ref[:, :n_valid], "bf16", "o")
    parity(ht.numpy(), ht_ref, "bf16", "ht")
    # slot starts hold h0 bit for bit
    j = 0
    for n in range(SLOTS):
        L = int(cu[n + 1]) - int(cu[n])
        if L > 0:
            assert torch.equal(hs[0, j], d["h0"][n].float())
        j += (L + C - 1) // C


def test_states_without_h0_start_at_zero():
    need_gpu()
    C, D = 64, 128
    d = kda_synth.chunk_inputs(1, 150, 2, D, D, dtype=torch.bfloat16, seed=117)
    d["h0"] = None
    o, ht, hs = _run(d, "fused", C)
    assert torch.equal(hs[:, 0], torch.zeros_like(hs[:, 0]))
    _, _, it = _oracle(d, C)
    parity(hs.numpy().reshape(-1, 2, D, D), it["hc"], "bf16", "h_states")
