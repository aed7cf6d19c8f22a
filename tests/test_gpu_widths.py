"""GPU parity at head widths other than K = V in {64, 128, 256}.

"FLA KDA Skill", section "Correctness checklist", lists D != Dv among the
forward's axes, and "Add fused recurrent_kda ...", section "Test Plan", tests
non-power-of-two K/V masking. Widths here are multiples of 8 up to 256; the
kernels run in the next tile width (64, 128, 256) with the rest masked. The
oracle is the FP64 token recurrence at the real widths. Every case has a ragged
tail (T not a multiple of the chunk) and an initial state.
"""
import numpy as np
import pytest
import torch

import kda_synth
import oracle
from oracle.chunked import chunked_forward
from kda_testlib import f64, need_gpu, parity

pytestmark = pytest.mark.gpu

# (K, V): value side narrower, wider, both non-powers of two, a tile and a half,
# and one pair whose tile is 256 (the staged schedule only)
PAIRS = [(128, 64), (64, 128), (96, 96), (72, 120), (48, 200)]


def _gate(d):
    return oracle.gate(oracle.GATE_SAFE, f64(d["x"]), f64(d["A_log"]), f64(d["dt_bias"]), -5.0)


def _chunk(d, schedule, C=64, cu=None):
    from gated_delta_rule_gate_amd import chunk_kda

    dd = {k: (v.cuda() if v is not None else None) for k, v in d.items()}
    cu_d = None if cu is None else torch.from_numpy(np.asarray(cu, dtype=np.int32)).cuda()
    o, ht = chunk_kda(dd["q"], dd["k"], dd["v"], dd["x"], dd["beta"], dd["h0"], cu_seqlens=cu_d,
                      output_final_state=True, chunk_size=C, gate_kind="safe", A_log=dd["A_log"],
                      dt_bias=dd["dt_bias"], lower_bound=-5.0, schedule=schedule)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), ht.cpu().numpy()


@pytest.mark.parametrize("schedule,K,V", [(s_, k_, v_) for s_ in ("auto", "split", "staged") for k_, v_ in PAIRS]
                         + [("pipe", k_, v_) for k_, v_ in PAIRS if 64 < max(k_, v_) <= 128] + [("pipe", 80, 128)])
def test_chunk_widths(schedule, K, V):
    need_gpu()
    B, T, H = 2, 203, 2
    d = kda_synth.chunk_inputs(B, T, H, K, V, dtype=torch.bfloat16, seed=1200 + K + V)
    if schedule == "split" and max(K, V) > 128:
        from gated_delta_rule_gate_amd import KdaError

        with pytest.raises(KdaError, match="UNSUPPORTED"):  # its tiles stop at 128
            _chunk(d, schedule)
        return
    o, ht = _chunk(d, schedule)
    assert o.shape == (B, T, H, V) and ht.shape == (B, H, K, V)
    o_ref, ht_ref = oracle.recurrent(f64(d["q"]), f64(d["k"]), f64(d["v"]), _gate(d), f64(d["beta"]),
                                     h0=f64(d["h0"]))
    parity(o, o_ref, "bf16", "o")
    parity(ht, ht_ref, "bf16", "ht")


@pytest.mark.parametrize("K,V", [(128, 64), (96, 96)])
def test_chunk_widths_fp32(K, V):
    need_gpu()
    d = kda_synth.chunk_inputs(1, 150, 2, K, V, dtype=torch.float32, seed=1300 + K + V)
    o, ht = _chunk(d, "auto", C=32)
    o_ref, ht_ref = oracle.recurrent(f64(d["q"]), f64(d["k"]), f64(d["v"]), _gate(d), f64(d["beta"]),
                                     h0=f64(d["h0"]))
    parity(o, o_ref, "fp32", "o")
    parity(ht, ht_ref, "fp32", "ht")


@pytest.mark.parametrize("schedule", ["auto", "split", "staged", "pipe"])
def test_chunk_widths_packed_states(schedule):
    """K != V, packed with an empty slot and few (sequence, head) pairs, with the
    chunk-start states in the [K, V] layout of h0."""
    from gated_delta_rule_gate_amd import chunk_kda

    need_gpu()
    K, V, H, SLOTS, CAP, C = 96, 64, 2, 4, 330, 64
    cu = kda_synth.varlen_offsets(131, n_slots=SLOTS, n_empty=1, total=300, max_len=CAP)
    d = kda_synth.chunk_inputs(1, CAP, H, K, V, dtype=torch.bfloat16, seed=131, n_slots=SLOTS)
    dd = {k: (v.cuda() if v is not None else None) for k, v in d.items()}
    cu_d = torch.from_numpy(np.asarray(cu, dtype=np.int32)).cuda()
    o, ht, hs = chunk_kda(dd["q"], dd["k"], dd["v"], dd["x"], dd["beta"], dd["h0"], cu_seqlens=cu_d,
                          output_final_state=True, chunk_size=C, gate_kind="safe", A_log=dd["A_log"],
                          dt_bias=dd["dt_bias"], lower_bound=-5.0, schedule=schedule,
                          return_intermediate_states=True)
    torch.cuda.synchronize()
    o_ref, ht_ref, it = chunked_forward(f64(d["q"]), f64(d["k"]), f64(d["v"]), _gate(d), f64(d["beta"]),
                                        h0=f64(d["h0"]), cu_seqlens=cu, chunk_size=C, emit=True)
    n = int(cu[-1])
    nch = it["hc"].shape[0]
    parity(o.float().cpu().numpy()[:, :n], o_ref[:, :n], "bf16", "o")
    parity(ht.cpu().numpy(), ht_ref, "bf16", "ht")
    parity(hs.cpu().numpy()[0, :nch], it["hc"], "bf16", "h_states")


@pytest.mark.parametrize("T", [1, 64])
@pytest.mark.parametrize("K,V", [(96, 96), (128, 64), (72, 200), (256, 136)])
def test_recurrent_widths(T, K, V):
    from gated_delta_rule_gate_amd import recurrent_kda

    need_gpu()
    N, H = 8, 2
    d = kda_synth.chunk_inputs(N, T, H, K, V, dtype=torch.bfloat16, seed=1400 + K + V + T)
    d["g"] = kda_synth.log2_gate(d["x"].numpy(), d["A_log"].numpy(), d["dt_bias"].numpy())
    dd = {k: (v.cuda() if v is not None else None) for k, v in d.items()}
    o, ht = recurrent_kda(dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"], dd["h0"], output_final_state=True)
    torch.cuda.synchronize()
    o_ref, ht_ref = oracle.recurrent(f64(d["q"]), f64(d["k"]), f64(d["v"]), f64(d["g"]), f64(d["beta"]),
                                     h0=f64(d["h0"]), g_is_log2=True)
    parity(o.float().cpu().numpy(), o_ref, "bf16", "o")
    parity(ht.cpu().numpy(), ht_ref, "bf16", "ht")
