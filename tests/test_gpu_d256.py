"""GPU parity of the fused schedule at tile width 256 (K, V up to 256), which runs
32-row chunks: one wave per 16-column tile, sixteen waves per (sequence, head).

The widths of the contract shape B8 T2048 H32 D256 ("[examples] Read only the
causal columns ...", Benchmarks, forward table), gate modes of "FLA KDA Skill",
section "Gate modes", ragged tails, packed slots with empty ones, non-power-of-two
widths inside the 256 tile, and the value-column split that few pairs take.
"""
import numpy as np
import pytest
import torch

import kda_synth
import oracle
from kda_testlib import f64, need_gpu, parity
from test_gpu_chunk import gpu_run, make, oracle_run

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("gate", ["safe", "softplus", "loge"])
def test_fused_d256_gates(gate):
    need_gpu()
    d = make(2, 150, 3, 256, torch.bfloat16, 2560, gate=gate)
    o, ht = gpu_run(d, gate, "fused", C=32)
    o_ref, ht_ref = oracle_run(d, gate)
    parity(o, o_ref, "bf16", "o")
    parity(ht, ht_ref, "bf16", "ht")


@pytest.mark.parametrize("K,V", [(256, 136), (200, 256), (136, 176)])
def test_fused_d256_widths(K, V):
    """Widths inside the 256 tile, masked; the oracle runs at the real widths."""
    from gated_delta_rule_gate_amd import chunk_kda

    need_gpu()
    d = kda_synth.chunk_inputs(2, 97, 2, K, V, dtype=torch.bfloat16, seed=2570 + K + V)
    dd = {k: (v.cuda() if v is not None else None) for k, v in d.items()}
    o, ht = chunk_kda(dd["q"], dd["k"], dd["v"], dd["x"], dd["beta"], dd["h0"], output_final_state=True,
                      chunk_size=32, gate_kind="safe", A_log=dd["A_log"], dt_bias=dd["dt_bias"], lower_bound=-5.0,
                      schedule="fused")
    torch.cuda.synchronize()
    g = oracle.gate(oracle.GATE_SAFE, f64(d["x"]), f64(d["A_log"]), f64(d["dt_bias"]), -5.0)
    o_ref, ht_ref = oracle.recurrent(f64(d["q"]), f64(d["k"]), f64(d["v"]), g, f64(d["beta"]), h0=f64(d["h0"]))
    parity(o.float().cpu().numpy(), o_ref, "bf16", "o")
    parity(ht.cpu().numpy(), ht_ref, "bf16", "ht")


def test_fused_d256_packed():
    """Packed slots, empty ones passing their state through bit for bit; one pair per
    slot and head, so few pairs: the value columns split over several workgroups."""
    need_gpu()
    lens = [0, 70, 33, 1, 0, 129]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    cap = int(cu[-1]) + 11
    d = make(1, cap, 2, 256, torch.bfloat16, 2580, n_slots=len(lens))
    o, ht = gpu_run(d, "safe", "fused", cu=cu, C=32)
    o_ref, ht_ref = oracle_run(d, "safe", cu=cu)
    parity(o[:, : int(cu[-1])], o_ref[:, : int(cu[-1])], "bf16", "o")
    parity(ht, ht_ref, "bf16", "ht")
    h0 = d["h0"].numpy()
    for n, L in enumerate(lens):
        if L == 0:
            assert np.array_equal(ht[n].view(np.uint32), h0[n].view(np.uint32))


def test_fused_d256_chunk_states():
    """The chunk-start states at 32-row chunks against the oracle's chunked form,
    which emits them; o and ht as well."""
    from gated_delta_rule_gate_amd import chunk_kda
    from oracle.chunked import chunked_forward

    need_gpu()
    B, T, H, D, C = 1, 100, 2, 256, 32
    d = make(B, T, H, D, torch.bfloat16, 2590)
    dd = {k: (v.cuda() if v is not None else None) for k, v in d.items()}
    o, ht, hs = chunk_kda(dd["q"], dd["k"], dd["v"], dd["x"], dd["beta"], dd["h0"], output_final_state=True,
                          chunk_size=C, gate_kind="safe", A_log=dd["A_log"], dt_bias=dd["dt_bias"],
                          lower_bound=-5.0, schedule="fused", return_intermediate_states=True)
    torch.cuda.synchronize()
    g = oracle.gate(oracle.GATE_SAFE, f64(d["x"]), f64(d["A_log"]), f64(d["dt_bias"]), -5.0)
    o_ref, ht_ref, it = chunked_forward(f64(d["q"]), f64(d["k"]), f64(d["v"]), g, f64(d["beta"]),
                                        h0=f64(d["h0"]), chunk_size=C, emit=True)
    NT = (T + C - 1) // C
    parity(hs.cpu().numpy().reshape(B * NT, H, D, D), it["hc"], "bf16", "h_states")
    parity(o.float().cpu().numpy(), o_ref, "bf16", "o")
    parity(ht.cpu().numpy(), ht_ref, "bf16", "ht")
