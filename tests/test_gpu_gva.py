"""GPU parity with grouped value heads (GVA: more value heads than q/k heads).

"FLA KDA Skill", section "Correctness checklist", lists MHA and GVA (HV > H)
among the axes a change must cover. The pages fix no head mapping; the reading
here is contiguous groups: value head h uses q/k head h / (H / Hk), as
torch.repeat_interleave lays them out. v, g, beta, o and the states carry the H
value heads. The oracle runs the plain multi-head recurrence on q and k with
each head repeated for its group.
"""
import pytest
import torch

import kda_synth
import oracle
from kda_testlib import f64, need_gpu, parity

pytestmark = pytest.mark.gpu


def _case(B, T, H, Hk, D, seed, gate="safe"):
    d = kda_synth.chunk_inputs(B, T, H, D, D, dtype=torch.bfloat16, seed=seed)
    d["q"] = d["q"][:, :, :Hk].contiguous()  # the first Hk heads serve as the q/k heads
    d["k"] = d["k"][:, :, :Hk].contiguous()
    if gate == "log2":
        d["g"] = kda_synth.log2_gate(d["x"].numpy(), d["A_log"].numpy(), d["dt_bias"].numpy())
    return d


def _oracle(d, H, gate="safe"):
    G = H // d["q"].shape[2]
    q = f64(d["q"].repeat_interleave(G, dim=2))
    k = f64(d["k"].repeat_interleave(G, dim=2))
    if gate == "log2":
        return oracle.recurrent(q, k, f64(d["v"]), f64(d["g"]), f64(d["beta"]), h0=f64(d["h0"]), g_is_log2=True)
    g = oracle.gate(oracle.GATE_SAFE, f64(d["x"]), f64(d["A_log"]), f64(d["dt_bias"]), -5.0)
    return oracle.recurrent(q, k, f64(d["v"]), g, f64(d["beta"]), h0=f64(d["h0"]))


@pytest.mark.parametrize("schedule", ["fused", "split", "staged", "pipe"])
@pytest.mark.parametrize("Hk", [1, 2])
def test_chunk_gva(schedule, Hk):
    from gated_delta_rule_gate_amd import chunk_kda

    need_gpu()
    H = 4
    d = _case(2, 150, H, Hk, 128, 900 + Hk)
    dd = {k: (v.cuda() if v is not None else None) for k, v in d.items()}
    o, ht = chunk_kda(dd["q"], dd["k"], dd["v"], dd["x"], dd["beta"], dd["h0"], output_final_state=True,
                      gate_kind="safe", A_log=dd["A_log"], dt_bias=dd["dt_bias"], lower_bound=-5.0,
                      schedule=schedule)
    torch.cuda.synchronize()
    assert o.shape == (2, 150, H, 128) and ht.shape == (2, H, 128, 128)
    o_ref, ht_ref = _oracle(d, H)
    parity(o.float().cpu().numpy(), o_ref, "bf16", "o")
    parity(ht.cpu().numpy(), ht_ref, "bf16", "ht")


@pytest.mark.parametrize("Hk", [1, 2])
def test_recurrent_gva(Hk):
    from gated_delta_rule_gate_amd import recurrent_kda

    need_gpu()
    H = 4
    d = _case(8, 3, H, Hk, 128, 950 + Hk, gate="log2")
    dd = {k: (v.cuda() if v is not None else None) for k, v in d.items()}
    o, ht = recurrent_kda(dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"], dd["h0"], output_final_state=True)
    torch.cuda.synchronize()
    o_ref, ht_ref = _oracle(d, H, gate="log2")
    parity(o.float().cpu().numpy(), o_ref, "bf16", "o")
    parity(ht.cpu().numpy(), ht_ref, "bf16", "ht")


def test_gva_rejects_indivisible_heads():
    from gated_delta_rule_gate_amd import chunk_kda

    need_gpu()
    d = _case(1, 64, 3, 2, 128, 990)
    dd = {k: (v.cuda() if v is not None else None) for k, v in d.items()}
    with pytest.raises(ValueError):
        chunk_kda(dd["q"], dd["k"], dd["v"], dd["x"], dd["beta"], dd["h0"], A_log=dd["A_log"],
                  dt_bias=dd["dt_bias"])
