"""GPU parity with beta given as raw logits (the sigmoid runs in the kernels).

"FLA KDA Skill", section "Correctness checklist": raw beta logits and
post-sigmoid beta. The oracle maps the same fp32 logits through its FP64
sigmoid (oracle.beta_from_logits) and runs the token recurrence. Logits are
N(0, 2) with every eleventh one at +-20, so some tokens have beta ~ 1 and some
~ 2e-9.
"""
import numpy as np
import pytest
import torch

import kda_synth
import oracle
from kda_testlib import f64, need_gpu, parity

pytestmark = pytest.mark.gpu


def _logits(shape, seed):
    rng = np.random.default_rng(seed)
    x = (2.0 * rng.standard_normal(shape)).astype(np.float32)
    flat = x.reshape(-1)
    flat[::11] = 20.0
    flat[5::11] = -20.0
    return torch.from_numpy(x)


@pytest.mark.parametrize("schedule,C", [(s_, c_) for s_ in ("fused", "split", "staged") for c_ in (64, 32)]
                         + [("pipe", 64)])
def test_chunk_beta_logits(schedule, C):
    from gated_delta_rule_gate_amd import chunk_kda

    need_gpu()
    d = kda_synth.chunk_inputs(2, 203, 3, 128, 128, dtype=torch.bfloat16, seed=1700 + C)
    d["beta"] = _logits(d["beta"].shape, 1701 + C)
    dd = {k: (v.cuda() if v is not None else None) for k, v in d.items()}
    o, ht = chunk_kda(dd["q"], dd["k"], dd["v"], dd["x"], dd["beta"], dd["h0"], output_final_state=True,
                      chunk_size=C, gate_kind="safe", A_log=dd["A_log"], dt_bias=dd["dt_bias"], lower_bound=-5.0,
                      schedule=schedule, beta_logits=True)
    torch.cuda.synchronize()
    g = oracle.gate(oracle.GATE_SAFE, f64(d["x"]), f64(d["A_log"]), f64(d["dt_bias"]), -5.0)
    o_ref, ht_ref = oracle.recurrent(f64(d["q"]), f64(d["k"]), f64(d["v"]), g,
                                     oracle.beta_from_logits(f64(d["beta"])), h0=f64(d["h0"]))
    parity(o.float().cpu().numpy(), o_ref, "bf16", "o")
    parity(ht.cpu().numpy(), ht_ref, "bf16", "ht")


def test_recurrent_beta_logits():
    from gated_delta_rule_gate_amd import recurrent_kda

    need_gpu()
    d = kda_synth.chunk_inputs(8, 64, 2, 128, 128, dtype=torch.bfloat16, seed=1710)
    d["g"] = kda_synth.log2_gate(d["x"].numpy(), d["A_log"].numpy(), d["dt_bias"].numpy())
    d["beta"] = _logits(d["beta"].shape, 1711)
    dd = {k: (v.cuda() if v is not None else None) for k, v in d.items()}
    o, ht = recurrent_kda(dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"], dd["h0"], output_final_state=True,
                          beta_logits=True)
    torch.cuda.synchronize()
    o_ref, ht_ref = oracle.recurrent(f64(d["q"]), f64(d["k"]), f64(d["v"]), f64(d["g"]),
                                     oracle.beta_from_logits(f64(d["beta"])), h0=f64(d["h0"]), g_is_log2=True)
    parity(o.float().cpu().numpy(), o_ref, "bf16", "o")
    parity(ht.cpu().numpy(), ht_ref, "bf16", "ht")
