"""GPU parity at the gate's numerical extremes.

"FLA KDA Skill", section "Correctness checklist", asks for these whenever the
gate or the decay math changes: lower_bound -5 and close to 0, large positive
and negative g + dt_bias, extreme A_log, long cumulative decay, chunk and
ragged varlen boundaries. Heads here span exp(A_log) from 1e-3 to 1e3, and the
raw gate input holds stretches saturated at +-30 between N(0, 1) stretches, so
per-token decays run from none to the bound (safe gate) or far past it
(softplus, whose decay is unbounded). The oracle evaluates the same gates in
FP64.

The chunk path keeps the chunk-local cumsum b in FP32, as the pages' kernels do
("FLA KDA Skill", section "Safe gate numerical note"). An unbounded softplus
decay of ~1e6 per token would leave b ~ 1e8 within a chunk, where FP32 spacing
(~8) swamps the small per-pair differences, so the chunk-path softplus heads
stop at exp(A_log) = 16 (decays up to ~700 per token in log2, b spacing below
0.01). The recurrent kernel exponentiates each token's decay on its own and
takes the full range.
"""
import numpy as np
import pytest
import torch

import kda_synth
import oracle
from kda_testlib import f64, need_gpu, parity

pytestmark = pytest.mark.gpu

H, D = 4, 128
A_LOG = {"wide": np.log(np.array([1e-3, 1.0, 16.0, 1e3])).astype(np.float32),
         "chunk_softplus": np.log(np.array([1e-3, 0.1, 1.0, 16.0])).astype(np.float32)}
GK = {"safe": oracle.GATE_SAFE, "softplus": oracle.GATE_SOFTPLUS}


def _case(B, T, seed, n_slots=None, a_log="wide"):
    d = kda_synth.chunk_inputs(B, T, H, D, D, dtype=torch.bfloat16, seed=seed, n_slots=n_slots)
    x = d["x"].numpy().copy()
    t = np.arange(T)
    x[:, (t // 37) % 3 == 1] = 30.0   # saturated high
    x[:, (t // 37) % 3 == 2] = -30.0  # saturated low
    d["x"] = torch.from_numpy(x)
    d["A_log"] = torch.from_numpy(A_LOG[a_log].copy())
    return d


def _oracle(d, gate, lb, cu=None):
    g = oracle.gate(GK[gate], f64(d["x"]), f64(d["A_log"]), f64(d["dt_bias"]), lb)
    return oracle.recurrent(f64(d["q"]), f64(d["k"]), f64(d["v"]), g, f64(d["beta"]), h0=f64(d["h0"]),
                            cu_seqlens=cu)


def _chunk(d, gate, lb, schedule, cu=None):
    from gated_delta_rule_gate_amd import chunk_kda

    dd = {k: (v.cuda() if v is not None else None) for k, v in d.items()}
    cu_d = None if cu is None else torch.from_numpy(np.asarray(cu, dtype=np.int32)).cuda()
    o, ht = chunk_kda(dd["q"], dd["k"], dd["v"], dd["x"], dd["beta"], dd["h0"], cu_seqlens=cu_d,
                      output_final_state=True, chunk_size=64, gate_kind=gate, A_log=dd["A_log"],
                      dt_bias=dd["dt_bias"], lower_bound=lb, schedule=schedule)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), ht.cpu().numpy()


@pytest.mark.parametrize("schedule,gate,lb", [(s_, g_, l_) for s_ in ("fused", "split", "staged")
                                              for g_, l_ in (("safe", -5.0), ("safe", -1e-3), ("softplus", -5.0))]
                         + [("pipe", "safe", -5.0), ("pipe", "safe", -1e-3)])
def test_chunk_gate_extremes(schedule, gate, lb):
    need_gpu()
    d = _case(2, 333, 1600, a_log="chunk_softplus" if gate == "softplus" else "wide")
    o, ht = _chunk(d, gate, lb, schedule)
    o_ref, ht_ref = _oracle(d, gate, lb)
    parity(o, o_ref, "bf16", "o")
    parity(ht, ht_ref, "bf16", "ht")


@pytest.mark.parametrize("schedule", ["fused", "split", "staged", "pipe"])
def test_chunk_long_decay_packed(schedule):
    """A long slot (2048 tokens) beside short ragged ones, bound close to 0, so
    the cumulative decay stays near 1 over the whole sequence."""
    need_gpu()
    lens = [2048, 3, 0, 131, 70]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    d = _case(1, int(cu[-1]) + 9, 1601, n_slots=len(lens))
    o, ht = _chunk(d, "safe", -1e-3, schedule, cu=cu)
    o_ref, ht_ref = _oracle(d, "safe", -1e-3, cu=cu)
    n = int(cu[-1])
    parity(o[:, :n], o_ref[:, :n], "bf16", "o")
    parity(ht, ht_ref, "bf16", "ht")


@pytest.mark.parametrize("gate,lb", [("safe", -1e-3), ("softplus", -5.0)])
def test_recurrent_gate_extremes(gate, lb):
    from gated_delta_rule_gate_amd import recurrent_kda

    need_gpu()
    d = _case(4, 150, 1602)
    dd = {k: (v.cuda() if v is not None else None) for k, v in d.items()}
    o, ht = recurrent_kda(dd["q"], dd["k"], dd["v"], dd["x"], dd["beta"], dd["h0"], output_final_state=True,
                          gate_kind=gate, A_log=dd["A_log"], dt_bias=dd["dt_bias"], lower_bound=lb)
    torch.cuda.synchronize()
    o_ref, ht_ref = _oracle(d, gate, lb)
    parity(o.float().cpu().numpy(), o_ref, "bf16", "o")
    parity(ht.cpu().numpy(), ht_ref, "bf16", "ht")
