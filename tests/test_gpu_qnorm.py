"""GPU parity of the q_l2norm option: raw q in, normalisation deferred to the output.

The option ("Add fused recurrent_kda ...", stacked description of the fused
q-l2norm option) scales each output row by 1/sqrt(|q_r|^2 + 1e-6) instead of
normalising q first. The oracle normalises the same raw q bytes explicitly in
FP64 (oracle.l2norm_rows) and runs the token recurrence. Raw rows span the
pages' test range of scales 1e-3..1e3, with some rows exactly zero.
"""
import numpy as np
import pytest
import torch

import kda_synth
import oracle
from kda_testlib import f64, need_gpu, parity

pytestmark = pytest.mark.gpu


def _raw_q(q, seed):
    """Rows of the l2-normalised q scaled by log-uniform factors in [1e-3, 1e3]; every
    seventh row zero. Returned in q's dtype."""
    rng = np.random.default_rng(seed)
    s = np.exp(rng.uniform(np.log(1e-3), np.log(1e3), size=q.shape[:-1])).astype(np.float32)
    s[..., ::7] = 0.0
    return (q.float() * torch.from_numpy(s)[..., None]).to(q.dtype).contiguous()


def _chunk_case(B, T, H, D, seed, n_slots=None):
    d = kda_synth.chunk_inputs(B, T, H, D, D, dtype=torch.bfloat16, seed=seed, n_slots=n_slots)
    d["q"] = _raw_q(d["q"], seed + 1)
    return d


def _oracle_chunk(d, cu=None):
    g = oracle.gate(oracle.GATE_SAFE, f64(d["x"]), f64(d["A_log"]), f64(d["dt_bias"]), -5.0)
    qn = oracle.l2norm_rows(f64(d["q"]))
    return oracle.recurrent(qn, f64(d["k"]), f64(d["v"]), g, f64(d["beta"]), h0=f64(d["h0"]), cu_seqlens=cu)


def _gpu_chunk(d, schedule, cu=None, C=64, q_l2norm=True):
    from gated_delta_rule_gate_amd import chunk_kda

    dd = {k: (v.cuda() if v is not None else None) for k, v in d.items()}
    cu_d = None if cu is None else torch.from_numpy(np.asarray(cu, dtype=np.int32)).cuda()
    o, ht = chunk_kda(dd["q"], dd["k"], dd["v"], dd["x"], dd["beta"], dd["h0"], cu_seqlens=cu_d,
                      output_final_state=True, chunk_size=C, gate_kind="safe", A_log=dd["A_log"],
                      dt_bias=dd["dt_bias"], lower_bound=-5.0, schedule=schedule, q_l2norm=q_l2norm)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), ht.cpu().numpy()


@pytest.mark.parametrize("schedule,D,C", [(s_, d_, c_) for s_ in ("fused", "split", "staged")
                                          for d_, c_ in ((128, 64), (128, 32), (64, 64))] + [("pipe", 128, 64)])
def test_chunk_q_l2norm(schedule, D, C):
    need_gpu()
    d = _chunk_case(2, 203, 3, D, 700 + D + C)
    o, ht = _gpu_chunk(d, schedule, C=C)
    o_ref, ht_ref = _oracle_chunk(d)
    parity(o, o_ref, "bf16", "o")
    parity(ht, ht_ref, "bf16", "ht")
    zero = d["q"].float().abs().sum(-1).numpy() == 0
    assert zero.any() and np.all(o[zero] == 0.0), "rows of zero q must give zero output"


def test_chunk_q_l2norm_packed_and_value_split():
    """Packed slots (one empty) and few (sequence, head) pairs, so the fused kernel
    also splits the value columns."""
    need_gpu()
    cu = kda_synth.varlen_offsets(71, n_slots=4, n_empty=1, total=300, max_len=300)
    d = _chunk_case(1, 320, 2, 128, 71, n_slots=4)
    o, ht = _gpu_chunk(d, "fused", cu=cu)
    o_ref, ht_ref = _oracle_chunk(d, cu=cu)
    n = int(cu[-1])
    parity(o[:, :n], o_ref[:, :n], "bf16", "o")
    parity(ht, ht_ref, "bf16", "ht")


def test_chunk_q_l2norm_flag_off_is_unchanged():
    """Without the flag the same raw q is used as given (the contract's normalised q)."""
    need_gpu()
    d = _chunk_case(1, 130, 2, 128, 77)
    o, _ = _gpu_chunk(d, "fused", q_l2norm=False)
    g = oracle.gate(oracle.GATE_SAFE, f64(d["x"]), f64(d["A_log"]), f64(d["dt_bias"]), -5.0)
    o_ref, _ = oracle.recurrent(f64(d["q"]), f64(d["k"]), f64(d["v"]), g, f64(d["beta"]), h0=f64(d["h0"]))
    rel = np.linalg.norm(o - o_ref) / np.linalg.norm(o_ref)
    assert rel < 5e-3


@pytest.mark.parametrize("T", [1, 64])
def test_recurrent_q_l2norm(T):
    from gated_delta_rule_gate_amd import recurrent_kda

    need_gpu()
    N, H, D = 16, 4, 128
    d = kda_synth.chunk_inputs(N, T, H, D, D, dtype=torch.bfloat16, seed=800 + T)
    d["q"] = _raw_q(d["q"], 801 + T)
    d["g"] = kda_synth.log2_gate(d["x"].numpy(), d["A_log"].numpy(), d["dt_bias"].numpy())
    dd = {k: (v.cuda() if v is not None else None) for k, v in d.items()}
    o, ht = recurrent_kda(dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"], dd["h0"], output_final_state=True,
                          q_l2norm=True)
    torch.cuda.synchronize()
    qn = oracle.l2norm_rows(f64(d["q"]))
    o_ref, ht_ref = oracle.recurrent(qn, f64(d["k"]), f64(d["v"]), f64(d["g"]), f64(d["beta"]), h0=f64(d["h0"]),
                                     g_is_log2=True)
    parity(o.float().cpu().numpy(), o_ref, "bf16", "o")
    parity(ht.cpu().numpy(), ht_ref, "bf16", "ht")
