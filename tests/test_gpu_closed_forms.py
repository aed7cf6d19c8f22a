"""GPU results against closed forms of special cases, with no oracle recurrence.

Each case reduces the gated delta rule to something with its own plain answer
("FLA KDA Skill", section "Correctness checklist", and the method's
recurrence as the pages define it), evaluated here in FP64 and compared with
every chunk schedule and with the recurrent kernel at real widths (K = V =
128, a ragged tail, several chunks):

* g = 0: no decay, so the state follows the textbook delta rule
  S_t = (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T and o_t = scale S_t^T q_t.
* beta = 0: nothing is written, the initial state only decays:
  o_t = scale (q_t * e^{G_t})^T h0 and ht = Diag(e^{G_T}) h0, G = cumsum(g).
* beta = 1 and q = k with |k| = 1 exactly (sixteen entries of +-1/4): the
  update overwrites the state's read-out along k, so o_t = v_t / sqrt(K)
  whatever the gate.
* axis-aligned keys k_t = +-e_i: the state's rows decouple into scalar
  recursions, row i_t <- (1 - beta_t) alpha row + beta_t (+-v_t), the others
  only decay, under the safe and the softplus gate.

The gate of the last case comes from the oracle's gate function (pinned on
its own); everything else is the closed form.
"""
import math

import numpy as np
import pytest
import torch

import kda_synth
import oracle
from kda_testlib import f64, need_gpu, parity

pytestmark = pytest.mark.gpu

B, T, H, K = 2, 203, 2, 128
SCALE = 1.0 / math.sqrt(K)
CHUNK_SCHEDULES = ["fused", "split", "staged"]


def _base(seed):
    return kda_synth.chunk_inputs(B, T, H, K, K, dtype=torch.bfloat16, seed=seed)


def _run(d, path, gate, g, lb=-5.0):
    """o [B, T, H, V] and ht [B, H, K, V] from the chunk path (schedule) or the recurrent kernel."""
    from gated_delta_rule_gate_amd import chunk_kda, recurrent_kda

    dev = lambda t: None if t is None else t.cuda()
    kw = dict(gate_kind=gate, A_log=dev(d["A_log"]), dt_bias=dev(d["dt_bias"]), lower_bound=lb)
    args = (dev(d["q"]), dev(d["k"]), dev(d["v"]), dev(g), dev(d["beta"]), dev(d["h0"]))
    if path == "recurrent":
        o, ht = recurrent_kda(*args, output_final_state=True, **kw)
    else:
        o, ht = chunk_kda(*args, output_final_state=True, chunk_size=64, schedule=path, **kw)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), ht.cpu().numpy()


def _bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)


@pytest.mark.parametrize("path", CHUNK_SCHEDULES + ["recurrent"])
def test_no_decay_is_the_delta_rule(path):
    need_gpu()
    d = _base(2100)
    g = torch.zeros((B, T, H, K), dtype=torch.float32)
    o, ht = _run(d, path, "loge", g)
    q, k, v, beta, h0 = f64(d["q"]), f64(d["k"]), f64(d["v"]), f64(d["beta"]), f64(d["h0"])
    o_ref = np.zeros_like(v)
    ht_ref = np.zeros_like(h0)
    for b in range(B):
        for h in range(H):
            S = h0[b, h].copy()
            for t in range(T):
                kt, bt = k[b, t, h], beta[b, t, h]
                S = S - bt * np.outer(kt, kt @ S) + bt * np.outer(kt, v[b, t, h])
                o_ref[b, t, h] = SCALE * (S.T @ q[b, t, h])
            ht_ref[b, h] = S
    parity(o, o_ref, "bf16", "o")
    parity(ht, ht_ref, "bf16", "ht")


@pytest.mark.parametrize("path", CHUNK_SCHEDULES + ["recurrent"])
def test_zero_beta_only_decays_the_initial_state(path):
    need_gpu()
    d = _base(2101)
    d["beta"] = torch.zeros((B, T, H), dtype=torch.float32)
    g64 = -0.2 * np.abs(f64(d["x"]))  # natural-log decays in (-inf, 0]
    g = torch.from_numpy(g64.astype(np.float32))
    o, ht = _run(d, path, "loge", g)
    G = np.cumsum(f64(g), axis=1)  # [B, T, H, K]
    q, h0 = f64(d["q"]), f64(d["h0"])
    o_ref = SCALE * np.einsum("bthk,bhkv->bthv", q * np.exp(G), h0)
    ht_ref = np.exp(G[:, -1])[..., None] * h0
    parity(o, o_ref, "bf16", "o")
    parity(ht, ht_ref, "bf16", "ht")


@pytest.mark.parametrize("path", CHUNK_SCHEDULES + ["pipe", "recurrent"])
def test_unit_beta_with_query_equal_key_returns_v(path):
    need_gpu()
    d = _base(2102)
    rng = np.random.default_rng(2102)
    kk = np.zeros((B, T, H, K), dtype=np.float32)
    for idx in np.ndindex(B, T, H):
        ch = rng.choice(K, size=16, replace=False)
        kk[idx + (ch,)] = rng.choice([-0.25, 0.25], size=16)  # |k| = 1 exactly, also in bf16
    d["k"] = _bf16(kk)
    d["q"] = d["k"].clone()
    d["beta"] = torch.ones((B, T, H), dtype=torch.float32)
    o, _ = _run(d, path, "safe", d["x"])
    parity(o, f64(d["v"]) * SCALE, "bf16", "o")


@pytest.mark.parametrize("path,gate", [(p_, g_) for p_ in CHUNK_SCHEDULES + ["recurrent"]
                                        for g_ in ("safe", "softplus")] + [("pipe", "safe")])
def test_axis_aligned_keys_decouple_rows(path, gate):
    need_gpu()
    d = _base(2103 + (gate == "softplus"))
    rng = np.random.default_rng(2103)
    idx = rng.integers(0, K, size=(B, T, H))
    sign = rng.choice([-1.0, 1.0], size=(B, T, H))
    kk = np.zeros((B, T, H, K), dtype=np.float32)
    np.put_along_axis(kk, idx[..., None], sign[..., None].astype(np.float32), axis=-1)
    d["k"] = _bf16(kk)
    if gate == "softplus":  # keep the unbounded decay moderate: exp(A_log) in [0.1, 1]
        d["A_log"] = torch.from_numpy(np.log(rng.uniform(0.1, 1.0, size=H)).astype(np.float32))
    kind = oracle.GATE_SAFE if gate == "safe" else oracle.GATE_SOFTPLUS
    lb = -5.0
    g = oracle.gate(kind, f64(d["x"]), f64(d["A_log"]), f64(d["dt_bias"]), lb)  # natural log, [B, T, H, K]
    o, ht = _run(d, path, gate, d["x"], lb=lb)
    q, v, beta, h0 = f64(d["q"]), f64(d["v"]), f64(d["beta"]), f64(d["h0"])
    o_ref = np.zeros_like(v)
    ht_ref = np.zeros_like(h0)
    for b in range(B):
        for h in range(H):
            S = h0[b, h].copy()
            for t in range(T):
                S *= np.exp(g[b, t, h])[:, None]
                i, bt = idx[b, t, h], beta[b, t, h]
                S[i] = (1.0 - bt) * S[i] + bt * sign[b, t, h] * v[b, t, h]
                o_ref[b, t, h] = SCALE * (S.T @ q[b, t, h])
            ht_ref[b, h] = S
    parity(o, o_ref, "bf16", "o")
    parity(ht, ht_ref, "bf16", "ht")
