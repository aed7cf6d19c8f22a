"""GPU parity of the chunked backward (kda_chunk_bwd) against the FP64 oracle.

The oracle's gradients come from reverse mode through the token recurrence
(oracle.recurrent_bwd, pinned on the CPU by central finite differences) and the
gate activation's derivative (oracle.gate_bwd, pinned the same way). The loss
is L = sum(do * o) + sum(dht * ht) with seeded N(0, 1) do and 0.1 N(0, 1) dht.

Bounds (gradients span orders of magnitude, so both are relative to the
reference tensor's largest entry):
  fp32 inputs: rel-RMS <= 1e-4 and max-abs <= 1e-4 * max(1, max|ref|)
  bf16 inputs: rel-RMS <= 5e-3 and max-abs <= 2e-2 * max(1, max|ref|)
dA_log and ddt_bias are sums over every token. Their terms are the per-token
gate gradients times a factor, and those terms are already bounded element by
element through dg. For a head whose decay is steep, the FP32 chunked form
reaches a true gradient of ~1e-10 as a difference of O(1e-2) terms, so a sum
of such terms cannot match to a fraction of its own size. The sums are checked
in two parts instead:
  (a) against the oracle, with each entry bounded by 1e-4 (fp32) or 5e-3
      (bf16) times the L1 norm of its terms plus the summed error of the GPU's
      own terms against the oracle's;
  (b) as the sum of the GPU's own terms, to 1e-5 of their L1 norm (FP32
      accumulation).
"""
import os

import numpy as np
import pytest
import torch

import kda_synth
import oracle
from kda_testlib import f64, need_gpu

pytestmark = pytest.mark.gpu

BOUNDS = {"fp32": (1e-4, 1e-4), "bf16": (5e-3, 2e-2)}
GK = {"safe": oracle.GATE_SAFE, "softplus": oracle.GATE_SOFTPLUS, "loge": oracle.GATE_LOGE}


def grad_parity(got, want, kind, what):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    assert np.isfinite(got).all(), "%s: non-finite values" % what
    rel_b, abs_b = BOUNDS[kind]
    diff = got - want
    den = float(np.sqrt(np.sum(want * want)))
    rel = float(np.sqrt(np.sum(diff * diff)) / den) if den > 0 else float(np.sqrt(np.sum(diff * diff)))
    mx = float(np.abs(diff).max()) if diff.size else 0.0
    ref = max(1.0, float(np.abs(want).max()) if want.size else 0.0)
    log = os.environ.get("KDA_PARITY_LOG")
    if log:
        with open(log, "a") as f:
            f.write("%s | %s | %s | max-abs/ref %.3e | rel-RMS %.3e\n" % (
                os.environ.get("PYTEST_CURRENT_TEST", "?").split(" ")[0], what, kind, mx / ref, rel))
    assert rel <= rel_b, "%s: rel-RMS %.3e > %.1e (max-abs %.3e)" % (what, rel, rel_b, mx)
    assert mx <= abs_b * ref, "%s: max-abs %.3e > %.1e * %.3g" % (what, mx, abs_b, ref)


def sum_parity(got, want, l1, term_err, own_sum, own_l1, kind, what):
    tol = {"fp32": 1e-4, "bf16": 5e-3}[kind]
    got, want, l1, term_err, own_sum, own_l1 = (np.asarray(a, dtype=np.float64)
                                                for a in (got, want, l1, term_err, own_sum, own_l1))
    assert np.isfinite(got).all(), "%s: non-finite values" % what
    err = np.abs(got - want)
    bound = tol * l1 + term_err
    assert np.all(err <= bound + 1e-30), "%s: error %.3e over its bound %.3e" % (
        what, float(np.max(err - bound)), float(bound[np.argmax(err - bound)]))
    own = np.abs(got - own_sum)
    assert np.all(own <= 1e-5 * own_l1 + 1e-30), "%s: not the sum of its own terms (%.3e)" % (what, float(own.max()))


def _case(B, T, H, K, V, dtype, seed, gate, n_slots=None):
    d = kda_synth.chunk_inputs(B, T, H, K, V, dtype=dtype, seed=seed, n_slots=n_slots)
    rng = np.random.default_rng(seed + 77)
    N = B if n_slots is None else n_slots
    d["do"] = torch.from_numpy(rng.standard_normal((B, T, H, V)).astype(np.float32)).to(dtype)
    d["dht"] = torch.from_numpy((0.1 * rng.standard_normal((N, H, K, V))).astype(np.float32))
    if gate == "loge":
        d["x"] = (-0.3 * d["x"].abs()).contiguous()
    return d


def _run(d, gate, C, cu=None, beta_logits=False):
    from gated_delta_rule_gate_amd import chunk_kda_bwd

    dd = {k: (v.cuda() if v is not None else None) for k, v in d.items()}
    cu_d = None if cu is None else torch.from_numpy(np.asarray(cu, dtype=np.int32)).cuda()
    out = chunk_kda_bwd(dd["q"], dd["k"], dd["v"], dd["x"], dd["beta"], dd["do"], dd["h0"], dht=dd["dht"],
                        cu_seqlens=cu_d, chunk_size=C, gate_kind=gate, A_log=dd["A_log"], dt_bias=dd["dt_bias"],
                        lower_bound=-5.0, beta_logits=beta_logits)
    torch.cuda.synchronize()
    return {k: (None if v is None else v.float().cpu().numpy()) for k, v in out.items()}


def _oracle(d, gate, cu=None, beta_logits=False):
    x = f64(d["x"])
    g = oracle.gate(GK[gate], x, f64(d["A_log"]), f64(d["dt_bias"]), -5.0)
    beta = f64(d["beta"])
    if beta_logits:
        beta = oracle.beta_from_logits(beta)
    dq, dk, dv, dg, dbeta, dh0 = oracle.recurrent_bwd(f64(d["q"]), f64(d["k"]), f64(d["v"]), g, beta, f64(d["do"]),
                                                      dht=f64(d["dht"]), h0=f64(d["h0"]), cu_seqlens=cu)
    if cu is not None:
        n = int(cu[-1])
        dg = dg.copy()
        dg[:, n:] = 0.0
    dx, dA, ddt = oracle.gate_bwd(GK[gate], x, dg, f64(d["A_log"]), f64(d["dt_bias"]), -5.0)
    if beta_logits:
        dbeta = dbeta * beta * (1.0 - beta)
    out = dict(dq=dq, dk=dk, dv=dv, dg=dx, dbeta=dbeta, dh0=dh0, dA_log=dA, ddt_bias=ddt)
    if dA is not None:
        # dA_log sums dx * wA over tokens and channels, ddt_bias sums dx over tokens:
        # safe wA = x + dt; softplus wA = g / (dg/dx) = softplus(z) / sigmoid(z)
        z = x + f64(d["dt_bias"])
        if gate == "safe":
            out["wA"] = z
        else:
            out["wA"] = np.logaddexp(0.0, z) / oracle.beta_from_logits(z)
    return out


def _compare(got, want, kind, rows=None):
    for name in ("dq", "dk", "dv", "dg", "dbeta"):
        g, w = got[name], want[name]
        if rows is not None:
            g, w = g[:, :rows], w[:, :rows]
        grad_parity(g, w, kind, name)
    grad_parity(got["dh0"], want["dh0"], kind, "dh0")
    if want["dA_log"] is not None:
        lead = tuple(range(want["dg"].ndim - 2))
        dx_ref = want["dg"] if rows is None else want["dg"][:, :rows]
        dx_gpu = got["dg"].astype(np.float64) if rows is None else got["dg"][:, :rows].astype(np.float64)
        wA = want["wA"] if rows is None else want["wA"][:, :rows]
        tsum = lambda a: np.sum(a, axis=lead)
        sum_parity(got["ddt_bias"], want["ddt_bias"], tsum(np.abs(dx_ref)), tsum(np.abs(dx_gpu - dx_ref)),
                   tsum(dx_gpu), tsum(np.abs(dx_gpu)), kind, "ddt_bias")
        sum_parity(got["dA_log"], want["dA_log"], tsum(np.abs(dx_ref * wA)).sum(-1),
                   tsum(np.abs((dx_gpu - dx_ref) * wA)).sum(-1), tsum(dx_gpu * wA).sum(-1),
                   tsum(np.abs(dx_gpu * wA)).sum(-1), kind, "dA_log")


@pytest.mark.parametrize("C", [64, 32])
@pytest.mark.parametrize("gate", ["safe", "softplus", "loge"])
def test_bwd_fp32(gate, C):
    need_gpu()
    d = _case(2, 150, 2, 64, 64, torch.float32, 1800 + C, gate)
    _compare(_run(d, gate, C), _oracle(d, gate), "fp32")


@pytest.mark.parametrize("C", [64, 32])
@pytest.mark.parametrize("D", [128, 64])
def test_bwd_bf16(D, C):
    need_gpu()
    d = _case(2, 203, 2, D, D, torch.bfloat16, 1810 + C + D, "safe")
    _compare(_run(d, "safe", C), _oracle(d, "safe"), "bf16")


def test_bwd_packed_empty_slots_and_logits():
    need_gpu()
    lens = [70, 0, 130, 5]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    d = _case(1, int(cu[-1]) + 11, 2, 128, 128, torch.bfloat16, 1820, "safe", n_slots=len(lens))
    got = _run(d, "safe", 64, cu=cu, beta_logits=True)
    want = _oracle(d, "safe", cu=cu, beta_logits=True)
    _compare(got, want, "bf16", rows=int(cu[-1]))
    assert np.array_equal(got["dh0"][1], d["dht"][1].numpy()), "an empty slot's dh0 is dht"


@pytest.mark.parametrize("K,V", [(128, 64), (96, 72)])
def test_bwd_widths(K, V):
    need_gpu()
    d = _case(1, 140, 2, K, V, torch.float32, 1830 + K + V, "softplus")
    _compare(_run(d, "softplus", 64), _oracle(d, "softplus"), "fp32")


@pytest.mark.parametrize("B,T,H,D,C,gate", [(2, 1000, 32, 128, 64, "safe"), (2, 1000, 64, 64, 32, "safe"),
                                             (2, 600, 16, 64, 64, "softplus")])
def test_bwd_many_items(B, T, H, D, C, gate):
    """More (chunk, head) items than compute units, each sequence ending in a ragged
    chunk: the contraction and WY kernels' persistent workgroups walk several items
    with the next item's loads in flight, and at 4096 items the staged gate step's
    workgroups (four per compute unit) do as well."""
    need_gpu()
    d = _case(B, T, H, D, D, torch.bfloat16, 1840 + H + C, gate)
    _compare(_run(d, gate, C), _oracle(d, gate), "bf16")
