"""GPU parity of kda_recurrent_fwd (fused token-sequential recurrence) against the FP64 oracle."""
import math

import numpy as np
import pytest
import torch

import kda_synth
import oracle
from kda_testlib import f64, need_gpu, parity

pytestmark = pytest.mark.gpu

GK = {"loge": oracle.GATE_LOGE, "safe": oracle.GATE_SAFE, "softplus": oracle.GATE_SOFTPLUS}


def _inputs(B, T, H, K, V, dtype, seed, gate, n_slots=None, with_h0=True):
    kk = max(K, V)
    d = kda_synth.chunk_inputs(B, T, H, kk, kk, dtype=dtype, seed=seed, with_h0=with_h0, n_slots=n_slots)
    d["q"] = d["q"][..., :K].contiguous()
    d["k"] = d["k"][..., :K].contiguous()
    # re-normalising after truncation is the caller's job; the oracle sees the same bytes
    d["v"] = d["v"][..., :V].contiguous()
    d["x"] = d["x"][..., :K].contiguous()
    d["dt_bias"] = d["dt_bias"][:, :K].contiguous()
    if d["h0"] is not None:
        d["h0"] = d["h0"][..., :K, :V].contiguous()
    if gate == "log2":
        d["g"] = kda_synth.log2_gate(d["x"].numpy(), d["A_log"].numpy(), d["dt_bias"].numpy())
    elif gate == "loge":
        d["g"] = (-0.5 * d["x"].abs()).contiguous()
    else:
        d["g"] = d["x"]
    return d


def _oracle(d, gate, cu=None, lb=-5.0):
    if gate == "log2":
        g, is2 = f64(d["g"]), True
    elif gate == "loge":
        g, is2 = f64(d["g"]), False
    else:
        g, is2 = oracle.gate(GK[gate], f64(d["x"]), f64(d["A_log"]), f64(d["dt_bias"]), lb), False
    return oracle.recurrent(f64(d["q"]), f64(d["k"]), f64(d["v"]), g, f64(d["beta"]), h0=f64(d["h0"]),
                            cu_seqlens=cu, g_is_log2=is2)


def _gpu(d, gate, cu=None, inplace=False, out=None):
    from gated_delta_rule_gate_amd import recurrent_kda

    dd = {k: (v.cuda() if v is not None else None) for k, v in d.items()}
    cu_d = None if cu is None else torch.from_numpy(np.asarray(cu, dtype=np.int32)).cuda()
    fs = dd["h0"] if inplace else None
    o, ht = recurrent_kda(dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"], dd["h0"], cu_seqlens=cu_d,
                          output_final_state=True, gate_kind=gate, A_log=dd["A_log"], dt_bias=dd["dt_bias"],
                          final_state=fs, out=None if out is None else out.cuda())
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), ht.cpu().numpy()


@pytest.mark.parametrize("gate", ["log2", "loge", "safe", "softplus"])
def test_dense_fp32(gate):
    need_gpu()
    d = _inputs(2, 37, 2, 64, 64, torch.float32, 101, gate)
    o, ht = _gpu(d, gate)
    o_ref, ht_ref = _oracle(d, gate)
    parity(o, o_ref, "fp32", "o")
    parity(ht, ht_ref, "fp32", "ht")


@pytest.mark.parametrize("K,V", [(128, 128), (64, 128), (128, 64), (256, 256), (256, 64)])
def test_dense_bf16_widths(K, V):
    need_gpu()
    d = _inputs(2, 50, 3, K, V, torch.bfloat16, 102, "log2")
    o, ht = _gpu(d, "log2")
    o_ref, ht_ref = _oracle(d, "log2")
    parity(o, o_ref, "bf16", "o")
    parity(ht, ht_ref, "bf16", "ht")


def test_decode_full_size_in_place():
    """256 sequences x 1 token, H 64, K = V = 128, bf16, log2 gate, state updated in place."""
    need_gpu()
    d = _inputs(256, 1, 64, 128, 128, torch.bfloat16, 1004, "log2")
    o, ht = _gpu(d, "log2", inplace=True)
    o_ref, ht_ref = _oracle(d, "log2")
    parity(o, o_ref, "bf16", "o")
    parity(ht, ht_ref, "bf16", "ht")


def test_prefill_64_tokens_sampled():
    """The 64-token prefill through the same kernel; the oracle checks 8 sampled sequences
    (each sequence is independent, so a slice of the batch is an exact sub-problem)."""
    need_gpu()
    d = _inputs(256, 64, 64, 128, 128, torch.bfloat16, 1005, "log2")
    o, ht = _gpu(d, "log2")
    idx = [0, 1, 77, 128, 199, 254, 255, 31]
    sub = {k: (v[idx].contiguous() if (v is not None and v.dim() >= 3) else v) for k, v in d.items()}
    o_ref, ht_ref = _oracle(sub, "log2")
    parity(o[idx], o_ref, "bf16", "o")
    parity(ht[idx], ht_ref, "bf16", "ht")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_packed_empty_slots_and_tail(dtype):
    """Empty slots first, inside and last pass their state through bit for bit; rows past
    the last offset are neither read (NaN-poisoned inputs) nor written (sentinel kept)."""
    need_gpu()
    lens = [0, 17, 1, 0, 40, 3, 0]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    cap = int(cu[-1]) + 9
    d = _inputs(1, cap, 2, 64, 64, dtype, 103, "safe", n_slots=len(lens))
    for key in ("q", "k", "v", "x"):
        d[key][:, int(cu[-1]):] = float("nan")
    d["beta"][:, int(cu[-1]):] = float("nan")
    sentinel = torch.full((1, cap, 2, 64), 7.0, dtype=dtype)
    o, ht = _gpu(d, "safe", cu=cu, out=sentinel)
    o_ref, ht_ref = _oracle(d, "safe", cu=cu)
    name = "fp32" if dtype == torch.float32 else "bf16"
    parity(o[:, : int(cu[-1])], o_ref[:, : int(cu[-1])], name, "o")
    parity(ht, ht_ref, name, "ht")
    assert (o[:, int(cu[-1]):] == 7.0).all()
    h0 = d["h0"].numpy()
    for n, L in enumerate(lens):
        if L == 0:
            assert np.array_equal(ht[n].view(np.uint32), h0[n].view(np.uint32))


def test_packed_no_initial_state_gives_zero_for_empty():
    need_gpu()
    lens = [5, 0, 9]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    d = _inputs(1, 14, 2, 64, 64, torch.float32, 104, "log2", n_slots=3, with_h0=False)
    o, ht = _gpu(d, "log2", cu=cu)
    o_ref, ht_ref = _oracle(d, "log2", cu=cu)
    parity(o, o_ref, "fp32", "o")
    parity(ht, ht_ref, "fp32", "ht")
    assert not ht[1].any()


def test_dyadic_exact_case_fp32():
    """Dyadic inputs (entries +-1/8 at K = 64, log2 gates in {0,-1,-2}, beta in quarters): the
    exact result is representable and the FP32 kernel must land within the fp32 bound."""
    need_gpu()
    rng = np.random.default_rng(105)
    T, K, V = 8, 64, 64
    q = rng.choice([-0.125, 0.125], size=(1, T, 1, K)).astype(np.float32)
    k = rng.choice([-0.125, 0.125], size=(1, T, 1, K)).astype(np.float32)
    v = rng.integers(-3, 4, size=(1, T, 1, V)).astype(np.float32)
    g = rng.integers(-2, 1, size=(1, T, 1, K)).astype(np.float32)
    beta = (rng.integers(1, 5, size=(1, T, 1)) / 4.0).astype(np.float32)
    h0 = (rng.integers(-4, 5, size=(1, 1, K, V)) / 8.0).astype(np.float32)
    d = dict(q=torch.from_numpy(q), k=torch.from_numpy(k), v=torch.from_numpy(v), g=torch.from_numpy(g),
             beta=torch.from_numpy(beta), h0=torch.from_numpy(h0), x=None, A_log=None, dt_bias=None)
    o, ht = _gpu(d, "log2")
    o_ref, ht_ref = _oracle(d, "log2")
    parity(o, o_ref, "fp32", "o")
    parity(ht, ht_ref, "fp32", "ht")


def test_rejects_grad_and_bad_args():
    need_gpu()
    from gated_delta_rule_gate_amd import KdaError, recurrent_kda

    d = _inputs(1, 4, 1, 64, 64, torch.float32, 106, "log2")
    dd = {k: (v.cuda() if v is not None else None) for k, v in d.items()}
    qg = dd["q"].clone().requires_grad_(True)
    with pytest.raises(RuntimeError, match="requires grad"):
        recurrent_kda(qg, dd["k"], dd["v"], dd["g"], dd["beta"])
    with pytest.raises(KdaError, match="GATE"):
        recurrent_kda(dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"], gate_kind="safe")  # no A_log
    with pytest.raises(KdaError, match="GATE"):
        recurrent_kda(dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"], gate_kind="safe", A_log=dd["A_log"],
                      lower_bound=-6.0)
    q44 = torch.zeros((1, 4, 1, 44), device="cuda")  # widths are multiples of 8
    with pytest.raises(KdaError, match="UNSUPPORTED"):
        recurrent_kda(q44, q44, dd["v"], q44, dd["beta"])
