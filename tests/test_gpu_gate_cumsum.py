"""GPU parity of kda_gate_cumsum (step (1) on its own) against the oracle's
chunk-local cumsum, and of kda_chunk_fwd fed the pre-cumsummed gate
(KDA_GATE_LOG2_CUMSUM) against the token recurrence on the original gate."""
import math

import numpy as np
import pytest
import torch

import kda_synth
import oracle
from kda_testlib import f64, need_gpu, parity

pytestmark = pytest.mark.gpu

GK = {"loge": oracle.GATE_LOGE, "safe": oracle.GATE_SAFE, "softplus": oracle.GATE_SOFTPLUS}


def _inputs(B, T, H, K, seed, gate, n_slots=None):
    d = kda_synth.chunk_inputs(B, T, H, K, K, dtype=torch.bfloat16, seed=seed, n_slots=n_slots)
    if gate == "loge":
        d["g"] = (-0.3 * d["x"].abs()).contiguous()
    elif gate == "log2":
        d["g"] = (-0.3 / math.log(2.0) * d["x"].abs()).contiguous()
    else:
        d["g"] = d["x"]
    return d


def _natural_gate(d, gate):
    """Per-token natural-log decay the oracle uses for this gate kind."""
    if gate == "loge":
        return f64(d["g"])
    if gate == "log2":
        return f64(d["g"]) * math.log(2.0)
    return oracle.gate(GK[gate], f64(d["x"]), f64(d["A_log"]), f64(d["dt_bias"]), -5.0)


def _gpu_cumsum(d, gate, C, cu=None, out=None):
    from gated_delta_rule_gate_amd import gate_cumsum

    dev = {k: (v.cuda() if v is not None else None) for k, v in d.items()}
    cu_d = None if cu is None else torch.from_numpy(np.asarray(cu, dtype=np.int32)).cuda()
    b = gate_cumsum(dev["g"], chunk_size=C, gate_kind=gate, A_log=dev["A_log"], dt_bias=dev["dt_bias"],
                    lower_bound=-5.0, cu_seqlens=cu_d, out=None if out is None else out.cuda())
    torch.cuda.synchronize()
    return b.cpu().numpy()


def _check_b(got, want):
    err = np.abs(got.astype(np.float64) - want)
    assert np.isfinite(got).all()
    assert err.max() <= 1e-5 * max(1.0, np.abs(want).max()) + 1e-5, err.max()


@pytest.mark.parametrize("gate", ["safe", "softplus", "loge", "log2"])
@pytest.mark.parametrize("C", [1, 32, 64])
def test_gate_cumsum_dense_ragged(gate, C):
    """B2 T200 (three full chunks and a ragged one per sequence) H3 K128."""
    need_gpu()
    d = _inputs(2, 200, 3, 128, 2000 + C, gate)
    got = _gpu_cumsum(d, gate, C)
    want = oracle.chunk_cumsum_log2(_natural_gate(d, gate), chunk_size=C)
    _check_b(got, want)


@pytest.mark.parametrize("K", [64, 256, 40, 96, 200])  # and non-powers of two (multiples of 8)
def test_gate_cumsum_widths(K):
    need_gpu()
    d = _inputs(1, 150, 2, K, 2100 + K, "safe")
    _check_b(_gpu_cumsum(d, "safe", 64), oracle.chunk_cumsum_log2(_natural_gate(d, "safe"), chunk_size=64))


@pytest.mark.parametrize("C", [1, 32, 64])
def test_gate_cumsum_packed(C):
    """Empty slots first, inside and last; slot starts off the 64-row grid (carry-in);
    the NaN-poisoned tail is neither read nor written."""
    need_gpu()
    lens = [0, 70, 64, 1, 0, 129, 17, 0]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    end = int(cu[-1])
    d = _inputs(1, end + 37, 2, 128, 2200 + C, "safe", n_slots=len(lens))
    d["x"][:, end:] = float("nan")
    sentinel = torch.full(d["g"].shape, 7.0, dtype=torch.float32)
    got = _gpu_cumsum(d, "safe", C, cu=cu, out=sentinel)
    want = oracle.chunk_cumsum_log2(_natural_gate(d, "safe"), cu_seqlens=cu, chunk_size=C)
    _check_b(got[:, :end], want[:, :end])
    assert (got[:, end:] == 7.0).all()


def test_gate_cumsum_per_token_is_exact():
    """chunk_size 1: a log2 gate comes back bit for bit, a natural-log gate as its
    fp32 product with log2(e) (the rounding the kernels apply)."""
    need_gpu()
    d = _inputs(1, 96, 2, 128, 2300, "log2")
    got = _gpu_cumsum(d, "log2", 1)
    assert np.array_equal(got.view(np.uint32), d["g"].numpy().view(np.uint32))
    d = _inputs(1, 96, 2, 128, 2301, "loge")
    got = _gpu_cumsum(d, "loge", 1)
    want = d["g"].numpy() * np.float32(1.4426950408889634)
    assert np.array_equal(got.view(np.uint32), want.astype(np.float32).view(np.uint32))


def test_gate_cumsum_rejects_overlap():
    need_gpu()
    from gated_delta_rule_gate_amd import KdaError, gate_cumsum

    g = torch.zeros((1, 64, 1, 128), dtype=torch.float32, device="cuda")
    with pytest.raises(KdaError):
        gate_cumsum(g, chunk_size=64, gate_kind="loge", out=g)
    with pytest.raises(KdaError):
        gate_cumsum(g, chunk_size=16, gate_kind="loge")


@pytest.mark.parametrize("schedule", ["fused", "split", "staged"])
@pytest.mark.parametrize("C", [64, 32])
def test_chunk_with_precumsummed_gate(schedule, C):
    """kda_gate_cumsum then kda_chunk_fwd(LOG2_CUMSUM) equals the recurrence on the raw gate,
    packed with empty slots."""
    need_gpu()
    from gated_delta_rule_gate_amd import chunk_kda, gate_cumsum

    lens = [0, 70, 129, 0, 33]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    d = _inputs(1, int(cu[-1]) + 11, 2, 128, 2400 + C, "softplus", n_slots=len(lens))
    dev = {k: (v.cuda() if v is not None else None) for k, v in d.items()}
    cu_d = torch.from_numpy(cu).cuda()
    b = gate_cumsum(dev["g"], chunk_size=C, gate_kind="softplus", A_log=dev["A_log"], dt_bias=dev["dt_bias"],
                    cu_seqlens=cu_d, out=torch.zeros_like(dev["g"]))
    o, ht = chunk_kda(dev["q"], dev["k"], dev["v"], b, dev["beta"], dev["h0"], cu_seqlens=cu_d,
                      output_final_state=True, chunk_size=C, gate_kind="log2_cumsum", schedule=schedule)
    torch.cuda.synchronize()
    g = _natural_gate(d, "softplus")
    o_ref, ht_ref = oracle.recurrent(f64(d["q"]), f64(d["k"]), f64(d["v"]), g, f64(d["beta"]), h0=f64(d["h0"]),
                                     cu_seqlens=cu)
    end = int(cu[-1])
    parity(o.float().cpu().numpy()[:, :end], o_ref[:, :end], "bf16", "o")
    parity(ht.cpu().numpy(), ht_ref, "bf16", "ht")


@pytest.mark.parametrize("schedule", ["auto", "staged"])
@pytest.mark.parametrize("K,V", [(64, 128), (96, 96), (48, 200)])
def test_precumsummed_gate_narrow_keys(schedule, K, V):
    """The pre-cumsummed gate has K channels per row while the kernels run at the
    tile width max(K, V) rounded up: every schedule must read it at its own
    stride. Packed with an empty slot, against the recurrence on the raw gate."""
    need_gpu()
    from gated_delta_rule_gate_amd import chunk_kda, gate_cumsum

    lens = [70, 0, 129, 33]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    d = kda_synth.chunk_inputs(1, int(cu[-1]) + 7, 2, K, V, dtype=torch.bfloat16, seed=2450 + K + V,
                               n_slots=len(lens))
    dev = {k: (v.cuda() if v is not None else None) for k, v in d.items()}
    cu_d = torch.from_numpy(cu).cuda()
    b = gate_cumsum(dev["x"], chunk_size=64, gate_kind="softplus", A_log=dev["A_log"], dt_bias=dev["dt_bias"],
                    cu_seqlens=cu_d, out=torch.zeros_like(dev["x"]))
    o, ht = chunk_kda(dev["q"], dev["k"], dev["v"], b, dev["beta"], dev["h0"], cu_seqlens=cu_d,
                      output_final_state=True, chunk_size=64, gate_kind="log2_cumsum", schedule=schedule)
    torch.cuda.synchronize()
    g = oracle.gate(oracle.GATE_SOFTPLUS, f64(d["x"]), f64(d["A_log"]), f64(d["dt_bias"]), -5.0)
    o_ref, ht_ref = oracle.recurrent(f64(d["q"]), f64(d["k"]), f64(d["v"]), g, f64(d["beta"]), h0=f64(d["h0"]),
                                     cu_seqlens=cu)
    end = int(cu[-1])
    parity(o.float().cpu().numpy()[:, :end], o_ref[:, :end], "bf16", "o")
    parity(ht.cpu().numpy(), ht_ref, "bf16", "ht")
