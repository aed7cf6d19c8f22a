"""GPU parity of kda_chunk_fwd (chunked prefill) against the FP64 oracle.

All schedules (six staged kernels, the fused persistent kernel, and the
split pair of a per-chunk key-side kernel and a per-sequence state kernel) are
compared element by element with the token recurrence on the same seeded
inputs; the full-size shapes compare sampled (sequence, head) pairs, each an
exact sub-problem the oracle computes on its own.
"""
import numpy as np
import pytest
import torch

import kda_synth
import oracle
from kda_testlib import expect_unsupported, f64, need_gpu, parity, pipe_refuses

pytestmark = pytest.mark.gpu

GK = {"loge": oracle.GATE_LOGE, "safe": oracle.GATE_SAFE, "softplus": oracle.GATE_SOFTPLUS}


def make(B, T, H, D, dtype, seed, gate="safe", with_h0=True, n_slots=None):
    d = kda_synth.chunk_inputs(B, T, H, D, D, dtype=dtype, seed=seed, with_h0=with_h0, n_slots=n_slots)
    d["g"] = (-0.3 * d["x"].abs()).contiguous() if gate == "loge" else d["x"]
    return d


def oracle_run(d, gate, cu=None, lb=-5.0):
    if gate == "loge":
        g = f64(d["g"])
    else:
        g = oracle.gate(GK[gate], f64(d["x"]), f64(d["A_log"]), f64(d["dt_bias"]), lb)
    return oracle.recurrent(f64(d["q"]), f64(d["k"]), f64(d["v"]), g, f64(d["beta"]), h0=f64(d["h0"]),
                            cu_seqlens=cu)


def gpu_run(d, gate, schedule, cu=None, C=64, lb=-5.0, out=None, inplace=False):
    from gated_delta_rule_gate_amd import chunk_kda

    dd = {k: (v.cuda() if v is not None else None) for k, v in d.items()}
    cu_d = None if cu is None else torch.from_numpy(np.asarray(cu, dtype=np.int32)).cuda()
    o, ht = chunk_kda(dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"], dd["h0"], cu_seqlens=cu_d,
                      output_final_state=True, chunk_size=C, gate_kind=gate, A_log=dd["A_log"],
                      dt_bias=dd["dt_bias"], lower_bound=lb, schedule=schedule,
                      out=None if out is None else out.cuda(), final_state=dd["h0"] if inplace else None)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), ht.cpu().numpy()


def oracle_pairs(d, gate, pairs):
    os_, hts = [], []
    for b, h in pairs:
        one = {k: None for k in d}
        for key in ("q", "k", "v", "g", "x"):
            one[key] = d[key][b:b + 1, :, h:h + 1].contiguous()
        one["beta"] = d["beta"][b:b + 1, :, h:h + 1].contiguous()
        one["h0"] = None if d["h0"] is None else d["h0"][b:b + 1, h:h + 1].contiguous()
        one["A_log"] = d["A_log"][h:h + 1]
        one["dt_bias"] = d["dt_bias"][h:h + 1]
        o, ht = oracle_run(one, gate)
        os_.append(o[0, :, 0])
        hts.append(ht[0, 0])
    return np.stack(os_), np.stack(hts)


SCHEDULES = ["fused", "split", "staged", "pipe"]


def expect_fused_unsupported(d, cu=None, schedule="fused"):
    from gated_delta_rule_gate_amd import KdaError

    with pytest.raises(KdaError, match="UNSUPPORTED"):
        gpu_run(d, "safe", schedule, cu=cu)


@pytest.mark.parametrize("schedule", SCHEDULES)
@pytest.mark.parametrize("C", [64, 32])
def test_fp32_small_config(schedule, C):
    """fp32, B1 T256 H2 K=V=64, safe gate, h0 = 0, final state returned (the fused
    kernel takes bf16 only: fp32 runs the staged schedule, also under "auto")."""
    need_gpu()
    d = make(1, 256, 2, 64, torch.float32, 1000, with_h0=False)
    if schedule in ("fused", "split", "pipe"):
        expect_fused_unsupported(d, schedule=schedule)
        schedule = "auto"
    o, ht = gpu_run(d, "safe", schedule, C=C)
    o_ref, ht_ref = oracle_run(d, "safe")
    parity(o, o_ref, "fp32", "o")
    parity(ht, ht_ref, "fp32", "ht")


@pytest.mark.parametrize("schedule", SCHEDULES)
@pytest.mark.parametrize("gate", ["safe", "softplus", "loge"])
@pytest.mark.parametrize("C", [64, 32])
def test_bf16_ragged(schedule, gate, C):
    """bf16, T not a multiple of the chunk (several chunks and a ragged tail)."""
    need_gpu()
    d = make(2, 203, 3, 128, torch.bfloat16, 200 + C, gate=gate)
    if pipe_refuses(schedule, gate, C):
        return expect_unsupported(lambda: gpu_run(d, gate, schedule, C=C))
    o, ht = gpu_run(d, gate, schedule, C=C)
    o_ref, ht_ref = oracle_run(d, gate)
    parity(o, o_ref, "bf16", "o")
    parity(ht, ht_ref, "bf16", "ht")


@pytest.mark.parametrize("schedule", SCHEDULES)
@pytest.mark.parametrize("D", [64, 256])
def test_bf16_widths(schedule, D):
    need_gpu()
    d = make(2, 150, 2, D, torch.bfloat16, 300 + D)
    if pipe_refuses(schedule, K=D):
        return expect_unsupported(lambda: gpu_run(d, "safe", schedule))
    if schedule in ("fused", "split") and D == 256:
        from gated_delta_rule_gate_amd import KdaError

        with pytest.raises(KdaError, match="UNSUPPORTED"):  # the fused tile needs D <= 128
            gpu_run(d, "safe", schedule)
        return
    o, ht = gpu_run(d, "safe", schedule)
    o_ref, ht_ref = oracle_run(d, "safe")
    parity(o, o_ref, "bf16", "o")
    parity(ht, ht_ref, "bf16", "ht")


@pytest.mark.parametrize("schedule", SCHEDULES)
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_packed_empty_slots_tail(schedule, dtype):
    """Empty slots (first, inside, last) pass their state through bit for bit; the tail past
    the last offset is NaN-poisoned on input and must keep its sentinel in o."""
    need_gpu()
    lens = [0, 70, 64, 1, 0, 129, 17, 0]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    cap = int(cu[-1]) + 37
    D = 64 if dtype == torch.float32 else 128
    d = make(1, cap, 2, D, dtype, 400, gate="safe", n_slots=len(lens))
    if schedule in ("fused", "split", "pipe") and dtype == torch.float32:
        expect_fused_unsupported(d, cu, schedule)
        schedule = "auto"
    end = int(cu[-1])
    for key in ("q", "k", "v", "g"):
        d[key][:, end:] = float("nan")
    d["beta"][:, end:] = float("nan")
    sentinel = torch.full((1, cap, 2, D), 3.0, dtype=dtype)
    o, ht = gpu_run(d, "safe", schedule, cu=cu, out=sentinel)
    o_ref, ht_ref = oracle_run(d, "safe", cu=cu)
    name = "fp32" if dtype == torch.float32 else "bf16"
    parity(o[:, :end], o_ref[:, :end], name, "o")
    parity(ht, ht_ref, name, "ht")
    assert (o[:, end:] == 3.0).all()
    h0 = d["h0"].numpy()
    for n, L in enumerate(lens):
        if L == 0:
            assert np.array_equal(ht[n].view(np.uint32), h0[n].view(np.uint32)), n


@pytest.mark.parametrize("schedule", SCHEDULES)
def test_short_and_single_token(schedule):
    need_gpu()
    for T in (1, 5, 16, 17):
        d = make(1, T, 2, 128, torch.bfloat16, 500 + T)
        o, ht = gpu_run(d, "safe", schedule)
        o_ref, ht_ref = oracle_run(d, "safe")
        parity(o, o_ref, "bf16", "o T=%d" % T)
        parity(ht, ht_ref, "bf16", "ht T=%d" % T)


@pytest.mark.parametrize("schedule", SCHEDULES)
def test_split_resume_and_in_place(schedule):
    """run(x[0:T]) == run(x[T1:T] | h0 = run(x[0:T1]).ht); ht may alias h0."""
    need_gpu()
    d = make(1, 300, 2, 128, torch.bfloat16, 600)
    o_full, ht_full = gpu_run(d, "safe", schedule)
    T1 = 128
    a = {k: (v[:, :T1].contiguous() if (v is not None and k in ("q", "k", "v", "g", "x", "beta")) else v)
         for k, v in d.items()}
    b = {k: (v[:, T1:].contiguous() if (v is not None and k in ("q", "k", "v", "g", "x", "beta")) else v)
         for k, v in d.items()}
    oa, ha = gpu_run(a, "safe", schedule)
    b["h0"] = torch.from_numpy(ha)
    ob, hb = gpu_run(b, "safe", schedule, inplace=True)
    parity(np.concatenate([oa, ob], axis=1), o_full, "bf16", "o")
    parity(hb, ht_full, "bf16", "ht")


def test_recurrent_chunk_cross_check():
    """kda_recurrent_fwd with the per-token log2 gate equals kda_chunk_fwd on the same decay."""
    need_gpu()
    from gated_delta_rule_gate_amd import recurrent_kda

    for dtype, D, schedule, name in ((torch.float32, 64, "auto", "fp32"), (torch.bfloat16, 128, "fused", "bf16")):
        d = make(2, 130, 2, D, dtype, 700)
        g = oracle.gate(oracle.GATE_SAFE, f64(d["x"]), f64(d["A_log"]), f64(d["dt_bias"]), -5.0)
        d["g"] = torch.from_numpy(g.astype(np.float32))
        oc, hc = gpu_run(d, "loge", schedule)
        dd = {k: (v.cuda() if v is not None else None) for k, v in d.items()}
        orr, hr = recurrent_kda(dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"], dd["h0"], output_final_state=True,
                                gate_kind="loge")
        torch.cuda.synchronize()
        parity(oc, orr.float().cpu().numpy(), name, "o chunk vs recurrent")
        parity(hc, hr.cpu().numpy(), name, "ht chunk vs recurrent")


def test_config_b4_t2048_h16_full():
    """B4 T2048 H16 K=V=128 bf16, C=64, safe gate, h0 ~ 0.1 N(0,1): every output checked."""
    need_gpu()
    d = make(4, 2048, 16, 128, torch.bfloat16, 1001)
    o, ht = gpu_run(d, "safe", "auto")
    o_ref, ht_ref = oracle_run(d, "safe")
    parity(o, o_ref, "bf16", "o")
    parity(ht, ht_ref, "bf16", "ht")


def test_headline_full():
    """The headline B4 T4096 H64 K=V=128 bf16, C=64, safe gate, h0 and ht, in the launch
    configuration the benchmark times: every output of every (sequence, head) pair
    against the oracle (about 3 s of FP64 recurrence on the host cores)."""
    need_gpu()
    d = make(4, 4096, 64, 128, torch.bfloat16, 1002)
    o, ht = gpu_run(d, "safe", "auto")
    o_ref, ht_ref = oracle_run(d, "safe")
    parity(o, o_ref, "bf16", "o")
    parity(ht, ht_ref, "bf16", "ht")


@pytest.mark.parametrize("shape", [(1, 8192, 96, 128), (2, 16384, 16, 128), (8, 2048, 32, 256), (8, 1024, 8, 64)])
def test_contract_shapes_sampled(shape):
    """The other contract shapes, in the launch configuration the benchmark times; the
    oracle checks sampled (sequence, head) pairs in full."""
    need_gpu()
    B, T, H, D = shape
    d = make(B, T, H, D, torch.bfloat16, 1002 + B * 7 + H)
    o, ht = gpu_run(d, "safe", "auto")
    rng = np.random.default_rng(B * 1000 + H)
    pairs = [(0, 0), (B - 1, H - 1)] + [(int(rng.integers(B)), int(rng.integers(H))) for _ in range(2)]
    o_ref, ht_ref = oracle_pairs(d, "safe", pairs)
    got_o = np.stack([o[b, :, h] for b, h in pairs])
    got_h = np.stack([ht[b, h] for b, h in pairs])
    parity(got_o, o_ref, "bf16", "o")
    parity(got_h, ht_ref, "bf16", "ht")


@pytest.mark.parametrize("schedule", SCHEDULES + ["recurrent"])
def test_long_sequence(schedule):
    """One 65536-token sequence (1024 chunks in one chain; token offsets past
    2^24 elements), two heads, safe gate with the bound close to 0 so the state
    keeps its history: every output against the oracle."""
    need_gpu()
    from gated_delta_rule_gate_amd import recurrent_kda

    B, T, H, D = 1, 65536, 2, 128
    d = make(B, T, H, D, torch.bfloat16, 1700)
    lb = -0.05
    if schedule == "recurrent":
        dd = {k: (v.cuda() if v is not None else None) for k, v in d.items()}
        o, ht = recurrent_kda(dd["q"], dd["k"], dd["v"], dd["x"], dd["beta"], dd["h0"], output_final_state=True,
                              gate_kind="safe", A_log=dd["A_log"], dt_bias=dd["dt_bias"], lower_bound=lb)
        torch.cuda.synchronize()
        o, ht = o.float().cpu().numpy(), ht.cpu().numpy()
    else:
        o, ht = gpu_run(d, "safe", schedule, lb=lb)
    o_ref, ht_ref = oracle_run(d, "safe", lb=lb)
    parity(o, o_ref, "bf16", "o")
    parity(ht, ht_ref, "bf16", "ht")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("pairs", [144, 96, 48, 6])
def test_value_column_split(D, pairs):
    """The fused kernel splits the value columns over 1, 2, 4 or 8 workgroups per
    (sequence, head) so that few pairs still cover 256 compute units: every split
    checked in full, with an h0, a ragged tail and several chunks."""
    need_gpu()
    B = 3 if pairs % 3 == 0 else 2
    d = make(B, 70, pairs // B, D, torch.bfloat16, 500 + pairs + D)
    o, ht = gpu_run(d, "safe", "fused")
    o_ref, ht_ref = oracle_run(d, "safe")
    parity(o, o_ref, "bf16", "o")
    parity(ht, ht_ref, "bf16", "ht")


@pytest.mark.parametrize("schedule", ["auto", "fused"])
def test_config_varlen_softplus(schedule):
    """Packed capacity 16384, H16 D128, 10 slots (two empty), terminal offset 512 below
    capacity, non-safe softplus gate, h0 per slot: every head and slot in full, the
    empty slots' states bit for bit."""
    need_gpu()
    cu = kda_synth.varlen_offsets(1003)
    assert cu[-1] == 15872 and len(cu) == 11
    d = make(1, 16384, 16, 128, torch.bfloat16, 1003, gate="softplus", n_slots=10)
    o, ht = gpu_run(d, "softplus", schedule, cu=cu)
    o_ref, ht_ref = oracle_run(d, "softplus", cu=cu)
    end = int(cu[-1])
    parity(o[:, :end], o_ref[:, :end], "bf16", "o")
    parity(ht, ht_ref, "bf16", "ht")
    empty = [n for n in range(10) if cu[n] == cu[n + 1]]
    assert len(empty) == 2
    for n in empty:
        assert np.array_equal(ht[n].view(np.uint32), d["h0"][n].numpy().view(np.uint32)), \
            "empty slot %d state not passed through" % n


def test_empty_batch():
    """T = 0: no tokens, NULL token pointers; every final state is its h0 bit for bit
    (every schedule and the recurrent kernel), the chunk cumsum writes nothing, and
    the backward returns dh0 = dht and zero parameter gradients."""
    need_gpu()
    from gated_delta_rule_gate_amd import chunk_kda, chunk_kda_bwd, gate_cumsum, recurrent_kda

    B, H, D = 2, 3, 128
    d = make(B, 0, H, D, torch.bfloat16, 1800)
    dd = {k: (v.cuda() if v is not None else None) for k, v in d.items()}
    h0 = d["h0"].numpy()
    kw = dict(gate_kind="safe", A_log=dd["A_log"], dt_bias=dd["dt_bias"], lower_bound=-5.0)
    for schedule in SCHEDULES:
        o, ht = chunk_kda(dd["q"], dd["k"], dd["v"], dd["x"], dd["beta"], dd["h0"], output_final_state=True,
                          schedule=schedule, **kw)
        torch.cuda.synchronize()
        assert o.shape == (B, 0, H, D)
        assert np.array_equal(ht.cpu().numpy().view(np.uint32), h0.view(np.uint32)), schedule
    o, ht = recurrent_kda(dd["q"], dd["k"], dd["v"], dd["x"], dd["beta"], dd["h0"], output_final_state=True, **kw)
    torch.cuda.synchronize()
    assert np.array_equal(ht.cpu().numpy().view(np.uint32), h0.view(np.uint32))
    b = gate_cumsum(dd["x"], chunk_size=64, **kw)
    torch.cuda.synchronize()
    assert b.shape == (B, 0, H, D)
    dht = torch.randn((B, H, D, D), dtype=torch.float32, device="cuda")
    do = torch.empty((B, 0, H, D), dtype=torch.bfloat16, device="cuda")
    g = chunk_kda_bwd(dd["q"], dd["k"], dd["v"], dd["x"], dd["beta"], do, dd["h0"], dht=dht, **kw)
    torch.cuda.synchronize()
    assert torch.equal(g["dh0"], dht)
    assert g["dq"].shape == (B, 0, H, D) and g["dg"].shape == (B, 0, H, D)
    assert not g["dA_log"].any() and not g["ddt_bias"].any()


@pytest.mark.parametrize("offsets,T,want", [
    ([0, 70, 134, 135, 135, 264], 300, 0),     # valid, an empty slot, tail below capacity
    ([0, 0, 0], 0, 0),                         # all empty, zero capacity
    ([0, 70, 60, 200], 300, 1),                # a decreasing offset
    ([-4, 10, 20], 300, 2),                    # negative first offset
    ([0, 70, 301], 300, 4),                    # past the capacity
    ([5, 3, 400], 300, 1 | 4),                 # several at once
    (list(range(0, 3000, 3)), 2997, 0),        # many slots (several rounds of the check's loop)
    (list(range(0, 3000, 3))[:700] + [5] + list(range(2100, 2997, 3)), 2997, 1),
])
def test_check_offsets(offsets, T, want):
    """The device-side check of the packed-offset contract, one flag bit per violation."""
    need_gpu()
    from gated_delta_rule_gate_amd import check_offsets

    cu = torch.tensor(offsets, dtype=torch.int32, device="cuda")
    assert check_offsets(cu, T) == want


@pytest.mark.parametrize("D,C,gate", [(64, 32, "softplus"), (128, 64, "safe")])
def test_staged_many_items(D, C, gate):
    """The staged chain with more (chunk, head) items than its gate step's persistent
    workgroups (four per compute unit), each sequence ending in a ragged chunk; the
    state scan runs one workgroup per (sequence, head) for bf16 inputs."""
    need_gpu()
    H = 4096 // D
    d = make(2, 1000, H, D, torch.bfloat16, 3300 + D, gate=gate)
    o, ht = gpu_run(d, gate, "staged", C=C)
    o_ref, ht_ref = oracle_run(d, gate)
    parity(o, o_ref, "bf16", "o")
    parity(ht, ht_ref, "bf16", "ht")
