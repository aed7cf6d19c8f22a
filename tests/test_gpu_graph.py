"""HIP-graph replay of the entry points.

Neither call reads a device value on the host, allocates inside the library or
issues a memset, so each can be captured once and replayed ("attention-gym"
page, "Agent note": graph-capturable, cu_seqlens on the device). Every replay
here runs on inputs and cu_seqlens rewritten in place since the capture, with
eager calls and synchronisations between the replays, and must equal an eager
call on the same inputs bit for bit (both run the same kernels, which hold no
state between calls).
"""
import numpy as np
import pytest
import torch

import kda_synth
from kda_testlib import need_gpu

pytestmark = pytest.mark.gpu

CAP, H, D, SLOTS = 1536, 4, 128, 5


def _chunk_case(seed):
    d = kda_synth.chunk_inputs(1, CAP, H, D, D, dtype=torch.bfloat16, seed=seed, n_slots=SLOTS)
    cu = kda_synth.varlen_offsets(seed, n_slots=SLOTS, n_empty=1, total=CAP - 64 - seed % 37, max_len=CAP)
    d["cu"] = torch.from_numpy(cu)
    return d


def _refill(dst, src):
    for key, t in src.items():
        if t is not None:
            dst[key].copy_(t)


@pytest.mark.parametrize("schedule", ["auto", "split", "staged", "pipe"])
def test_chunk_graph_replay_with_new_offsets(schedule):
    from gated_delta_rule_gate_amd import chunk_kda

    need_gpu()
    first = _chunk_case(11)
    dev = {k: v.cuda() for k, v in first.items() if v is not None}
    o_g = torch.zeros((1, CAP, H, D), dtype=torch.bfloat16, device="cuda")
    ht_g = torch.empty((SLOTS, H, D, D), dtype=torch.float32, device="cuda")

    def call(o, ht):
        chunk_kda(dev["q"], dev["k"], dev["v"], dev["x"], dev["beta"], dev["h0"], cu_seqlens=dev["cu"],
                  chunk_size=64, gate_kind="safe", A_log=dev["A_log"], dt_bias=dev["dt_bias"], lower_bound=-5.0,
                  schedule=schedule, out=o, final_state=ht)

    call(o_g, ht_g)  # warm-up outside the capture (loads the library, compiles nothing)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(o_g, ht_g)
    torch.cuda.synchronize()

    o_e = torch.zeros_like(o_g)
    ht_e = torch.empty_like(ht_g)
    for rep, seed in enumerate([12, 13, 14, 15]):
        case = _chunk_case(seed)
        _refill(dev, {k: v for k, v in case.items() if v is not None})
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        call(o_e, ht_e)  # eager, same inputs
        torch.cuda.synchronize()
        n_valid = int(case["cu"][-1])
        assert torch.equal(o_g[:, :n_valid], o_e[:, :n_valid]), "replay %d: o differs from the eager call" % rep
        assert torch.equal(ht_g, ht_e), "replay %d: ht differs from the eager call" % rep
        # the replay really used the new offsets: an empty slot passes h0 through
        cu = case["cu"].numpy()
        for n in range(SLOTS):
            if cu[n] == cu[n + 1]:
                assert torch.equal(ht_g[n], dev["h0"][n])


def test_recurrent_graph_replay_in_place_state():
    from gated_delta_rule_gate_amd import recurrent_kda

    need_gpu()
    N, T = 8, 4

    def case(seed):
        d = kda_synth.chunk_inputs(N, T, H, D, D, dtype=torch.bfloat16, seed=seed)
        d["g"] = kda_synth.log2_gate(d["x"].numpy(), d["A_log"].numpy(), d["dt_bias"].numpy())
        return d

    first = case(21)
    dev = {k: v.cuda() for k, v in first.items() if v is not None}
    state_g = dev["h0"].clone()
    o_g = torch.empty((N, T, H, D), dtype=torch.bfloat16, device="cuda")

    def call(state, o):
        recurrent_kda(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], state, final_state=state, out=o)

    warm = state_g.clone()
    call(warm, o_g)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(state_g, o_g)
    torch.cuda.synchronize()
    state_g.copy_(dev["h0"])  # the capture itself ran nothing

    o_e = torch.empty_like(o_g)
    for rep, seed in enumerate([22, 23, 24]):
        _refill(dev, {k: v for k, v in case(seed).items() if v is not None and k != "h0"})
        state_e = state_g.clone()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        call(state_e, o_e)
        torch.cuda.synchronize()
        assert torch.equal(o_g, o_e), "replay %d: o differs from the eager call" % rep
        assert torch.equal(state_g, state_e), "replay %d: state differs from the eager call" % rep
        assert not torch.equal(state_g, dev["h0"]), "the replay did not advance the state"


def test_gate_cumsum_graph_replay():
    from gated_delta_rule_gate_amd import gate_cumsum

    need_gpu()
    d = kda_synth.chunk_inputs(2, 200, H, D, D, dtype=torch.bfloat16, seed=31)
    x = d["x"].cuda()
    A_log, dt_bias = d["A_log"].cuda(), d["dt_bias"].cuda()
    out_g = torch.empty_like(x)
    gate_cumsum(x, chunk_size=64, A_log=A_log, dt_bias=dt_bias, out=out_g)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gate_cumsum(x, chunk_size=64, A_log=A_log, dt_bias=dt_bias, out=out_g)
    rng = np.random.default_rng(32)
    for rep in range(3):
        x.copy_(torch.from_numpy(rng.standard_normal(x.shape).astype(np.float32)))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        out_e = gate_cumsum(x, chunk_size=64, A_log=A_log, dt_bias=dt_bias)
        torch.cuda.synchronize()
        assert torch.equal(out_g, out_e), "replay %d differs from the eager call" % rep


def test_chunk_bwd_graph_replay():
    """The backward allocates nothing inside the library and never syncs: captured
    once with its workspace and outputs fixed, each replay on rewritten inputs
    equals an eager call bit for bit."""
    from gated_delta_rule_gate_amd import _binding as kb

    need_gpu()
    import ctypes

    first = _chunk_case(41)
    dev = {k: v.cuda() for k, v in first.items() if v is not None}
    rng = np.random.default_rng(42)
    do = torch.from_numpy(rng.standard_normal((1, CAP, H, D)).astype(np.float32)).to(torch.bfloat16).cuda()
    a = kb.make_args(dev["q"], dev["v"], H, SLOTS, "safe", chunk_size=64, A_log=dev["A_log"], dt_bias=dev["dt_bias"],
                     lower_bound=-5.0, schedule="staged")
    L = kb.lib()
    ws = torch.empty((int(L.kda_chunk_bwd_workspace_bytes(ctypes.byref(a))),), dtype=torch.uint8, device="cuda")

    def outputs():
        return dict(dq=torch.zeros_like(dev["q"]), dk=torch.zeros_like(dev["k"]), dv=torch.zeros_like(dev["v"]),
                    dg=torch.zeros_like(dev["x"]), dbeta=torch.zeros_like(dev["beta"]),
                    dh0=torch.zeros_like(dev["h0"]), dA=torch.zeros((H,), device="cuda"),
                    ddt=torch.zeros((H, D), device="cuda"))

    def call(o):
        P = kb._ptr
        kb.check(L.kda_chunk_bwd(ctypes.byref(a), P(dev["q"]), P(dev["k"]), P(dev["v"]), P(dev["x"]), P(dev["beta"]),
                                 P(dev["h0"]), P(dev["cu"]), P(do), None, P(o["dq"]), P(o["dk"]), P(o["dv"]),
                                 P(o["dg"]), P(o["dbeta"]), P(o["dh0"]), P(o["dA"]), P(o["ddt"]), P(ws),
                                 ctypes.c_size_t(ws.numel()), kb._stream()))

    og = outputs()
    call(og)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(og)
    torch.cuda.synchronize()
    for rep, seed in enumerate([43, 44, 45]):
        case = _chunk_case(seed)
        _refill(dev, {k: v for k, v in case.items() if v is not None})
        do.copy_(torch.from_numpy(rng.standard_normal(do.shape).astype(np.float32)).to(torch.bfloat16))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        oe = outputs()
        call(oe)
        torch.cuda.synchronize()
        n = int(case["cu"][-1])
        for key in ("dq", "dk", "dv", "dg", "dbeta"):
            assert torch.equal(og[key][:, :n], oe[key][:, :n]), "replay %d: %s differs" % (rep, key)
        for key in ("dh0", "dA", "ddt"):
            assert torch.equal(og[key], oe[key]), "replay %d: %s differs" % (rep, key)
