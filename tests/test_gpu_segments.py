"""GPU parity of the split schedule's chain-parallel state scan against the FP64 oracle.

kda_args.segment cuts each (sequence, head) chain into segments of that many
chunks: later segments run from the identity and from zero side by side, their
affine maps h_out = M h_in + B are chained in fp32 afterwards, and E h_in is
added to each chunk's o_local. The cases force segment lengths from one chunk
to longer than the sequence, over ragged tails, packed slots shorter than one
segment (and empty ones, whose state passes through bit for bit), every gate
kind, q l2-normalisation, K != V with padded channels, grouped value heads, a
state updated in place and a missing h0; the long case checks the cumulative
decay of a 64-chunk chain against the serial scan and the oracle ("FLA KDA
Skill", section "Correctness checklist": CP paths, long-sequence cumulative
decay, chunk boundaries, ragged varlen boundaries).
"""
import numpy as np
import pytest
import torch

import kda_synth
import oracle
from kda_testlib import f64, need_gpu, parity

pytestmark = pytest.mark.gpu

GK = {"loge": oracle.GATE_LOGE, "safe": oracle.GATE_SAFE, "softplus": oracle.GATE_SOFTPLUS}


def _make(B, T, H, K, V, seed, gate="safe", with_h0=True, n_slots=None, Hk=None):
    d = kda_synth.chunk_inputs(B, T, H, K, V, dtype=torch.bfloat16, seed=seed, with_h0=with_h0, n_slots=n_slots)
    if Hk is not None:  # the first Hk heads serve as the q/k heads (value head h reads h / (H / Hk))
        d["q"] = d["q"][:, :, :Hk].contiguous()
        d["k"] = d["k"][:, :, :Hk].contiguous()
    d["g"] = (-0.3 * d["x"].abs()).contiguous() if gate == "loge" else d["x"]
    return d


def _oracle(d, gate, cu=None):
    if gate == "loge":
        g = f64(d["g"])
    else:
        kind = GK["softplus" if gate == "log2_cumsum" else gate]
        g = oracle.gate(kind, f64(d["x"]), f64(d["A_log"]), f64(d["dt_bias"]), -5.0)
    G = d["v"].shape[2] // d["q"].shape[2]
    q = f64(d["q"].repeat_interleave(G, dim=2)) if G > 1 else f64(d["q"])
    k = f64(d["k"].repeat_interleave(G, dim=2)) if G > 1 else f64(d["k"])
    return oracle.recurrent(q, k, f64(d["v"]), g, f64(d["beta"]),
                            h0=None if d["h0"] is None else f64(d["h0"]), cu_seqlens=cu)


def _gpu(d, gate, segment, cu=None, C=64, out=None, inplace=False, q_l2norm=False, schedule="split"):
    from gated_delta_rule_gate_amd import chunk_kda, gate_cumsum

    dd = {k: (v.cuda() if v is not None else None) for k, v in d.items()}
    cu_d = None if cu is None else torch.from_numpy(np.asarray(cu, dtype=np.int32)).cuda()
    g, kind = dd["g"], gate
    if gate == "log2_cumsum":
        g = gate_cumsum(dd["x"], chunk_size=C, cu_seqlens=cu_d, gate_kind="softplus", A_log=dd["A_log"],
                        dt_bias=dd["dt_bias"])
    o, ht = chunk_kda(dd["q"], dd["k"], dd["v"], g, dd["beta"], dd["h0"], cu_seqlens=cu_d,
                      output_final_state=True, chunk_size=C, gate_kind=kind, A_log=dd["A_log"],
                      dt_bias=dd["dt_bias"], lower_bound=-5.0, schedule=schedule, segment=segment,
                      out=None if out is None else out.cuda(), final_state=dd["h0"] if inplace else None,
                      q_l2norm=q_l2norm)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), ht.cpu().numpy()


@pytest.mark.parametrize("segment", [1, 2, 3, 5, 9])
def test_dense_segment_lengths(segment):
    """B2 T300 H2 D128 (five chunks, the last of 44 rows): one-chunk segments, a
    segment of three beside one of two, and one segment longer than the sequence."""
    need_gpu()
    d = _make(2, 300, 2, 128, 128, 5100 + segment)
    o, ht = _gpu(d, "safe", segment)
    o_ref, ht_ref = _oracle(d, "safe")
    parity(o, o_ref, "bf16", "o")
    parity(ht, ht_ref, "bf16", "ht")


@pytest.mark.parametrize("gate", ["softplus", "loge", "log2_cumsum"])
def test_gate_kinds(gate):
    need_gpu()
    d = _make(1, 400, 3, 128, 128, 5110, gate=gate)
    o, ht = _gpu(d, gate, 2)
    o_ref, ht_ref = _oracle(d, gate)
    parity(o, o_ref, "bf16", "o")
    parity(ht, ht_ref, "bf16", "ht")


@pytest.mark.parametrize("C,D", [(32, 128), (64, 64), (32, 64)])
def test_chunk_and_width(C, D):
    need_gpu()
    d = _make(2, 333, 2, D, D, 5120 + C + D)
    o, ht = _gpu(d, "safe", 3, C=C)
    o_ref, ht_ref = _oracle(d, "safe")
    parity(o, o_ref, "bf16", "o")
    parity(ht, ht_ref, "bf16", "ht")


@pytest.mark.parametrize("K,V", [(96, 128), (128, 72), (64, 40)])
def test_padded_widths(K, V):
    """Channels past K and columns past V run as zeros in the tile: the columns of M
    for padded channels only decay and never reach o or ht."""
    need_gpu()
    d = _make(2, 260, 2, K, V, 5130 + K + V)
    o, ht = _gpu(d, "safe", 2)
    o_ref, ht_ref = _oracle(d, "safe")
    parity(o, o_ref, "bf16", "o")
    parity(ht, ht_ref, "bf16", "ht")


def test_grouped_heads_and_qnorm():
    """Four value heads over two q/k heads, raw q normalised inside (the row scales
    reach E and o_local alike)."""
    need_gpu()
    d = _make(1, 320, 4, 128, 128, 5140, Hk=2)
    raw = d["q"].float() * torch.linspace(0.5, 3.0, 320).reshape(1, 320, 1, 1)
    d["q"] = raw.to(torch.bfloat16)
    o, ht = _gpu(d, "safe", 2, q_l2norm=True)
    dn = dict(d)
    dn["q"] = torch.from_numpy(oracle.l2norm_rows(f64(d["q"])))
    o_ref, ht_ref = _oracle(dn, "safe")
    parity(o, o_ref, "bf16", "o")
    parity(ht, ht_ref, "bf16", "ht")


def test_packed_slots():
    """Packed slots: empty ones (state bit for bit), one-token, shorter than a
    segment, exactly one segment, several segments with a ragged tail. Rows past
    the last offset hold NaN and their output rows keep the sentinel."""
    need_gpu()
    lens = [0, 200, 1, 64, 0, 520, 130, 0]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    end = int(cu[-1])
    cap = end + 23
    d = _make(1, cap, 2, 128, 128, 5150, n_slots=len(lens))
    for key in ("q", "k", "v", "x"):
        d[key][:, end:] = float("nan")
    d["g"] = d["x"]
    d["beta"][:, end:] = float("nan")
    sentinel = torch.full((1, cap, 2, 128), 5.0, dtype=torch.bfloat16)
    o, ht = _gpu(d, "safe", 2, cu=cu, out=sentinel)
    o_ref, ht_ref = _oracle(d, "safe", cu=cu)
    parity(o[:, :end], o_ref[:, :end], "bf16", "o")
    parity(ht, ht_ref, "bf16", "ht")
    assert (o[:, end:] == 5.0).all()
    h0 = d["h0"].numpy()
    for n, L in enumerate(lens):
        if L == 0:
            assert np.array_equal(ht[n].view(np.uint32), h0[n].view(np.uint32)), n


def test_state_in_place_and_no_h0():
    need_gpu()
    d = _make(2, 270, 2, 128, 128, 5160)
    o_ref, ht_ref = _oracle(d, "safe")
    o, ht = _gpu(d, "safe", 2, inplace=True)
    parity(o, o_ref, "bf16", "o")
    parity(ht, ht_ref, "bf16", "ht")
    d = _make(2, 270, 2, 128, 128, 5161, with_h0=False)
    o, ht = _gpu(d, "safe", 1)
    o_ref, ht_ref = _oracle(d, "safe")
    parity(o, o_ref, "bf16", "o")
    parity(ht, ht_ref, "bf16", "ht")


def test_long_chain_against_serial():
    """A 64-chunk chain (T 4096) in eight segments against the oracle, and against
    the serial scan of the same kernels within the same bounds."""
    need_gpu()
    d = _make(1, 4096, 2, 128, 128, 5170)
    o, ht = _gpu(d, "safe", 8)
    o_s, ht_s = _gpu(d, "safe", -1)
    o_ref, ht_ref = _oracle(d, "safe")
    parity(o, o_ref, "bf16", "o")
    parity(ht, ht_ref, "bf16", "ht")
    parity(o, o_s.astype(np.float64), "bf16", "o vs serial")
    parity(ht, ht_s.astype(np.float64), "bf16", "ht vs serial")


def test_auto_segment_choice():
    """AUTO cuts the chain where the serial scan leaves compute units idle (few long
    sequences) and keeps it whole where the pairs fill the device."""
    need_gpu()
    from gated_delta_rule_gate_amd import resolved_schedule, resolved_segment

    q = torch.empty((2, 16384, 16, 128), dtype=torch.bfloat16, device="meta")
    assert resolved_schedule(q, q, 16, 2) == "split"
    assert resolved_segment(q, q, 16, 2) > 0
    q = torch.empty((4, 4096, 64, 128), dtype=torch.bfloat16, device="meta")
    assert resolved_segment(q, q, 64, 4) == 0
    assert resolved_segment(q, q, 64, 4, schedule="split", segment=-1) == 0
    assert resolved_segment(q, q, 64, 4, schedule="split", segment=7) == 7
