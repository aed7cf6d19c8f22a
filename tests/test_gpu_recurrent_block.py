"""GPU parity of the blocked recurrence (bf16, K = V = 128, sequences longer than
one token), which kda_recurrent_fwd runs for such calls, against the FP64 oracle.

The kernel scans 16-token blocks in the WY form of the chunked path; a block whose
in-block gate range could overflow the midpoint-offset operands ("FLA KDA Skill",
section "Safe gate numerical note") is evaluated one token at a time by the same
code. The cases below cover both: moderate gates (every block on the blocked
path), the softplus gate with large A_log (long in-block decays), a log2 gate with
-300 and -inf entries (those blocks must take the per-token path), block tails,
packed slots with empty and one-token slots, and the state updated in place.
"""
import numpy as np
import pytest
import torch

import kda_synth
import oracle
from kda_testlib import f64, need_gpu, parity

pytestmark = pytest.mark.gpu

GK = {"loge": oracle.GATE_LOGE, "safe": oracle.GATE_SAFE, "softplus": oracle.GATE_SOFTPLUS}


def _case(N, T, H, seed, gate, n_slots=None):
    d = kda_synth.chunk_inputs(N, T, H, 128, 128, dtype=torch.bfloat16, seed=seed, n_slots=n_slots)
    if gate == "log2":
        d["g"] = kda_synth.log2_gate(d["x"].numpy(), d["A_log"].numpy(), d["dt_bias"].numpy())
    elif gate == "loge":
        d["g"] = (-0.5 * d["x"].abs()).contiguous()
    else:
        d["g"] = d["x"]
    return d


def _oracle(d, gate, cu=None):
    if gate in ("log2", "loge"):
        g, is2 = f64(d["g"]), gate == "log2"
    else:
        g, is2 = oracle.gate(GK[gate], f64(d["x"]), f64(d["A_log"]), f64(d["dt_bias"]), -5.0), False
    return oracle.recurrent(f64(d["q"]), f64(d["k"]), f64(d["v"]), g, f64(d["beta"]), h0=f64(d["h0"]),
                            cu_seqlens=cu, g_is_log2=is2)


def _gpu(d, gate, cu=None, inplace=False, out=None):
    from gated_delta_rule_gate_amd import recurrent_kda

    dd = {k: (v.cuda() if v is not None else None) for k, v in d.items()}
    cu_d = None if cu is None else torch.from_numpy(np.asarray(cu, dtype=np.int32)).cuda()
    o, ht = recurrent_kda(dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"], dd["h0"], cu_seqlens=cu_d,
                          output_final_state=True, gate_kind=gate, A_log=dd["A_log"], dt_bias=dd["dt_bias"],
                          final_state=dd["h0"] if inplace else None, out=None if out is None else out.cuda())
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), ht.cpu().numpy()


@pytest.mark.parametrize("gate", ["log2", "loge", "safe", "softplus"])
@pytest.mark.parametrize("T", [45, 64, 2])
def test_block_gate_kinds(gate, T):
    """Full blocks, a 13-token tail (T = 45) and a two-token sequence."""
    need_gpu()
    d = _case(3, T, 2, 1300 + T, gate)
    o, ht = _gpu(d, gate)
    o_ref, ht_ref = _oracle(d, gate)
    parity(o, o_ref, "bf16", "o")
    parity(ht, ht_ref, "bf16", "ht")


def test_block_softplus_strong_decay():
    """A_log = log 16 on every head: softplus decays of tens of log2 units per token
    push most blocks past the operand range, so they run token by token."""
    need_gpu()
    d = _case(2, 70, 4, 1310, "softplus")
    d["A_log"] = torch.full_like(d["A_log"], float(np.log(16.0)))
    d["x"] = (d["x"] + 2.0).contiguous()
    d["g"] = d["x"]
    o, ht = _gpu(d, "softplus")
    o_ref, ht_ref = _oracle(d, "softplus")
    parity(o, o_ref, "bf16", "o")
    parity(ht, ht_ref, "bf16", "ht")


def test_block_extreme_log2_gate():
    """Isolated -300 and -inf log2 gates (a full reset of one channel) inside and at
    the edges of blocks. (Every gate mode of "FLA KDA Skill", section "Gate modes",
    yields a non-positive log decay, so no case grows the state.)"""
    need_gpu()
    d = _case(2, 48, 2, 1320, "log2")
    g = d["g"].numpy().copy()
    g[0, 5, 0, :7] = -300.0
    g[0, 16, 1, 30:40] = -np.inf
    g[1, 31, 0, 100] = -np.inf
    g[1, 33, 1, :] = -300.0
    d["g"] = torch.from_numpy(g)
    o, ht = _gpu(d, "log2")
    o_ref, ht_ref = _oracle(d, "log2")
    parity(o, o_ref, "bf16", "o")
    parity(ht, ht_ref, "bf16", "ht")


def test_block_packed_slots():
    """Packed slots: empty ones pass their state through bit for bit, a one-token slot,
    block tails; rows past the last offset hold NaN and are never read, and their
    output rows keep the sentinel."""
    need_gpu()
    lens = [0, 17, 1, 0, 40, 3, 0, 33]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    cap = int(cu[-1]) + 9
    d = _case(1, cap, 2, 1330, "safe", n_slots=len(lens))
    for key in ("q", "k", "v", "x"):
        d[key][:, int(cu[-1]):] = float("nan")
    d["g"] = d["x"]
    d["beta"][:, int(cu[-1]):] = float("nan")
    sentinel = torch.full((1, cap, 2, 128), 7.0, dtype=torch.bfloat16)
    o, ht = _gpu(d, "safe", cu=cu, out=sentinel)
    o_ref, ht_ref = _oracle(d, "safe", cu=cu)
    parity(o[:, : int(cu[-1])], o_ref[:, : int(cu[-1])], "bf16", "o")
    parity(ht, ht_ref, "bf16", "ht")
    assert (o[:, int(cu[-1]):] == 7.0).all()
    h0 = d["h0"].numpy()
    for n, L in enumerate(lens):
        if L == 0:
            assert np.array_equal(ht[n].view(np.uint32), h0[n].view(np.uint32))


def test_block_state_in_place():
    need_gpu()
    d = _case(4, 37, 3, 1340, "log2")
    o_ref, ht_ref = _oracle(d, "log2")
    o, ht = _gpu(d, "log2", inplace=True)
    parity(o, o_ref, "bf16", "o")
    parity(ht, ht_ref, "bf16", "ht")


def test_block_no_initial_state():
    need_gpu()
    d = _case(2, 33, 2, 1350, "log2")
    d["h0"] = None
    o, ht = _gpu(d, "log2")
    o_ref, ht_ref = _oracle(d, "log2")
    parity(o, o_ref, "bf16", "o")
    parity(ht, ht_ref, "bf16", "ht")
