"""Per-step GPU parity of the staged chunk schedule against the oracle's chunked form.

Each step runs alone on the chunked form's own FP64 intermediates (written into
the workspace as fp32), so a failure points at one kernel: (1) gate cumsum,
(2) grams, (3) triangular solve, (4) WY factors, (5) state scan, (6) output.
"""
import numpy as np
import pytest
import torch

import kda_synth
import oracle
from kda_testlib import f64, need_gpu

pytestmark = pytest.mark.gpu


def rel_rms(got, want):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    return float(np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-300))


def setup(dtype, D, gate="safe", C=64, lens=None, seed=900):
    from gated_delta_rule_gate_amd._binding import StagedRun

    if lens is None:
        B, T, N, cu = 2, 150, 2, None
    else:
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        B, T, N = 1, int(cu[-1]) + 11, len(lens)
    d = kda_synth.chunk_inputs(B, T, 2, D, D, dtype=dtype, seed=seed, n_slots=N)
    kind = oracle.GATE_SAFE if gate == "safe" else oracle.GATE_SOFTPLUS
    g = oracle.gate(kind, f64(d["x"]), f64(d["A_log"]), f64(d["dt_bias"]), -5.0)
    o2, h2, it = oracle.chunked_forward(f64(d["q"]), f64(d["k"]), f64(d["v"]), g, f64(d["beta"]), h0=f64(d["h0"]),
                                        cu_seqlens=cu, chunk_size=C, anchored=(gate == "safe"), emit=True)
    dd = {k: v.cuda() for k, v in d.items()}
    cu_d = None if cu is None else torch.from_numpy(cu).cuda()
    run = StagedRun(dd["q"], dd["k"], dd["v"], dd["x"], dd["beta"], dd["h0"], cu_seqlens=cu_d, chunk_size=C,
                    gate_kind=gate, A_log=dd["A_log"], dt_bias=dd["dt_bias"], lower_bound=-5.0)
    run.run("index")
    valid = np.ones(B * T, dtype=bool) if cu is None else (np.arange(T) < cu[-1])
    return run, it, o2, h2, valid, B, T


def put(run, name, arr, B, T):
    """Writes an oracle intermediate into the workspace (fp32; rows outside the contract as 0)."""
    a = arr if name == "hc" else arr.reshape(B * T, *arr.shape[2:])
    t = torch.nan_to_num(torch.from_numpy(np.ascontiguousarray(a).astype(np.float32)), nan=0.0)
    run.views[name][: t.shape[0]].copy_(t.cuda())


def get(run, name):
    torch.cuda.synchronize()
    return run.views[name].cpu().numpy()


CASES = [(torch.float32, 64, "safe"), (torch.bfloat16, 128, "safe"), (torch.bfloat16, 128, "softplus"),
         (torch.bfloat16, 256, "safe")]


@pytest.mark.parametrize("dtype,D,gate", CASES)
def test_stage_gate(dtype, D, gate):
    need_gpu()
    run, it, _, _, valid, B, T = setup(dtype, D, gate)
    run.run("gate")
    got = get(run, "b")[valid]
    want = it["b"].reshape(B * T, 2, D)[valid]
    err = np.abs(got - want)
    assert err.max() <= 1e-5 * max(1.0, np.abs(want).max()) + 1e-5, err.max()


@pytest.mark.parametrize("dtype,D,gate", CASES)
def test_stage_grams(dtype, D, gate):
    need_gpu()
    run, it, _, _, valid, B, T = setup(dtype, D, gate)
    put(run, "b", it["b"], B, T)
    run.run("grams")
    for name in ("Akk", "Aqk"):
        got = get(run, name)[valid]
        want = it[name].reshape(B * T, 2, -1)[valid]
        if dtype == torch.float32:
            assert np.abs(got - want).max() <= 1e-5, (name, np.abs(got - want).max())
        else:
            assert rel_rms(got, want) <= 1e-2, (name, rel_rms(got, want))


@pytest.mark.parametrize("dtype,D,gate", CASES)
def test_stage_solve(dtype, D, gate):
    need_gpu()
    run, it, _, _, valid, B, T = setup(dtype, D, gate)
    put(run, "Akk", it["Akk"], B, T)
    run.run("solve")
    got = get(run, "T")[valid]
    want = it["T"].reshape(B * T, 2, -1)[valid]
    assert np.abs(got - want).max() <= 2e-5 * max(1.0, np.abs(want).max()), np.abs(got - want).max()
    # residual of the GPU's inverse itself: (I + A_kk) T = I on every chunk (rows of a
    # partial chunk past its end do not exist)
    C = got.shape[-1]
    A = it["Akk"].reshape(B, T, 2, C)
    Tg = got.reshape(B, T, 2, C)
    worst = 0.0
    for b in range(B):
        for c0 in range(0, T, C):
            L = min(C, T - c0)
            for h in range(2):
                M = np.eye(L) + np.tril(A[b, c0:c0 + L, h, :L], -1)
                Ti = Tg[b, c0:c0 + L, h, :L].astype(np.float64)
                R = M @ Ti - np.eye(L)
                bound = 1e-5 * max(1.0, np.abs(M).sum(1).max() * np.abs(Ti).sum(1).max())
                assert np.abs(R).max() <= bound, (b, c0, h, np.abs(R).max(), bound)
                worst = max(worst, np.abs(R).max())


@pytest.mark.parametrize("dtype,D,gate", CASES)
def test_stage_wy(dtype, D, gate):
    need_gpu()
    run, it, _, _, valid, B, T = setup(dtype, D, gate)
    put(run, "b", it["b"], B, T)
    put(run, "T", it["T"], B, T)
    run.run("wy")
    for name in ("w", "u"):
        got = get(run, name)[valid]
        want = it[name].reshape(B * T, 2, D)[valid]
        if dtype == torch.float32:
            assert np.abs(got - want).max() <= 1e-4, (name, np.abs(got - want).max())
        else:
            assert rel_rms(got, want) <= 1e-2, (name, rel_rms(got, want))


@pytest.mark.parametrize("dtype,D,gate", CASES)
@pytest.mark.parametrize("lens", [None, [0, 70, 64, 1, 0, 129]])
def test_stage_scan(dtype, D, gate, lens):
    need_gpu()
    run, it, _, h2, valid, B, T = setup(dtype, D, gate, lens=lens)
    put(run, "b", it["b"], B, T)
    put(run, "w", it["w"], B, T)
    put(run, "u", it["u"], B, T)
    run.run("scan")
    got = get(run, "vnew")[valid]
    want = it["vnew"].reshape(B * T, 2, D)[valid]
    tol = 1e-4 if dtype == torch.float32 else 1e-2
    assert rel_rms(got, want) <= tol, rel_rms(got, want)
    nch = it["hc"].shape[0]
    assert rel_rms(get(run, "hc")[:nch], it["hc"]) <= tol
    torch.cuda.synchronize()
    assert rel_rms(run.ht.cpu().numpy(), h2) <= tol


@pytest.mark.parametrize("dtype,D,gate", CASES)
def test_stage_output(dtype, D, gate):
    need_gpu()
    run, it, o2, _, valid, B, T = setup(dtype, D, gate)
    put(run, "b", it["b"], B, T)
    put(run, "Aqk", it["Aqk"], B, T)
    put(run, "vnew", it["vnew"], B, T)
    put(run, "hc", it["hc"], B, T)
    run.run("output")
    torch.cuda.synchronize()
    got = run.o.float().cpu().numpy().reshape(B * T, 2, D)[valid]
    want = o2.reshape(B * T, 2, D)[valid]
    if dtype == torch.float32:
        assert np.abs(got - want).max() <= 1e-4, np.abs(got - want).max()
    else:
        assert rel_rms(got, want) <= 5e-3, rel_rms(got, want)
