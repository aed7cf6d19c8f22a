"""Benchmark of the KDA forward on one MI355X.

Headline workload: chunk_kda forward, B4 T4096 H64 K=V=128, bf16 q/k/v, fp32
gate input / beta / state, chunk 64, safe gate (lower bound -5) activated in
the kernel, initial state 0.1 N(0,1), final state returned. Synthetic seeded
inputs (kda_synth), resident in HBM before timing.

One JSON line on stdout:
  value          Mtokens/s (tokens = B*T per call) from HIP events around each
                 kda_chunk_fwd launch on its stream; the 512 MiB cache-flush
                 write between calls sits outside the events.
  roofline       the dominant kernel (the fused chunk kernel: one launch per
                 call) against HBM: algorithmic bytes per launch (q, k, v, gate,
                 beta, o, h0, ht counted once) / its mean launch time.
  cpu_baseline   the FP64 oracle on the host cores over the same workload
                 (4 sequences, 64 heads, 4096 tokens, gate included), 3 timed runs.
  recurrent_decode  kda_recurrent_fwd: 256 sequences x 1 token, H64 D128, bf16,
                 log2 gate, fp32 state read and written in place.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0


def alg_bytes_chunk(B, T, H, D, dtype_bytes=2, N=None, with_h0=True, with_ht=True):
    """Bytes the method must move once: q, k, v, o in dtype; gate input fp32; beta fp32; h0, ht fp32."""
    N = B if N is None else N
    per_token_head = dtype_bytes * (2 * D + D) + 4 * D + 4 + dtype_bytes * D
    state = 4 * N * H * D * D
    return B * T * H * per_token_head + state * (int(with_h0) + int(with_ht))


def alg_flops_chunk(B, T, H, D, C=64):
    """Block-causal flops per token-head: state products, grams, WY, A_qk v_new, solve."""
    NC = C // 16
    pbar = 16 * (NC + 1) / 2
    per = 6 * D * D + 2 * (2 * D) * pbar + (2 * D + 2 * D) * pbar + 2 * D * pbar + C * C / 3
    return B * T * H * per


# per single-kernel schedule: the sources its kernel is built from and the
# committed counter summary of its HBM traffic at the headline shape
_HEADERS = ("chunk_fused_layout.h", "chunk_fused_tiles.h", "chunk_tiles.h", "kda_device.h", "kda_launch.h")
TRAFFIC = {
    "fused": (("chunk_fused.hip",) + _HEADERS, "fused_chunk_b4t4096h64d128_traffic.txt", "fused_chunk_kernel"),
    "pipe": (("chunk_pipe.hip",) + _HEADERS, "pipe_chunk_b4t4096h64d128_traffic.txt", "pipe_chunk_kernel"),
}
# kept for the traffic summaries' own commands
FUSED_SOURCES = TRAFFIC["fused"][0]


def kernel_source_sha(sched="fused"):
    """sha256 over the sources the schedule's chunk kernel is built from."""
    h = hashlib.sha256()
    for name in TRAFFIC[sched][0]:
        with open(os.path.join(ROOT, "gated_delta_rule_gate_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(sched):
    """HBM bytes per launch from the committed counter summary, or None when the
    kernel sources changed since the counters were taken."""
    if sched not in TRAFFIC:
        return None
    path = os.path.join(ROOT, "profiles", TRAFFIC[sched][1])
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            key, val = line.split(":", 1)
            vals[key.strip()] = val.strip()
    if vals.get("source_sha256") != kernel_source_sha(sched):
        return None
    try:
        return int(float(vals["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


RAMP_S = 0.3  # seconds of load before each timed measurement


def gpu_ramp(buf, seconds=0.3):
    """Keeps the GPU busy with a plain fill kernel for about `seconds` before any
    timing: from idle, the part needs on the order of 100 ms of load to reach its
    working clock, and calls timed earlier run up to 15% slower. The fill is not
    the measured step, touches none of its data, and the flush before every timed
    call evicts what it leaves in the caches. (A bf16 matmul ramp measured slower.)"""
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(64):
            buf.zero_()
        torch.cuda.synchronize()


def workspace_for(q, v, H, N, C, schedule, gate_kind):
    """The call's workspace, allocated once so that no timed call allocates."""
    from gated_delta_rule_gate_amd import workspace_bytes

    n = workspace_bytes(q, v, H, N, chunk_size=C, schedule=schedule, gate_kind=gate_kind)
    return torch.empty((max(n, 256),), dtype=torch.uint8, device=q.device)


def event_time_ms(fn, steps, warmup, flush=None):
    """Mean / median / p10 / p90 of per-call HIP event times (ms) on the current stream.
    Warm-up calls run with the same flush as the timed ones."""
    for _ in range(warmup):
        if flush is not None:
            flush()
        fn()
    torch.cuda.synchronize()
    times = []
    st = torch.cuda.current_stream()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        if flush is not None:
            flush()
        starts[i].record(st)
        fn()
        ends[i].record(st)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    times = np.array([s.elapsed_time(e) for s, e in zip(starts, ends)])
    return dict(mean=float(times.mean()), median=float(np.median(times)), p10=float(np.percentile(times, 10)),
                p90=float(np.percentile(times, 90)), wall_ms=wall * 1e3)


def cpu_baseline(d, H, T, threads, runs=3):
    """The FP64 oracle (token recurrence + gate activation) on the whole headline
    workload: one untimed run, then the mean of ``runs`` timed runs."""
    import oracle
    from kda_synth import to_f64

    q, k, v, x, beta, h0 = (to_f64(d[n]) for n in ("q", "k", "v", "x", "beta", "h0"))
    A_log, dt = to_f64(d["A_log"]), to_f64(d["dt_bias"])

    def once():
        g = oracle.gate(oracle.GATE_SAFE, x, A_log, dt, -5.0)
        oracle.recurrent(q, k, v, g, beta, h0=h0, nthreads=threads)

    once()
    t0 = time.perf_counter()
    for _ in range(runs):
        once()
    dt_s = (time.perf_counter() - t0) / runs
    nseq = q.shape[0]
    tokens = nseq * T
    return dict(value=tokens / dt_s / 1e6, unit="Mtokens/s", cores=threads, kind="oracle",
                sample="all %d sequences x %d heads x %d tokens (FP64 token recurrence + gate), "
                       "mean of %d runs after 1 untimed, %.2f s per run" % (nseq, H, T, runs, dt_s))


def bench_decode(steps, warmup):
    import kda_synth
    from gated_delta_rule_gate_amd import recurrent_kda

    N, H, D = 256, 64, 128
    d = kda_synth.chunk_inputs(N, 1, H, D, D, dtype=torch.bfloat16, seed=1004)
    g2 = kda_synth.log2_gate(d["x"].numpy(), d["A_log"].numpy(), d["dt_bias"].numpy())
    dev = {k: v.cuda() for k, v in d.items() if v is not None}
    g2 = g2.cuda()
    state = dev["h0"]
    o = torch.empty((N, 1, H, D), dtype=torch.bfloat16, device="cuda")

    def step():
        recurrent_kda(dev["q"], dev["k"], dev["v"], g2, dev["beta"], state, final_state=state, out=o)

    t = event_time_ms(step, steps, warmup)
    nbytes = 2 * 4 * N * H * D * D + N * H * (2 * 3 * D + 4 * D + 4 + 2 * D)
    gbs = nbytes / (t["median"] * 1e-3) / 1e9
    return dict(config="256 seq x 1 token, H64 K=V=128, bf16, log2 gate, state in place", ms=t["median"],
                GBps=gbs, hbm_frac=gbs / HBM_PEAK_GBS, Mtokens_per_s=N / (t["median"] * 1e-3) / 1e6)


def bench_bwd(B, T, H, D, steps, warmup, C=64):
    """Flushed-cache HIP-event timing of kda_chunk_bwd (forward recompute included)
    on the headline shape: safe gate, bf16, h0 and dht given."""
    import kda_synth
    from gated_delta_rule_gate_amd import chunk_kda_bwd

    d = kda_synth.chunk_inputs(B, T, H, D, D, dtype=torch.bfloat16, seed=1002)
    dev = {k: v.cuda() for k, v in d.items() if v is not None}
    del d
    gen = torch.Generator(device="cuda").manual_seed(1003)
    do = torch.randn((B, T, H, D), device="cuda", generator=gen).to(torch.bfloat16)
    dht = 0.1 * torch.randn((B, H, D, D), device="cuda", generator=gen)
    flush_buf = torch.empty((512 << 20,), dtype=torch.uint8, device="cuda")

    def step():
        chunk_kda_bwd(dev["q"], dev["k"], dev["v"], dev["x"], dev["beta"], do, dev["h0"], dht=dht, chunk_size=C,
                      gate_kind="safe", A_log=dev["A_log"], dt_bias=dev["dt_bias"], lower_bound=-5.0)

    # the part leaves its idle clock only under load: ramp it first, as for the headline
    gpu_ramp(flush_buf, RAMP_S)
    t = event_time_ms(step, steps, warmup, flush=lambda: flush_buf.zero_())
    nbytes = alg_bytes_bwd(B, T, H, D)
    return {"config": "chunk_kda bwd B%d T%d H%d K=V=%d bf16, C=%d, safe gate, h0 + dht; forward recompute "
                      "included" % (B, T, H, D, C),
            "ms": round(t["mean"], 4), "Mtokens_per_s": round(B * T / (t["mean"] * 1e-3) / 1e6, 3),
            "alg_bytes": nbytes, "roofline_frac": round(nbytes / (t["mean"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}


def alg_bytes_bwd(B, T, H, D, dtype_bytes=2):
    """Bytes the backward must move once: it reads q, k, v, do (dtype) and the gate
    input x (fp32), beta, h0 and dht; it writes dq, dk, dv (dtype), dx (fp32),
    dbeta and dh0 (dA_log and ddt_bias are per head and negligible)."""
    per_elem = 4 * dtype_bytes + 4 + 3 * dtype_bytes + 4
    return B * T * H * (per_elem * D + 4 + 4) + 3 * B * H * D * D * 4


def bench_fp32_small(steps, warmup):
    """The fp32 configuration: B1 T256 H2 K=V=64, C=64, safe gate, h0 = 0 and the
    final state returned (one chunk chain of four chunks per head)."""
    import kda_synth
    from gated_delta_rule_gate_amd import chunk_kda, resolved_schedule

    B, T, H, D = 1, 256, 2, 64
    d = kda_synth.chunk_inputs(B, T, H, D, D, dtype=torch.float32, seed=1001, with_h0=False)
    dev = {k: v.cuda() for k, v in d.items() if v is not None}
    o = torch.empty((B, T, H, D), dtype=torch.float32, device="cuda")
    ht = torch.empty((B, H, D, D), dtype=torch.float32, device="cuda")
    ws = workspace_for(dev["q"], dev["v"], H, B, 64, "auto", "safe")

    def step():
        chunk_kda(dev["q"], dev["k"], dev["v"], dev["x"], dev["beta"], None, chunk_size=64, gate_kind="safe",
                  A_log=dev["A_log"], dt_bias=dev["dt_bias"], lower_bound=-5.0, out=o, final_state=ht, workspace=ws)

    t = event_time_ms(step, steps, warmup)
    ms = t["median"]
    nbytes = alg_bytes_chunk(B, T, H, D, dtype_bytes=4, with_h0=False)
    return {"config": "chunk_kda fwd fp32 B1 T256 H2 K=V=64, C=64, safe gate lb=-5, h0=0, ht", "ms": round(ms, 5),
            "Mtokens_per_s": round(B * T / (ms * 1e-3) / 1e6, 3),
            "roofline_frac": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 6),
            "schedule": resolved_schedule(dev["q"], dev["v"], H, B, chunk_size=64)}


def bench_prefill(steps, warmup):
    """recurrent_kda over 256 sequences x 64 tokens (the recurrent prefill), H64 K=V=128 bf16, log2 gate."""
    import kda_synth
    from gated_delta_rule_gate_amd import recurrent_kda

    N, T, H, D = 256, 64, 64, 128
    d = kda_synth.chunk_inputs(N, T, H, D, D, dtype=torch.bfloat16, seed=1004)
    g2 = kda_synth.log2_gate(d["x"].numpy(), d["A_log"].numpy(), d["dt_bias"].numpy()).cuda()
    dev = {k: v.cuda() for k, v in d.items() if v is not None}
    o = torch.empty((N, T, H, D), dtype=torch.bfloat16, device="cuda")
    ht = torch.empty_like(dev["h0"])
    flush_buf = torch.empty((512 << 20,), dtype=torch.uint8, device="cuda")

    def step():
        recurrent_kda(dev["q"], dev["k"], dev["v"], g2, dev["beta"], dev["h0"], final_state=ht, out=o)

    # the part leaves its idle clock only under load: ramp it first, as for the headline
    gpu_ramp(flush_buf, RAMP_S)
    t = event_time_ms(step, steps, warmup, flush=lambda: flush_buf.zero_())
    return dict(config="256 seq x 64 tokens, H64 K=V=128, bf16, log2 gate, h0 + ht", ms=round(t["mean"], 4),
                Mtokens_per_s=round(N * T / (t["mean"] * 1e-3) / 1e6, 3))


def bench_varlen(steps, warmup, schedule="auto"):
    """chunk_kda on the packed workload: capacity 16384, ten slots (two empty) holding 15872
    tokens, H16 K=V=128 bf16, softplus gate, h0 per slot."""
    import kda_synth
    from gated_delta_rule_gate_amd import chunk_kda

    CAP, H, D, SLOTS = 16384, 16, 128, 10
    cu = torch.from_numpy(kda_synth.varlen_offsets(1003, n_slots=SLOTS, n_empty=2, total=15872, max_len=4096))
    d = kda_synth.chunk_inputs(1, CAP, H, D, D, dtype=torch.bfloat16, seed=1003, n_slots=SLOTS)
    dev = {k: v.cuda() for k, v in d.items() if v is not None}
    cu_d = cu.cuda()
    o = torch.empty((1, CAP, H, D), dtype=torch.bfloat16, device="cuda")
    ht = torch.empty_like(dev["h0"])
    flush_buf = torch.empty((512 << 20,), dtype=torch.uint8, device="cuda")
    ws = workspace_for(dev["q"], dev["v"], H, SLOTS, 64, schedule, "softplus")

    def step():
        chunk_kda(dev["q"], dev["k"], dev["v"], dev["x"], dev["beta"], dev["h0"], cu_seqlens=cu_d, chunk_size=64,
                  gate_kind="softplus", A_log=dev["A_log"], dt_bias=dev["dt_bias"], out=o, final_state=ht,
                  schedule=schedule, workspace=ws)

    # the part leaves its idle clock only under load: ramp it first, as for the headline
    gpu_ramp(flush_buf, RAMP_S)
    t = event_time_ms(step, steps, warmup, flush=lambda: flush_buf.zero_())
    n = int(cu[-1])
    nbytes = n * H * (2 * 3 * D + 4 * D + 4 + 2 * D) + 2 * 4 * SLOTS * H * D * D
    return dict(config="packed, capacity 16384, 10 slots (2 empty), 15872 tokens, H16 K=V=128 bf16, softplus, h0+ht",
                ms=round(t["mean"], 4), Mtokens_per_s=round(n / (t["mean"] * 1e-3) / 1e6, 3),
                roofline_frac=round(nbytes / (t["mean"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4))


def alg_bytes_general(B, T, H, Hk, K, V, n_chunks=0, dtype_bytes=2):
    """Bytes moved once: q, k (Hk heads), v and o (H heads) in dtype; gate input fp32; beta fp32;
    h0 and ht fp32; plus n_chunks chunk-start states fp32 when those are returned."""
    tokens = B * T
    return (tokens * (2 * Hk * K * dtype_bytes + 2 * H * V * dtype_bytes + H * K * 4 + H * 4)
            + 2 * B * H * K * V * 4 + n_chunks * H * K * V * 4)


def bench_variants(steps, warmup):
    """The headline call (B4 T4096 H64, C=64, safe gate, h0 + ht, flushed caches) and its
    variants: q_l2norm on raw q, beta as logits, the chunk-start states returned, grouped
    value heads (16 q/k heads), K != V and a non-power-of-two width, chunk size 32, and the
    plain call replayed from a HIP graph. Each variant's fraction is of its own algorithmic bytes."""
    import kda_synth
    from gated_delta_rule_gate_amd import chunk_kda, resolved_schedule

    B, T, H, C = 4, 4096, 64, 64
    flush_buf = torch.empty((512 << 20,), dtype=torch.uint8, device="cuda")
    flush = lambda: flush_buf.zero_()
    out = []

    def run(name, K, V, Hk=H, chunk=C, **kw):
        d = kda_synth.chunk_inputs(B, T, H, K, V, dtype=torch.bfloat16, seed=1002)
        dev = {k: v.cuda() for k, v in d.items() if v is not None}
        del d
        if Hk != H:
            dev["q"] = dev["q"][:, :, :Hk].contiguous()
            dev["k"] = dev["k"][:, :, :Hk].contiguous()
        o = torch.empty((B, T, H, V), dtype=torch.bfloat16, device="cuda")
        ht = torch.empty((B, H, K, V), dtype=torch.float32, device="cuda")
        n_chunks = B * ((T + chunk - 1) // chunk) if kw.get("return_intermediate_states") else 0
        hs = torch.empty((B, n_chunks // B, H, K, V), dtype=torch.float32, device="cuda") if n_chunks else None
        extra = dict(intermediate_states=hs) if hs is not None else {}
        kw2 = {k: v for k, v in kw.items() if k not in ("return_intermediate_states", "graph")}

        def step():
            chunk_kda(dev["q"], dev["k"], dev["v"], dev["x"], dev["beta"], dev["h0"], chunk_size=chunk, gate_kind="safe",
                      A_log=dev["A_log"], dt_bias=dev["dt_bias"], lower_bound=-5.0, out=o, final_state=ht, **extra,
                      **kw2)

        fn = step
        if kw.get("graph"):
            step()  # the first call builds what the capture then reuses
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step()
            fn = g.replay
        # the part leaves its idle clock only under load: ramp it first, as for the headline
        gpu_ramp(flush_buf, RAMP_S)
        t = event_time_ms(fn, steps, warmup, flush=flush)
        nbytes = alg_bytes_general(B, T, H, Hk, K, V, n_chunks)
        out.append({"variant": name, "ms": round(t["mean"], 4),
                    "Mtokens_per_s": round(B * T / (t["mean"] * 1e-3) / 1e6, 3),
                    "alg_bytes": nbytes, "roofline_frac": round(nbytes / (t["mean"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                    "schedule": resolved_schedule(dev["q"], dev["v"], H, B, chunk_size=chunk)})
        del dev, o, ht, hs
        torch.cuda.empty_cache()

    run("plain", 128, 128)
    run("q_l2norm (raw q)", 128, 128, q_l2norm=True)
    run("beta as logits", 128, 128, beta_logits=True)
    run("chunk-start states returned", 128, 128, return_intermediate_states=True)
    run("GVA: 16 q/k heads for 64 value heads", 128, 128, Hk=16)
    run("K=128, V=64", 128, 64)
    run("K=V=96 (tile 128)", 96, 96)
    run("chunk size 32", 128, 128, chunk=32)
    run("HIP graph replay", 128, 128, graph=True)
    return out


def copy_bandwidth():
    """Device copy of 1 GiB (read + write), for context beside the roofline."""
    src = torch.ones((1 << 28,), dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    t = event_time_ms(lambda: dst.copy_(src), 10, 2)
    return round(2 * src.numel() * 4 / (t["median"] * 1e-3) / 1e9, 1)


def cpu_model():
    """The host CPU as /proc/cpuinfo names it, with its family / model / stepping numbers."""
    info = {}
    try:
        for line in open("/proc/cpuinfo"):
            if ":" in line:
                key, val = (x.strip() for x in line.split(":", 1))
                if key in ("model name", "cpu family", "model", "stepping") and key not in info:
                    info[key] = val
            if not line.strip() and info:
                break
    except OSError:
        pass
    if not info:
        return "unknown"
    return "%s (family %s, model %s, stepping %s)" % (info.get("model name", "?"), info.get("cpu family", "?"),
                                                      info.get("model", "?"), info.get("stepping", "?"))


def affinity_ranges(cpus):
    """A CPU id set as a compact range list, e.g. '0-15,32-47'."""
    cpus = sorted(cpus)
    out, i = [], 0
    while i < len(cpus):
        j = i
        while j + 1 < len(cpus) and cpus[j + 1] == cpus[j] + 1:
            j += 1
        out.append(str(cpus[i]) if i == j else "%d-%d" % (cpus[i], cpus[j]))
        i = j + 1
    return ",".join(out)


def cpu_threads():
    """Threads for the oracle: every CPU this process may run on (its affinity mask),
    capped by OMP_NUM_THREADS where the host sets it (the CPU share allotted per GPU)."""
    allowed = os.sched_getaffinity(0)
    cap = os.environ.get("OMP_NUM_THREADS")
    n = len(allowed)
    if cap and cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    return max(1, n), allowed


SWEEP_SHAPES = [(1, 8192, 96, 128), (2, 16384, 16, 128), (4, 2048, 16, 128), (4, 4096, 64, 128),
                   (8, 2048, 32, 256), (8, 1024, 8, 64)]


def bench_shape(B, T, H, D, steps, warmup, schedule="auto", C=64):
    """Flushed-cache HIP-event timing of kda_chunk_fwd on one synthetic shape (safe gate)."""
    import kda_synth
    from gated_delta_rule_gate_amd import chunk_kda, resolved_schedule

    d = kda_synth.chunk_inputs(B, T, H, D, D, dtype=torch.bfloat16, seed=1002)
    dev = {k: v.cuda() for k, v in d.items() if v is not None}
    del d
    o = torch.empty((B, T, H, D), dtype=torch.bfloat16, device="cuda")
    ht = torch.empty((B, H, D, D), dtype=torch.float32, device="cuda")
    flush_buf = torch.empty((512 << 20,), dtype=torch.uint8, device="cuda")
    ws = workspace_for(dev["q"], dev["v"], H, B, C, schedule, "safe")

    def step():
        chunk_kda(dev["q"], dev["k"], dev["v"], dev["x"], dev["beta"], dev["h0"], chunk_size=C, gate_kind="safe",
                  A_log=dev["A_log"], dt_bias=dev["dt_bias"], lower_bound=-5.0, schedule=schedule, out=o,
                  final_state=ht, workspace=ws)

    # the part leaves its idle clock only under load: ramp it first, as for the headline
    gpu_ramp(flush_buf, RAMP_S)
    t = event_time_ms(step, steps, warmup, flush=lambda: flush_buf.zero_())
    ms = t["mean"]
    nbytes = alg_bytes_chunk(B, T, H, D)
    return {"shape": "B%d T%d H%d D%d" % (B, T, H, D), "ms": round(ms, 4),
            "Mtokens_per_s": round(B * T / (ms * 1e-3) / 1e6, 3),
            "roofline_frac": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "schedule": resolved_schedule(dev["q"], dev["v"], H, B, chunk_size=C, schedule=schedule)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--schedule", default="auto", choices=["auto", "pipe", "fused", "split", "staged"])
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle timing")
    ap.add_argument("--no-decode", action="store_true", help="skip the recurrent decode figure")
    ap.add_argument("--shape", default="4,4096,64,128", help="B,T,H,D")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration under rocprofv3)")
    ap.add_argument("--sweep", action="store_true", help="also time a sweep of six shapes (and, where AUTO chose fused or split, the other one)")
    ap.add_argument("--no-bwd", action="store_true", help="skip the backward figure")
    ap.add_argument("--variants", action="store_true",
                    help="also time the headline call's variants (q_l2norm, beta logits, states, GVA, widths, C=32, graph)")
    ap.add_argument("--no-varlen", action="store_true", help="skip the packed-batch and copy figures")
    ap.add_argument("--no-prefill", action="store_true", help="skip the 64-token recurrent prefill figure")
    ap.add_argument("--ramp-s", type=float, default=0.3,
                    help="seconds of a plain fill kernel before the warm-up, to bring the GPU to its working clock")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: this build runs on one GPU only (the op has no cross-GPU path); "
              "--gpus %d is not supported" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(2)

    import kda_synth
    from gated_delta_rule_gate_amd import chunk_kda, lib, resolved_schedule

    lib()
    B, T, H, D = (int(x) for x in args.shape.split(","))
    C = 64
    d = kda_synth.chunk_inputs(B, T, H, D, D, dtype=torch.bfloat16, seed=1002)
    dev = {k: v.cuda() for k, v in d.items() if v is not None}
    sched = resolved_schedule(dev["q"], dev["v"], H, B, chunk_size=C, schedule=args.schedule)
    o = torch.empty((B, T, H, D), dtype=torch.bfloat16, device="cuda")
    ht = torch.empty((B, H, D, D), dtype=torch.float32, device="cuda")
    flush_buf = torch.empty((512 << 20,), dtype=torch.uint8, device="cuda")
    ws = workspace_for(dev["q"], dev["v"], H, B, C, args.schedule, "safe")

    def step():
        chunk_kda(dev["q"], dev["k"], dev["v"], dev["x"], dev["beta"], dev["h0"], chunk_size=C, gate_kind="safe",
                  A_log=dev["A_log"], dt_bias=dev["dt_bias"], lower_bound=-5.0, schedule=args.schedule, out=o,
                  final_state=ht, workspace=ws)

    def flush():
        flush_buf.zero_()

    if args.calib_copy:
        # one elementwise dispatch that reads 1 GiB and writes 1 GiB (counter calibration)
        src = torch.ones((1 << 28,), dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.add(src, 1.0, out=dst)
        torch.cuda.synchronize()

    gpu_ramp(flush_buf, args.ramp_s)
    cold = event_time_ms(step, args.steps, args.warmup, flush=flush)
    warm = event_time_ms(step, max(5, args.steps // 2), 1)
    ms = cold["mean"]
    tokens = B * T
    value = tokens / (ms * 1e-3) / 1e6
    nbytes = alg_bytes_chunk(B, T, H, D)
    flops = alg_flops_chunk(B, T, H, D, C)
    achieved = nbytes / (ms * 1e-3) / 1e9
    line = {
        "metric": "chunk_kda fwd Mtokens/s (B4 T4096 H64 D128 bf16) + % of roofline",
        "value": round(value, 3),
        "unit": "Mtokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "chunk_kda fwd B%d T%d H%d K=V=%d bf16, C=%d, safe gate lb=-5, h0+ht" % (B, T, H, D, C),
                   "B": B, "T": T, "H": H, "D": D, "chunk": C, "schedule": args.schedule, "runs": sched,
                   "cache": "flushed"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(sched) if (B, T, H, D) == (4, 4096, 64, 128) else None,
                     "kernel": {"fused": "fused_chunk_kernel", "pipe": "pipe_chunk_kernel",
                                "split": "split_key_kernel + split_state_kernel"}.get(sched, "staged chain"),
                     "alg_bytes_per_launch": nbytes,
                     "alg_tflops": round(flops / (ms * 1e-3) / 1e12, 2),
                     "mfma_frac": round(flops / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)},
        "timing_ms": {"cold_mean": round(cold["mean"], 4), "cold_p10": round(cold["p10"], 4),
                      "cold_p90": round(cold["p90"], 4), "warm_median": round(warm["median"], 4)},
    }
    if not args.no_decode:
        line["recurrent_decode"] = bench_decode(max(10, args.steps), 3)
    if not args.no_decode and not args.no_prefill:
        line["recurrent_prefill"] = bench_prefill(max(5, args.steps // 2), 2)
    if not args.no_varlen:
        line["fp32_small"] = bench_fp32_small(max(10, args.steps), 3)
        line["varlen"] = bench_varlen(max(5, args.steps // 2), 2)
        line["copy_GBps"] = copy_bandwidth()
    if not args.no_bwd and args.schedule != "fused":
        line["backward"] = bench_bwd(B, T, H, D, steps=max(3, args.steps // 4), warmup=1, C=C)
    if args.variants or args.sweep:
        del dev, o, ht, flush_buf
        torch.cuda.empty_cache()
    if args.variants:
        line["variants"] = bench_variants(max(5, args.steps // 2), 2)
    if args.sweep:
        from gated_delta_rule_gate_amd import KdaError
        line["shape_sweep"] = []
        for shp in SWEEP_SHAPES:
            r = bench_shape(*shp, steps=max(5, args.steps // 2), warmup=2)
            if r["schedule"] in ("fused", "split"):  # the schedule AUTO passed over, for comparison
                other = "split" if r["schedule"] == "fused" else "fused"
                try:
                    ms = bench_shape(*shp, steps=max(5, args.steps // 2), warmup=2, schedule=other)["ms"]
                except KdaError:  # that schedule does not take this shape (split stops at width 128)
                    ms = None
                r["other"] = {"schedule": other, "ms": ms}
            line["shape_sweep"].append(r)
            torch.cuda.empty_cache()
    if not args.no_cpu:
        threads, allowed = cpu_threads()
        line["cpu_baseline"] = cpu_baseline(d, H, T, threads)
        line["cpu_baseline"]["cpu_model"] = cpu_model()
        line["cpu_baseline"]["nproc"] = os.cpu_count()
        line["cpu_baseline"]["affinity"] = affinity_ranges(allowed)
        line["cpu_baseline"]["omp_num_threads"] = os.environ.get("OMP_NUM_THREADS")
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
