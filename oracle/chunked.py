"""O2: the chunked form of the KDA forward pass, numpy FP64 (test infrastructure).

TEST INFRASTRUCTURE ONLY (see the package docstring). Written from the
recurrence: within a chunk of L <= C tokens that starts from state h,

  (1) b_r   = log2(e) * sum_{s<=r} g_s       inclusive, chunk-local, base 2
  (2) A_kk[r,s] = beta_r * sum_i k_r[i] k_s[i] 2^(b_r[i]-b_s[i])    s < r
      A_qk[r,s] = scale  * sum_i q_r[i] k_s[i] 2^(b_r[i]-b_s[i])    s <= r
  (3) T = (I + A_kk)^-1                       unit lower triangular
  (4) w = T (beta * k * 2^b),   u = T (beta * v)
  (5) v_new = u - w h ;  h <- Diag(2^b_L) h + (k * 2^(b_L - b))^T v_new
  (6) o = scale (q * 2^b) h + A_qk v_new

with b_L the cumsum at the chunk's last valid row. Chunks restart at every
sequence start and never straddle two sequences.

The grams are formed per 16x16 sub-block, as "FLA KDA Skill" describes in
section "Safe gate numerical note": a diagonal block factors the decay through
a midpoint row m of its own block, 2^(b_r-b_m) * 2^(b_m-b_s); an off-diagonal
block (i, j<i) factors it through the first row n of block i,
2^(b_r-b_n) * 2^(b_n-b_s), both exponents non-positive for a decaying gate.
Only the causal blocks j <= i are formed ("[examples] Read only the causal
columns in chunk_fwd_A_diag_anchored", description). ``anchored=False``
evaluates 2^(b_r-b_s) per pair instead (the token-parallel form that "FLA
KDA Skill", section "Safe vs non-safe intra path", uses for a non-safe gate).
In exact arithmetic both are the same number.
"""
import math

import numpy as np
from scipy.linalg import solve_triangular

RCP_LN2 = 1.0 / math.log(2.0)
SUB = 16  # sub-chunk rows


def _chunk(qc, kc, vc, gc, bc, h, scale, anchored, mid):
    """One chunk of L rows starting from state h [K, V]. Returns a dict."""
    L = kc.shape[0]
    b = np.cumsum(gc, axis=0) * RCP_LN2
    Akk = np.zeros((L, L))
    Aqk = np.zeros((L, L))
    nblk = (L + SUB - 1) // SUB
    for i in range(nblk):
        R = slice(SUB * i, min(SUB * i + SUB, L))
        for j in range(i + 1):
            S = slice(SUB * j, min(SUB * j + SUB, L))
            if anchored:
                if i == j:
                    a = b[min(SUB * i + mid, L - 1)]  # midpoint row, clamped to the last valid row
                else:
                    a = b[SUB * i]  # first row of the row block
                row = np.exp2(b[R] - a)
                col = np.exp2(a - b[S])
                gqk = (qc[R] * row) @ (kc[S] * col).T
                gkk = (kc[R] * row) @ (kc[S] * col).T
            else:
                # only causal pairs s <= r enter the grams: the exponent of every other
                # pair is masked before exponentiating (it would be positive)
                diff = b[R][:, None, :] - b[S][None, :, :]
                if i == j:
                    causal = np.arange(R.start, R.stop)[:, None] >= np.arange(S.start, S.stop)[None, :]
                    diff = np.where(causal[:, :, None], diff, -np.inf)
                E = np.exp2(diff)
                gqk = np.einsum("ri,si,rsi->rs", qc[R], kc[S], E)
                gkk = np.einsum("ri,si,rsi->rs", kc[R], kc[S], E)
            Aqk[R, S] = gqk
            Akk[R, S] = gkk
    Aqk = np.tril(Aqk) * scale
    Akk = np.tril(Akk, -1) * bc[:, None]
    eye = np.eye(L)
    Tm = solve_triangular(eye + Akk, eye, lower=True, unit_diagonal=True)
    gam = np.exp2(b)
    w = Tm @ (bc[:, None] * kc * gam)
    u = Tm @ (bc[:, None] * vc)
    vnew = u - w @ h
    o = scale * (qc * gam) @ h + Aqk @ vnew
    bL = b[L - 1]
    h_next = np.exp2(bL)[:, None] * h + (kc * np.exp2(bL - b)).T @ vnew
    return dict(b=b, Akk=Akk, Aqk=Aqk, T=Tm, w=w, u=u, vnew=vnew, o=o, h_next=h_next)


def chunked_forward(q, k, v, g, beta, h0=None, cu_seqlens=None, scale=None, chunk_size=64,
                    anchored=True, mid=8, emit=False):
    """O2 over a batch. Shapes as in ``oracle.recurrent``; g is the natural-log decay.

    Returns (o, ht) or, with ``emit``, (o, ht, inter) where ``inter`` holds the
    intermediates in the token-major layouts the chunk kernels use:
      b [B,T,H,K]; Akk, Aqk, T [B,T,H,C] (column = row within the chunk);
      w [B,T,H,K]; u, vnew [B,T,H,V]; hc [n_chunks,H,K,V], the state at the
      start of each chunk, chunks enumerated slot by slot.
    """
    q, k, v, g, beta = (np.asarray(a, dtype=np.float64) for a in (q, k, v, g, beta))
    B, T, H, K = q.shape
    V = v.shape[-1]
    C = int(chunk_size)
    if cu_seqlens is None:
        cu = np.arange(B + 1) * T
    else:
        assert B == 1
        cu = np.asarray(cu_seqlens, dtype=np.int64)
    N = len(cu) - 1
    if scale is None:
        scale = 1.0 / math.sqrt(K)
    qf, kf, vf, gf = (a.reshape(B * T, H, -1) for a in (q, k, v, g))
    bf = beta.reshape(B * T, H)
    o = np.full((B * T, H, V), np.nan)
    ht = np.zeros((N, H, K, V))
    inter = None
    if emit:
        inter = dict(b=np.full((B * T, H, K), np.nan), Akk=np.zeros((B * T, H, C)),
                     Aqk=np.zeros((B * T, H, C)), T=np.zeros((B * T, H, C)),
                     w=np.full((B * T, H, K), np.nan), u=np.full((B * T, H, V), np.nan),
                     vnew=np.full((B * T, H, V), np.nan), hc=[])
    hcs = []
    for n in range(N):
        s0, s1 = int(cu[n]), int(cu[n + 1])
        nch = (s1 - s0 + C - 1) // C
        slot_states = np.zeros((nch, H, K, V))
        for hh in range(H):
            h = np.zeros((K, V)) if h0 is None else np.asarray(h0, dtype=np.float64).reshape(N, H, K, V)[n, hh].copy()
            for c in range(nch):
                t0, t1 = s0 + c * C, min(s0 + (c + 1) * C, s1)
                L = t1 - t0
                slot_states[c, hh] = h
                r = _chunk(qf[t0:t1, hh], kf[t0:t1, hh], vf[t0:t1, hh], gf[t0:t1, hh], bf[t0:t1, hh],
                           h, scale, anchored, mid)
                o[t0:t1, hh] = r["o"]
                if emit:
                    inter["b"][t0:t1, hh] = r["b"]
                    inter["Akk"][t0:t1, hh, :L] = r["Akk"]
                    inter["Aqk"][t0:t1, hh, :L] = r["Aqk"]
                    inter["T"][t0:t1, hh, :L] = r["T"]
                    inter["w"][t0:t1, hh] = r["w"]
                    inter["u"][t0:t1, hh] = r["u"]
                    inter["vnew"][t0:t1, hh] = r["vnew"]
                h = r["h_next"]
            ht[n, hh] = h
        if h0 is not None and s0 == s1:
            ht[n] = np.asarray(h0, dtype=np.float64).reshape(N, H, K, V)[n]
        hcs.append(slot_states)
    o = o.reshape(B, T, H, V)
    if not emit:
        return o, ht
    for key in ("b", "Akk", "Aqk", "T", "w", "u", "vnew"):
        inter[key] = inter[key].reshape((B, T) + inter[key].shape[1:])
    inter["hc"] = np.concatenate(hcs, axis=0) if hcs else np.zeros((0, H, K, V))
    return o, ht, inter


def chunk_cumsum_log2(g, cu_seqlens=None, chunk_size=64, g_is_log2=False):
    """Step (1) alone: b = log2(e) * (running sum of g from the start of each chunk).

    g is the per-token decay [B, T, H, K] (natural log, or log2 with
    ``g_is_log2``). Chunks of ``chunk_size`` rows restart at every sequence
    start ("FLA KDA Skill", section "Safe gate numerical note": the RCP_LN2
    conversion of the chunk-local cumsum). chunk_size 1 is the per-token log2
    decay. Rows outside the packed contract are NaN.
    """
    g = np.asarray(g, dtype=np.float64)
    B, T, H, K = g.shape
    unit = 1.0 if g_is_log2 else RCP_LN2
    cu = np.arange(B + 1) * T if cu_seqlens is None else np.asarray(cu_seqlens, dtype=np.int64)
    gf = g.reshape(B * T, H, K)
    out = np.full_like(gf, np.nan)
    C = int(chunk_size)
    for n in range(len(cu) - 1):
        s0, s1 = int(cu[n]), int(cu[n + 1])
        run = np.zeros((H, K))
        for t in range(s0, s1):
            if (t - s0) % C == 0:
                run = np.zeros((H, K))
            run = run + gf[t] * unit
            out[t] = run
    return out.reshape(B, T, H, K)
