"""Pins of the FP64 oracle against facts the mathematics fixes (CPU only).

Each test checks the oracle against something other than itself: exact rational
brute force, closed forms of special cases, limits that reduce to textbook
rules, library routines, and invariants (split/resume, packing, pass-through).
A dropped term, a wrong sign or index or a transposed operand in the
recurrence, the gate activations or the chunked form fails at least one.
"""
import math
from fractions import Fraction as Fr

import numpy as np
import pytest
from scipy.special import expit

import oracle
from oracle import chunk_cumsum_log2, chunked_forward


def _l2(x):
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True))


def _case(seed, B=1, T=40, H=2, K=8, V=6, gate="safe", lb=-5.0):
    rng = np.random.default_rng(seed)
    q = _l2(rng.standard_normal((B, T, H, K)))
    k = _l2(rng.standard_normal((B, T, H, K)))
    v = rng.standard_normal((B, T, H, V))
    beta = expit(rng.standard_normal((B, T, H)))
    x = rng.standard_normal((B, T, H, K))
    A_log = np.log(rng.uniform(1, 16, size=H))
    dt = rng.standard_normal((H, K))
    if gate == "safe":
        g = oracle.gate(oracle.GATE_SAFE, x, A_log, dt, lb)
    elif gate == "softplus":
        g = oracle.gate(oracle.GATE_SOFTPLUS, x, A_log, dt)
    else:
        g = -0.1 * np.abs(x)
    return q, k, v, g, beta


# ----------------------------------------------------------------------------------------
# Exact brute force: explicit matrix products over rationals, T <= 8
# ----------------------------------------------------------------------------------------

def _mm(A, B):
    return [[sum(A[i][p] * B[p][j] for p in range(len(B))) for j in range(len(B[0]))] for i in range(len(A))]


def _product_form(q, k, v, g2, beta, S0, scale):
    """S_t = P(t,0) S0 + sum_{u<=t} P(t,u) beta_u k_u v_u^T, P(t,u) = M_t ... M_{u+1},
    M_t = (I - beta_t k_t k_t^T) Diag(2^g_t); o_t = S_t^T q_t * scale. Exact rationals."""
    T, K, V = len(q), len(q[0]), len(v[0])
    M = []
    for t in range(T):
        alpha = [Fr(2) ** g2[t][i] for i in range(K)]
        M.append([[((1 if i == j else 0) - beta[t] * k[t][i] * k[t][j]) * alpha[j] for j in range(K)]
                  for i in range(K)])
    eye = [[Fr(int(i == j)) for j in range(K)] for i in range(K)]
    outs, S_t = [], None
    for t in range(T):
        P = eye
        acc = [[Fr(0)] * V for _ in range(K)]
        for u in range(t, -1, -1):  # P = M_t ... M_{u+1} before adding term u
            rank1 = [[beta[u] * k[u][i] * v[u][j] for j in range(V)] for i in range(K)]
            term = _mm(P, rank1)
            acc = [[acc[i][j] + term[i][j] for j in range(V)] for i in range(K)]
            P = _mm(P, M[u])
        init = _mm(P, S0)
        S_t = [[acc[i][j] + init[i][j] for j in range(V)] for i in range(K)]
        outs.append([sum(S_t[i][j] * q[t][i] for i in range(K)) * scale for j in range(V)])
    return outs, S_t


@pytest.mark.parametrize("K,V,T,seed", [(4, 4, 6, 0), (4, 3, 8, 1), (16, 4, 5, 2)])
def test_exact_bruteforce_dyadic(oracle_mod, K, V, T, seed):
    rng = np.random.default_rng(seed)
    e = Fr(1, int(math.isqrt(K)))  # entries +-1/sqrt(K): unit rows, exact scale
    sgn = lambda shape: rng.choice([-1, 1], size=shape)
    qs, ks = sgn((T, K)), sgn((T, K))
    vs = rng.integers(-3, 4, size=(T, V))
    g2 = rng.integers(-2, 1, size=(T, K))
    bq = rng.choice([1, 2, 3, 4], size=T)
    s0 = rng.integers(-4, 5, size=(K, V))
    q = [[e * int(a) for a in row] for row in qs]
    k = [[e * int(a) for a in row] for row in ks]
    v = [[Fr(int(a)) for a in row] for row in vs]
    beta = [Fr(int(b), 4) for b in bq]
    S0 = [[Fr(int(a), 8) for a in row] for row in s0]
    scale = e
    o_ex, S_ex = _product_form(q, k, v, g2.tolist(), beta, S0, scale)

    f = lambda rows: np.array([[float(a) for a in r] for r in rows])
    o, ht = oracle.recurrent(f(q)[None, :, None], f(k)[None, :, None], f(v)[None, :, None],
                             g2.astype(float)[None, :, None], np.array([float(b) for b in beta])[None, :, None],
                             h0=f(S0)[None, None], scale=float(scale), g_is_log2=True)
    np.testing.assert_allclose(o[0, :, 0], f(o_ex), rtol=0, atol=1e-13)
    np.testing.assert_allclose(ht[0, 0], f(S_ex), rtol=0, atol=1e-13)

    # the same case through the natural-log gate: g = g2 * ln 2
    o2, ht2 = oracle.recurrent(f(q)[None, :, None], f(k)[None, :, None], f(v)[None, :, None],
                               (g2 * math.log(2.0))[None, :, None], np.array([float(b) for b in beta])[None, :, None],
                               h0=f(S0)[None, None], scale=float(scale))
    np.testing.assert_allclose(o2[0, :, 0], f(o_ex), rtol=0, atol=1e-12)
    np.testing.assert_allclose(ht2[0, 0], f(S_ex), rtol=0, atol=1e-12)


def _product_form_applied(q, k, v, g2, beta, S0, scale):
    """The explicit product form of ``_product_form``, with each P(t, u) applied to its
    operand one factor at a time (M_{u+1} first), so that K = 64 stays cheap in
    exact rationals: S_t = P(t, 0) S0 + sum_{u <= t} P(t, u) beta_u k_u v_u^T."""
    T, K, V = len(q), len(q[0]), len(v[0])

    def apply_M(t, X):  # M_t X = (I - beta_t k_t k_t^T) Diag(2^g_t) X for a K x n matrix X
        DX = [[(Fr(2) ** g2[t][i]) * X[i][j] for j in range(len(X[0]))] for i in range(K)]
        kDX = [sum(k[t][i] * DX[i][j] for i in range(K)) for j in range(len(X[0]))]
        return [[DX[i][j] - beta[t] * k[t][i] * kDX[j] for j in range(len(X[0]))] for i in range(K)]

    outs, S_t = [], None
    for t in range(T):
        S_t = [[Fr(0)] * V for _ in range(K)]
        for u in range(-1, t + 1):  # u = -1 stands for the initial state
            X = S0 if u < 0 else [[beta[u] * k[u][i] * v[u][j] for j in range(V)] for i in range(K)]
            for w in range(u + 1, t + 1):
                X = apply_M(w, X)
            S_t = [[S_t[i][j] + X[i][j] for j in range(V)] for i in range(K)]
        outs.append([sum(S_t[i][j] * q[t][i] for i in range(K)) * scale for j in range(V)])
    return outs, S_t


def test_exact_bruteforce_dyadic_k64(oracle_mod):
    """K = V = 64, the chunk kernels' smallest tile width: keys and queries of entries
    +-1/8 (unit rows, scale 1/8 exact), log2 gates in {0, -1, -2}, beta in quarters,
    small-integer values and an initial state in eighths; the oracle's recurrence
    against the exact product form, in the log2 and the natural-log gate."""
    K = V = 64
    T = 3
    rng = np.random.default_rng(64)
    e = Fr(1, 8)
    q = [[e * int(a) for a in row] for row in rng.choice([-1, 1], size=(T, K))]
    k = [[e * int(a) for a in row] for row in rng.choice([-1, 1], size=(T, K))]
    v = [[Fr(int(a)) for a in row] for row in rng.integers(-3, 4, size=(T, V))]
    g2 = rng.integers(-2, 1, size=(T, K))
    beta = [Fr(int(b), 4) for b in rng.choice([1, 2, 3, 4], size=T)]
    S0 = [[Fr(int(a), 8) for a in row] for row in rng.integers(-4, 5, size=(K, V))]
    o_ex, S_ex = _product_form_applied(q, k, v, g2.tolist(), beta, S0, e)

    f = lambda rows: np.array([[float(a) for a in r] for r in rows])
    b = np.array([float(x) for x in beta])[None, :, None]
    o, ht = oracle.recurrent(f(q)[None, :, None], f(k)[None, :, None], f(v)[None, :, None],
                             g2.astype(float)[None, :, None], b, h0=f(S0)[None, None], scale=float(e),
                             g_is_log2=True)
    np.testing.assert_allclose(o[0, :, 0], f(o_ex), rtol=0, atol=1e-12)
    np.testing.assert_allclose(ht[0, 0], f(S_ex), rtol=0, atol=1e-12)
    o2, ht2 = oracle.recurrent(f(q)[None, :, None], f(k)[None, :, None], f(v)[None, :, None],
                               (g2 * math.log(2.0))[None, :, None], b, h0=f(S0)[None, None], scale=float(e))
    np.testing.assert_allclose(o2[0, :, 0], f(o_ex), rtol=0, atol=1e-11)
    np.testing.assert_allclose(ht2[0, 0], f(S_ex), rtol=0, atol=1e-11)


def test_product_forms_agree():
    """The two exact product forms (whole P(t, u) matrices, and factors applied one at
    a time) are the same rationals on a small case."""
    rng = np.random.default_rng(11)
    K, V, T = 4, 3, 5
    e = Fr(1, 2)
    q = [[e * int(a) for a in row] for row in rng.choice([-1, 1], size=(T, K))]
    k = [[e * int(a) for a in row] for row in rng.choice([-1, 1], size=(T, K))]
    v = [[Fr(int(a)) for a in row] for row in rng.integers(-3, 4, size=(T, V))]
    g2 = rng.integers(-2, 1, size=(T, K)).tolist()
    beta = [Fr(int(b), 4) for b in rng.choice([1, 2, 3, 4], size=T)]
    S0 = [[Fr(int(a), 8) for a in row] for row in rng.integers(-4, 5, size=(K, V))]
    assert _product_form(q, k, v, g2, beta, S0, e) == _product_form_applied(q, k, v, g2, beta, S0, e)


# ----------------------------------------------------------------------------------------
# Closed forms and limits
# ----------------------------------------------------------------------------------------

def test_scalar_closed_form(oracle_mod):
    """K = V = 1, k = +-1: s_t = (1-b_t) a_t s_{t-1} + b_t k_t v_t, solved as a sum."""
    rng = np.random.default_rng(3)
    T = 50
    k = rng.choice([-1.0, 1.0], size=T)
    q = rng.choice([-1.0, 1.0], size=T)
    v = rng.standard_normal(T)
    beta = rng.uniform(0, 1, size=T)
    g = -rng.uniform(0, 0.3, size=T)
    s0 = 0.7
    fac = (1 - beta) * np.exp(g)
    s = np.empty(T)
    for t in range(T):
        P_0t = np.prod(fac[: t + 1])
        terms = [beta[u] * k[u] * v[u] * np.prod(fac[u + 1: t + 1]) for u in range(t + 1)]
        s[t] = P_0t * s0 + sum(terms)
    o, ht = oracle.recurrent(q[None, :, None, None], k[None, :, None, None], v[None, :, None, None],
                             g[None, :, None, None], beta[None, :, None], h0=np.array([[[[s0]]]]), scale=1.0)
    np.testing.assert_allclose(o[0, :, 0, 0], q * s, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(ht[0, 0, 0, 0], s[-1], rtol=1e-12)


def test_zero_gate_is_plain_delta_rule(oracle_mod):
    """g = 0: S_t = (I - beta k k^T) S_{t-1} + beta k v^T, with the explicit projector matrix."""
    q, k, v, _, beta = _case(4, T=30, H=1, K=8, V=5)
    g = np.zeros_like(q)
    h0 = 0.3 * np.random.default_rng(5).standard_normal((1, 1, 8, 5))
    o, ht = oracle.recurrent(q, k, v, g, beta, h0=h0)
    S = h0[0, 0].copy()
    for t in range(30):
        kt = k[0, t, 0][:, None]
        S = (np.eye(8) - beta[0, t, 0] * kt @ kt.T) @ S + beta[0, t, 0] * kt @ v[0, t, 0][None, :]
        np.testing.assert_allclose(o[0, t, 0], S.T @ q[0, t, 0] / math.sqrt(8), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(ht[0, 0], S, rtol=1e-12, atol=1e-13)


def test_zero_beta_pure_decay(oracle_mod):
    """beta = 0: o_t = scale (q_t * e^{G_t})^T h0, ht = Diag(e^{G_T}) h0, G = cumsum(g)."""
    q, k, v, g, _ = _case(6, T=25, H=2, K=8, V=4)
    beta = np.zeros(q.shape[:3])
    h0 = np.random.default_rng(7).standard_normal((1, 2, 8, 4))
    o, ht = oracle.recurrent(q, k, v, g, beta, h0=h0)
    G = np.cumsum(g, axis=1)
    for h in range(2):
        want = np.einsum("tk,kv->tv", q[0, :, h] * np.exp(G[0, :, h]), h0[0, h]) / math.sqrt(8)
        np.testing.assert_allclose(o[0, :, h], want, rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(ht[0, h], np.exp(G[0, -1, h])[:, None] * h0[0, h], rtol=1e-12, atol=1e-300)


def test_small_beta_limit_is_gated_linear_attention(oracle_mod):
    """h0 = 0, beta = eps * bhat: o / eps -> GLA with S_t = Diag(a_t) S_{t-1} + bhat_t k_t v_t^T."""
    q, k, v, g, bh = _case(8, T=40, H=1, K=8, V=4, gate="safe")
    eps = 1e-7
    o, _ = oracle.recurrent(q, k, v, g, eps * bh)
    S = np.zeros((8, 4))
    ref = np.empty((40, 4))
    for t in range(40):
        S = np.exp(g[0, t, 0])[:, None] * S + bh[0, t, 0] * np.outer(k[0, t, 0], v[0, t, 0])
        ref[t] = S.T @ q[0, t, 0] / math.sqrt(8)
    np.testing.assert_allclose(o[0, :, 0] / eps, ref, rtol=1e-5, atol=1e-6)


def test_unit_beta_query_equals_key(oracle_mod):
    """beta = 1 and q = k (unit norm): S_t^T k_t = v_t, so o_t = v_t / sqrt(K)."""
    _, k, v, g, _ = _case(9, T=30, H=2, K=16, V=8)
    beta = np.ones(k.shape[:3])
    h0 = np.random.default_rng(10).standard_normal((1, 2, 16, 8))
    o, _ = oracle.recurrent(k, k, v, g, beta, h0=h0)
    np.testing.assert_allclose(o, v / 4.0, rtol=0, atol=1e-12)


def test_axis_aligned_keys_decouple_rows(oracle_mod):
    """k_t = s_t e_{i_t}: row i is a scalar EMA, (1-b) a S[i] + s b v at its tokens, a S[i] elsewhere."""
    rng = np.random.default_rng(11)
    T, K, V = 60, 8, 5
    idx = rng.integers(0, K, size=T)
    sg = rng.choice([-1.0, 1.0], size=T)
    k = np.zeros((1, T, 1, K))
    k[0, np.arange(T), 0, idx] = sg
    q = _l2(rng.standard_normal((1, T, 1, K)))
    v = rng.standard_normal((1, T, 1, V))
    beta = rng.uniform(0, 1, size=(1, T, 1))
    g = -rng.uniform(0, 0.5, size=(1, T, 1, K))
    h0 = rng.standard_normal((1, 1, K, V))
    o, ht = oracle.recurrent(q, k, v, g, beta, h0=h0)
    rows = h0[0, 0].copy()
    for t in range(T):
        for i in range(K):
            a = math.exp(g[0, t, 0, i])
            if i == idx[t]:
                rows[i] = (1 - beta[0, t, 0]) * a * rows[i] + sg[t] * beta[0, t, 0] * v[0, t, 0]
            else:
                rows[i] = a * rows[i]
        np.testing.assert_allclose(o[0, t, 0], rows.T @ q[0, t, 0] / math.sqrt(K), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(ht[0, 0], rows, rtol=1e-12, atol=1e-13)


# ----------------------------------------------------------------------------------------
# Gate activations against library routines
# ----------------------------------------------------------------------------------------

def test_gate_activations(oracle_mod):
    rng = np.random.default_rng(12)
    x = 4 * rng.standard_normal((7, 3, 5))
    A_log = np.log(rng.uniform(1, 16, size=3))
    dt = rng.standard_normal((3, 5))
    z = np.exp(A_log)[:, None] * (x + dt)
    g = oracle.gate(oracle.GATE_SAFE, x, A_log, dt, -5.0)
    np.testing.assert_allclose(g, -5.0 * expit(z), rtol=1e-14, atol=1e-300)
    g = oracle.gate(oracle.GATE_SOFTPLUS, x, A_log, dt)
    np.testing.assert_allclose(g, -np.exp(A_log)[:, None] * np.logaddexp(0.0, x + dt), rtol=1e-13)
    # special points: sigmoid(0) = 1/2, softplus(0) = ln 2
    xz = -np.broadcast_to(dt, (1, 3, 5)).copy()
    np.testing.assert_array_equal(oracle.gate(oracle.GATE_SAFE, xz, A_log, dt, -3.0), -1.5)
    np.testing.assert_allclose(oracle.gate(oracle.GATE_SOFTPLUS, xz, A_log, dt),
                               np.broadcast_to(-np.exp(A_log)[:, None] * math.log(2.0), (1, 3, 5)), rtol=1e-15)
    # pre-gated mode is the identity; the safe gate stays inside [lower_bound, 0)
    np.testing.assert_array_equal(oracle.gate(oracle.GATE_LOGE, x, A_log, dt), x)
    gs = oracle.gate(oracle.GATE_SAFE, x, A_log, dt, -5.0)
    assert gs.min() >= -5.0 and gs.max() < 0.0


# ----------------------------------------------------------------------------------------
# Invariants: split/resume, packing, empty slots
# ----------------------------------------------------------------------------------------

def test_split_resume(oracle_mod):
    q, k, v, g, beta = _case(13, T=70, H=2, K=8, V=4)
    h0 = np.random.default_rng(14).standard_normal((1, 2, 8, 4))
    o, ht = oracle.recurrent(q, k, v, g, beta, h0=h0)
    T1 = 29
    oa, ha = oracle.recurrent(q[:, :T1], k[:, :T1], v[:, :T1], g[:, :T1], beta[:, :T1], h0=h0)
    ob, hb = oracle.recurrent(q[:, T1:], k[:, T1:], v[:, T1:], g[:, T1:], beta[:, T1:], h0=ha)
    np.testing.assert_allclose(np.concatenate([oa, ob], axis=1), o, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(hb, ht, rtol=1e-13, atol=1e-15)


def test_packed_equals_dense_and_empty_slots(oracle_mod):
    lens = [13, 0, 40, 1, 0, 22]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    Ttot = int(cu[-1]) + 5  # a tail beyond the last offset
    q, k, v, g, beta = _case(15, T=Ttot, H=2, K=8, V=4)
    h0 = np.random.default_rng(16).standard_normal((len(lens), 2, 8, 4))
    o, ht = oracle.recurrent(q, k, v, g, beta, h0=h0, cu_seqlens=cu)
    assert np.isnan(o[0, cu[-1]:]).all()  # the tail is untouched
    for n, L in enumerate(lens):
        s = slice(int(cu[n]), int(cu[n + 1]))
        if L == 0:
            np.testing.assert_array_equal(ht[n], h0[n])
            continue
        od, hd = oracle.recurrent(q[:, s], k[:, s], v[:, s], g[:, s], beta[:, s], h0=h0[n:n + 1])
        np.testing.assert_array_equal(o[:, s], od)
        np.testing.assert_array_equal(ht[n], hd[0])
    _, ht0 = oracle.recurrent(q, k, v, g, beta, h0=None, cu_seqlens=cu)
    assert not ht0[1].any() and not ht0[4].any()


# ----------------------------------------------------------------------------------------
# O2 (chunked form) against O1 (recurrence)
# ----------------------------------------------------------------------------------------

@pytest.mark.parametrize("C", [32, 64])
@pytest.mark.parametrize("anchored,mid,gate", [(True, 8, "safe"), (True, 0, "safe"), (True, 15, "safe"),
                                               (False, 8, "safe"), (False, 8, "softplus")])
def test_chunked_matches_recurrence(oracle_mod, C, anchored, mid, gate):
    q, k, v, g, beta = _case(17, B=2, T=150, H=2, K=16, V=8, gate=gate)
    h0 = 0.1 * np.random.default_rng(18).standard_normal((2, 2, 16, 8))
    o1, h1 = oracle.recurrent(q, k, v, g, beta, h0=h0)
    o2, h2 = chunked_forward(q, k, v, g, beta, h0=h0, chunk_size=C, anchored=anchored, mid=mid)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-12 * max(1.0, np.abs(o1).max()))
    np.testing.assert_allclose(h2, h1, rtol=0, atol=1e-12 * max(1.0, np.abs(h1).max()))


def test_chunked_packed_and_intermediates(oracle_mod):
    lens = [0, 70, 64, 5, 0, 129]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    q, k, v, g, beta = _case(19, T=int(cu[-1]) + 7, H=2, K=16, V=8, gate="safe")
    h0 = 0.1 * np.random.default_rng(20).standard_normal((len(lens), 2, 16, 8))
    C = 64
    o1, h1 = oracle.recurrent(q, k, v, g, beta, h0=h0, cu_seqlens=cu)
    o2, h2, it = chunked_forward(q, k, v, g, beta, h0=h0, cu_seqlens=cu, chunk_size=C, emit=True)
    valid = slice(0, int(cu[-1]))
    np.testing.assert_allclose(o2[:, valid], o1[:, valid], rtol=0, atol=1e-12)
    np.testing.assert_allclose(h2, h1, rtol=0, atol=1e-12)
    np.testing.assert_array_equal(h2[0], h0[0])
    np.testing.assert_array_equal(h2[4], h0[4])
    # chunk-start states equal the recurrence's state after the preceding prefix
    ci = 0
    for n, L in enumerate(lens):
        for c in range((L + C - 1) // C):
            t_end = int(cu[n]) + c * C
            s = slice(int(cu[n]), t_end)
            if t_end == int(cu[n]):
                want = h0[n]
            else:
                _, want = oracle.recurrent(q[:, s], k[:, s], v[:, s], g[:, s], beta[:, s], h0=h0[n:n + 1])
                want = want[0]
            np.testing.assert_allclose(it["hc"][ci], want, rtol=0, atol=1e-12)
            ci += 1
    assert ci == it["hc"].shape[0]
    # (I + A_kk) T = I on every chunk; A_kk strictly lower, A_qk lower
    for n, L in enumerate(lens):
        for c in range((L + C - 1) // C):
            t0 = int(cu[n]) + c * C
            Lc = min(C, L - c * C)
            for hh in range(2):
                A = it["Akk"][0, t0:t0 + Lc, hh, :Lc]
                Tm = it["T"][0, t0:t0 + Lc, hh, :Lc]
                np.testing.assert_allclose((np.eye(Lc) + A) @ Tm, np.eye(Lc), atol=1e-12)
                assert np.all(np.triu(A) == 0)
                assert np.all(np.triu(it["Aqk"][0, t0:t0 + Lc, hh, :Lc], 1) == 0)


def test_chunked_gram_matches_pairwise_definition(oracle_mod):
    """A_qk and A_kk of the anchored form equal the per-pair sums of their definition."""
    q, k, v, g, beta = _case(21, T=64, H=1, K=8, V=4, gate="safe")
    _, _, it = chunked_forward(q, k, v, g, beta, chunk_size=64, emit=True)
    G = np.cumsum(g[0, :, 0], axis=0)
    qq, kk, bb = q[0, :, 0], k[0, :, 0], beta[0, :, 0]
    for r in range(64):
        for s in range(64):
            d = np.sum(qq[r] * kk[s] * np.exp(G[r] - G[s])) / math.sqrt(8) if s <= r else 0.0
            e = bb[r] * np.sum(kk[r] * kk[s] * np.exp(G[r] - G[s])) if s < r else 0.0
            assert abs(it["Aqk"][0, r, 0, s] - d) <= 1e-12 * max(1, abs(d))
            assert abs(it["Akk"][0, r, 0, s] - e) <= 1e-12 * max(1, abs(e))


# ----------------------------------------------------------------------------------------
# Step (1) alone: the chunk-local cumsum in log2 units
# ----------------------------------------------------------------------------------------

def test_chunk_cumsum_pins(oracle_mod):
    """C = 1 is g / ln 2; a chunk spanning the sequence is numpy's cumsum; every chunk
    restarts; packed slots equal dense runs of their own rows; rows outside are NaN;
    the chunked form's own b agrees."""
    rng = np.random.default_rng(31)
    g = -np.abs(rng.standard_normal((2, 100, 3, 8)))
    ln2 = math.log(2.0)
    np.testing.assert_allclose(chunk_cumsum_log2(g, chunk_size=1), g / ln2, rtol=1e-15, atol=0)
    np.testing.assert_allclose(chunk_cumsum_log2(g, chunk_size=128), np.cumsum(g, axis=1) / ln2, rtol=1e-13)
    b32 = chunk_cumsum_log2(g, chunk_size=32)
    for c0 in range(0, 100, 32):
        np.testing.assert_allclose(b32[:, c0:c0 + 32], np.cumsum(g[:, c0:c0 + 32], axis=1) / ln2, rtol=1e-13)
    np.testing.assert_allclose(chunk_cumsum_log2(g / ln2, chunk_size=32, g_is_log2=True), b32, rtol=1e-13)

    lens = [0, 70, 5, 0, 33]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    gp = -np.abs(rng.standard_normal((1, int(cu[-1]) + 9, 2, 8)))
    bp = chunk_cumsum_log2(gp, cu_seqlens=cu, chunk_size=32)
    for n, L in enumerate(lens):
        s0 = int(cu[n])
        if L:
            np.testing.assert_allclose(bp[:, s0:s0 + L], chunk_cumsum_log2(gp[:, s0:s0 + L], chunk_size=32),
                                       rtol=1e-15)
    assert np.isnan(bp[:, int(cu[-1]):]).all()
    q, k, v, _, beta = _case(33, T=gp.shape[1], H=2, K=8, V=4)
    _, _, it = chunked_forward(q, k, v, gp, beta, cu_seqlens=cu, chunk_size=32, emit=True)
    valid = slice(0, int(cu[-1]))
    np.testing.assert_allclose(bp[:, valid], it["b"][:, valid], rtol=1e-13, atol=1e-13)


# ----------------------------------------------------------------------------------------
# The explicit q normalisation behind the q_l2norm option
# ----------------------------------------------------------------------------------------

def test_l2norm_rows_pins(oracle_mod):
    """Rows whose squared norm plus eps is exactly 1 come back unchanged; zero rows stay
    zero; large rows reach unit norm (eps negligible); tiny rows are divided by
    sqrt(eps); each row is normalised on its own."""
    f = oracle_mod.l2norm_rows
    eps = 1e-6
    b = math.sqrt(0.64 - eps)
    x = np.array([[0.6, b, 0.0], [0.0, 0.0, math.sqrt(1.0 - eps)], [0.0, 0.0, 0.0]])
    np.testing.assert_allclose(f(x), x, rtol=0, atol=1e-15)
    big = np.array([[3e6, 4e6, 0.0]])
    np.testing.assert_allclose(f(big), [[0.6, 0.8, 0.0]], rtol=1e-12, atol=0)
    tiny = np.array([[3e-9, -4e-9, 0.0]])
    np.testing.assert_allclose(f(tiny), tiny / math.sqrt(eps), rtol=1e-9, atol=0)
    rows = np.concatenate([big, tiny, x], axis=0)[None, :, None, :]  # [1, T, 1, K] like q
    together = f(rows)
    for t in range(rows.shape[1]):
        np.testing.assert_allclose(together[0, t, 0], f(rows[:, t:t + 1])[0, 0, 0], rtol=1e-15, atol=0)


def test_beta_from_logits_pins(oracle_mod):
    """sigma(0) = 1/2, sigma(ln 3) = 3/4 and sigma(-ln 3) = 1/4 exactly; sigma(x) +
    sigma(-x) = 1; the far tails are 1 and e^x without overflow."""
    f = oracle_mod.beta_from_logits
    np.testing.assert_allclose(f(np.array([0.0, math.log(3.0), -math.log(3.0)])), [0.5, 0.75, 0.25],
                               rtol=0, atol=1e-15)
    x = np.linspace(-30, 30, 121)
    np.testing.assert_allclose(f(x) + f(-x), 1.0, rtol=0, atol=1e-15)
    assert f(np.array([800.0]))[0] == 1.0
    np.testing.assert_allclose(f(np.array([-700.0]))[0], math.exp(-700.0), rtol=1e-12)


def _fd_grad(f, x, eps=1e-6):
    """Central finite differences of the scalar f at every element of x (in place, restored)."""
    gr = np.zeros_like(x)
    flat, gflat = x.reshape(-1), gr.reshape(-1)
    for i in range(flat.size):
        keep = flat[i]
        flat[i] = keep + eps
        fp = f()
        flat[i] = keep - eps
        fm = f()
        flat[i] = keep
        gflat[i] = (fp - fm) / (2 * eps)
    return gr


def test_recurrent_bwd_finite_differences(oracle_mod):
    """The reverse-mode gradients of the token recurrence equal central finite
    differences of L = sum(do * o) + sum(dht * ht) through the forward oracle, for
    every input element, on a packed batch with an empty slot (whose dh0 is dht)."""
    rng = np.random.default_rng(41)
    lens = [3, 0, 5]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T, H, K, V, N = int(cu[-1]) + 2, 2, 3, 2, len(lens)
    q = rng.standard_normal((1, T, H, K))
    k = rng.standard_normal((1, T, H, K)) / math.sqrt(K)
    v = rng.standard_normal((1, T, H, V))
    g = -rng.uniform(0.05, 0.6, (1, T, H, K))
    beta = rng.uniform(0.1, 0.9, (1, T, H))
    h0 = rng.standard_normal((N, H, K, V))
    do = rng.standard_normal((1, T, H, V))
    dht = rng.standard_normal((N, H, K, V))
    n = int(cu[-1])

    def loss():
        o, ht = oracle_mod.recurrent(q, k, v, g, beta, h0=h0, cu_seqlens=cu)
        return float(np.sum(do[:, :n] * o[:, :n]) + np.sum(dht * ht))

    dq, dk, dv, dg, db, dh0 = oracle_mod.recurrent_bwd(q, k, v, g, beta, do, dht=dht, h0=h0, cu_seqlens=cu)
    for name, x, got in (("q", q, dq), ("k", k, dk), ("v", v, dv), ("g", g, dg), ("beta", beta, db),
                         ("h0", h0, dh0)):
        want = _fd_grad(loss, x)
        if got.shape[:2] == (1, T):
            got, want = got[:, :n], want[:, :n]
        np.testing.assert_allclose(got, want, rtol=1e-6, atol=1e-8, err_msg=name)
    np.testing.assert_array_equal(dh0[1], dht[1])  # empty slot
    assert np.isnan(dq[:, n:]).all()


@pytest.mark.parametrize("kind", [0, 1, 2])
def test_gate_bwd_finite_differences(oracle_mod, kind):
    """gate_bwd equals central finite differences of sum(w * gate(x)) in x, A_log and dt_bias."""
    rng = np.random.default_rng(42 + kind)
    T, H, K = 5, 2, 3
    x = 2.0 * rng.standard_normal((1, T, H, K))
    A_log = rng.uniform(-1.0, 2.0, H)
    dt = rng.standard_normal((H, K))
    w = rng.standard_normal((1, T, H, K))
    lb = -3.0
    f = lambda: float(np.sum(w * oracle_mod.gate(kind, x, A_log, dt, lb)))
    dx, dA, ddt = oracle_mod.gate_bwd(kind, x, w, A_log, dt, lb)
    np.testing.assert_allclose(dx, _fd_grad(f, x), rtol=1e-6, atol=1e-9)
    if kind == oracle_mod.GATE_LOGE:
        assert dA is None and ddt is None
        return
    np.testing.assert_allclose(dA, _fd_grad(f, A_log), rtol=1e-6, atol=1e-9)
    np.testing.assert_allclose(ddt, _fd_grad(f, dt), rtol=1e-6, atol=1e-9)
