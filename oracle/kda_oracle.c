/*
 * FP64 CPU oracle for the Kimi Delta Attention (KDA) forward pass.
 *
 * TEST INFRASTRUCTURE ONLY. Only tests/, the smoke check and the CPU-baseline
 * leg of the benchmark may load this library. It shares no code, header,
 * table or helper with the HIP library; it is plain, slow, obviously correct C.
 *
 * What it computes (token by token, per slot and head):
 *
 *   alpha_t = exp(g_t)      (natural-log gate)  or  exp2(g_t)  (log2 gate)
 *   S'      = Diag(alpha_t) S
 *   delta_t = beta_t (v_t - S'^T k_t)
 *   S       = S' + k_t delta_t^T            == (I - beta k k^T) Diag(alpha) S + beta k v^T
 *   o_t     = S^T q_t * scale               (scale = 1/sqrt(K) by default)
 *
 * This is the gated delta rule with a per-channel decay. The query scale of
 * 1/sqrt(K), the FP32 state with one leading entry per logical sequence, the
 * packed int32 offsets and the bitwise pass-through of empty slots follow
 * "Add fused recurrent_kda for decode and inference prefill" (attention-gym
 * PR #317), section "Agent note". The per-token log2 gate of the recurrent
 * entry point is described in the same section. The gate activations follow
 * "FLA KDA Skill", section "Gate modes".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Gate kinds understood by kda_oracle_gate. */
#define ORACLE_GATE_LOGE 0     /* g already holds the natural-log decay          */
#define ORACLE_GATE_SAFE 1     /* lower_bound * sigmoid(exp(A_log) * (x + dt))   */
#define ORACLE_GATE_SOFTPLUS 2 /* -exp(A_log) * softplus(x + dt)                 */

/*
 * Gate activation ("FLA KDA Skill", section "Gate modes").
 *   x        [T, H, K]  raw gate input (or the decay itself for LOGE)
 *   A_log    [H]
 *   dt_bias  [H, K] or NULL (treated as 0)
 * Output g [T, H, K]: natural-log decay per token and channel.
 * softplus(z) is evaluated as log1p(exp(z)) directly; in FP64 exp(z) overflows
 * only for z > 709, far outside any input this oracle is given, and for those
 * it returns z (the exact limit) to stay finite.
 */
void kda_oracle_gate(int kind, int64_t T, int H, int K, const double *x, const double *A_log,
                     const double *dt_bias, double lower_bound, double *g) {
  for (int64_t t = 0; t < T; ++t) {
    for (int h = 0; h < H; ++h) {
      for (int i = 0; i < K; ++i) {
        int64_t idx = (t * H + h) * (int64_t)K + i;
        double z = x[idx] + (dt_bias ? dt_bias[(int64_t)h * K + i] : 0.0);
        if (kind == ORACLE_GATE_LOGE) {
          g[idx] = x[idx];
        } else if (kind == ORACLE_GATE_SAFE) {
          double a = exp(A_log[h]) * z;
          g[idx] = lower_bound * (1.0 / (1.0 + exp(-a)));
        } else {
          double sp = (z > 700.0) ? z : log1p(exp(z));
          g[idx] = -exp(A_log[h]) * sp;
        }
      }
    }
  }
}

/*
 * Token-by-token recurrence.
 *   N, H, K, V     slots, heads, key and value widths
 *   cu             [N+1] int32 token offsets (dense batches use 0, T, 2T, ...)
 *   q, k           [T_total, H, K]
 *   v              [T_total, H, V]
 *   g              [T_total, H, K] per-token decay, natural log (g_is_log2 == 0)
 *                  or log2 (g_is_log2 == 1)
 *   beta           [T_total, H]
 *   scale          query scale
 *   h0             [N, H, K, V] or NULL (zero initial state)
 *   o              [T_total, H, V]; rows outside [cu[0], cu[N]) are not touched
 *   ht             [N, H, K, V] or NULL; an empty slot gets h0 (or zeros) unchanged
 *   nthreads       OpenMP threads (<= 0: runtime default)
 */
void kda_oracle_recurrent(int N, int H, int K, int V, const int32_t *cu, const double *q,
                          const double *k, const double *v, const double *g, int g_is_log2,
                          const double *beta, double scale, const double *h0, double *o,
                          double *ht, int nthreads) {
  int64_t pairs = (int64_t)N * H;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
  for (int64_t p = 0; p < pairs; ++p) {
    int n = (int)(p / H);
    int h = (int)(p % H);
    double *S = (double *)malloc(sizeof(double) * (size_t)K * V);
    double *d = (double *)malloc(sizeof(double) * (size_t)V);
    const double *S0 = h0 ? h0 + p * (int64_t)K * V : NULL;
    for (int64_t e = 0; e < (int64_t)K * V; ++e) S[e] = S0 ? S0[e] : 0.0;

    for (int64_t t = cu[n]; t < cu[n + 1]; ++t) {
      const double *qt = q + (t * H + h) * (int64_t)K;
      const double *kt = k + (t * H + h) * (int64_t)K;
      const double *vt = v + (t * H + h) * (int64_t)V;
      const double *gt = g + (t * H + h) * (int64_t)K;
      double bt = beta[t * H + h];
      /* S' = Diag(alpha) S */
      for (int i = 0; i < K; ++i) {
        double a = g_is_log2 ? exp2(gt[i]) : exp(gt[i]);
        for (int j = 0; j < V; ++j) S[(int64_t)i * V + j] *= a;
      }
      /* delta = beta (v - S'^T k) */
      for (int j = 0; j < V; ++j) {
        double acc = 0.0;
        for (int i = 0; i < K; ++i) acc += S[(int64_t)i * V + j] * kt[i];
        d[j] = bt * (vt[j] - acc);
      }
      /* S = S' + k delta^T */
      for (int i = 0; i < K; ++i)
        for (int j = 0; j < V; ++j) S[(int64_t)i * V + j] += kt[i] * d[j];
      /* o = S^T q * scale */
      double *ot = o + (t * H + h) * (int64_t)V;
      for (int j = 0; j < V; ++j) {
        double acc = 0.0;
        for (int i = 0; i < K; ++i) acc += S[(int64_t)i * V + j] * qt[i];
        ot[j] = acc * scale;
      }
    }
    if (ht) {
      double *dst = ht + p * (int64_t)K * V;
      if (cu[n] == cu[n + 1] && S0) {
        memcpy(dst, S0, sizeof(double) * (size_t)K * V); /* empty slot: pass-through */
      } else {
        memcpy(dst, S, sizeof(double) * (size_t)K * V);
      }
    }
    free(S);
    free(d);
  }
}

/*
 * Backward of kda_oracle_recurrent (natural-log gate) by reverse-mode through
 * the token recurrence, for the loss L = sum(do * o) + sum(dht * ht). With
 * P_t = Diag(alpha_t) S_{t-1}, delta_t = beta_t (v_t - P_t^T k_t),
 * S_t = P_t + k_t delta_t^T and o_t = scale S_t^T q_t, one reverse step takes
 * the gradient dS of S_t to that of S_{t-1}:
 *
 *   dS     += scale q_t do_t^T                 dq_t   = scale S_t do_t
 *   ddelta  = dS^T k_t                         dk_t   = dS delta_t - beta_t P_t ddelta
 *   dv_t    = beta_t ddelta                    dbeta_t = ddelta . (v_t - P_t^T k_t)
 *   dP      = dS - beta_t k_t ddelta^T
 *   dg_t[i] = alpha_t[i] sum_j dP[i, j] S_{t-1}[i, j]      (d/dg of exp(g) = exp(g))
 *   dS      = Diag(alpha_t) dP
 *
 * The forward states of the slot are kept whole (plain and slow: test sizes
 * only). Outputs: dq, dk [T_total, H, K]; dv [T_total, H, V]; dg [T_total, H, K]
 * (gradient of the per-token natural-log gate); dbeta [T_total, H]; dh0
 * [N, H, K, V] or NULL. Rows outside [cu[0], cu[N]) are not touched. dht may be
 * NULL (zero).
 */
void kda_oracle_recurrent_bwd(int N, int H, int K, int V, const int32_t *cu, const double *q,
                              const double *k, const double *v, const double *g, const double *beta,
                              double scale, const double *h0, const double *dout, const double *dht,
                              double *dq, double *dk, double *dv, double *dg, double *dbeta, double *dh0,
                              int nthreads) {
  int64_t pairs = (int64_t)N * H;
  const int64_t KV = (int64_t)K * V;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
  for (int64_t p = 0; p < pairs; ++p) {
    int n = (int)(p / H);
    int h = (int)(p % H);
    int64_t t0 = cu[n], len = cu[n + 1] - cu[n];
    /* states S_{t0-1} .. S_{t0+len-1}: Sall + (t - t0 + 1) * KV holds S_t */
    double *Sall = (double *)malloc(sizeof(double) * (size_t)((len + 1) * KV));
    double *dS = (double *)malloc(sizeof(double) * (size_t)KV);
    double *P = (double *)malloc(sizeof(double) * (size_t)KV);
    double *dlt = (double *)malloc(sizeof(double) * (size_t)V);
    double *u = (double *)malloc(sizeof(double) * (size_t)V);
    double *ddl = (double *)malloc(sizeof(double) * (size_t)V);
    const double *S0 = h0 ? h0 + p * KV : NULL;
    for (int64_t e = 0; e < KV; ++e) Sall[e] = S0 ? S0[e] : 0.0;
    /* forward, keeping every state */
    for (int64_t s = 0; s < len; ++s) {
      int64_t t = t0 + s;
      const double *kt = k + (t * H + h) * (int64_t)K;
      const double *vt = v + (t * H + h) * (int64_t)V;
      const double *gt = g + (t * H + h) * (int64_t)K;
      double bt = beta[t * H + h];
      const double *Sp = Sall + s * KV;
      double *Sn = Sall + (s + 1) * KV;
      for (int i = 0; i < K; ++i)
        for (int j = 0; j < V; ++j) Sn[(int64_t)i * V + j] = exp(gt[i]) * Sp[(int64_t)i * V + j];
      for (int j = 0; j < V; ++j) {
        double acc = 0.0;
        for (int i = 0; i < K; ++i) acc += Sn[(int64_t)i * V + j] * kt[i];
        dlt[j] = bt * (vt[j] - acc);
      }
      for (int i = 0; i < K; ++i)
        for (int j = 0; j < V; ++j) Sn[(int64_t)i * V + j] += kt[i] * dlt[j];
    }
    /* reverse */
    for (int64_t e = 0; e < KV; ++e) dS[e] = dht ? dht[p * KV + e] : 0.0;
    for (int64_t s = len - 1; s >= 0; --s) {
      int64_t t = t0 + s;
      const double *qt = q + (t * H + h) * (int64_t)K;
      const double *kt = k + (t * H + h) * (int64_t)K;
      const double *vt = v + (t * H + h) * (int64_t)V;
      const double *gt = g + (t * H + h) * (int64_t)K;
      const double *dot = dout + (t * H + h) * (int64_t)V;
      double bt = beta[t * H + h];
      const double *Sp = Sall + s * KV;      /* S_{t-1} */
      const double *St = Sall + (s + 1) * KV; /* S_t */
      double *dqt = dq + (t * H + h) * (int64_t)K;
      double *dkt = dk + (t * H + h) * (int64_t)K;
      double *dvt = dv + (t * H + h) * (int64_t)V;
      double *dgt = dg + (t * H + h) * (int64_t)K;
      /* o_t = scale S_t^T q_t */
      for (int i = 0; i < K; ++i) {
        double acc = 0.0;
        for (int j = 0; j < V; ++j) acc += St[(int64_t)i * V + j] * dot[j];
        dqt[i] = scale * acc;
        for (int j = 0; j < V; ++j) dS[(int64_t)i * V + j] += scale * qt[i] * dot[j];
      }
      /* rebuild P_t, delta_t and P_t^T k_t */
      for (int i = 0; i < K; ++i)
        for (int j = 0; j < V; ++j) P[(int64_t)i * V + j] = exp(gt[i]) * Sp[(int64_t)i * V + j];
      for (int j = 0; j < V; ++j) {
        double acc = 0.0;
        for (int i = 0; i < K; ++i) acc += P[(int64_t)i * V + j] * kt[i];
        u[j] = acc;
        dlt[j] = bt * (vt[j] - acc);
      }
      /* S_t = P_t + k_t delta_t^T */
      double db = 0.0;
      for (int j = 0; j < V; ++j) {
        double acc = 0.0;
        for (int i = 0; i < K; ++i) acc += dS[(int64_t)i * V + j] * kt[i];
        ddl[j] = acc;
        dvt[j] = bt * acc;
        db += acc * (vt[j] - u[j]);
      }
      dbeta[t * H + h] = db;
      for (int i = 0; i < K; ++i) {
        double a1 = 0.0, a2 = 0.0;
        for (int j = 0; j < V; ++j) {
          a1 += dS[(int64_t)i * V + j] * dlt[j];
          a2 += P[(int64_t)i * V + j] * ddl[j];
        }
        dkt[i] = a1 - bt * a2;
      }
      /* dP = dS - beta k ddelta^T ; dg ; dS_{t-1} = Diag(alpha) dP */
      for (int i = 0; i < K; ++i) {
        double al = exp(gt[i]), acc = 0.0;
        for (int j = 0; j < V; ++j) {
          double dp = dS[(int64_t)i * V + j] - bt * kt[i] * ddl[j];
          acc += dp * Sp[(int64_t)i * V + j];
          dS[(int64_t)i * V + j] = al * dp;
        }
        dgt[i] = al * acc;
      }
    }
    if (dh0) memcpy(dh0 + p * KV, dS, sizeof(double) * (size_t)KV);
    free(Sall);
    free(dS);
    free(P);
    free(dlt);
    free(u);
    free(ddl);
  }
}
