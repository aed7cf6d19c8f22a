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
