// Host side of the C ABI declared in include/kda.h: argument validation,
// workspace carving and kernel launches on the caller's stream. No host
// synchronisation, no allocation, no host read of device memory.
#include <math.h>
#include <stdio.h>
#include <string.h>

#include "../../include/kda.h"
#include "kda_launch.h"

namespace {

thread_local char g_last_error[256] = "";

kda_status hip_status(hipError_t e) {
  if (e == hipSuccess) return KDA_OK;
  snprintf(g_last_error, sizeof(g_last_error), "%s: %s", hipGetErrorName(e), hipGetErrorString(e));
  return KDA_ERR_HIP;
}

bool aligned16(const void *p) { return p == nullptr || (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool width_ok(int d) { return d == 64 || d == 128 || d == 256; }

// Checks shared by both entry points.
kda_status check_common(const kda_args *a, const void *q, const void *k, const void *v, const float *g,
                        const float *beta, const float *h0, const void *o, const float *ht, bool recurrent) {
  if (!a) return KDA_ERR_NULL;
  if (a->B < 1 || a->T < 0 || a->H < 1 || a->N < 0) return KDA_ERR_SHAPE;
  if (a->K < 1 || a->V < 1) return KDA_ERR_SHAPE;
  if (a->dtype != KDA_BF16 && a->dtype != KDA_F32) return KDA_ERR_DTYPE;
  if (!q || !k || !v || !g || !beta || !o) return KDA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(g) || !aligned16(o) || !aligned16(h0) ||
      !aligned16(ht))
    return KDA_ERR_ALIGN;
  switch (a->gate_kind) {
    case KDA_GATE_LOGE:
      break;
    case KDA_GATE_LOG2:
      if (!recurrent) return KDA_ERR_GATE;
      break;
    case KDA_GATE_SAFE:
      if (!a->A_log) return KDA_ERR_GATE;
      if (!(a->lower_bound >= -5.0f && a->lower_bound < 0.0f)) return KDA_ERR_GATE;
      break;
    case KDA_GATE_SOFTPLUS:
      if (!a->A_log) return KDA_ERR_GATE;
      break;
    default:
      return KDA_ERR_GATE;
  }
  if (!width_ok(a->K) || !width_ok(a->V)) return KDA_ERR_UNSUPPORTED;
  return KDA_OK;
}

int n_slots(const kda_args *a, const int32_t *cu) { return cu ? a->N : a->B; }

kda_status check_slots(const kda_args *a, const int32_t *cu) {
  if (cu) {
    if (a->B != 1) return KDA_ERR_SHAPE;
  } else if (a->N != a->B) {
    return KDA_ERR_SHAPE;
  }
  return KDA_OK;
}

float resolve_scale(const kda_args *a) { return a->scale > 0.f ? a->scale : 1.0f / sqrtf((float)a->K); }

}  // namespace

extern "C" const char *kda_status_string(kda_status s) {
  switch (s) {
    case KDA_OK: return "KDA_OK";
    case KDA_ERR_NULL: return "KDA_ERR_NULL: a required pointer is NULL";
    case KDA_ERR_SHAPE: return "KDA_ERR_SHAPE: inconsistent or out-of-range sizes";
    case KDA_ERR_DTYPE: return "KDA_ERR_DTYPE: unknown dtype";
    case KDA_ERR_CHUNK: return "KDA_ERR_CHUNK: unsupported chunk size";
    case KDA_ERR_GATE: return "KDA_ERR_GATE: invalid gate kind, A_log or lower bound";
    case KDA_ERR_ALIGN: return "KDA_ERR_ALIGN: a tensor is not 16-byte aligned";
    case KDA_ERR_WORKSPACE: return "KDA_ERR_WORKSPACE: workspace missing or too small";
    case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED: valid but not implemented";
    case KDA_ERR_HIP: return "KDA_ERR_HIP: a HIP launch failed";
  }
  return "unknown kda_status";
}

extern "C" const char *kda_last_error(void) { return g_last_error; }

extern "C" kda_status kda_recurrent_fwd(const kda_args *a, const void *q, const void *k, const void *v,
                                        const float *g, const float *beta, const float *h0,
                                        const int32_t *cu_seqlens, void *o, float *ht, void *stream) {
  kda_status s = check_common(a, q, k, v, g, beta, h0, o, ht, true);
  if (s != KDA_OK) return s;
  if ((s = check_slots(a, cu_seqlens)) != KDA_OK) return s;
  kda::RecurrentParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.g = g;
  p.beta = beta;
  p.h0 = h0;
  p.cu = cu_seqlens;
  p.o = o;
  p.ht = ht;
  p.A_log = a->A_log;
  p.dt_bias = a->dt_bias;
  p.lower_bound = a->lower_bound;
  p.scale = resolve_scale(a);
  p.gate_kind = (int)a->gate_kind;
  p.B = a->B;
  p.T = a->T;
  p.H = a->H;
  p.K = a->K;
  p.V = a->V;
  p.N = n_slots(a, cu_seqlens);
  p.is_bf16 = a->dtype == KDA_BF16;
  return hip_status(kda::launch_recurrent(p, (hipStream_t)stream));
}

extern "C" size_t kda_chunk_workspace_bytes(const kda_args *a) {
  (void)a;
  return 0;
}

extern "C" kda_status kda_chunk_fwd(const kda_args *a, const void *q, const void *k, const void *v, const float *g,
                                    const float *beta, const float *h0, const int32_t *cu_seqlens, void *o,
                                    float *ht, void *workspace, size_t ws_bytes, void *stream) {
  (void)a; (void)q; (void)k; (void)v; (void)g; (void)beta; (void)h0; (void)cu_seqlens; (void)o; (void)ht;
  (void)workspace; (void)ws_bytes; (void)stream;
  return KDA_ERR_UNSUPPORTED;
}
