// Host side of the C ABI declared in include/kda.h: argument validation,
// workspace carving and kernel launches on the caller's stream. No host
// synchronisation, no allocation, no host read of device memory.
#include <math.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "../../include/kda.h"
#include "../../include/kda_stages.h"
#include "kda_launch.h"

namespace {

thread_local char g_last_error[256] = "";

kda_status hip_status(hipError_t e) {
  if (e == hipSuccess) return KDA_OK;
  snprintf(g_last_error, sizeof(g_last_error), "%s: %s", hipGetErrorName(e), hipGetErrorString(e));
  return KDA_ERR_HIP;
}

bool aligned16(const void *p) { return p == nullptr || (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Widths of q/k (K) and v (V): multiples of 8 up to 256, so every row of a
// 16-byte aligned tensor starts 16-byte aligned. The kernels run at the tile
// width pad_width(max(K, V)) and mask the rest.
// Heads per call: one chunk's 64 rows of a [*, H, 256] fp32 tensor then span under
// 2^28 bytes, so the kernels' 32-bit in-chunk offsets and their out-of-range
// sentinels (2^30 and above) never meet.
constexpr int kMaxHeads = 4096;

bool width_ok(int d) { return d >= 8 && d <= 256 && d % 8 == 0; }
int pad_width(int d) { return d <= 64 ? 64 : (d <= 128 ? 128 : 256); }

// Checks shared by both entry points.
kda_status check_common(const kda_args *a, const void *q, const void *k, const void *v, const float *g,
                        const float *beta, const float *h0, const void *o, const float *ht, bool recurrent) {
  if (!a) return KDA_ERR_NULL;
  if (a->B < 1 || a->T < 0 || a->H < 1 || a->H > kMaxHeads || a->N < 0) return KDA_ERR_SHAPE;
  if (a->q_l2norm != 0 && a->q_l2norm != 1) return KDA_ERR_SHAPE;
  if (a->beta_logits != 0 && a->beta_logits != 1) return KDA_ERR_SHAPE;
  if (a->Hk < 0 || (a->Hk > 0 && a->H % a->Hk != 0)) return KDA_ERR_SHAPE;
  if (a->K < 1 || a->V < 1) return KDA_ERR_SHAPE;
  if (a->dtype != KDA_BF16 && a->dtype != KDA_F32) return KDA_ERR_DTYPE;
  // with no tokens (T == 0) the token tensors are never touched and may be NULL
  if (a->T > 0 && (!q || !k || !v || !g || !beta || !o)) return KDA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(g) || !aligned16(o) || !aligned16(h0) ||
      !aligned16(ht))
    return KDA_ERR_ALIGN;
  switch (a->gate_kind) {
    case KDA_GATE_LOGE:
      break;
    case KDA_GATE_LOG2:
      if (!recurrent) return KDA_ERR_GATE;
      break;
    case KDA_GATE_LOG2_CUMSUM:
      if (recurrent) return KDA_ERR_GATE;
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

extern "C" kda_status kda_check_offsets(const int32_t *cu_seqlens, int N, int T, int32_t *flags, void *stream) {
  if (!cu_seqlens || !flags) return KDA_ERR_NULL;
  if (N < 0 || T < 0) return KDA_ERR_SHAPE;
  return hip_status(kda::launch_check_offsets(cu_seqlens, N, T, flags, (hipStream_t)stream));
}

// ---------------------------------------------------------------------------------------------
// step (1) on its own
// ---------------------------------------------------------------------------------------------
extern "C" kda_status kda_gate_cumsum(const kda_args *a, const float *g_in, const int32_t *cu_seqlens,
                                      int chunk_size, float *g_out, void *stream) {
  if (!a) return KDA_ERR_NULL;
  if (a->B < 1 || a->T < 0 || a->H < 1 || a->H > kMaxHeads || a->N < 0 || a->K < 1) return KDA_ERR_SHAPE;
  if (a->T > 0 && (!g_in || !g_out)) return KDA_ERR_NULL;
  if (!aligned16(g_in) || !aligned16(g_out)) return KDA_ERR_ALIGN;
  if (chunk_size != 1 && chunk_size != 32 && chunk_size != 64) return KDA_ERR_CHUNK;
  switch (a->gate_kind) {
    case KDA_GATE_LOGE:
    case KDA_GATE_LOG2:
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
  if (!width_ok(a->K)) return KDA_ERR_UNSUPPORTED;
  kda_status s = check_slots(a, cu_seqlens);
  if (s != KDA_OK) return s;
  const size_t bytes = sizeof(float) * (size_t)a->B * a->T * a->H * a->K;
  const char *i0 = reinterpret_cast<const char *>(g_in), *o0 = reinterpret_cast<const char *>(g_out);
  if (bytes > 0 && i0 < o0 + bytes && o0 < i0 + bytes) return KDA_ERR_SHAPE;  // overlapping in/out
  kda::GateCumsumParams p{};
  p.g = g_in;
  p.out = g_out;
  p.cu = cu_seqlens;
  p.A_log = a->A_log;
  p.dt_bias = a->dt_bias;
  p.lower_bound = a->lower_bound;
  p.gate_kind = (int)a->gate_kind;
  p.B = a->B;
  p.T = a->T;
  p.H = a->H;
  p.K = a->K;
  p.N = n_slots(a, cu_seqlens);
  p.C = chunk_size;
  return hip_status(kda::launch_gate_cumsum(p, (hipStream_t)stream));
}

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
  p.q_l2norm = a->q_l2norm;
  p.Hk = a->Hk > 0 ? a->Hk : a->H;
  p.beta_logits = a->beta_logits;
  return hip_status(kda::launch_recurrent(p, (hipStream_t)stream));
}

// ---------------------------------------------------------------------------------------------
// chunked prefill
// ---------------------------------------------------------------------------------------------
namespace {

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool chunk_shape_ok(const kda_args *a) {
  if (!a) return false;
  if (a->B < 1 || a->T < 0 || a->H < 1 || a->H > kMaxHeads || a->N < 0) return false;
  if (!width_ok(a->K) || !width_ok(a->V)) return false;
  if (a->chunk_size != 32 && a->chunk_size != 64) return false;
  return true;
}

// Upper bound of the number of chunks: dense B * ceil(T/C); packed ceil(T/C) + N
// (each slot adds at most one partial chunk).
int64_t max_chunks(const kda_args *a, bool packed) {
  const int64_t nt = ((int64_t)a->T + a->chunk_size - 1) / a->chunk_size;
  return packed ? nt + a->N : (int64_t)a->B * nt;
}

struct WsLayout {
  size_t off[9];
  size_t total;
};

// The staged workspace is laid out for the packed bound of chunks, so one
// layout serves dense and packed calls with the same sizes.
WsLayout staged_layout(const kda_args *a) {
  WsLayout L{};
  const size_t rows = (size_t)a->B * a->T * a->H;
  const size_t D = pad_width(std::max(a->K, a->V)), C = a->chunk_size;
  const size_t nch = (size_t)std::max<int64_t>(max_chunks(a, true), max_chunks(a, false));
  const size_t sz[9] = {sizeof(int32_t) * (a->N + 1), 4 * rows * D, 4 * rows * C, 4 * rows * C, 4 * rows * C,
                        4 * rows * D, 4 * rows * D, 4 * rows * D, 4 * nch * a->H * (size_t)a->K * a->V};
  size_t cur = 0;
  for (int i = 0; i < 9; ++i) {
    L.off[i] = cur;
    cur += align_up(sz[i]);
  }
  L.total = cur;
  return L;
}

// AUTO on a shape the fused kernel takes: split when its cost model says so.
// Depends on the arguments' sizes (and the device's compute units) only, so
// kda_chunk_workspace_bytes makes the same choice.
bool auto_split(const kda_args *a) {
  const int64_t chain = ((int64_t)a->T + a->chunk_size - 1) / a->chunk_size;
  const int64_t items = std::max<int64_t>(max_chunks(a, true), max_chunks(a, false)) * a->H;
  return kda::split_preferred(chain, (int64_t)a->N * a->H, items, pad_width(std::max(a->K, a->V)));
}

// AUTO at tile width 256 with 64-row chunks: the fused kernel takes 32-row chunks
// at this width (its LDS holds a 32-row chunk of 256 channels), which give the
// same o and ht up to rounding; the chunk-start states keep the requested chunk.
// A gate cumsummed by the caller is chunk-local to the requested chunk size, so
// it keeps that size (and the staged schedule).
bool auto_fused_c32(const kda_args *a) {
  return a->schedule == KDA_SCHED_AUTO && a->dtype == KDA_BF16 && a->chunk_size == 64 &&
         a->gate_kind != KDA_GATE_LOG2_CUMSUM && pad_width(std::max(a->K, a->V)) == 256;
}

bool use_split(const kda_args *a, const kda::ChunkParams &p) {
  if (!kda::split_supported(p)) return false;
  return a->schedule == KDA_SCHED_SPLIT || (a->schedule == KDA_SCHED_AUTO && auto_split(a));
}

// The pipelined fused kernel: when named, or under AUTO / FUSED where it takes the
// arguments and there are more (sequence, head) pairs than half the compute units
// (fewer leave the serial fused kernel room to split value columns).
bool use_pipe(const kda_args *a, const kda::ChunkParams &p) {
  if (!kda::pipe_supported(p)) return false;
  if (a->schedule == KDA_SCHED_PIPE) return true;
  if (a->schedule != KDA_SCHED_AUTO) return false;  // an explicit schedule runs its own kernel
  return !use_split(a, p) && 2 * (int64_t)a->N * a->H > kda::device_cus();
}

bool use_fused(const kda_args *a, const kda::ChunkParams &p) {
  if (a->schedule != KDA_SCHED_AUTO && a->schedule != KDA_SCHED_FUSED) return false;
  return kda::fused_supported(p) && !use_split(a, p) && !use_pipe(a, p);
}

bool schedule_known(const kda_args *a) {
  return a->schedule == KDA_SCHED_AUTO || a->schedule == KDA_SCHED_STAGED || a->schedule == KDA_SCHED_FUSED ||
         a->schedule == KDA_SCHED_SPLIT || a->schedule == KDA_SCHED_PIPE;
}

// The fields of ChunkParams that the schedule choice reads.
kda::ChunkParams shape_params(const kda_args *a) {
  kda::ChunkParams p{};
  p.D = pad_width(std::max(a->K, a->V));
  p.C = a->chunk_size;
  p.is_bf16 = a->dtype == KDA_BF16;
  p.gate_kind = (int)a->gate_kind;
  return p;
}

// Chunks per segment of the split schedule's state side (0: the serial chain):
// args->segment when set, else the cost model's choice for a dense batch's chain
// of ceil(T / C) chunks. A packed batch (N != B) keeps the serial chain unless
// asked: its lengths are on the device, and the capacity bounds its longest
// slot only loosely.
int seg_len_for(const kda_args *a) {
  if (a->segment < 0) return 0;
  if (a->segment > 0) return a->segment;
  if (a->N != a->B) return 0;
  const int64_t nt = ((int64_t)a->T + a->chunk_size - 1) / a->chunk_size;
  return kda::split_segment_len(nt, (int64_t)a->N * a->H, pad_width(std::max(a->K, a->V)), a->chunk_size);
}

// Upper bound of the segments of a split call (packed or dense sizes).
int64_t seg_bound(const kda_args *a, int len) {
  const int64_t nt = ((int64_t)a->T + a->chunk_size - 1) / a->chunk_size;
  return std::max<int64_t>(kda::split_segment_bound(a->B, a->N, nt, true, len),
                           kda::split_segment_bound(a->B, a->N, nt, false, len));
}

// Split schedule: the chunk prefix, then the key side's records for every
// (chunk, head) of the packed or dense bound; with segments, the segment
// prefix, E and o_local per (chunk, head), [M | B] and the incoming state per
// (segment, head).
size_t split_ws_bytes(const kda_args *a) {
  const int64_t nch = std::max<int64_t>(max_chunks(a, true), max_chunks(a, false));
  const int D = pad_width(std::max(a->K, a->V));
  size_t b = align_up(sizeof(int32_t) * (a->N + 1)) + align_up(kda::split_workspace_bytes(a->chunk_size, D, nch * a->H));
  const int len = seg_len_for(a);
  if (len > 0)
    b += align_up(sizeof(int32_t) * (a->N + 1)) +
         align_up(kda::split_segment_bytes(a->chunk_size, D, nch * a->H, seg_bound(a, len) * a->H));
  return b;
}

kda_status prepare_chunk(const kda_args *a, const void *q, const void *k, const void *v, const float *g,
                         const float *beta, const float *h0, const int32_t *cu, void *o, float *ht, void *ws,
                         size_t ws_bytes, kda::ChunkParams &p) {
  kda_status s = check_common(a, q, k, v, g, beta, h0, o, ht, false);
  if (s != KDA_OK) return s;
  if ((s = check_slots(a, cu)) != KDA_OK) return s;
  if (a->chunk_size != 32 && a->chunk_size != 64) return KDA_ERR_CHUNK;
  if (!schedule_known(a)) return KDA_ERR_SHAPE;
  p = kda::ChunkParams{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.g = g;
  p.beta = beta;
  p.h0 = h0;
  p.cu = cu;
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
  p.D = pad_width(std::max(a->K, a->V));
  p.Kr = a->K;
  p.Vr = a->V;
  p.N = n_slots(a, cu);
  p.C = a->chunk_size;
  p.is_bf16 = a->dtype == KDA_BF16;
  p.q_l2norm = a->q_l2norm;
  p.Hk = a->Hk > 0 ? a->Hk : a->H;
  p.beta_logits = a->beta_logits;
  p.max_chunks = (int)max_chunks(a, cu != nullptr);
  if ((a->schedule == KDA_SCHED_FUSED && !kda::fused_supported(p)) ||
      (a->schedule == KDA_SCHED_SPLIT && !kda::split_supported(p)))
    return KDA_ERR_UNSUPPORTED;
  if (a->schedule == KDA_SCHED_PIPE && !kda::pipe_supported(p)) return KDA_ERR_UNSUPPORTED;
  const size_t need = kda_chunk_workspace_bytes(a);
  if (need > 0 && (!ws || ws_bytes < need)) return KDA_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(ws) & (kAlign - 1)) != 0) return KDA_ERR_ALIGN;
  char *base = static_cast<char *>(ws);
  if (use_fused(a, p) || use_pipe(a, p)) {
    p.chunk_off = reinterpret_cast<int32_t *>(base);
  } else if (use_split(a, p)) {
    const int64_t nch = std::max<int64_t>(max_chunks(a, true), max_chunks(a, false));
    const size_t bf = (size_t)nch * a->H * 2 * (3 * (size_t)p.C * p.D + (size_t)p.C * p.C);
    p.chunk_off = reinterpret_cast<int32_t *>(base);
    p.sws = base + align_up(sizeof(int32_t) * (a->N + 1));
    p.swf = reinterpret_cast<float *>(static_cast<char *>(p.sws) + bf);
    p.seg_len = seg_len_for(a);
    if (p.seg_len > 0) {
      p.seg_max = (int)seg_bound(a, p.seg_len);
      char *sb = static_cast<char *>(p.sws) + align_up(kda::split_workspace_bytes(p.C, p.D, nch * a->H));
      p.seg_off = reinterpret_cast<int32_t *>(sb);
      sb += align_up(sizeof(int32_t) * (a->N + 1));
      const size_t ch = (size_t)nch * a->H * p.C * p.D;
      p.seg_e = sb;
      p.seg_ol = reinterpret_cast<float *>(sb + 2 * ch);
      p.seg_mb = reinterpret_cast<float *>(sb + 6 * ch);
      p.seg_sin = p.seg_mb + (size_t)p.seg_max * a->H * p.D * 2 * p.D;  // bf16 fragments
    }
  } else {
    const WsLayout L = staged_layout(a);
    p.chunk_off = reinterpret_cast<int32_t *>(base + L.off[0]);
    p.b = reinterpret_cast<float *>(base + L.off[1]);
    p.Akk = reinterpret_cast<float *>(base + L.off[2]);
    p.Aqk = reinterpret_cast<float *>(base + L.off[3]);
    p.Tm = reinterpret_cast<float *>(base + L.off[4]);
    p.w = reinterpret_cast<float *>(base + L.off[5]);
    p.u = reinterpret_cast<float *>(base + L.off[6]);
    p.vnew = reinterpret_cast<float *>(base + L.off[7]);
    p.hc = reinterpret_cast<float *>(base + L.off[8]);
  }
  return KDA_OK;
}

kda_status run_stage(const kda::ChunkParams &p, int stage, hipStream_t st) {
  switch (stage) {
    case KDA_STAGE_INDEX: return hip_status(kda::launch_chunk_index(p, st));
    case KDA_STAGE_GATE: return hip_status(kda::launch_stage_gate(p, st));
    case KDA_STAGE_GRAMS: return hip_status(kda::launch_stage_grams(p, st));
    case KDA_STAGE_SOLVE: return hip_status(kda::launch_stage_solve(p, st));
    case KDA_STAGE_WY: return hip_status(kda::launch_stage_wy(p, st));
    case KDA_STAGE_SCAN: return hip_status(kda::launch_stage_scan(p, st));
    case KDA_STAGE_OUTPUT: return hip_status(kda::launch_stage_output(p, st));
  }
  return KDA_ERR_SHAPE;
}

}  // namespace

extern "C" size_t kda_chunk_workspace_bytes(const kda_args *a) {
  if (!chunk_shape_ok(a)) return 0;
  const kda::ChunkParams p = shape_params(a);
  if (a->schedule == KDA_SCHED_PIPE) return kda::pipe_supported(p) ? align_up(sizeof(int32_t) * (a->N + 1)) : 0;
  if (a->schedule == KDA_SCHED_SPLIT) return kda::split_supported(p) ? split_ws_bytes(a) : 0;
  if (a->schedule == KDA_SCHED_AUTO && kda::split_supported(p) && auto_split(a)) return split_ws_bytes(a);
  if (a->schedule != KDA_SCHED_STAGED && kda::fused_supported(p)) return align_up(sizeof(int32_t) * (a->N + 1));
  if (a->schedule == KDA_SCHED_FUSED) return 0;
  return staged_layout(a).total;
}

extern "C" int kda_chunk_schedule(const kda_args *a) {
  if (!chunk_shape_ok(a) || !schedule_known(a)) return -1;
  const kda::ChunkParams p = shape_params(a);
  if ((a->schedule == KDA_SCHED_FUSED && !kda::fused_supported(p)) ||
      (a->schedule == KDA_SCHED_SPLIT && !kda::split_supported(p)))
    return -1;
  if (a->schedule == KDA_SCHED_PIPE && !kda::pipe_supported(p)) return -1;
  if (auto_fused_c32(a)) return KDA_SCHED_FUSED;
  if (use_pipe(a, p)) return KDA_SCHED_PIPE;
  if (use_split(a, p)) return KDA_SCHED_SPLIT;
  if (use_fused(a, p)) return KDA_SCHED_FUSED;
  return KDA_SCHED_STAGED;
}

extern "C" int kda_chunk_segment(const kda_args *a) {
  if (kda_chunk_schedule(a) != KDA_SCHED_SPLIT) return 0;
  return seg_len_for(a);
}

extern "C" size_t kda_staged_workspace_offset(const kda_args *a, kda_ws_field field) {
  if (!chunk_shape_ok(a) || (int)field < 0 || (int)field > 8) return (size_t)-1;
  return staged_layout(a).off[(int)field];
}

namespace {

// states: the caller asked for the chunk-start states (they follow its chunk size)
kda_status run_chunk(const kda_args *a, const kda::ChunkParams &p, hipStream_t st, bool states) {
  kda_status s;
  if (auto_fused_c32(a) && !states) {
    // the same o and ht as 64-row chunks, up to rounding, on chip
    kda::ChunkParams q = p;
    q.C = 32;
    q.hc = nullptr;  // p.hc points into the staged layout of the workspace: no states here
    return hip_status(kda::launch_fused(q, st));
  }
  if (use_pipe(a, p)) {
    // the chunk prefix only numbers the chunk-start states
    if (p.hc && p.cu && (s = run_stage(p, KDA_STAGE_INDEX, st)) != KDA_OK) return s;
    return hip_status(kda::launch_pipe(p, st));
  }
  if (use_fused(a, p)) {
    // the fused kernel reads the chunk prefix only to number the chunk-start states
    if (p.hc && p.cu && (s = run_stage(p, KDA_STAGE_INDEX, st)) != KDA_OK) return s;
    return hip_status(kda::launch_fused(p, st));
  }
  if (use_split(a, p)) {
    kda::ChunkParams q = p;
    if (states) q.seg_len = 0;  // the chunk-start states come from the serial chain
    if (q.cu && (s = run_stage(q, KDA_STAGE_INDEX, st)) != KDA_OK) return s;
    return hip_status(kda::launch_split(q, st));
  }
  for (int stage = KDA_STAGE_INDEX; stage <= KDA_STAGE_OUTPUT; ++stage)
    if ((s = run_stage(p, stage, st)) != KDA_OK) return s;
  return KDA_OK;
}

}  // namespace

extern "C" kda_status kda_chunk_fwd(const kda_args *a, const void *q, const void *k, const void *v, const float *g,
                                    const float *beta, const float *h0, const int32_t *cu_seqlens, void *o,
                                    float *ht, void *workspace, size_t ws_bytes, void *stream) {
  kda::ChunkParams p;
  kda_status s = prepare_chunk(a, q, k, v, g, beta, h0, cu_seqlens, o, ht, workspace, ws_bytes, p);
  if (s != KDA_OK) return s;
  return run_chunk(a, p, (hipStream_t)stream, false);
}

// ---------------------------------------------------------------------------------------------
// kda_chunk_fwd without a caller workspace: the intermediates live in a static
// device array. In host code the array's name is a host-side stand-in; the
// device address comes from hipGetSymbolAddress, looked up once per device.
// ---------------------------------------------------------------------------------------------
namespace {

constexpr size_t kNoAllocBytes = (size_t)64 << 20;
__device__ __align__(256) char scratch[kNoAllocBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch`.
kda_status scratch_address(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (dev < 0 || dev >= kMaxDevices) {
    snprintf(g_last_error, sizeof(g_last_error), "device %d beyond the %d devices the static array covers", dev,
             kMaxDevices);
    return KDA_ERR_UNSUPPORTED;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e);
    if (!p) {
      snprintf(g_last_error, sizeof(g_last_error), "hipGetSymbolAddress returned NULL for the static array");
      return KDA_ERR_HIP;
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return KDA_OK;
}

}  // namespace

extern "C" size_t kda_chunk_noalloc_max_bytes(void) { return kNoAllocBytes; }

extern "C" kda_status kda_chunk_fwd_noalloc(const kda_args *a, const void *q, const void *k, const void *v,
                                            const float *g, const float *beta, const float *h0,
                                            const int32_t *cu_seqlens, void *o, float *ht, void *stream) {
  if (!a) return KDA_ERR_NULL;
  kda_args s = *a;
  size_t need = kda_chunk_workspace_bytes(&s);
  if (need > kNoAllocBytes && s.schedule == KDA_SCHED_AUTO) {
    kda_args f = s;
    f.schedule = KDA_SCHED_FUSED;
    const int r = kda_chunk_schedule(&f);
    if (r == KDA_SCHED_FUSED || r == KDA_SCHED_PIPE) {
      s = f;
      need = kda_chunk_workspace_bytes(&s);
    }
  }
  if (need > kNoAllocBytes) {
    snprintf(g_last_error, sizeof(g_last_error),
             "the schedule for these arguments needs %zu bytes of workspace; the static array holds %zu", need,
             kNoAllocBytes);
    return KDA_ERR_WORKSPACE;
  }
  void *ws = nullptr;
  kda_status st = scratch_address(&ws);
  if (st != KDA_OK) return st;
  return kda_chunk_fwd(&s, q, k, v, g, beta, h0, cu_seqlens, o, ht, ws, kNoAllocBytes, stream);
}

extern "C" size_t kda_chunk_states_count(const kda_args *a, int packed) {
  if (!chunk_shape_ok(a)) return 0;
  if (packed ? a->B != 1 : a->N != a->B) return 0;
  return (size_t)max_chunks(a, packed != 0);
}

extern "C" kda_status kda_chunk_fwd_states(const kda_args *a, const void *q, const void *k, const void *v,
                                           const float *g, const float *beta, const float *h0,
                                           const int32_t *cu_seqlens, void *o, float *ht, float *h_states,
                                           void *workspace, size_t ws_bytes, void *stream) {
  kda::ChunkParams p;
  kda_status s = prepare_chunk(a, q, k, v, g, beta, h0, cu_seqlens, o, ht, workspace, ws_bytes, p);
  if (s != KDA_OK) return s;
  if (!h_states && kda_chunk_states_count(a, cu_seqlens != nullptr) > 0) return KDA_ERR_NULL;
  if (!aligned16(h_states)) return KDA_ERR_ALIGN;
  if (h_states) p.hc = h_states;  // the staged scan writes the chunk-start states here, not in the workspace
  return run_chunk(a, p, (hipStream_t)stream, h_states != nullptr);
}

extern "C" kda_status kda_chunk_stage(const kda_args *a, kda_stage stage, const void *q, const void *k,
                                      const void *v, const float *g, const float *beta, const float *h0,
                                      const int32_t *cu_seqlens, void *o, float *ht, void *workspace,
                                      size_t ws_bytes, void *stream) {
  if (!a) return KDA_ERR_NULL;
  if (a->schedule != KDA_SCHED_STAGED) return KDA_ERR_SHAPE;
  kda::ChunkParams p;
  kda_status s = prepare_chunk(a, q, k, v, g, beta, h0, cu_seqlens, o, ht, workspace, ws_bytes, p);
  if (s != KDA_OK) return s;
  return run_stage(p, (int)stage, (hipStream_t)stream);
}

namespace {

// Workspace of kda_chunk_bwd: the staged forward's layout, then the backward's
// own fp32 intermediates (BwdParams in kda_launch.h), each 256-byte aligned.
struct BwdLayout {
  size_t fwd, off[13], total;
};

BwdLayout bwd_layout(const kda_args *a) {
  kda_args s = *a;
  s.schedule = KDA_SCHED_STAGED;
  BwdLayout L{};
  L.fwd = staged_layout(&s).total;
  const size_t rows = (size_t)a->B * a->T * a->H;
  const size_t D = pad_width(std::max(a->K, a->V)), C = a->chunk_size;
  const size_t nch = (size_t)std::max<int64_t>(max_chunks(a, true), max_chunks(a, false));
  // dvn, dqt, dkt, dw, dXw, dAqk, dT, dAkk, dbp, dhn, dlam, ddt_part, dA_part
  const size_t sz[13] = {4 * rows * D, 4 * rows * D, 4 * rows * D, 4 * rows * D, 4 * rows * D,
                         4 * rows * C, 4 * rows * C, 4 * rows * C, 4 * rows,
                         4 * nch * a->H * (size_t)a->K * a->V, 4 * nch * a->H * D, 4 * nch * a->H * D,
                         4 * nch * a->H};
  size_t cur = L.fwd;
  for (int i = 0; i < 13; ++i) {
    L.off[i] = cur;
    cur += align_up(sz[i]);
  }
  L.total = cur;
  return L;
}

bool bwd_shape_ok(const kda_args *a) {
  if (!chunk_shape_ok(a)) return false;
  return pad_width(std::max(a->K, a->V)) <= 128;
}

}  // namespace

extern "C" size_t kda_chunk_bwd_workspace_bytes(const kda_args *a) {
  if (!bwd_shape_ok(a)) return 0;
  return bwd_layout(a).total;
}

extern "C" kda_status kda_chunk_bwd(const kda_args *a, const void *q, const void *k, const void *v, const float *g,
                                    const float *beta, const float *h0, const int32_t *cu_seqlens,
                                    const void *d_o, const float *dht, void *dq, void *dk, void *dv, float *dg,
                                    float *dbeta, float *dh0, float *dA_log, float *ddt_bias, void *workspace,
                                    size_t ws_bytes, void *stream) {
  if (!a) return KDA_ERR_NULL;
  if (a->T > 0 && (!d_o || !dq || !dk || !dv || !dg || !dbeta)) return KDA_ERR_NULL;
  if (!aligned16(d_o) || !aligned16(dht) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv) || !aligned16(dg) ||
      !aligned16(dh0))
    return KDA_ERR_ALIGN;
  kda_args s = *a;
  s.schedule = KDA_SCHED_STAGED;
  kda::ChunkParams p;
  // o is never written here: the forward is recomputed up to the state scan only
  kda_status st = prepare_chunk(&s, q, k, v, g, beta, h0, cu_seqlens, const_cast<void *>(d_o), nullptr, workspace,
                                ws_bytes, p);
  if (st != KDA_OK) return st;
  if (a->gate_kind == KDA_GATE_LOG2_CUMSUM) return KDA_ERR_UNSUPPORTED;
  if (a->q_l2norm) return KDA_ERR_UNSUPPORTED;
  if (a->Hk != 0 && a->Hk != a->H) return KDA_ERR_UNSUPPORTED;
  if (!bwd_shape_ok(a)) return KDA_ERR_UNSUPPORTED;
  const BwdLayout L = bwd_layout(a);
  if (ws_bytes < L.total) return KDA_ERR_WORKSPACE;
  char *base = static_cast<char *>(workspace);
  kda::BwdParams b{};
  b.dout = d_o;
  b.dht = dht;
  b.dq = dq;
  b.dk = dk;
  b.dv = dv;
  b.dg = dg;
  b.dbeta = dbeta;
  b.dh0 = dh0;
  b.dA_log = dA_log;
  b.ddt = (a->gate_kind == KDA_GATE_LOGE) ? nullptr : ddt_bias;
  if (a->gate_kind == KDA_GATE_LOGE) b.dA_log = nullptr;
  float **slots[13] = {&b.dvn, &b.dqt, &b.dkt, &b.dw, &b.dXw, &b.dAqk, &b.dT, &b.dAkk, &b.dbp, &b.dhn, &b.dlam,
                       &b.ddt_part, &b.dA_part};
  for (int i = 0; i < 13; ++i) *slots[i] = reinterpret_cast<float *>(base + L.off[i]);
  hipStream_t hs = (hipStream_t)stream;
  for (int stage = KDA_STAGE_INDEX; stage <= KDA_STAGE_SCAN; ++stage)
    if ((st = run_stage(p, stage, hs)) != KDA_OK) return st;
  return hip_status(kda::launch_bwd(p, b, hs));
}
