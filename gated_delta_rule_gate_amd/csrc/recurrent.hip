// Fused token-sequential KDA recurrence (decode and inference prefill).
//
// One workgroup of 256 threads owns a (sequence, head, value-block) and scans
// its tokens with the [K, BV] FP32 state held in registers, computing in FP32
// whatever the input dtype ("Add fused recurrent_kda for decode and inference
// prefill", section "Agent note"). Per token, with S' = Diag(2^g) S:
//
//   delta = beta (v - S'^T k)
//   o     = scale S_t^T q = scale (S'^T q + (k . q) delta)
//   S     = S' + k delta^T
//
// so both column reductions (S'^T k and S'^T q) happen in one pass over the
// state, and o needs no second pass after the rank-1 update. With q_l2norm, o
// is also scaled by 1/sqrt(|q|^2 + eps), which normalises q after the fact
// (o is linear in q).
//
// Thread layout: thread = (column group cg of 4 adjacent columns, row group rg);
// it holds RPT rows x 4 columns. A wave's 16-byte loads of the state cover whole
// 512-byte rows, so the state streams through HBM fully coalesced.
//
// Widths K and V that are not 64, 128 or 256 run in the next larger tile
// (KP rows, value blocks of BV columns): channels past K enter as zeros and the
// state rows and value columns past the real widths are neither loaded nor
// stored, which leaves every reduction exact.
#include "kda_device.h"
#include "kda_launch.h"

// State traffic cache policy: 0 = default, 1 = non-temporal stores,
// 2 = non-temporal loads and stores, 3 = non-temporal loads only
// (the state is touched once per call).
#ifndef KDA_REC_STATE_NT
#define KDA_REC_STATE_NT 2
#endif
// Threads per workgroup (256 or 512).
#ifndef KDA_REC_THREADS
#define KDA_REC_THREADS 256
#endif
// Widest value block per workgroup (128 or 64 columns).
#ifndef KDA_REC_MAX_BV
#define KDA_REC_MAX_BV 128
#endif

namespace kda {

__device__ __forceinline__ f32x4_t load_state4(const float *p) {
#if KDA_REC_STATE_NT >= 2
  return __builtin_nontemporal_load(reinterpret_cast<const f32x4_t *>(p));
#else
  return *reinterpret_cast<const f32x4_t *>(p);
#endif
}

__device__ __forceinline__ void store_state4(float *p, f32x4_t v) {
#if KDA_REC_STATE_NT == 1 || KDA_REC_STATE_NT == 2
  __builtin_nontemporal_store(v, reinterpret_cast<f32x4_t *>(p));
#else
  *reinterpret_cast<f32x4_t *>(p) = v;
#endif
}

template <int K, int BV>
struct RecCfg {
  static constexpr int kThreads = KDA_REC_THREADS;
  static constexpr int kCG = BV / 4;             // column groups
  static constexpr int kRG = kThreads / kCG;     // row groups
  static constexpr int kRPT = K / kRG;           // rows per thread
  static_assert(kThreads % kCG == 0 && K % kRG == 0, "tile");
};

// FULL: K == KP and V a multiple of BV, so no row or column needs a mask and
// the widths are compile-time constants.
template <typename Tin, int KP, int BV, bool FULL>
__global__ __launch_bounds__(KDA_REC_THREADS) void recurrent_kernel(RecurrentParams p) {
  using Cfg = RecCfg<KP, BV>;
  constexpr int RPT = Cfg::kRPT, CG = Cfg::kCG, RG = Cfg::kRG;
  const int K = FULL ? KP : p.K;
  const int nvb = FULL ? p.V / BV : (p.V + BV - 1) / BV;
  const int vb = blockIdx.x % nvb;
  const int nh = blockIdx.x / nvb;
  const int n = nh / p.H, h = nh % p.H;
  const int tid = threadIdx.x;
  const int cg = tid % CG, rg = tid / CG;
  const int row0 = rg * RPT;
  const int col0 = vb * BV + cg * 4;
  const bool col_ok = FULL || col0 < p.V;  // four columns, all inside V or none (V % 4 == 0)

  const SlotRange sr = slot_range(p.cu, n, p.T);
  const int64_t sbase = ((int64_t)(n * p.H + h) * K) * p.V;

  // ---- state load (FP32, registers) ----
  f32x4_t S[RPT];
  if (p.h0) {
#pragma unroll
    for (int r = 0; r < RPT; ++r)
      S[r] = (FULL || (col_ok && row0 + r < K)) ? load_state4(p.h0 + sbase + (int64_t)(row0 + r) * p.V + col0)
                                                : f32x4_t{0.f, 0.f, 0.f, 0.f};
  } else {
#pragma unroll
    for (int r = 0; r < RPT; ++r) S[r] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  __shared__ float s_k[2][KP], s_q[2][KP], s_a[2][KP];
  __shared__ float s_v[2][BV];
  __shared__ float s_red[2][RG][BV];
  __shared__ float s_d[BV];
  constexpr int NWAVE = Cfg::kThreads / 64;
  __shared__ float s_kq[2][NWAVE], s_qq[2][NWAVE];
  __shared__ float s_beta[2];

  const float expA = (p.gate_kind == kGateSafe || p.gate_kind == kGateSoftplus) ? fast_exp2(p.A_log[h] * kLog2e) : 0.f;
  const float dt = (p.dt_bias && tid < K) ? p.dt_bias[h * K + tid] : 0.f;

  const Tin *qp = reinterpret_cast<const Tin *>(p.q);
  const Tin *kp = reinterpret_cast<const Tin *>(p.k);
  const Tin *vp = reinterpret_cast<const Tin *>(p.v);
  Tin *op = reinterpret_cast<Tin *>(p.o);

  // registers holding the next token's raw inputs
  float nk = 0.f, nq = 0.f, ng = 0.f, nv = 0.f, nb = 0.f;
  auto fetch = [&](int i) {
    const int64_t t = sr.t0 + i;
    const int64_t th = t * p.H + h, thk = t * p.Hk + h / (p.H / p.Hk);
    if (tid < K) {
      nk = to_f32(kp[thk * K + tid]);
      nq = to_f32(qp[thk * K + tid]);
      ng = p.g[th * K + tid];
    }
    if (tid < BV && (FULL || vb * BV + tid < p.V)) nv = to_f32(vp[th * p.V + vb * BV + tid]);
    if (tid == 0) nb = p.beta_logits ? sigmoid_f32(p.beta[th]) : p.beta[th];
  };
  if (sr.len > 0) fetch(0);

  for (int i = 0; i < sr.len; ++i) {
    const int buf = i & 1;
    // ---- phase A: stage this token's inputs in LDS, prefetch the next ----
    float kq = 0.f, qq = 0.f;
    if (tid < KP) {  // channels >= K hold zeros (never fetched)
      s_k[buf][tid] = nk;
      s_q[buf][tid] = nq;
      s_a[buf][tid] = fast_exp2(gate_log2(p.gate_kind, ng, dt, expA, p.lower_bound));
      kq = nk * nq;
      qq = nq * nq;
    }
    if (tid < BV) s_v[buf][tid] = nv;
    if (tid == 0) s_beta[buf] = nb;
    // k . q : wave reduction, one partial per wave
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) kq += __shfl_xor(kq, off);
    if ((tid & 63) == 0) s_kq[buf][tid >> 6] = kq;
    if (p.q_l2norm) {  // |q|^2 for the deferred normalisation of q
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) qq += __shfl_xor(qq, off);
      if ((tid & 63) == 0) s_qq[buf][tid >> 6] = qq;
    }
    if (i + 1 < sr.len) fetch(i + 1);
    __syncthreads();

    // ---- phase B: decay and the two column reductions ----
    f32x4_t pk = {0.f, 0.f, 0.f, 0.f}, pq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
      const float a = s_a[buf][row0 + r];
      const float kr = s_k[buf][row0 + r];
      const float qr = s_q[buf][row0 + r];
      S[r] *= a;
      pk += S[r] * kr;
      pq += S[r] * qr;
    }
    *reinterpret_cast<f32x4_t *>(&s_red[0][rg][cg * 4]) = pk;
    *reinterpret_cast<f32x4_t *>(&s_red[1][rg][cg * 4]) = pq;
    __syncthreads();

    // ---- phase C: delta and the output ----
    if (tid < BV) {  // columns >= V compute zeros and are not stored
      float sk = 0.f, sq = 0.f;
#pragma unroll
      for (int g2 = 0; g2 < RG; ++g2) {
        sk += s_red[0][g2][tid];
        sq += s_red[1][g2][tid];
      }
      float kqs = 0.f;
#pragma unroll
      for (int w = 0; w < NWAVE; ++w) kqs += s_kq[buf][w];
      const float d = s_beta[buf] * (s_v[buf][tid] - sk);
      s_d[tid] = d;
      const int64_t th = (sr.t0 + i) * p.H + h;
      float os = p.scale;
      if (p.q_l2norm) {
        float qqs = 0.f;
#pragma unroll
        for (int w = 0; w < NWAVE; ++w) qqs += s_qq[buf][w];
        os *= rsqrtf(qqs + kQNormEps);
      }
      if (FULL || vb * BV + tid < p.V) op[th * p.V + vb * BV + tid] = from_f32<Tin>(os * (sq + kqs * d));
    }
    __syncthreads();

    // ---- phase D: rank-1 update ----
    const f32x4_t d4 = *reinterpret_cast<const f32x4_t *>(&s_d[cg * 4]);
#pragma unroll
    for (int r = 0; r < RPT; ++r) S[r] += s_k[buf][row0 + r] * d4;
  }

  // ---- state store ----
  if (p.ht && !(sr.len == 0 && p.ht == p.h0)) {
#pragma unroll
    for (int r = 0; r < RPT; ++r)
      if (FULL || (col_ok && row0 + r < K)) store_state4(p.ht + sbase + (int64_t)(row0 + r) * p.V + col0, S[r]);
  }
}

template <typename Tin, int KP, int BV>
static hipError_t launch_rec(const RecurrentParams &p, hipStream_t st) {
  const int grid = p.N * p.H * ((p.V + BV - 1) / BV);
  if (grid == 0) return hipSuccess;
  if (p.K == KP && p.V % BV == 0)
    hipLaunchKernelGGL((recurrent_kernel<Tin, KP, BV, true>), dim3(grid), dim3(RecCfg<KP, BV>::kThreads), 0, st, p);
  else
    hipLaunchKernelGGL((recurrent_kernel<Tin, KP, BV, false>), dim3(grid), dim3(RecCfg<KP, BV>::kThreads), 0, st, p);
  return hipGetLastError();
}

template <typename Tin, int KP>
static hipError_t launch_rec_k(const RecurrentParams &p, hipStream_t st) {
  // value block: 128 columns when V allows (one 64 KB contiguous state block at K = 128)
  if (KDA_REC_MAX_BV >= 128 && p.V % 128 == 0) return launch_rec<Tin, KP, 128>(p, st);
  return launch_rec<Tin, KP, 64>(p, st);
}

template <typename Tin>
static hipError_t launch_rec_t(const RecurrentParams &p, hipStream_t st) {
  if (p.K < 1 || p.K > 256 || p.V < 1 || p.V > 256) return hipErrorInvalidValue;
  if (p.K <= 64) return launch_rec_k<Tin, 64>(p, st);
  if (p.K <= 128) return launch_rec_k<Tin, 128>(p, st);
  return launch_rec_k<Tin, 256>(p, st);
}

hipError_t launch_recurrent(const RecurrentParams &p, hipStream_t st) {
  if (recurrent_block_supported(p)) return launch_recurrent_block(p, st);
  return p.is_bf16 ? launch_rec_t<bf16_t>(p, st) : launch_rec_t<float>(p, st);
}

}  // namespace kda
