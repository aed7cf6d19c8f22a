// The fused schedule of the chunked KDA forward: one persistent workgroup per
// (sequence, head) walks the sequence's chunks in order and runs steps (1)-(6)
// for each chunk entirely on chip. Inputs are read from HBM exactly once and
// only o and the final state are written; the [D, D] FP32 state lives in MFMA
// accumulator registers for the whole sequence (each of the NT/64 waves owns
// a 16*NVW-column strip of it).
//
// The next chunk's raw inputs are loaded into registers while the current
// chunk computes, so HBM latency overlaps the on-chip work.
//
// LDS per chunk (bf16, C = 64, D = 128: about 144 KB):
//   q (-> q~ in place), k, v (-> w after the WY step), gate (-> b), A_kk and
//   T (-> k~^T after the WY step), A_qk, beta, b_L, 2^b_L, dt_bias.
#include "chunk_tiles.h"
#include "kda_launch.h"

// Threads per workgroup of the fused kernel (0: 512 when the state has at
// least 8 column tiles, else 256). A build-time knob for tuning.
#ifndef KDA_FUSED_THREADS
#define KDA_FUSED_THREADS 0
#endif

namespace kda {

template <typename Tin, int C, int D, int NT>
struct FusedSmem {
  using TL = Tile<Tin, C, D>;
  static constexpr size_t tin_tile = sizeof(Tin) * C * TL::LDT;
  static constexpr size_t q = 0;
  static constexpr size_t k = q + tin_tile;
  static constexpr size_t v = k + tin_tile;
  static constexpr size_t b = v + tin_tile;
  static constexpr size_t akk = b + sizeof(float) * C * TL::LDB;
  static constexpr size_t t = akk + sizeof(float) * C * TL::LDA;
  static constexpr size_t aqk = t + sizeof(float) * C * TL::LDA;
  static constexpr size_t beta = aqk + sizeof(float) * C * TL::LDA;
  static constexpr size_t bl = beta + sizeof(float) * C;
  static constexpr size_t decay = bl + sizeof(float) * D;
  static constexpr size_t dt = decay + sizeof(float) * D;
  static constexpr size_t seg = dt + sizeof(float) * D;
  static constexpr size_t end = seg + sizeof(float) * NT;
  // k~^T [D][C] reuses the A_kk + T region once the WY step has consumed T, when it fits
  static constexpr size_t kt_bytes = sizeof(Tin) * D * TL::LDKT;
  static constexpr bool kt_alias = kt_bytes <= 2 * sizeof(float) * C * TL::LDA;
  static constexpr size_t kt = kt_alias ? akk : end;
  static constexpr size_t total = kt_alias ? end : end + kt_bytes;
};

// One chunk's raw inputs held in registers between the HBM load and the LDS store.
template <typename Tin, int C, int D, int NT>
struct ChunkRegs {
  static constexpr int EPV = 16 / (int)sizeof(Tin);
  static constexpr int VPR = D / EPV, NVT = C * VPR, IT = (NVT + NT - 1) / NT;  // q, k, v tiles
  static constexpr int XPR = D / 4, NVX = C * XPR, IX = (NVX + NT - 1) / NT;    // gate tile (fp32)
  u32x4_t q[IT], k[IT], v[IT];
  f32x4_t x[IX];
  float beta;

  // The chunk's first element is a uniform base pointer; each vector is a
  // 32-bit unsigned element offset from it, so the loads take the
  // scalar-base + vector-offset form.
  __device__ __forceinline__ void load(const ChunkParams &p, int64_t t0, int L, int h) {
    const unsigned ld = (unsigned)p.H * D;
    const int64_t base = t0 * (int64_t)ld + (int64_t)h * D;
    const Tin *gq = reinterpret_cast<const Tin *>(p.q) + base;
    const Tin *gk = reinterpret_cast<const Tin *>(p.k) + base;
    const Tin *gv = reinterpret_cast<const Tin *>(p.v) + base;
    const float *gx = p.g + base;
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int idx = it * NT + tid_opaque();
      const int r = idx / VPR, c = (idx % VPR) * EPV;
      const bool ok = (NVT % NT == 0 || idx < NVT) && r < L;
      const unsigned off = (unsigned)r * ld + (unsigned)c;
      const u32x4_t z = {0u, 0u, 0u, 0u};
      q[it] = ok ? *reinterpret_cast<const u32x4_t *>(gq + off) : z;
      k[it] = ok ? *reinterpret_cast<const u32x4_t *>(gk + off) : z;
      v[it] = ok ? *reinterpret_cast<const u32x4_t *>(gv + off) : z;
    }
#pragma unroll
    for (int it = 0; it < IX; ++it) {
      const int idx = it * NT + tid_opaque();
      const int r = idx / XPR, c = (idx % XPR) * 4;
      const bool ok = (NVX % NT == 0 || idx < NVX) && r < L;
      const unsigned off = (unsigned)r * ld + (unsigned)c;
      x[it] = ok ? *reinterpret_cast<const f32x4_t *>(gx + off) : zero4();
    }
    const int r = tid_opaque();
    beta = (r < C && r < L) ? p.beta[(t0 + r) * p.H + h] : 0.f;
  }

  // q, k, v to their tiles; the gate input, activated, to sB (rows >= L: 0)
  template <int GK>
  __device__ __forceinline__ void store(Tin *sQ, Tin *sK, Tin *sV, float *sB, float *sBeta, const float *sDt, int L,
                                        float expA, float lower_bound) const {
    using TL = Tile<Tin, C, D>;
    wait_vmem();
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int idx = it * NT + tid_opaque();
      const int r = idx / VPR, c = (idx % VPR) * EPV;
      if (NVT % NT == 0 || idx < NVT) {
        *reinterpret_cast<u32x4_t *>(sQ + r * TL::LDT + c) = q[it];
        *reinterpret_cast<u32x4_t *>(sK + r * TL::LDT + c) = k[it];
        *reinterpret_cast<u32x4_t *>(sV + r * TL::LDT + c) = v[it];
      }
    }
#pragma unroll
    for (int it = 0; it < IX; ++it) {
      const int idx = it * NT + tid_opaque();
      const int r = idx / XPR, c = (idx % XPR) * 4;
      if (NVX % NT == 0 || idx < NVX) {
        const f32x4_t dt = *reinterpret_cast<const f32x4_t *>(sDt + c);
        f32x4_t la;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // rows >= L were loaded as zeros, so the activation is finite there; select, no branch
          const float a = gate_log2(GK, x[it][e], dt[e], expA, lower_bound);
          la[e] = (r < L) ? a : 0.f;
        }
        *reinterpret_cast<f32x4_t *>(sB + r * TL::LDB + c) = la;
      }
    }
    if (tid_opaque() < C) sBeta[tid_opaque()] = beta;
  }
};

template <typename Tin, int C, int D, int NT, int GK>
__global__ __launch_bounds__(NT) void fused_chunk_kernel(ChunkParams p) {
  using TL = Tile<Tin, C, D>;
  using S = FusedSmem<Tin, C, D, NT>;
  constexpr bool SAFE = (GK == kGateSafe);
  constexpr int NW = NT / 64, NC = TL::NC, DT = TL::DT, LDT = TL::LDT, LDB = TL::LDB;
  constexpr int NVW = DT / NW;  // value tiles per wave
  constexpr int NWT = DT / NW;  // w column tiles per wave
  static_assert(DT % NW == 0 && NVW >= 1, "strip split");

  extern __shared__ __align__(16) char smem[];
  Tin *sQ = reinterpret_cast<Tin *>(smem + S::q);
  Tin *sK = reinterpret_cast<Tin *>(smem + S::k);
  Tin *sV = reinterpret_cast<Tin *>(smem + S::v);  // v, then w
  float *sB = reinterpret_cast<float *>(smem + S::b);
  float *sAkk = reinterpret_cast<float *>(smem + S::akk);
  float *sT = reinterpret_cast<float *>(smem + S::t);
  Tin *sKT = reinterpret_cast<Tin *>(smem + S::kt);
  float *sAqk = reinterpret_cast<float *>(smem + S::aqk);
  float *sBeta = reinterpret_cast<float *>(smem + S::beta);
  float *sBL = reinterpret_cast<float *>(smem + S::bl);
  float *sDecay = reinterpret_cast<float *>(smem + S::decay);
  float *sDt = reinterpret_cast<float *>(smem + S::dt);
  float *sSeg = reinterpret_cast<float *>(smem + S::seg);

  const int nh = blockIdx.x;
  const int n = nh / p.H, h = nh % p.H;
  const int lane = tid_opaque() & 63, wid = tid_opaque() >> 6;
  const int n16 = lane & 15, grp = lane >> 4;
  const int col0 = wid * NVW * 16;
  const SlotRange sr = slot_range(p.cu, n, p.T);
  const int nch = (sr.len + C - 1) / C;
  const int64_t sbase = (int64_t)nh * D * D;
  const int64_t ld = (int64_t)p.H * D;
  const float expA = (GK == kGateSafe || GK == kGateSoftplus) ? fast_exp2(p.A_log[h] * kLog2e) : 0.f;
  for (int i = tid_opaque(); i < D; i += NT) sDt[i] = p.dt_bias ? p.dt_bias[h * D + i] : 0.f;

  f32x4_t hs[DT][NVW];
  if (p.h0) {
    load_strip<DT, NVW>(hs, p.h0 + sbase, D, col0, D);
  } else {
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int v = 0; v < NVW; ++v) hs[t][v] = zero4();
  }

  ChunkRegs<Tin, C, D, NT> regs;
  if (nch > 0) regs.load(p, sr.t0, min(C, sr.len), h);
  __syncthreads();  // sDt visible

  for (int c = 0; c < nch; ++c) {
    const int64_t t0 = sr.t0 + (int64_t)c * C;
    const int L = min(C, sr.len - c * C);
    const int64_t off = t0 * ld + h * D;
    regs.template store<GK>(sQ, sK, sV, sB, sBeta, sDt, L, expA, p.lower_bound);
    __syncthreads();
    if (c + 1 < nch) regs.load(p, t0 + C, min(C, sr.len - (c + 1) * C), h);  // in flight during this chunk

    // (1)
    if constexpr (GK == kGateLog2Cumsum) gate_pad<NT, C, D>(sB, LDB, sBL, L);
    else gate_cumsum<NT, C, D>(sB, LDB, sBL, sSeg);
    for (int i = tid_opaque(); i < D; i += NT) sDecay[i] = fast_exp2(sBL[i]);
    // (2)
    grams<Tin, NT, C, D, SAFE>(sQ, sK, sB, sBeta, p.scale, sAkk, sAqk, TL::LDA, L, C);
    __syncthreads();
    // (3)
    solve<NT, C>(sAkk, sT);
    // (4) w column tiles wid + NW*j; u on this wave's own value strip
    f32x4_t wacc[NC][NWT], uv[NC][NVW];
#pragma unroll
    for (int j = 0; j < NWT; ++j)
      tri_mm<Tin, C, NWT>(sT, wid + NW * j, wacc, j, [&](int r, int col) {
        return sBeta[r] * to_f32(sK[r * LDT + col]) * fast_exp2(sB[r * LDB + col]);
      });
#pragma unroll
    for (int v = 0; v < NVW; ++v)
      tri_mm<Tin, C, NVW>(sT, wid * NVW + v, uv, v, [&](int r, int col) { return sBeta[r] * to_f32(sV[r * LDT + col]); });
    __syncthreads();
    // w -> the v tile, q~ in place, k~^T over A_kk/T
#pragma unroll
    for (int j = 0; j < NWT; ++j)
#pragma unroll
      for (int i = 0; i < NC; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          sV[(16 * i + 4 * grp + e) * LDT + 16 * (wid + NW * j) + n16] = from_f32<Tin>(wacc[i][j][e]);
    make_qtilde<Tin, NT, C, D>(sQ, sB, p.scale);
    make_ktilde_t<Tin, NT, C, D>(sKT, sK, sB, sBL);
    __syncthreads();
    // (5) + (6)
    f32x4_t p1[NC][NVW], o[NC][NVW];
#pragma unroll
    for (int i = 0; i < NC; ++i)
#pragma unroll
      for (int v = 0; v < NVW; ++v) {
        p1[i][v] = zero4();
        o[i][v] = zero4();
      }
    rows_times_state<Tin, C, D, NVW, true>(p1, o, sV, sQ, hs);
#pragma unroll
    for (int i = 0; i < NC; ++i)
#pragma unroll
      for (int v = 0; v < NVW; ++v) uv[i][v] = uv[i][v] - p1[i][v];
    causal_times<Tin, C, NVW>(o, sAqk, uv);
    state_update<Tin, C, D, NVW>(hs, sKT, TL::LDKT, uv, sDecay);
    // o through the (now unused) cumsum tile, then 16-byte row stores
    stage_strip<NC, NVW>(sB, LDB, col0, o);
    __syncthreads();
    store_rows_from_f32<Tin, NT, C, D>(reinterpret_cast<Tin *>(p.o) + off, ld, sB, LDB, L);
    __syncthreads();
  }
  if (p.ht && !(sr.len == 0 && p.ht == p.h0)) store_strip<float, DT, NVW>(p.ht + sbase, D, col0, D, hs);
}

bool fused_supported(const ChunkParams &p) {
  if (p.is_bf16) return p.D == 64 || p.D == 128;
  return p.D == 64;
}

namespace {

template <typename Tin, int C, int D, int NT, int GK>
hipError_t launch_fused_g(const ChunkParams &p, hipStream_t st) {
  const size_t smem = FusedSmem<Tin, C, D, NT>::total;
  auto kern = fused_chunk_kernel<Tin, C, D, NT, GK>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)smem);
  if (e != hipSuccess) {
    (void)hipGetLastError();  // do not leave the error for the next launch to report
    return e;
  }
  hipLaunchKernelGGL(kern, dim3(p.N * p.H), dim3(NT), smem, st, p);
  return hipGetLastError();
}

template <typename Tin, int C, int D>
hipError_t launch_fused_t(const ChunkParams &p, hipStream_t st) {
  constexpr int NT = (KDA_FUSED_THREADS > 0) ? KDA_FUSED_THREADS : ((D / 16 >= 8) ? 512 : 256);
  if (p.N * p.H == 0) return hipSuccess;
  switch (p.gate_kind) {
    case kGateSafe: return launch_fused_g<Tin, C, D, NT, kGateSafe>(p, st);
    case kGateSoftplus: return launch_fused_g<Tin, C, D, NT, kGateSoftplus>(p, st);
    case kGateLogE: return launch_fused_g<Tin, C, D, NT, kGateLogE>(p, st);
    case kGateLog2Cumsum: return launch_fused_g<Tin, C, D, NT, kGateLog2Cumsum>(p, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_fused(const ChunkParams &p, hipStream_t st) {
  if (p.is_bf16) {
    if (p.C == 64 && p.D == 128) return launch_fused_t<bf16_t, 64, 128>(p, st);
    if (p.C == 64 && p.D == 64) return launch_fused_t<bf16_t, 64, 64>(p, st);
    if (p.C == 32 && p.D == 128) return launch_fused_t<bf16_t, 32, 128>(p, st);
    if (p.C == 32 && p.D == 64) return launch_fused_t<bf16_t, 32, 64>(p, st);
  } else {
    if (p.C == 64 && p.D == 64) return launch_fused_t<float, 64, 64>(p, st);
    if (p.C == 32 && p.D == 64) return launch_fused_t<float, 32, 64>(p, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace kda
