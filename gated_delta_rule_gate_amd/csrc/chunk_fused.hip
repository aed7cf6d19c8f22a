// The fused schedule of the chunked KDA forward: one persistent workgroup per
// (sequence, head) walks the sequence's chunks in order and runs steps (1)-(6)
// for each chunk entirely on chip. Inputs are read from HBM exactly once and
// only o and the final state are written; the [D, D] FP32 state lives in MFMA
// accumulator registers for the whole sequence (each of the four waves owns a
// 16*NVW-column strip of it).
//
// LDS per chunk (bf16, C = 64, D = 128: about 141 KB):
//   q (-> q~ in place), k, v (-> w after the WY step), x (-> b), A_kk and T
//   (-> k~^T after the WY step), A_qk, beta, b_L, 2^b_L.
#include "chunk_tiles.h"
#include "kda_launch.h"

namespace kda {

namespace {
constexpr int kNT = 256;
}

template <typename Tin, int C, int D>
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
  static constexpr size_t seg = decay + sizeof(float) * D;
  static constexpr size_t end = seg + sizeof(float) * kNT;
  // k~^T [D][C] reuses the A_kk + T region once the WY step has consumed T, when it fits
  static constexpr size_t kt_bytes = sizeof(Tin) * D * TL::LDKT;
  static constexpr bool kt_alias = kt_bytes <= 2 * sizeof(float) * C * TL::LDA;
  static constexpr size_t kt = kt_alias ? akk : end;
  static constexpr size_t total = kt_alias ? end : end + kt_bytes;
};

template <typename Tin, int C, int D, bool SAFE>
__global__ __launch_bounds__(256) void fused_chunk_kernel(ChunkParams p) {
  using TL = Tile<Tin, C, D>;
  using S = FusedSmem<Tin, C, D>;
  constexpr int NW = kNT / 64, NC = TL::NC, DT = TL::DT, LDT = TL::LDT, LDB = TL::LDB;
  constexpr int NVW = DT / NW;  // value tiles per wave
  constexpr int NWT = DT / NW;  // w column tiles per wave
  static_assert(DT % NW == 0, "strip split");

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
  float *sSeg = reinterpret_cast<float *>(smem + S::seg);

  const int nh = blockIdx.x;
  const int n = nh / p.H, h = nh % p.H;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int n16 = lane & 15, grp = lane >> 4;
  const int col0 = wid * NVW * 16;
  const SlotRange sr = slot_range(p.cu, n, p.T);
  const int nch = (sr.len + C - 1) / C;
  const int64_t sbase = (int64_t)nh * D * D;
  const int64_t ld = (int64_t)p.H * D;
  const float expA =
      (p.gate_kind == kGateSafe || p.gate_kind == kGateSoftplus) ? fast_exp2(p.A_log[h] * kLog2e) : 0.f;
  const float *dt = p.dt_bias ? p.dt_bias + h * D : nullptr;

  f32x4_t hs[DT][NVW];
  if (p.h0) {
    load_strip<DT, NVW>(hs, p.h0 + sbase, D, col0, D);
  } else {
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int v = 0; v < NVW; ++v) hs[t][v] = zero4();
  }

  for (int c = 0; c < nch; ++c) {
    const int64_t t0 = sr.t0 + (int64_t)c * C;
    const int L = min(C, sr.len - c * C);
    const int64_t off = t0 * ld + h * D;
    load_rows<Tin, kNT, C, D>(sQ, LDT, reinterpret_cast<const Tin *>(p.q) + off, ld, L);
    load_rows<Tin, kNT, C, D>(sK, LDT, reinterpret_cast<const Tin *>(p.k) + off, ld, L);
    load_rows<Tin, kNT, C, D>(sV, LDT, reinterpret_cast<const Tin *>(p.v) + off, ld, L);
    load_rows<float, kNT, C, D>(sB, LDB, p.g + off, ld, L);
    for (int r = threadIdx.x; r < C; r += kNT) sBeta[r] = (r < L) ? p.beta[(t0 + r) * p.H + h] : 0.f;
    __syncthreads();

    // (1)
    gate_cumsum<kNT, C, D>(sB, LDB, sBL, sSeg, L, p.gate_kind, dt, expA, p.lower_bound);
    for (int i = threadIdx.x; i < D; i += kNT) sDecay[i] = fast_exp2(sBL[i]);
    // (2)
    grams<Tin, kNT, C, D, SAFE>(sQ, sK, sB, sBeta, p.scale, sAkk, sAqk, TL::LDA, L, C);
    __syncthreads();
    // (3)
    solve<kNT, C>(sAkk, sT);
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
    make_qtilde<Tin, kNT, C, D>(sQ, sB, p.scale);
    make_ktilde_t<Tin, kNT, C, D>(sKT, sK, sB, sBL);
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
    store_strip<Tin, NC, NVW>(reinterpret_cast<Tin *>(p.o) + off, ld, col0, L, o);
    __syncthreads();
  }
  if (p.ht && !(sr.len == 0 && p.ht == p.h0)) store_strip<float, DT, NVW>(p.ht + sbase, D, col0, D, hs);
}

bool fused_supported(const ChunkParams &p) {
  if (p.is_bf16) return p.D == 64 || p.D == 128;
  return p.D == 64;
}

namespace {
template <typename Tin, int C, int D>
hipError_t launch_fused_t(const ChunkParams &p, hipStream_t st) {
  const size_t smem = FusedSmem<Tin, C, D>::total;
  const int grid = p.N * p.H;
  if (grid == 0) return hipSuccess;
  auto kern = (p.gate_kind == kGateSafe) ? fused_chunk_kernel<Tin, C, D, true> : fused_chunk_kernel<Tin, C, D, false>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)smem);
  if (e != hipSuccess) {
    (void)hipGetLastError();  // do not leave the error for the next launch to report
    return e;
  }
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kNT), smem, st, p);
  return hipGetLastError();
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
