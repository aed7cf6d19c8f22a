// The staged schedule of the chunked KDA forward: one kernel per step, with
// the fp32 intermediates in the caller's workspace. Steps (1)-(4) and (6)
// run one workgroup per (chunk, head); the scan (5) runs one workgroup per
// (sequence, head, 64-column value block) and walks the chunks in order.
// Grids are sized from capacity; workgroups past the last chunk exit at once,
// so no launch depends on a host read of cu_seqlens.
#include "../../include/kda.h"
#include "chunk_fused_tiles.h"
#include "chunk_loc.h"
#include "chunk_tiles.h"
#include "kda_launch.h"

namespace kda {

namespace {

constexpr int kNT = 256;  // threads per workgroup in every chunk kernel

__device__ __forceinline__ float head_expA(const ChunkParams &p, int h) {
  return (p.gate_kind == kGateSafe || p.gate_kind == kGateSoftplus) ? fast_exp2(p.A_log[h] * kLog2e) : 0.f;
}

template <int C>
__device__ __forceinline__ void load_beta(float *sBeta, const ChunkParams &p, int64_t t0, int h, int L) {
  for (int r = threadIdx.x; r < C; r += kNT) {
    float b = (r < L) ? p.beta[(t0 + r) * p.H + h] : 0.f;
    if (p.beta_logits && r < L) b = sigmoid_f32(b);
    sBeta[r] = b;
  }
}

template <int ROWS, int COLS, int LDS>
__device__ __forceinline__ void store_rows_f32(float *g, int64_t ldg, const float *s, int L) {
  for (int idx = threadIdx.x; idx < ROWS * COLS / 4; idx += kNT) {
    const int r = idx / (COLS / 4), c = (idx % (COLS / 4)) * 4;
    if (r < L) *reinterpret_cast<f32x4_t *>(g + (int64_t)r * ldg + c) = *reinterpret_cast<const f32x4_t *>(s + r * LDS + c);
  }
}

}  // namespace

// ---- chunk index: chunk_off[n] = sum_{m<n} ceil(len_m / C); with seg_len > 0
// also seg_off[n] = sum_{m<n} max(1, ceil(ceil(len_m / C) / seg_len)) ----
__global__ __launch_bounds__(256) void chunk_index_kernel(const int32_t *cu, int N, int C, int32_t *off, int seg_len,
                                                          int32_t *soff) {
  __shared__ int s[256], g[256];
  const int tid = threadIdx.x;
  int carry = 0, gcarry = 0;
  if (tid == 0) {
    off[0] = 0;
    if (seg_len > 0) soff[0] = 0;
  }
  for (int base = 0; base < N; base += 256) {
    const int n = base + tid;
    int cnt = 0, sc = 0;
    if (n < N) {
      const int len = cu[n + 1] - cu[n];
      cnt = len > 0 ? (len + C - 1) / C : 0;
      sc = seg_len > 0 ? max(1, (cnt + seg_len - 1) / seg_len) : 0;
    }
    s[tid] = cnt;
    g[tid] = sc;
    __syncthreads();
    for (int o = 1; o < 256; o <<= 1) {
      const int v = tid >= o ? s[tid - o] : 0;
      const int w = tid >= o ? g[tid - o] : 0;
      __syncthreads();
      s[tid] += v;
      g[tid] += w;
      __syncthreads();
    }
    if (n < N) {
      off[n + 1] = carry + s[tid];
      if (seg_len > 0) soff[n + 1] = gcarry + g[tid];
    }
    carry += s[255];
    gcarry += g[255];
    __syncthreads();
  }
}

// ---- (1) gate activation + chunk-local cumsum (base 2) ----
// Persistent workgroups walk (chunk, head) items: thread t owns channel t % D
// and RPS consecutive rows, the activation and the cumsum run in registers
// (the row parts' totals meet in LDS), and the next item's gate input is
// loaded while the current one is summed and stored.
template <int C, int D, int GK>
__global__ __launch_bounds__(kNT) void stage_gate_items_kernel(ChunkParams p) {
  constexpr int TPC = kNT / D, RPS = C / TPC;  // threads per channel, rows per thread
  static_assert(kNT % D == 0 && C % TPC == 0, "whole channels per thread group");
  __shared__ float sSeg[kNT];
  const int t = threadIdx.x, ch = t % D, part = t / D;
  const int total = p.cu ? p.chunk_off[p.N] : p.B * ((p.T + C - 1) / C);
  const int64_t items = (int64_t)total * p.H;
  const int ld = p.H * D, ldg = p.H * p.Kr;  // row strides (elements) within a chunk
  float x[RPS];
  auto load = [&](int64_t it) {
    ChunkLoc lc;
    locate_chunk(p, (int)(it / p.H), lc);
    const int h = (int)(it % p.H);
    const float *g = p.g + lc.t0 * (int64_t)ldg + h * p.Kr + ch;
#pragma unroll
    for (int i = 0; i < RPS; ++i) {
      const int r = part * RPS + i;
      x[i] = (r < lc.L && ch < p.Kr) ? g[r * ldg] : 0.f;
    }
  };
  int64_t it = blockIdx.x;
  if (it < items) load(it);
  for (; it < items; it += gridDim.x) {
    ChunkLoc lc;
    locate_chunk(p, (int)(it / p.H), lc);
    const int h = (int)(it % p.H), L = lc.L;
    float v[RPS];
    if constexpr (GK == kGateLog2Cumsum) {
      // a pre-cumsummed log2 gate already is b: only restrided to the tile width
#pragma unroll
      for (int i = 0; i < RPS; ++i) v[i] = x[i];
    } else {
      const float expA = head_expA(p, h);
      const float dt = (p.dt_bias && ch < p.Kr) ? p.dt_bias[h * p.Kr + ch] : 0.f;
#pragma unroll
      for (int i = 0; i < RPS; ++i) v[i] = (part * RPS + i < L) ? gate_log2(GK, x[i], dt, expA, p.lower_bound) : 0.f;
    }
    if (it + gridDim.x < items) load(it + gridDim.x);
    if constexpr (GK != kGateLog2Cumsum) {
#pragma unroll
      for (int i = 1; i < RPS; ++i) v[i] += v[i - 1];
      if constexpr (TPC > 1) {
        sSeg[part * D + ch] = v[RPS - 1];
        __syncthreads();
        float off = 0.f;
#pragma unroll
        for (int q = 0; q < TPC - 1; ++q)
          if (q < part) off += sSeg[q * D + ch];
#pragma unroll
        for (int i = 0; i < RPS; ++i) v[i] += off;
        __syncthreads();  // sSeg is rewritten by the next item
      }
    }
    float *b = p.b + lc.t0 * (int64_t)ld + h * D + ch;
#pragma unroll
    for (int i = 0; i < RPS; ++i) {
      const int r = part * RPS + i;
      if (r < L) b[r * ld] = v[i];
    }
  }
}

// ---- (2) intra-chunk grams ----
template <typename Tin, int C, int D, bool SAFE>
__global__ __launch_bounds__(256) void stage_grams_kernel(ChunkParams p) {
  ChunkLoc lc;
  if (!locate_chunk(p, blockIdx.x, lc)) return;
  const int h = blockIdx.y;
  using TL = Tile<Tin, C, D>;
  extern __shared__ __align__(16) char smem[];
  Tin *sQ = reinterpret_cast<Tin *>(smem);
  Tin *sK = sQ + C * TL::LDT;
  float *sB = reinterpret_cast<float *>(sK + C * TL::LDT);
  float *sBL = sB + C * TL::LDB;
  float *sBeta = sBL + D;
  const int64_t ld = (int64_t)p.H * D, ldc = (int64_t)p.H * C, ldk = (int64_t)p.Hk * p.Kr;
  const int64_t off = lc.t0 * ld + h * D, offk = lc.t0 * ldk + (h / (p.H / p.Hk)) * p.Kr;
  // every tile's loads in flight before the first LDS write
  RowsFetch<Tin, kNT, C, D> fq, fk;
  RowsFetch<float, kNT, C, D> fb;
  fq.fetch(reinterpret_cast<const Tin *>(p.q) + offk, ldk, lc.L, p.Kr);
  fk.fetch(reinterpret_cast<const Tin *>(p.k) + offk, ldk, lc.L, p.Kr);
  fb.fetch(p.b + off, ld, lc.L);
  load_beta<C>(sBeta, p, lc.t0, h, lc.L);
  fq.put(sQ, TL::LDT);
  fk.put(sK, TL::LDT);
  fb.put(sB, TL::LDB);
  __syncthreads();
  pad_cumsum<kNT, C, D>(sB, TL::LDB, sBL, lc.L);
  __syncthreads();
  grams<Tin, kNT, C, D, SAFE>(sQ, sK, sB, sBeta, p.scale, p.Akk + lc.t0 * ldc + h * C, p.Aqk + lc.t0 * ldc + h * C,
                             ldc, lc.L, lc.L);
}

// ---- (3) T = (I + A_kk)^-1 ----
template <int C>
__global__ __launch_bounds__(256) void stage_solve_kernel(ChunkParams p) {
  ChunkLoc lc;
  if (!locate_chunk(p, blockIdx.x, lc)) return;
  const int h = blockIdx.y;
  constexpr int LDA = C + 4;
  extern __shared__ __align__(16) char smem[];
  float *sAkk = reinterpret_cast<float *>(smem);
  float *sT = sAkk + C * LDA;
  const int64_t ldc = (int64_t)p.H * C;
  load_rows<float, kNT, C, C>(sAkk, LDA, p.Akk + lc.t0 * ldc + h * C, ldc, lc.L);
  __syncthreads();
  solve<kNT, C>(sAkk, sT);
  store_rows_f32<C, C, LDA>(p.Tm + lc.t0 * ldc + h * C, ldc, sT, lc.L);
}

// ---- (4) WY recompute: w = T (beta k 2^b), u = T (beta v) ----
template <typename Tin, int C, int D>
__global__ __launch_bounds__(256) void stage_wy_kernel(ChunkParams p) {
  ChunkLoc lc;
  if (!locate_chunk(p, blockIdx.x, lc)) return;
  const int h = blockIdx.y;
  using TL = Tile<Tin, C, D>;
  constexpr int NC = TL::NC, DT = TL::DT, LDT = TL::LDT, LDB = TL::LDB, NW = kNT / 64;
  extern __shared__ __align__(16) char smem[];
  float *sT = reinterpret_cast<float *>(smem);
  float *sBeta = sT + C * TL::LDA;
  Tin *sK = reinterpret_cast<Tin *>(sBeta + C);  // k, then beta k 2^b (rounded to Tin once, as an operand)
  Tin *sV = sK + C * LDT;
  const int64_t ld = (int64_t)p.H * D, ldc = (int64_t)p.H * C, ldk = (int64_t)p.Hk * p.Kr, ldv = (int64_t)p.H * p.Vr;
  const int64_t off = lc.t0 * ld + h * D, offk = lc.t0 * ldk + (h / (p.H / p.Hk)) * p.Kr;
  const int L = lc.L;
  // b of the chunk's rows, four channels per item, loaded beside the tiles (rows past L are never read)
  // (all of them before the tiles' barrier up to 8 vectors a thread; wider tiles take them in groups of 8 after it)
  constexpr int VPR = D / 4, NI = C * VPR, IB = (NI + kNT - 1) / kNT, GB = IB <= 8 ? IB : 8;
  auto load_b = [&](f32x4_t (&bv)[GB], int j0) {
#pragma unroll
    for (int j = 0; j < GB; ++j) {
      const int idx = (j0 + j) * kNT + threadIdx.x, r = idx / VPR, i = (idx % VPR) * 4;
      bv[j] = (idx < NI && r < L) ? *reinterpret_cast<const f32x4_t *>(p.b + off + (int64_t)r * ld + i) : zero4();
    }
  };
  auto scale_k = [&](const f32x4_t (&bv)[GB], int j0) {
#pragma unroll
    for (int j = 0; j < GB; ++j) {
      const int idx = (j0 + j) * kNT + threadIdx.x, r = idx / VPR, i = (idx % VPR) * 4;
      if (idx < NI && r < L) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          Tin &x = sK[r * LDT + i + e];
          x = from_f32<Tin>(sBeta[r] * to_f32(x) * fast_exp2(bv[j][e]));
        }
      }
    }
  };
  f32x4_t bv[GB];
  if constexpr (IB <= 8) load_b(bv, 0);
  // every tile's loads in flight before the first LDS write
  RowsFetch<float, kNT, C, C> ft;
  RowsFetch<Tin, kNT, C, D> fk, fv;
  ft.fetch(p.Tm + lc.t0 * ldc + h * C, ldc, L);
  fk.fetch(reinterpret_cast<const Tin *>(p.k) + offk, ldk, L, p.Kr);
  fv.fetch(reinterpret_cast<const Tin *>(p.v) + lc.t0 * ldv + h * p.Vr, ldv, L, p.Vr);
  load_beta<C>(sBeta, p, lc.t0, h, L);
  ft.put(sT, TL::LDA);
  fk.put(sK, LDT);
  fv.put(sV, LDT);
  __syncthreads();
  // beta k 2^b in place of k; rows past L stay zero
  if constexpr (IB <= 8) {
    scale_k(bv, 0);
  } else {
#pragma unroll 1
    for (int j0 = 0; j0 < IB; j0 += GB) {
      load_b(bv, j0);
      scale_k(bv, j0);
    }
  }
  __syncthreads();
  const int wid = threadIdx.x >> 6;
  for (int ct = wid; ct < 2 * DT; ct += NW) {
    f32x4_t acc[NC][1];
    if (ct < DT) {
      tri_mm<Tin, C, 1>(sT, ct, acc, 0, [&](int c, int col) { return to_f32(sK[c * LDT + col]); });
      store_strip<float, NC, 1>(p.w + off, ld, 16 * ct, lc.L, acc);
    } else {
      tri_mm<Tin, C, 1>(sT, ct - DT, acc, 0, [&](int c, int col) { return sBeta[c] * to_f32(sV[c * LDT + col]); });
      store_strip<float, NC, 1>(p.u + off, ld, 16 * (ct - DT), lc.L, acc);
    }
  }
}

// ---- (5) inter-chunk state scan, per (sequence, head, 64-column value block) ----
// k~^T = (k 2^(b_L - b))^T of one chunk into LDS [D][LDKT] (Tin), straight from
// the global rows of k and b (b_L read from the chunk's last row): four channels
// per item, and every load of a half of the items issued before its first LDS
// write, so the loads' latencies overlap.
template <typename Tin, int NT, int C, int D>
__device__ __forceinline__ void ktilde_t_from_global(Tin *sKT, const Tin *gK, int64_t ldk, const float *gB, int64_t ld,
                                                     int L, int kr) {
  using TL = Tile<Tin, C, D>;
  constexpr int VPR = D / 4, NI = C * VPR, IT = (NI + NT - 1) / NT, HALF = (IT + 1) / 2;
  const float *gBL = gB + (int64_t)(L - 1) * ld;
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    f32x4_t kv[HALF], ev[HALF];
#pragma unroll
    for (int j = 0; j < HALF; ++j) {
      const int idx = (hf * HALF + j) * NT + tid_opaque();
      const int r = idx / VPR, i = (idx % VPR) * 4;
      const bool ok = hf * HALF + j < IT && idx < NI && r < L && i < kr;  // kr % 8 == 0: all four or none
      if (ok) {
        const f32x4_t b = *reinterpret_cast<const f32x4_t *>(gB + (int64_t)r * ld + i);
        const f32x4_t bl = *reinterpret_cast<const f32x4_t *>(gBL + i);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          kv[j][e] = to_f32(gK[(int64_t)r * ldk + i + e]);
          ev[j][e] = bl[e] - b[e];
        }
      } else {
        kv[j] = zero4();
        ev[j] = zero4();
      }
    }
#pragma unroll
    for (int j = 0; j < HALF; ++j) {
      const int idx = (hf * HALF + j) * NT + tid_opaque();
      if (hf * HALF + j < IT && idx < NI) {
        const int r = idx / VPR, i = (idx % VPR) * 4;
#pragma unroll
        for (int e = 0; e < 4; ++e) sKT[(i + e) * TL::LDKT + r] = from_f32<Tin>(kv[j][e] * fast_exp2(ev[j][e]));
      }
    }
  }
}

template <typename Tin, int C, int D>
__global__ __launch_bounds__(256) void stage_scan_kernel(ChunkParams p) {
  using TL = Tile<Tin, C, D>;
  constexpr int BV = 64, NVW = 1, NC = TL::NC, DT = TL::DT, LDT = TL::LDT;
  const int nvb = (p.Vr + BV - 1) / BV;  // value blocks wholly past Vr would compute zeros
  const int vb = blockIdx.x % nvb, nh = blockIdx.x / nvb;
  const int n = nh / p.H, h = nh % p.H;
  const int wid = threadIdx.x >> 6;
  const int col0 = vb * BV + wid * 16;
  const SlotRange sr = slot_range(p.cu, n, p.T);
  const int nch = (sr.len + C - 1) / C;
  const int cbase = p.cu ? p.chunk_off[n] : n * ((p.T + C - 1) / C);
  const int Kr = p.Kr, Vr = p.Vr;
  const int64_t sbase = (int64_t)nh * Kr * Vr;  // states [Kr, Vr]
  const int64_t ld = (int64_t)p.H * D, ldk = (int64_t)p.Hk * Kr;
  const int hk = h / (p.H / p.Hk);  // q/k head of value head h

  extern __shared__ __align__(16) char smem[];
  Tin *sW = reinterpret_cast<Tin *>(smem);
  Tin *sKT = sW + C * LDT;
  float *sBL = reinterpret_cast<float *>(sKT + D * TL::LDKT);
  float *sDecay = sBL + D;

  f32x4_t hs[DT][NVW];
  if (p.h0) {
    load_strip<DT, NVW>(hs, p.h0 + sbase, Vr, col0, Kr, Vr);
  } else {
#pragma unroll
    for (int t = 0; t < DT; ++t) hs[t][0] = zero4();
  }
  for (int c = 0; c < nch; ++c) {
    const int64_t t0 = sr.t0 + (int64_t)c * C;
    const int L = min(C, sr.len - c * C);
    const int64_t off = t0 * ld + h * D;
    store_strip<float, DT, NVW>(p.hc + ((int64_t)(cbase + c) * p.H + h) * Kr * Vr, Vr, col0, Kr, hs, Vr);
    load_rows_cvt<Tin, kNT, C, D>(sW, LDT, p.w + off, ld, L);
    for (int i = threadIdx.x; i < D; i += kNT) sDecay[i] = fast_exp2(p.b[off + (int64_t)(L - 1) * ld + i]);
    ktilde_t_from_global<Tin, kNT, C, D>(sKT, reinterpret_cast<const Tin *>(p.k) + t0 * ldk + hk * Kr, ldk, p.b + off,
                                         ld, L, Kr);
    f32x4_t uv[NC][NVW];
    load_strip<NC, NVW>(uv, p.u + off, ld, col0, L);
    __syncthreads();
    f32x4_t p1[NC][NVW];
#pragma unroll
    for (int i = 0; i < NC; ++i) p1[i][0] = zero4();
    rows_times_state<Tin, C, D, NVW, false>(p1, p1, sW, sW, hs);
#pragma unroll
    for (int i = 0; i < NC; ++i) uv[i][0] = uv[i][0] - p1[i][0];
    store_strip<float, NC, NVW>(p.vnew + off, ld, col0, L, uv);
    state_update<Tin, C, D, NVW>(hs, sKT, TL::LDKT, uv, sDecay);
    __syncthreads();
  }
  if (p.ht && !(sr.len == 0 && p.ht == p.h0)) store_strip<float, DT, NVW>(p.ht + sbase, Vr, col0, Kr, hs, Vr);
}

// The same scan for bf16 inputs (D <= 128) with one workgroup per (sequence,
// head): D / 16 waves, wave w holding value columns 16w .. 16w + 15 of the state. The next
// chunk's w, k, b and u are loaded into registers while the current chunk
// computes. w goes to LDS as bf16 in the operand order of the product with the
// state (the contraction map of Mma<bf16_t>), k~ row-major, read for the state
// update with the transposing LDS load; every store is a wide one.
template <int C, int D>
struct ScanBf16Smem {
  static constexpr int LDT = D + 8;
  static constexpr size_t w = 0, k = w + 2 * C * LDT, decay = k + 2 * C * LDT;
  static constexpr size_t total = decay + 4 * D;
};

// position of channel x in the operand order of Mma<bf16_t> (inverse of kidx)
__device__ __forceinline__ int bf16_op_pos(int x) {
  const int w = x & 31;
  return (x & ~31) + 8 * ((w >> 2) & 3) + ((w >> 4) << 2) + (w & 3);
}

template <int C, int D>
struct ScanBf16Regs {
  static constexpr int NT = 4 * D, VPR = D / 8, NI = C * VPR, II = (NI + NT - 1) / NT;  // k vectors
  static constexpr int NF = C * D / 4, IF = (NF + NT - 1) / NT;                          // w vectors
  static_assert(NT % VPR == 0, "one channel vector per thread");
  u32x4_t k[II], w[IF];
  f32x4_t b[II][2], bl[2];
  f32x4_t u[C / 16];  // this wave's value columns of u (C layout)

  __device__ __forceinline__ void load(const ChunkParams &p, int64_t t0, int L, int h, int col0) {
    const int t = threadIdx.x;
    const int64_t ld = (int64_t)p.H * D, ldk = (int64_t)p.Hk * p.Kr;
    const bf16_t *gk = reinterpret_cast<const bf16_t *>(p.k) + t0 * ldk + (h / (p.H / p.Hk)) * p.Kr;
    const float *gb = p.b + t0 * ld + h * D, *gw = p.w + t0 * ld + h * D;
    const u32x4_t z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int it = 0; it < II; ++it) {
      const int idx = it * NT + t, r = idx / VPR, c = (idx % VPR) * 8;
      const bool ok = (NI % NT == 0 || idx < NI) && r < L;
      k[it] = ok && c < p.Kr ? *reinterpret_cast<const u32x4_t *>(gk + r * ldk + c) : z;
#pragma unroll
      for (int j = 0; j < 2; ++j)
        b[it][j] = ok ? *reinterpret_cast<const f32x4_t *>(gb + r * ld + c + 4 * j) : f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    const int c0 = (t % VPR) * 8;
#pragma unroll
    for (int j = 0; j < 2; ++j) bl[j] = *reinterpret_cast<const f32x4_t *>(gb + (int64_t)(L - 1) * ld + c0 + 4 * j);
#pragma unroll
    for (int it = 0; it < IF; ++it) {
      const int idx = it * NT + t, r = idx / (D / 4), c = (idx % (D / 4)) * 4;
      w[it] = ((NF % NT == 0 || idx < NF) && r < L) ? *reinterpret_cast<const u32x4_t *>(gw + r * ld + c) : z;
    }
    f32x4_t uu[C / 16][1];
    load_strip<C / 16, 1>(uu, p.u + t0 * ld + h * D, ld, col0, L);
#pragma unroll
    for (int i = 0; i < C / 16; ++i) u[i] = uu[i][0];
  }

  __device__ __forceinline__ void store(char *smem) const {
    using S = ScanBf16Smem<C, D>;
    const int t = threadIdx.x;
#pragma unroll
    for (int it = 0; it < II; ++it) {
      const int idx = it * NT + t, r = idx / VPR, c = (idx % VPR) * 8;
      if (NI % NT == 0 || idx < NI) {
        const bf16x8_t k8 = __builtin_bit_cast(bf16x8_t, k[it]);
        float kt[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) kt[e] = static_cast<float>(k8[e]) * fast_exp2(bl[e >> 2][e & 3] - b[it][e >> 2][e & 3]);
        *reinterpret_cast<bf16x8_t *>(smem + S::k + 2 * (r * S::LDT + c)) = pack_bf16x8(kt);
      }
    }
#pragma unroll
    for (int it = 0; it < IF; ++it) {
      const int idx = it * NT + t, r = idx / (D / 4), c = (idx % (D / 4)) * 4;
      if (NF % NT == 0 || idx < NF)
        *reinterpret_cast<bf16x4_t *>(smem + S::w + 2 * (r * S::LDT + bf16_op_pos(c))) =
            to_bf16x4(__builtin_bit_cast(f32x4_t, w[it]));
    }
    if (t < VPR) {
      float *sDecay = reinterpret_cast<float *>(smem + S::decay);
#pragma unroll
      for (int e = 0; e < 8; ++e) sDecay[t * 8 + e] = fast_exp2(bl[e >> 2][e & 3]);
    }
  }
};

template <int C, int D>
__global__ __launch_bounds__(4 * D) void stage_scan_bf16_kernel(ChunkParams p) {
  using S = ScanBf16Smem<C, D>;
  using M = Mma<bf16_t>;
  constexpr int NT = 4 * D, NC = C / 16, DT = D / 16, LDT = S::LDT;
  const int nh = blockIdx.x, n = nh / p.H, h = nh % p.H;
  const int wid = wave_id();
  const int n16 = tid_opaque() & 15, grp = (tid_opaque() & 63) >> 4;
  const int col0 = 16 * wid;
  const SlotRange sr = slot_range(p.cu, n, p.T);
  const int nch = (sr.len + C - 1) / C;
  const int cbase = p.cu ? p.chunk_off[n] : n * ((p.T + C - 1) / C);
  const int Kr = p.Kr, Vr = p.Vr;
  const int64_t sbase = (int64_t)nh * Kr * Vr;  // states [Kr, Vr]
  const int64_t ld = (int64_t)p.H * D;
  extern __shared__ __align__(16) char smem[];
  const bf16_t *sW = reinterpret_cast<const bf16_t *>(smem + S::w), *sK = reinterpret_cast<const bf16_t *>(smem + S::k);
  const float *sDecay = reinterpret_cast<const float *>(smem + S::decay);

  f32x4_t hs[DT][1];
  if (p.h0) {
    load_strip<DT, 1>(hs, p.h0 + sbase, Vr, col0, Kr, Vr);
  } else {
#pragma unroll
    for (int t = 0; t < DT; ++t) hs[t][0] = zero4();
  }
  ScanBf16Regs<C, D> R;
  if (nch > 0) R.load(p, sr.t0, min(C, sr.len), h, col0);
  for (int c = 0; c < nch; ++c) {
    const int64_t t0 = sr.t0 + (int64_t)c * C;
    const int L = min(C, sr.len - c * C);
    store_strip<float, DT, 1>(p.hc + ((int64_t)(cbase + c) * p.H + h) * Kr * Vr, Vr, col0, Kr, hs, Vr);
    R.store(smem);
    f32x4_t uv[NC];
#pragma unroll
    for (int i = 0; i < NC; ++i) uv[i] = R.u[i];
    __syncthreads();
    if (c + 1 < nch) R.load(p, t0 + C, min(C, sr.len - (c + 1) * C), h, col0);
    // v_new = u - w h (w in operand order, h's accumulators as the B operand)
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      f32x4_t col[DT];
#pragma unroll
      for (int t = 0; t < DT; ++t) col[t] = hs[t][0];
      const bf16x8_t fh = acc_frag<bf16_t, DT>(col, s);
#pragma unroll
      for (int i = 0; i < NC; ++i)
        uv[i] = uv[i] - M::mma(*reinterpret_cast<const bf16x8_t *>(sW + (16 * i + n16) * LDT + 32 * s + 8 * grp), fh,
                               zero4());
    }
    {
      f32x4_t vs[NC][1];
#pragma unroll
      for (int i = 0; i < NC; ++i) vs[i][0] = uv[i];
      store_strip<float, NC, 1>(p.vnew + t0 * ld + h * D, ld, col0, L, vs);
    }
    // h <- Diag(2^b_L) h + k~^T v_new (k~ through the transposing load, v_new's accumulators as B)
    const int lo = cfrag_lane_off(LDT);
#pragma unroll
    for (int t = 0; t < DT; ++t) {
      const f32x4_t dec = *reinterpret_cast<const f32x4_t *>(sDecay + 16 * t + 4 * grp);
      hs[t][0] = hs[t][0] * dec;
    }
#pragma unroll
    for (int kb = 0; kb < NC; ++kb) {
      const bf16x4_t fv = to_bf16x4(uv[kb]);
#pragma unroll
      for (int t = 0; t < DT; ++t) hs[t][0] = mma16(load_cfrag_at(sK + 16 * kb * LDT + 16 * t, lo), fv, hs[t][0]);
    }
    __syncthreads();
  }
  if (p.ht && !(sr.len == 0 && p.ht == p.h0)) store_strip<float, DT, 1>(p.ht + sbase, Vr, col0, Kr, hs, Vr);
}

// ---- (6) output o = q~ h_c + A_qk v_new, per (chunk, head, 64-column value block) ----
template <typename Tin, int C, int D>
__global__ __launch_bounds__(256) void stage_output_kernel(ChunkParams p) {
  ChunkLoc lc;
  if (!locate_chunk(p, blockIdx.x, lc)) return;
  const int h = blockIdx.y, vb = blockIdx.z;
  using TL = Tile<Tin, C, D>;
  constexpr int BV = 64, NVW = 1, NC = TL::NC, DT = TL::DT, LDT = TL::LDT, LDB = TL::LDB;
  const int wid = threadIdx.x >> 6;
  const int col0 = vb * BV + wid * 16;
  extern __shared__ __align__(16) char smem[];
  Tin *sQ = reinterpret_cast<Tin *>(smem);   // q, then q~ = scale q 2^b
  float *sAqk = reinterpret_cast<float *>(sQ + C * LDT);
  float *sQn = sAqk + C * TL::LDA;  // per row: 1/sqrt(|q|^2 + eps) with q_l2norm
  const int64_t ld = (int64_t)p.H * D, ldc = (int64_t)p.H * C, ldk = (int64_t)p.Hk * p.Kr, ldv = (int64_t)p.H * p.Vr;
  const int64_t off = lc.t0 * ld + h * D, offk = lc.t0 * ldk + (h / (p.H / p.Hk)) * p.Kr;
  const int L = lc.L;
  // b of the chunk's rows, four channels per item (before the tiles' barrier up to 8
  // vectors a thread; wider tiles take them in groups of 8 after it); rows past L stay zero
  constexpr int VPR = D / 4, NI = C * VPR, IB = (NI + kNT - 1) / kNT, GB = IB <= 8 ? IB : 8;
  auto load_b = [&](f32x4_t (&bv)[GB], int j0) {
#pragma unroll
    for (int j = 0; j < GB; ++j) {
      const int idx = (j0 + j) * kNT + threadIdx.x, r = idx / VPR, i = (idx % VPR) * 4;
      bv[j] = (idx < NI && r < L) ? *reinterpret_cast<const f32x4_t *>(p.b + off + (int64_t)r * ld + i) : zero4();
    }
  };
  auto scale_q = [&](const f32x4_t (&bv)[GB], int j0) {
#pragma unroll
    for (int j = 0; j < GB; ++j) {
      const int idx = (j0 + j) * kNT + threadIdx.x, r = idx / VPR, i = (idx % VPR) * 4;
      if (idx < NI && r < L) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          Tin &x = sQ[r * LDT + i + e];
          x = from_f32<Tin>(p.scale * to_f32(x) * fast_exp2(bv[j][e]));
        }
      }
    }
  };
  f32x4_t bv[GB];
  if constexpr (IB <= 8) load_b(bv, 0);
  // every tile's loads, and this wave's state and v_new strips, in flight before
  // the first LDS write
  RowsFetch<Tin, kNT, C, D> fq;
  RowsFetch<float, kNT, C, C> fa;
  fq.fetch(reinterpret_cast<const Tin *>(p.q) + offk, ldk, L, p.Kr);
  fa.fetch(p.Aqk + lc.t0 * ldc + h * C, ldc, L);
  f32x4_t hs[DT][NVW], vn[NC][NVW], o[NC][NVW];
  load_strip<DT, NVW>(hs, p.hc + ((int64_t)lc.gci * p.H + h) * p.Kr * p.Vr, p.Vr, col0, p.Kr, p.Vr);
  load_strip<NC, NVW>(vn, p.vnew + off, ld, col0, lc.L);
  fq.put(sQ, LDT);
  fa.put(sAqk, TL::LDA);
  __syncthreads();
  if (p.q_l2norm && threadIdx.x < C) {  // raw q: o is linear in each q row
    float ss = 0.f;
    for (int c = 0; c < D; ++c) {
      const float x = to_f32(sQ[threadIdx.x * LDT + c]);
      ss = fmaf(x, x, ss);
    }
    sQn[threadIdx.x] = rsqrtf(ss + kQNormEps);
  }
  __syncthreads();  // the row norms read raw q
  if constexpr (IB <= 8) {
    scale_q(bv, 0);
  } else {
#pragma unroll 1
    for (int j0 = 0; j0 < IB; j0 += GB) {
      load_b(bv, j0);
      scale_q(bv, j0);
    }
  }
#pragma unroll
  for (int i = 0; i < NC; ++i) o[i][0] = zero4();
  __syncthreads();
  rows_times_state<Tin, C, D, NVW, false>(o, o, sQ, sQ, hs);
  causal_times<Tin, C, NVW>(o, sAqk, vn);
  if (p.q_l2norm) {
    const int grp = (threadIdx.x & 63) >> 4;
#pragma unroll
    for (int i = 0; i < NC; ++i) o[i][0] = o[i][0] * *reinterpret_cast<const f32x4_t *>(sQn + 16 * i + 4 * grp);
  }
  store_strip<Tin, NC, NVW>(reinterpret_cast<Tin *>(p.o) + lc.t0 * ldv + h * p.Vr, ldv, col0, lc.L, o, p.Vr);
}

// ---------------------------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------------------------
namespace {

template <typename K>
hipError_t launch_dyn(K kernel, dim3 grid, size_t smem, hipStream_t st, const ChunkParams &p, int threads = kNT) {
  if (grid.x == 0 || grid.y == 0 || grid.z == 0) return hipSuccess;
  if (smem > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) {
      (void)hipGetLastError();  // do not leave the error for the next launch to report
      return e;
    }
  }
  hipLaunchKernelGGL(kernel, grid, dim3(threads), smem, st, p);
  return hipGetLastError();
}

// Calls f.template operator()<Tin, C, D>() for the runtime (dtype, C, D).
template <typename F>
hipError_t dispatch(const ChunkParams &p, F &&f) {
#define KDA_CASE(TIN, CC, DD) \
  if (p.C == CC && p.D == DD) return f.template operator()<TIN, CC, DD>();
  if (p.is_bf16) {
    KDA_CASE(bf16_t, 64, 128) KDA_CASE(bf16_t, 64, 64) KDA_CASE(bf16_t, 64, 256)
    KDA_CASE(bf16_t, 32, 128) KDA_CASE(bf16_t, 32, 64) KDA_CASE(bf16_t, 32, 256)
  } else {
    KDA_CASE(float, 64, 128) KDA_CASE(float, 64, 64) KDA_CASE(float, 64, 256)
    KDA_CASE(float, 32, 128) KDA_CASE(float, 32, 64) KDA_CASE(float, 32, 256)
  }
#undef KDA_CASE
  return hipErrorInvalidValue;
}

}  // namespace

// ---- offsets check: the device-side contract of cu_seqlens, as flag bits ----
__global__ __launch_bounds__(256) void check_offsets_kernel(const int32_t *cu, int N, int T, int32_t *flags) {
  __shared__ int s_bad;
  if (threadIdx.x == 0) s_bad = 0;
  __syncthreads();
  int bad = 0;
  for (int n = threadIdx.x; n < N; n += 256)
    if (cu[n + 1] < cu[n]) bad |= KDA_OFFSETS_DECREASE;
  if (threadIdx.x == 0) {
    if (cu[0] < 0) bad |= KDA_OFFSETS_NEGATIVE;
    if (cu[N] > T) bad |= KDA_OFFSETS_PAST_END;
  }
  if (bad) atomicOr(&s_bad, bad);
  __syncthreads();
  if (threadIdx.x == 0) flags[0] = s_bad;
}

hipError_t launch_check_offsets(const int32_t *cu, int N, int T, int32_t *flags, hipStream_t st) {
  hipLaunchKernelGGL(check_offsets_kernel, dim3(1), dim3(256), 0, st, cu, N, T, flags);
  return hipGetLastError();
}

hipError_t launch_chunk_index(const ChunkParams &p, hipStream_t st) {
  if (!p.cu) return hipSuccess;
  hipLaunchKernelGGL(chunk_index_kernel, dim3(1), dim3(256), 0, st, p.cu, p.N, p.C, p.chunk_off, p.seg_len,
                     p.seg_off);
  return hipGetLastError();
}

hipError_t launch_stage_gate(const ChunkParams &p, hipStream_t st) {
  return dispatch(p, [&]<typename Tin, int C, int D>() {
    // persistent workgroups, four per compute unit
    const dim3 grid((unsigned)std::min<int64_t>((int64_t)p.max_chunks * p.H, 4LL * device_cus()));
    switch (p.gate_kind) {
      case kGateSafe: return launch_dyn(stage_gate_items_kernel<C, D, kGateSafe>, grid, 0, st, p);
      case kGateSoftplus: return launch_dyn(stage_gate_items_kernel<C, D, kGateSoftplus>, grid, 0, st, p);
      case kGateLogE: return launch_dyn(stage_gate_items_kernel<C, D, kGateLogE>, grid, 0, st, p);
      case kGateLog2Cumsum: return launch_dyn(stage_gate_items_kernel<C, D, kGateLog2Cumsum>, grid, 0, st, p);
    }
    return hipErrorInvalidValue;
  });
}

hipError_t launch_stage_grams(const ChunkParams &p, hipStream_t st) {
  return dispatch(p, [&]<typename Tin, int C, int D>() {
    using TL = Tile<Tin, C, D>;
    const size_t smem = sizeof(Tin) * 2 * C * TL::LDT + sizeof(float) * (C * TL::LDB + D + C);
    if (p.gate_kind == kGateSafe)
      return launch_dyn(stage_grams_kernel<Tin, C, D, true>, dim3(p.max_chunks, p.H), smem, st, p);
    return launch_dyn(stage_grams_kernel<Tin, C, D, false>, dim3(p.max_chunks, p.H), smem, st, p);
  });
}

hipError_t launch_stage_solve(const ChunkParams &p, hipStream_t st) {
  const size_t smem = sizeof(float) * 2 * p.C * (p.C + 4);
  if (p.C == 64) return launch_dyn(stage_solve_kernel<64>, dim3(p.max_chunks, p.H), smem, st, p);
  return launch_dyn(stage_solve_kernel<32>, dim3(p.max_chunks, p.H), smem, st, p);
}

hipError_t launch_stage_wy(const ChunkParams &p, hipStream_t st) {
  return dispatch(p, [&]<typename Tin, int C, int D>() {
    using TL = Tile<Tin, C, D>;
    const size_t smem = sizeof(float) * (C * TL::LDA + C) + sizeof(Tin) * 2 * C * TL::LDT;
    return launch_dyn(stage_wy_kernel<Tin, C, D>, dim3(p.max_chunks, p.H), smem, st, p);
  });
}

hipError_t launch_stage_scan(const ChunkParams &p, hipStream_t st) {
  return dispatch(p, [&]<typename Tin, int C, int D>() {
    using TL = Tile<Tin, C, D>;
    const size_t smem = sizeof(Tin) * (C * TL::LDT + D * TL::LDKT) + sizeof(float) * 2 * D;
    if constexpr (sizeof(Tin) == 2 && D <= 128)  // 4 D threads: at D = 256 the state would not fit 128 VGPRs
      return launch_dyn(stage_scan_bf16_kernel<C, D>, dim3(p.N * p.H), ScanBf16Smem<C, D>::total, st, p, 4 * D);
    return launch_dyn(stage_scan_kernel<Tin, C, D>, dim3(p.N * p.H * ((p.Vr + 63) / 64)), smem, st, p);
  });
}

hipError_t launch_stage_output(const ChunkParams &p, hipStream_t st) {
  return dispatch(p, [&]<typename Tin, int C, int D>() {
    using TL = Tile<Tin, C, D>;
    const size_t smem = sizeof(Tin) * C * TL::LDT + sizeof(float) * (C * TL::LDA + C);
    return launch_dyn(stage_output_kernel<Tin, C, D>, dim3(p.max_chunks, p.H, (p.Vr + 63) / 64), smem, st, p);
  });
}

}  // namespace kda
