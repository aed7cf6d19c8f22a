// Per-chunk building blocks of the chunked KDA forward, operating on LDS tiles.
//
// Shared by the six standalone step kernels (chunk_stages.hip) and the fused
// persistent kernel (chunk_fused.hip). For one (sequence, head, chunk) of
// L <= C rows starting from state h:
//   (1) b    = cumsum(gate) in log2 units, chunk-local          (stage kernel)
//   (2) A_kk = beta_r sum_i k_r k_s 2^(b_r-b_s)   (s < r)         grams
//       A_qk = scale  sum_i q_r k_s 2^(b_r-b_s)   (s <= r)
//   (3) T    = (I + A_kk)^-1                                       solve
//   (4) w    = T (beta k 2^b),  u = T (beta v)                     tri_mm
//   (5) v_new = u - w h ;  h <- Diag(2^b_L) h + (k 2^(b_L-b))^T v_new
//   (6) o    = scale (q 2^b) h + A_qk v_new                       state_step
//
// MFMA conventions (gfx950, wave64). A 16x16 accumulator tile ("C layout")
// gives lane l the rows 4*(l/16)+e, e = 0..3, of column l%16. Operand A of
// a 16x16xKS product gives lane l row l%16, operand B column l%16; lane
// group l/16 supplies EPL contraction indices. Which contraction index each
// (group, element) slot carries is free as long as A and B agree; we pick
// the map kidx() under which a C-layout accumulator column is, unchanged, a
// valid B operand. The state h and the corrected values v_new therefore stay
// in accumulator registers across the whole chunk loop with no relayout.
#pragma once

#include <type_traits>

#include "kda_device.h"

namespace kda {

template <typename Tin>
struct Mma;

// bf16 operands: v_mfma_f32_16x16x32_bf16, 8 contraction indices per lane.
template <>
struct Mma<bf16_t> {
  static constexpr int KS = 32;
  static constexpr int EPL = 8;
  typedef bf16x8_t frag_t;
  // slots 0..3 -> rows 4g..4g+3 of tile 2s; slots 4..7 -> the same rows of tile 2s+1
  static __device__ __forceinline__ int kidx(int s, int grp, int e) {
    return 32 * s + ((e >> 2) << 4) + 4 * grp + (e & 3);
  }
  static __device__ __forceinline__ void set(frag_t &f, int e, float v) { f[e] = static_cast<bf16_t>(v); }
  static __device__ __forceinline__ f32x4_t mma(const frag_t &a, const frag_t &b, const f32x4_t &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

// fp32 operands: v_mfma_f32_16x16x4_f32, one contraction index per lane.
template <>
struct Mma<float> {
  static constexpr int KS = 4;
  static constexpr int EPL = 1;
  typedef float frag_t;
  // step s covers rows {4g + (s&3)} of tile s>>2
  static __device__ __forceinline__ int kidx(int s, int grp, int) { return 16 * (s >> 2) + 4 * grp + (s & 3); }
  static __device__ __forceinline__ void set(frag_t &f, int, float v) { f = v; }
  static __device__ __forceinline__ f32x4_t mma(const frag_t &a, const frag_t &b, const f32x4_t &c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
};

// B (or A) operand for contraction step s taken from C-layout accumulator
// tiles of one column: tiles[t] holds rows 16t..16t+15.
template <typename Tin, int NT_>
__device__ __forceinline__ typename Mma<Tin>::frag_t acc_frag(const f32x4_t (&tiles)[NT_], int s) {
  typename Mma<Tin>::frag_t f;
  if constexpr (std::is_same<Tin, bf16_t>::value) {
    const f32x4_t &a = tiles[2 * s], &b = tiles[2 * s + 1];
    f = __builtin_bit_cast(bf16x8_t, u32x4_t{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]),
                                             pack_bf16x2(b[0], b[1]), pack_bf16x2(b[2], b[3])});
  } else {
    f = tiles[s >> 2][s & 3];
  }
  return f;
}

__device__ __forceinline__ f32x4_t zero4() { return f32x4_t{0.f, 0.f, 0.f, 0.f}; }

// LDS geometry of one chunk.
template <typename Tin, int C_, int D_>
struct Tile {
  static constexpr int C = C_, D = D_;
  static constexpr int NC = C / 16;   // 16-row sub-chunks
  static constexpr int DT = D / 16;   // 16-wide channel tiles
  static constexpr int LDT = D + 8;   // row stride (elements) of q, k, v, w tiles [C][D] in Tin
  static constexpr int LDB = D + 4;   // row stride of the fp32 cumsum b [C][D]
  static constexpr int LDA = C + 4;   // row stride of the fp32 [C][C] matrices A_kk, T, A_qk
  static constexpr int LDKT = C + 8;  // row stride of the transposed [D][C] tile k~^T in Tin
  static_assert(C == 32 || C == 64, "chunk size");
  static_assert(D == 64 || D == 128 || D == 256, "head width");
};

// Range-checked loads through a raw buffer resource over [base, base + bytes):
// an offset at or past `bytes` reads zeros and touches no memory. The masked
// tile loads below are written with them, branch-free: a load behind a
// per-lane condition compiles to a branch around each load that waits for its
// data before the next one issues, which serialises the whole tile fetch.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}
constexpr uint32_t kOffNone = 0x80000000u;  // offset of an element to read as zero
__device__ __forceinline__ u32x4_t tile_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}

// L rows of COLS elements (global row stride ldg elements, L - 1 rows of it
// well below 2 GiB) fetched into registers, then written to an LDS tile of row
// stride lds; columns >= ncol (a multiple of the vector width) and rows
// L..ROWS-1 come out zero. 16-byte accesses. A kernel that fills several tiles
// fetches them all before the first put, so their loads are in flight
// together: a put waits for its own loads, which would otherwise hold back the
// next tile's.
template <typename T, int NT, int ROWS, int COLS>
struct RowsFetch {
  static constexpr int EPV = 16 / (int)sizeof(T);
  static constexpr int VPR = COLS / EPV, NV = ROWS * VPR, IT = (NV + NT - 1) / NT;
  u32x4_t buf[IT];

  __device__ __forceinline__ void fetch(const T *g, int64_t ldg, int L, int ncol = COLS) {
    const auto rs = tile_rsrc(g, L > 0 ? (uint32_t)(((int64_t)(L - 1) * ldg + ncol) * (int64_t)sizeof(T)) : 0u);
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int idx = it * NT + tid_opaque();
      const int r = idx / VPR, c = (idx % VPR) * EPV;
      const bool ok = (NV % NT == 0 || idx < NV) && r < L && c < ncol;
      buf[it] = tile_load16(rs, ok ? (uint32_t)(((int64_t)r * ldg + c) * (int64_t)sizeof(T)) : kOffNone);
    }
  }
  __device__ __forceinline__ void put(T *s, int lds) const {
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int idx = it * NT + tid_opaque();
      const int r = idx / VPR, c = (idx % VPR) * EPV;
      if (NV % NT == 0 || idx < NV) *reinterpret_cast<u32x4_t *>(s + r * lds + c) = buf[it];
    }
  }
};

// One tile on its own: fetch, then put.
template <typename T, int NT, int ROWS, int COLS>
__device__ __forceinline__ void load_rows(T *s, int lds, const T *g, int64_t ldg, int L, int ncol = COLS) {
  RowsFetch<T, NT, ROWS, COLS> f;
  f.fetch(g, ldg, L, ncol);
  f.put(s, lds);
}

// Same, converting fp32 global rows to the tile type T (used for the fp32
// intermediates of the staged schedule).
template <typename T, int NT, int ROWS, int COLS>
__device__ __forceinline__ void load_rows_cvt(T *s, int lds, const float *g, int64_t ldg, int L) {
  constexpr int VPR = COLS / 4, NV = ROWS * VPR, IT = (NV + NT - 1) / NT;
  const auto rs = tile_rsrc(g, L > 0 ? (uint32_t)(((int64_t)(L - 1) * ldg + COLS) * 4) : 0u);
  f32x4_t buf[IT];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int idx = it * NT + tid_opaque();
    const int r = idx / VPR, c = (idx % VPR) * 4;
    const bool ok = (NV % NT == 0 || idx < NV) && r < L;
    buf[it] = __builtin_bit_cast(f32x4_t, tile_load16(rs, ok ? (uint32_t)(((int64_t)r * ldg + c) * 4) : kOffNone));
  }
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int idx = it * NT + tid_opaque();
    const int r = idx / VPR, c = (idx % VPR) * 4;
    if (NV % NT == 0 || idx < NV) {
#pragma unroll
      for (int e = 0; e < 4; ++e) s[r * lds + c + e] = from_f32<T>(buf[it][e]);
    }
  }
}

// ---------------------------------------------------------------------------------------------
// (1) The chunk-local gate cumsum in log2 units (the staged step runs it in
// registers, chunk_stages.hip; the fused kernels in gate_cumsum_tables).
// ---------------------------------------------------------------------------------------------
// gate_pad: sB already holds the chunk-local cumsum for rows [0, L); rows >= L
// take row L-1's value (as the cumsum of a zero gate would) and sBL <- b[L-1].
template <int NT, int C, int D>
__device__ __forceinline__ void gate_pad(float *sB, int ldb, float *sBL, int L) {
  for (int idx = tid_opaque(); idx < (C - L) * D; idx += NT) {
    const int r = L + idx / D, c = idx % D;
    sB[r * ldb + c] = sB[(L - 1) * ldb + c];
  }
  for (int c = tid_opaque(); c < D; c += NT) sBL[c] = sB[(L - 1) * ldb + c];
  __syncthreads();
}

// ---------------------------------------------------------------------------------------------
// (2) intra-chunk grams over the causal 16x16 blocks (i, j <= i) only.
// Safe gate: diagonal blocks factor 2^(b_r-b_s) through the block's midpoint
// row, off-diagonal blocks through the first row of block i (both exponents
// non-positive) -- "FLA KDA Skill", section "Safe gate numerical note".
// Non-safe gate: diagonal blocks evaluate 2^(b_r-b_s) per pair (token-parallel
// form, "FLA KDA Skill", section "Safe vs non-safe intra path"); off-diagonal
// blocks use the same paired non-positive offsets.
// Blocks above the diagonal are written as zeros.
// ---------------------------------------------------------------------------------------------
// Outputs go to Akk / Aqk with row stride ldo (LDS or global); only rows < wlim
// are written.
template <typename Tin, int NT, int C, int D, bool SAFE>
__device__ void grams(const Tin *sQ, const Tin *sK, const float *sB, const float *sBeta, float scale, float *Akk,
                      float *Aqk, int64_t ldo, int L, int wlim) {
  using M = Mma<Tin>;
  using TL = Tile<Tin, C, D>;
  constexpr int NW = NT / 64, NC = TL::NC, NB = NC * (NC + 1) / 2;
  constexpr int LDT = TL::LDT, LDB = TL::LDB;
  const int lane = tid_opaque() & 63, wid = wave_id();
  const int n16 = lane & 15, grp = lane >> 4;

  for (int blk = wid; blk < NB; blk += NW) {
    int i = 0, j = blk;
    while (j > i) {
      j -= i + 1;
      ++i;
    }
    f32x4_t accQ = zero4(), accK = zero4();
    if (SAFE || i != j) {
      const int a = (i == j) ? 16 * i + 8 : 16 * i;  // anchor row
      const int rr = 16 * i + n16;                   // A-operand row
      const int cc = 16 * j + n16;                   // B-operand column token
#pragma unroll 2
      for (int s = 0; s < D / M::KS; ++s) {
        typename M::frag_t fq, fk, fc;
#pragma unroll
        for (int e = 0; e < M::EPL; ++e) {
          const int kk = M::kidx(s, grp, e);
          const float ba = sB[a * LDB + kk];
          const float er = fast_exp2(sB[rr * LDB + kk] - ba);
          const float ec = fast_exp2(ba - sB[cc * LDB + kk]);
          M::set(fq, e, to_f32(sQ[rr * LDT + kk]) * er);
          M::set(fk, e, to_f32(sK[rr * LDT + kk]) * er);
          M::set(fc, e, to_f32(sK[cc * LDT + kk]) * ec);
        }
        accQ = M::mma(fq, fc, accQ);
        accK = M::mma(fk, fc, accK);
      }
    } else {
      // token-parallel diagonal block: lane owns column token sc and rows 4*grp + e
      const int sc = 16 * i + n16;
      for (int kk = 0; kk < D; ++kk) {
        const float ks = to_f32(sK[sc * LDT + kk]);
        const float bs = sB[sc * LDB + kk];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * i + 4 * grp + e;
          const float f = (r >= sc) ? fast_exp2(sB[r * LDB + kk] - bs) : 0.f;
          const float kf = ks * f;
          accQ[e] += to_f32(sQ[r * LDT + kk]) * kf;
          accK[e] += to_f32(sK[r * LDT + kk]) * kf;
        }
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 16 * i + 4 * grp + e, s_ = 16 * j + n16;
      if (r < wlim) {
        Aqk[r * ldo + s_] = (s_ <= r && r < L) ? scale * accQ[e] : 0.f;
        Akk[r * ldo + s_] = (s_ < r && r < L) ? sBeta[r] * accK[e] : 0.f;
      }
    }
  }
#pragma unroll
  for (int it = 0; it < (C * C + NT - 1) / NT; ++it) {
    const int idx = it * NT + tid_opaque();
    const int r = idx / C, c = idx % C;
    if (idx < C * C && (c >> 4) > (r >> 4) && r < wlim) {
      Akk[r * ldo + c] = 0.f;
      Aqk[r * ldo + c] = 0.f;
    }
  }
}

// ---------------------------------------------------------------------------------------------
// (3) T = (I + A_kk)^-1 for strictly lower-triangular A_kk, blocked:
// the 16x16 diagonal blocks by forward substitution (one lane per column),
// then T_ij = -T_ii sum_{m=j}^{i-1} A_im T_mj level by level (i - j = 1, 2, ...)
// with fp32 MFMA. Reads sAkk, writes all of sT (upper blocks zero).
// ---------------------------------------------------------------------------------------------
template <int NT, int C>
__device__ void solve(const float *sAkk, float *sT) {
  constexpr int NW = NT / 64, NC = C / 16, LDA = C + 4;
  const int lane = tid_opaque() & 63, wid = wave_id();
  const int n16 = lane & 15, grp = lane >> 4;
#pragma unroll
  for (int it = 0; it < (C * C + NT - 1) / NT; ++it) {
    const int idx = it * NT + tid_opaque();
    const int r = idx / C, c = idx % C;
    if (idx < C * C && (c >> 4) > (r >> 4)) sT[r * LDA + c] = 0.f;
  }
  if (wid == NW - 1 && lane < 16 * NC) {
    // column c of T_ii solves (I + A_ii) x = e_c; right-looking so that each
    // step's 15 - s updates are independent
    const int i = lane >> 4, c = lane & 15;
    const float *A = sAkk + 16 * i * LDA + 16 * i;
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) x[r] = (r == c) ? 1.f : 0.f;
#pragma unroll
    for (int s = 0; s < 16; ++s) {
#pragma unroll
      for (int r = s + 1; r < 16; ++r) x[r] -= A[r * LDA + s] * x[s];
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) sT[(16 * i + r) * LDA + 16 * i + c] = x[r];
  }
  __syncthreads();
#pragma unroll
  for (int d = 1; d < NC; ++d) {
    for (int blk = wid; blk < NC - d; blk += NW) {
      const int j = blk, i = blk + d;
      f32x4_t P = zero4();
      for (int m = j; m < i; ++m) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float a = sAkk[(16 * i + n16) * LDA + 16 * m + 4 * grp + e];
          const float b = sT[(16 * m + 4 * grp + e) * LDA + 16 * j + n16];
          P = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, P, 0, 0, 0);
        }
      }
      f32x4_t R = zero4();
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float a = sT[(16 * i + n16) * LDA + 16 * i + 4 * grp + e];
        R = __builtin_amdgcn_mfma_f32_16x16x4f32(a, P[e], R, 0, 0, 0);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) sT[(16 * i + 4 * grp + e) * LDA + 16 * j + n16] = -R[e];
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------------------------
// (4) acc[i][v] = sum_c T[16i + r][c] X[c][16ct + n] for one 16-wide column tile ct,
// all row blocks i. Only the causal part of T (c <= 16i + 15) is visited.
// xval(c, col) returns X[c][col].
// ---------------------------------------------------------------------------------------------
template <typename Tin, int C, int NV, typename XF>
__device__ __forceinline__ void tri_mm(const float *sT, int ct, f32x4_t (&acc)[C / 16][NV], int v, XF xval) {
  using M = Mma<Tin>;
  constexpr int NC = C / 16, LDA = C + 4, NS = C / M::KS;
  const int lane = tid_opaque() & 63;
  const int n16 = lane & 15, grp = lane >> 4;
  const int col = 16 * ct + n16;
#pragma unroll
  for (int i = 0; i < NC; ++i) acc[i][v] = zero4();
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    typename M::frag_t fb;
#pragma unroll
    for (int e = 0; e < M::EPL; ++e) M::set(fb, e, xval(M::kidx(s, grp, e), col));
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      if (16 * (i + 1) <= s * M::KS) continue;  // T block entirely above the diagonal
      typename M::frag_t fa;
#pragma unroll
      for (int e = 0; e < M::EPL; ++e) M::set(fa, e, sT[(16 * i + n16) * LDA + M::kidx(s, grp, e)]);
      acc[i][v] = M::mma(fa, fb, acc[i][v]);
    }
  }
}

// q~ = scale * q * 2^b, in place (row-major).
template <typename Tin, int NT, int C, int D>
__device__ __forceinline__ void make_qtilde(Tin *sQ, const float *sB, float scale) {
  using TL = Tile<Tin, C, D>;
  constexpr int VPR = D / 4, IT = C * VPR / NT;
  static_assert(C * VPR % NT == 0, "tile");
#pragma unroll 4
  for (int it = 0; it < IT; ++it) {
    const int idx = it * NT + tid_opaque();
    const int r = idx / VPR, c = (idx % VPR) * 4;
    const f32x4_t b = *reinterpret_cast<const f32x4_t *>(sB + r * TL::LDB + c);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      sQ[r * TL::LDT + c + e] = from_f32<Tin>(scale * to_f32(sQ[r * TL::LDT + c + e]) * fast_exp2(b[e]));
  }
}

// k~^T [D][C] with k~[c][i] = k[c][i] * 2^(b_L[i] - b[c][i]).
template <typename Tin, int NT, int C, int D>
__device__ __forceinline__ void make_ktilde_t(Tin *sKT, const Tin *sK, const float *sB, const float *sBL) {
  using TL = Tile<Tin, C, D>;
  constexpr int IT = C * D / NT;
  static_assert(C * D % NT == 0, "tile");
#pragma unroll 4
  for (int it = 0; it < IT; ++it) {
    const int idx = it * NT + tid_opaque();
    const int c = idx % C, i = idx / C;  // consecutive threads walk the chunk rows
    const float v = to_f32(sK[c * TL::LDT + i]) * fast_exp2(sBL[i] - sB[c * TL::LDB + i]);
    sKT[i * TL::LDKT + c] = from_f32<Tin>(v);
  }
}

// Fills rows L..C-1 of an fp32 cumsum tile with row L-1 (rows past the end
// of a sequence carry a zero gate) and copies the last row to sBL.
template <int NT, int C, int D>
__device__ __forceinline__ void pad_cumsum(float *sB, int ldb, float *sBL, int L) {
  if (L < C) {
#pragma unroll
    for (int it = 0; it < C * D / NT; ++it) {
      const int idx = it * NT + tid_opaque();
      const int r = idx / D, c = idx % D;
      if (r >= L) sB[r * ldb + c] = (L > 0) ? sB[(L - 1) * ldb + c] : 0.f;
    }
  }
  __syncthreads();
  for (int c = tid_opaque(); c < D; c += NT) sBL[c] = sB[(C - 1) * ldb + c];
}

// Same from global rows: k [L][D] (row stride ld) and the fp32 cumsum b [L][D];
// rows >= L of k~^T are zero.
template <typename Tin, int NT, int C, int D>
__device__ __forceinline__ void make_ktilde_t_global(Tin *sKT, const Tin *gK, int64_t ldk, const float *gB,
                                                     int64_t ld, const float *sBL, int L, int kr) {
  using TL = Tile<Tin, C, D>;
  for (int idx = tid_opaque(); idx < C * D; idx += NT) {
    const int i = idx % D, c = idx / D;  // consecutive threads walk the channels (coalesced reads)
    float v = 0.f;
    if (c < L && i < kr) v = to_f32(gK[(int64_t)c * ldk + i]) * fast_exp2(sBL[i] - gB[(int64_t)c * ld + i]);
    sKT[i * TL::LDKT + c] = from_f32<Tin>(v);
  }
}

// ---------------------------------------------------------------------------------------------
// (5)/(6) on one wave's strip of NVW value tiles. h [D/16][NVW] and v_new
// [C/16][NVW] are C-layout accumulators (rows = channels / chunk rows).
// ---------------------------------------------------------------------------------------------

// out0 += A0 h and, when sA1 is given, out1 += A1 h; A0, A1: [C][D] row-major Tin
// (w and q~). Contraction over the D channels.
template <typename Tin, int C, int D, int NVW, bool TWO>
__device__ __forceinline__ void rows_times_state(f32x4_t (&out0)[C / 16][NVW], f32x4_t (&out1)[C / 16][NVW],
                                                 const Tin *sA0, const Tin *sA1, const f32x4_t (&h)[D / 16][NVW]) {
  using M = Mma<Tin>;
  using TL = Tile<Tin, C, D>;
  constexpr int NC = TL::NC, DT = TL::DT, LDT = TL::LDT, SD = D / M::KS;
  const int lane = tid_opaque() & 63;
  const int n16 = lane & 15, grp = lane >> 4;
#pragma unroll
  for (int s = 0; s < SD; ++s) {
    typename M::frag_t fh[NVW];
#pragma unroll
    for (int v = 0; v < NVW; ++v) {
      f32x4_t col[DT];
#pragma unroll
      for (int t = 0; t < DT; ++t) col[t] = h[t][v];
      fh[v] = acc_frag<Tin, DT>(col, s);
    }
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      typename M::frag_t f0, f1;
#pragma unroll
      for (int e = 0; e < M::EPL; ++e) {
        const int kk = M::kidx(s, grp, e);
        M::set(f0, e, to_f32(sA0[(16 * i + n16) * LDT + kk]));
        if (TWO) M::set(f1, e, to_f32(sA1[(16 * i + n16) * LDT + kk]));
      }
#pragma unroll
      for (int v = 0; v < NVW; ++v) {
        out0[i][v] = M::mma(f0, fh[v], out0[i][v]);
        if (TWO) out1[i][v] = M::mma(f1, fh[v], out1[i][v]);
      }
    }
  }
}

// o += A_qk v_new, A_qk: [C][C] fp32 (lower triangular; causal blocks only).
template <typename Tin, int C, int NVW>
__device__ __forceinline__ void causal_times(f32x4_t (&o)[C / 16][NVW], const float *sAqk,
                                             const f32x4_t (&vn)[C / 16][NVW]) {
  using M = Mma<Tin>;
  constexpr int NC = C / 16, LDA = C + 4, SC = C / M::KS;
  const int lane = tid_opaque() & 63;
  const int n16 = lane & 15, grp = lane >> 4;
#pragma unroll
  for (int s = 0; s < SC; ++s) {
    typename M::frag_t fv[NVW];
#pragma unroll
    for (int v = 0; v < NVW; ++v) {
      f32x4_t col[NC];
#pragma unroll
      for (int t = 0; t < NC; ++t) col[t] = vn[t][v];
      fv[v] = acc_frag<Tin, NC>(col, s);
    }
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      if (16 * (i + 1) <= s * M::KS) continue;
      typename M::frag_t fa;
#pragma unroll
      for (int e = 0; e < M::EPL; ++e) M::set(fa, e, sAqk[(16 * i + n16) * LDA + M::kidx(s, grp, e)]);
#pragma unroll
      for (int v = 0; v < NVW; ++v) o[i][v] = M::mma(fa, fv[v], o[i][v]);
    }
  }
}

// h <- Diag(2^b_L) h + k~^T v_new; sKT: [D][C] Tin with row stride ldkt; sDecay: [D].
template <typename Tin, int C, int D, int NVW>
__device__ __forceinline__ void state_update(f32x4_t (&h)[D / 16][NVW], const Tin *sKT, int ldkt,
                                             const f32x4_t (&vn)[C / 16][NVW], const float *sDecay) {
  using M = Mma<Tin>;
  constexpr int NC = C / 16, DT = D / 16, SC = C / M::KS;
  const int lane = tid_opaque() & 63;
  const int n16 = lane & 15, grp = lane >> 4;
#pragma unroll
  for (int t = 0; t < DT; ++t) {
    const f32x4_t dec = *reinterpret_cast<const f32x4_t *>(sDecay + 16 * t + 4 * grp);
#pragma unroll
    for (int v = 0; v < NVW; ++v) h[t][v] = h[t][v] * dec;
  }
#pragma unroll
  for (int s = 0; s < SC; ++s) {
    typename M::frag_t fv[NVW];
#pragma unroll
    for (int v = 0; v < NVW; ++v) {
      f32x4_t col[NC];
#pragma unroll
      for (int t = 0; t < NC; ++t) col[t] = vn[t][v];
      fv[v] = acc_frag<Tin, NC>(col, s);
    }
#pragma unroll
    for (int t = 0; t < DT; ++t) {
      typename M::frag_t fk;
#pragma unroll
      for (int e = 0; e < M::EPL; ++e) M::set(fk, e, to_f32(sKT[(16 * t + n16) * ldkt + M::kidx(s, grp, e)]));
#pragma unroll
      for (int v = 0; v < NVW; ++v) h[t][v] = M::mma(fk, fv[v], h[t][v]);
    }
  }
}

// Loads / stores a [ROWS][cols] fp32 strip into C-layout accumulator tiles:
// tile (t, v) covers rows 16t.., columns col0 + 16v... Rows >= L read as 0 /
// are not stored.
template <int RT, int NVW>
__device__ __forceinline__ void load_strip(f32x4_t (&x)[RT][NVW], const float *g, int64_t ld, int col0, int L,
                                           int ncol = 1 << 30) {
  const int lane = tid_opaque() & 63;
  const int n16 = lane & 15, grp = lane >> 4;
  // range-checked and branch-free (kOffNone and rows past L read zeros), so the
  // loads are issued back to back
  const int cend = ncol < col0 + 16 * NVW ? ncol : col0 + 16 * NVW;
  const auto rs = tile_rsrc(g, L > 0 && cend > 0 ? (uint32_t)(((int64_t)(L - 1) * ld + cend) * 4) : 0u);
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int v = 0; v < NVW; ++v)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * t + 4 * grp + e, c = col0 + 16 * v + n16;
        const uint32_t off = (r < L && c < ncol) ? (uint32_t)(((int64_t)r * ld + c) * 4) : kOffNone;
        x[t][v][e] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, (int)off, 0, 0));
      }
}

template <typename T, int RT, int NVW>
__device__ __forceinline__ void store_strip(T *g, int64_t ld, int col0, int L, const f32x4_t (&x)[RT][NVW],
                                            int ncol = 1 << 30) {
  const int lane = tid_opaque() & 63;
  const int n16 = lane & 15, grp = lane >> 4;
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int v = 0; v < NVW; ++v)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * t + 4 * grp + e, c = col0 + 16 * v + n16;
        if (r < L && c < ncol) g[(int64_t)r * ld + c] = from_f32<T>(x[t][v][e]);
      }
}

// The output strip of one wave (C-layout tiles: rows 16i.., columns col0 +
// 16v..) into an fp32 staging tile of row stride lds.
template <int NC, int NVW>
__device__ __forceinline__ void stage_strip(float *s, int lds, int col0, const f32x4_t (&x)[NC][NVW]) {
  const int lane = tid_opaque() & 63;
  const int n16 = lane & 15, grp = lane >> 4;
#pragma unroll
  for (int i = 0; i < NC; ++i)
#pragma unroll
    for (int v = 0; v < NVW; ++v)
#pragma unroll
      for (int e = 0; e < 4; ++e) s[(16 * i + 4 * grp + e) * lds + col0 + 16 * v + n16] = x[i][v][e];
}

// Rows [0, L) of an fp32 staging tile [C][D] to global rows of type T with
// 16-byte stores (all NT threads; a thread converts 16 / sizeof(T) adjacent
// elements of one row).
template <typename T, int NT, int C, int D>
__device__ __forceinline__ void store_rows_from_f32(T *g, int64_t ldg, const float *s, int lds, int L) {
  constexpr int EPV = 16 / (int)sizeof(T), VPR = D / EPV, NV = C * VPR;
  static_assert(NV % NT == 0, "tile");
#pragma unroll
  for (int it = 0; it < NV / NT; ++it) {
    const unsigned idx = it * NT + (unsigned)tid_opaque();
    const int r = idx / VPR, c = (idx % VPR) * EPV;
    if (r < L) {
      if constexpr (EPV == 8) {
        const f32x4_t a = *reinterpret_cast<const f32x4_t *>(s + r * lds + c);
        const f32x4_t b = *reinterpret_cast<const f32x4_t *>(s + r * lds + c + 4);
        *reinterpret_cast<u32x4_t *>(g + (int64_t)r * ldg + c) =
            u32x4_t{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]), pack_bf16x2(b[0], b[1]), pack_bf16x2(b[2], b[3])};
      } else {
        *reinterpret_cast<f32x4_t *>(g + (int64_t)r * ldg + c) = *reinterpret_cast<const f32x4_t *>(s + r * lds + c);
      }
    }
  }
}

}  // namespace kda
