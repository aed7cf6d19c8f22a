// Building blocks of the fused chunk kernel (bf16 operands, gfx950).
//
// Beyond the shared steps in chunk_tiles.h, the fused kernel
//  - solves (I + A_kk) [w | u] = [beta k 2^b | beta v] by blocked forward
//    substitution per 16-column tile, so no wave waits for another's columns
//    and only the four 16x16 diagonal inverses are formed explicitly;
//  - keeps w^T and k~ = k 2^(b_L - b) in LDS in the layouts their producers
//    write with wide stores, and reads the transposed MFMA operands with
//    ds_read_b64_tr_b16;
//  - forms q~, k~ and beta k 2^b in the grams from the same exponentials.
//
// ds_read_b64_tr_b16 (measured lane layout): within each 16-lane group g,
// source lane s supplies four consecutive 16-bit elements m[s][0..3] from its
// own address; destination lane 4a + b receives m[4e + a][b] for e = 0..3.
// Giving source lane s the address of M[k0 + 4g + s/4][n0 + 4(s%4)] of a
// row-major matrix M therefore hands lane l the C-layout column
// M[k0 + 4g + e][n0 + l%16], e = 0..3 -- a B operand of a 16x16x16 product,
// or, read from a transposed store, an A operand.
#pragma once

#include "chunk_tiles.h"

namespace kda {

typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));

// The lane's part of a transposed-load address into a row-major bf16 matrix
// of row stride ld: (4g + s/4) * ld + 4 (s % 4), g = lane / 16, s = lane % 16.
// Computed once per phase; the tile offsets k0 * ld + n0 are then immediates.
__device__ __forceinline__ int cfrag_lane_off(int ld) {
  const int lane = tid_opaque() & 63;
  const int g = lane >> 4, s = lane & 15;
  return (4 * g + (s >> 2)) * ld + 4 * (s & 3);
}

// Lane l of M (row-major bf16, ld % 4 == 0, n0 % 4 == 0), with lo = cfrag_lane_off(ld):
// {M[k0 + 4g + e][n0 + l%16]}, e = 0..3, g = (l%64)/16.
__device__ __forceinline__ bf16x4_t load_cfrag_at(const bf16_t *M, int lo) {
  const i16x4_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4_t __attribute__((address_space(3))) *)(M + lo));
  return __builtin_bit_cast(bf16x4_t, r);
}

__device__ __forceinline__ bf16x4_t load_cfrag(const bf16_t *M, int ld, int k0, int n0) {
  return load_cfrag_at(M + k0 * ld + n0, cfrag_lane_off(ld));
}

__device__ __forceinline__ f32x4_t mma16(const bf16x4_t &a, const bf16x4_t &b, const f32x4_t &c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4_t, a), __builtin_bit_cast(i16x4_t, b), c,
                                                    0, 0, 0);
}

__device__ __forceinline__ bf16x4_t to_bf16x4(const f32x4_t &x) {
  return __builtin_bit_cast(bf16x4_t, u32x2_t{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])});
}

__device__ __forceinline__ bf16x4_t pack_bf16x4(float a, float b, float c, float d) {
  return __builtin_bit_cast(bf16x4_t, u32x2_t{pack_bf16x2(a, b), pack_bf16x2(c, d)});
}

__device__ __forceinline__ f32x4_t to_f32x4(const bf16x4_t &x) {
  f32x4_t r;
#pragma unroll
  for (int e = 0; e < 4; ++e) r[e] = static_cast<float>(x[e]);
  return r;
}

// Two C-layout fragments (contraction rows k0.. and k0+16..) as the 8-slot
// operand of a 16x16x32 product under the kidx map of Mma<bf16_t>.
__device__ __forceinline__ bf16x8_t load_frag32_at(const bf16_t *M, int ld, int lo_off) {
  const bf16x4_t lo = load_cfrag_at(M, lo_off), hi = load_cfrag_at(M + 16 * ld, lo_off);
  bf16x8_t f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f[e] = lo[e];
    f[e + 4] = hi[e];
  }
  return f;
}

__device__ __forceinline__ bf16x8_t load_frag32(const bf16_t *M, int ld, int k0, int n0) {
  const bf16x4_t lo = load_cfrag(M, ld, k0, n0), hi = load_cfrag(M, ld, k0 + 16, n0);
  bf16x8_t f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f[e] = lo[e];
    f[e + 4] = hi[e];
  }
  return f;
}

// (1) The chunk-local cumsum b of the gate rows in sB (fp32, base 2, in place),
// with b_L in sBL, the chunk decay 2^b_L in sDecay and, for the safe gate, the
// anchor tables of each 16-row block i with midpoint m_i = b at row 16i + 8 and
// first row a_i: sT1 = scale 2^m_i, sT2 = 2^(b_L - m_i), sT0 = 2^(m_i - a_i).
// Each thread scans RPS consecutive rows of one channel; with RPS = 8 the thread
// of a block's first half also reads the raw gate of row 16i + 8 to reach m_i.
// Ends with a barrier.
template <int NT, int C, int D, bool SAFE>
__device__ __forceinline__ void gate_cumsum_tables(float *sB, int ldb, float *sBL, float *sSeg, float *sDecay,
                                                   float *sT0, float *sT1, float *sT2, float scale) {
  static_assert(NT % D == 0, "thread mapping: whole channels per thread group");
  constexpr int TPC = NT / D;  // threads per channel, each owning RPS consecutive rows
  constexpr int RPS = C / TPC;
  static_assert(RPS % 16 == 0 || RPS == 8, "segments and 16-row blocks nest");
  const int tid = tid_opaque(), col = tid % D, seg = tid / D;
  float vals[RPS];
#pragma unroll
  for (int i = 0; i < RPS; ++i) vals[i] = sB[(seg * RPS + i) * ldb + col];
  float g_mid = 0.f;  // RPS = 8: the raw gate of the next segment's first row
  if constexpr (SAFE && RPS == 8)
    if ((seg & 1) == 0) g_mid = sB[(seg * RPS + 8) * ldb + col];
#pragma unroll
  for (int i = 1; i < RPS; ++i) vals[i] += vals[i - 1];
  float bl = vals[RPS - 1];
  if constexpr (TPC > 1) {
    sSeg[seg * D + col] = vals[RPS - 1];
    __syncthreads();
    float off = 0.f, off_last = 0.f;
#pragma unroll
    for (int s2 = 0; s2 < TPC - 1; ++s2) {
      const float t = sSeg[s2 * D + col];
      if (s2 < seg) off += t;
      off_last += t;
    }
    bl = sSeg[(TPC - 1) * D + col] + off_last;  // the last row's value, summed in the same order
#pragma unroll
    for (int i = 0; i < RPS; ++i) vals[i] += off;
  }
#pragma unroll
  for (int i = 0; i < RPS; ++i) sB[(seg * RPS + i) * ldb + col] = vals[i];
  if (seg == 0) {
    sBL[col] = bl;
    sDecay[col] = fast_exp2(bl);
  }
  if constexpr (SAFE) {
    auto tables = [&](int blk, float a, float m) {
      sT1[blk * D + col] = scale * fast_exp2(m);
      sT2[blk * D + col] = fast_exp2(bl - m);
      sT0[blk * D + col] = fast_exp2(m - a);
    };
    if constexpr (RPS == 8) {
      if ((seg & 1) == 0) tables(seg / 2, vals[0], vals[7] + g_mid);
    } else {
#pragma unroll
      for (int j = 0; j < RPS; j += 16) tables((seg * RPS + j) / 16, vals[j], vals[j + 8]);
    }
  }
  __syncthreads();
}

// (3) T_ii = (I + A_ii)^-1 of one 16 x 16 diagonal block by blocked forward
// substitution on one wave: lane 16g + c holds rows 4g..4g+3 of column c. In
// stage k the lanes of group k finish their four rows (a 4-step chain), pass
// them to every lane of the same column, and the later groups subtract their
// part, so the chain crosses lanes four times instead of sixteen. -A_ii is
// read at its origin Ablk (fp32, row stride lda, strictly lower, beta folded),
// T_ii written as bf16 rows at Tblk (row stride ldt).
__device__ __forceinline__ void diag_inverse16(const float *Ablk, int lda, bf16_t *Tblk, int ldt) {
  const int lane = tid_opaque() & 63;
  const int g = lane >> 4, c = lane & 15;
  const float *A = Ablk + 4 * g * lda;
  f32x4_t a[4][4];  // rows 4g + e, column quads q
#pragma unroll
  for (int e = 0; e < 4; ++e)
#pragma unroll
    for (int q = 0; q < 4; ++q) a[e][q] = *reinterpret_cast<const f32x4_t *>(A + e * lda + 4 * q);
  float x[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) x[e] = (4 * g + e == c) ? 1.f : 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    float z[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      z[e] = x[e];
#pragma unroll
      for (int e2 = 0; e2 < e; ++e2) z[e] += a[e][k][e2] * z[e2];
    }
    const bool mine = (g == k);
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = mine ? z[e] : x[e];
    if (k == 3) break;
    float y[4];  // group k's finished rows of this column, in every group
#pragma unroll
    for (int e = 0; e < 4; ++e) y[e] = k == 0 ? row_bcast<0>(x[e]) : (k == 1 ? row_bcast<1>(x[e]) : row_bcast<2>(x[e]));
    const bool later = (g > k);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float acc = x[e];
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) acc += a[e][k][e2] * y[e2];
      x[e] = later ? acc : x[e];
    }
  }
  bf16_t *T = Tblk + 4 * g * ldt + c;
#pragma unroll
  for (int e = 0; e < 4; ++e) T[e * ldt] = static_cast<bf16_t>(x[e]);
}

// The same for diagonal block i of -A_kk in sAkk, into rows 16i.. of sTd.
__device__ __forceinline__ void diag_inverse_block(const float *sAkk, int lda, bf16_t *sTd, int ldt, int i) {
  diag_inverse16(sAkk + 16 * i * lda + 16 * i, lda, sTd + 16 * i * ldt, ldt);
}


// ---------------------------------------------------------------------------------------------
// (4) A 16-column tile of W = (I + A_kk)^-1 X for one or two right-hand sides
// (tile cta of Xa, and with TWO tile ctb of Xb with rows scaled by rowscale[r]), by blocked forward
// substitution: R_i = X_i - sum_{j<i} A_ij W_j, W_i = T_ii R_i, with sAkk
// holding -A_kk. X tiles are row-major bf16; A_ij and T_ii are read once for
// both. W comes back as
// C-layout accumulators, one per row block.
// ---------------------------------------------------------------------------------------------
template <int C, bool TWO>
__device__ __forceinline__ void wy_subst2(const bf16_t *sXa, int cta, const bf16_t *sXb, int ctb, int ldx,
                                          const float *rowscale, const float *sAkk, int lda, const bf16_t *sTd,
                                          int ldt, f32x4_t (&Wa)[C / 16], f32x4_t (&Wb)[C / 16]) {
  constexpr int NC = C / 16;
  const int lane = tid_opaque() & 63;
  const int n16 = lane & 15, grp = lane >> 4;
  const int lx = cfrag_lane_off(ldx);
  const float *aRow = sAkk + n16 * lda + 4 * grp;
  const bf16_t *tRow = sTd + n16 * ldt + 4 * grp;
  const float *rs = rowscale + 4 * grp;
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    f32x4_t Ra = to_f32x4(load_cfrag_at(sXa + 16 * i * ldx + 16 * cta, lx));
    f32x4_t Rb;
    if (TWO) {
      Rb = to_f32x4(load_cfrag_at(sXb + 16 * i * ldx + 16 * ctb, lx));
      Rb = Rb * *reinterpret_cast<const f32x4_t *>(rs + 16 * i);
    }
#pragma unroll
    for (int j = 0; j < i; ++j) {
      const bf16x4_t a = to_bf16x4(*reinterpret_cast<const f32x4_t *>(aRow + 16 * i * lda + 16 * j));
      Ra = mma16(a, to_bf16x4(Wa[j]), Ra);
      if (TWO) Rb = mma16(a, to_bf16x4(Wb[j]), Rb);
    }
    const bf16x4_t t = *reinterpret_cast<const bf16x4_t *>(tRow + 16 * i * ldt);
    Wa[i] = mma16(t, to_bf16x4(Ra), zero4());
    if (TWO) Wb[i] = mma16(t, to_bf16x4(Rb), zero4());
  }
}

// C-layout tiles of one 16-column tile ct of w into w^T [D][ldw] (bf16):
// lane writes w[16i + 4g .. 16i + 4g + 3][16ct + n16] as one 8-byte store.
template <int C>
__device__ __forceinline__ void store_wT(bf16_t *sWT, int ldw, int ct, const f32x4_t (&W)[C / 16]) {
  const int lane = tid_opaque() & 63;
  const int n16 = lane & 15, grp = lane >> 4;
#pragma unroll
  for (int i = 0; i < C / 16; ++i)
    *reinterpret_cast<bf16x4_t *>(sWT + (16 * ct + n16) * ldw + 16 * i + 4 * grp) = to_bf16x4(W[i]);
}

// ---------------------------------------------------------------------------------------------
// (5)/(6) on one wave's strip of NVW value tiles (h [D/16][NVW], C-layout).
// p1 = w h with w read from w^T; o is formed transposed, o^T = h^T q~^T with
// q~ row-major, so o[i][v] holds rows 16v.. of o^T (value columns) against
// chunk rows 16i + (lane % 16).
// ---------------------------------------------------------------------------------------------
template <int C, int D, int NVW>
__device__ __forceinline__ void w_times_state(f32x4_t (&p1)[C / 16][NVW], const bf16_t *sWT, int ldw,
                                              const f32x4_t (&h)[D / 16][NVW]) {
  using M = Mma<bf16_t>;
  constexpr int NC = C / 16, DT = D / 16, SD = D / 32;
  const int lw = cfrag_lane_off(ldw);
#pragma unroll
  for (int s = 0; s < SD; ++s) {
    bf16x8_t fh[NVW];
#pragma unroll
    for (int v = 0; v < NVW; ++v) {
      f32x4_t col[DT];
#pragma unroll
      for (int t = 0; t < DT; ++t) col[t] = h[t][v];
      fh[v] = acc_frag<bf16_t, DT>(col, s);
    }
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const bf16x8_t fw = load_frag32_at(sWT + 32 * s * ldw + 16 * i, ldw, lw);
#pragma unroll
      for (int v = 0; v < NVW; ++v) p1[i][v] = M::mma(fw, fh[v], p1[i][v]);
    }
  }
}

// o += (q~ h) transposed: h^T (the h fragment as the A operand) times q~^T,
// so a lane ends up with four adjacent value columns of one chunk row. Needs
// only q~ and the incoming state, so it runs beside the WY substitution.
template <int C, int D, int NVW>
__device__ __forceinline__ void q_times_state(f32x4_t (&o)[C / 16][NVW], const bf16_t *sQ, int ldt,
                                              const f32x4_t (&h)[D / 16][NVW]) {
  using M = Mma<bf16_t>;
  constexpr int NC = C / 16, DT = D / 16, SD = D / 32;
  const int lane = tid_opaque() & 63;
  const int n16 = lane & 15, grp = lane >> 4;
  const bf16_t *qRow = sQ + n16 * ldt + 8 * grp;  // q~ in operand order: 8 per lane and 32-channel block
#pragma unroll
  for (int s = 0; s < SD; ++s) {
    bf16x8_t fh[NVW];
#pragma unroll
    for (int v = 0; v < NVW; ++v) {
      f32x4_t col[DT];
#pragma unroll
      for (int t = 0; t < DT; ++t) col[t] = h[t][v];
      fh[v] = acc_frag<bf16_t, DT>(col, s);
    }
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const bf16x8_t fq = *reinterpret_cast<const bf16x8_t *>(qRow + 16 * i * ldt + 32 * s);
#pragma unroll
      for (int v = 0; v < NVW; ++v) o[i][v] = M::mma(fh[v], fq, o[i][v]);
    }
  }
}
// o^T += v_new^T A_qk^T with A_qk bf16 row-major [C][ldh] (causal blocks only);
// o in the transposed layout of wq_times_state.
template <int C, int NVW>
__device__ __forceinline__ void causal_times_h(f32x4_t (&o)[C / 16][NVW], const bf16_t *sAqh, int ldh,
                                               const f32x4_t (&vn)[C / 16][NVW]) {
  using M = Mma<bf16_t>;
  constexpr int NC = C / 16, SC = C / 32;
  const int lane = tid_opaque() & 63;
  const int n16 = lane & 15, grp = lane >> 4;
  const bf16_t *aRow = sAqh + n16 * ldh + 4 * grp;
#pragma unroll
  for (int s = 0; s < SC; ++s) {
    bf16x8_t fv[NVW];
#pragma unroll
    for (int v = 0; v < NVW; ++v) {
      f32x4_t col[NC];
#pragma unroll
      for (int t = 0; t < NC; ++t) col[t] = vn[t][v];
      fv[v] = acc_frag<bf16_t, NC>(col, s);
    }
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      if (16 * (i + 1) <= s * 32) continue;
      const bf16x4_t a0 = *reinterpret_cast<const bf16x4_t *>(aRow + 16 * i * ldh + 32 * s);
      const bf16x4_t a1 = *reinterpret_cast<const bf16x4_t *>(aRow + 16 * i * ldh + 32 * s + 16);
      bf16x8_t fa;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        fa[e] = a0[e];
        fa[e + 4] = a1[e];
      }
#pragma unroll
      for (int v = 0; v < NVW; ++v) o[i][v] = M::mma(fv[v], fa, o[i][v]);
    }
  }
}

// o (transposed accumulators, see wq_times_state) straight to global rows of
// type bf16: lane writes o[16i + l%16][col0 + 16v + 4g .. + 3] as 8 bytes; rows
// >= L are not written.
template <int C, int NVW>
__device__ __forceinline__ void store_oT(bf16_t *g, int64_t ldg, int col0, int L, const f32x4_t (&o)[C / 16][NVW],
                                         int ncol) {
  const int lane = tid_opaque() & 63;
  const int n16 = lane & 15, grp = lane >> 4;
#pragma unroll
  for (int i = 0; i < C / 16; ++i) {
    const int r = 16 * i + n16;
    if (r < L) {
#pragma unroll
      for (int v = 0; v < NVW; ++v) {
        const int c = col0 + 16 * v + 4 * grp;  // four columns, all below ncol or none (ncol % 4 == 0)
        if (c < ncol) *reinterpret_cast<bf16x4_t *>(g + (int64_t)r * ldg + c) = to_bf16x4(o[i][v]);
      }
    }
  }
}

// h <- Diag(2^b_L) h + k~^T v_new with k~ row-major [C][ldt].
// v_new as the bf16 operand fragments of the state update, one per 32 chunk rows.
template <int C, int NVW>
__device__ __forceinline__ void vnew_frags(bf16x8_t (&fv)[C / 32][NVW], const f32x4_t (&vn)[C / 16][NVW]) {
  constexpr int NC = C / 16;
#pragma unroll
  for (int s = 0; s < C / 32; ++s)
#pragma unroll
    for (int v = 0; v < NVW; ++v) {
      f32x4_t col[NC];
#pragma unroll
      for (int t = 0; t < NC; ++t) col[t] = vn[t][v];
      fv[s][v] = acc_frag<bf16_t, NC>(col, s);
    }
}

template <int C, int D, int NVW>
__device__ __forceinline__ void state_update_kt(f32x4_t (&h)[D / 16][NVW], const bf16_t *sKt, int ldt,
                                                const bf16x8_t (&fv)[C / 32][NVW], const float *sDecay) {
  using M = Mma<bf16_t>;
  constexpr int DT = D / 16, SC = C / 32;
  const int lane = tid_opaque() & 63;
  const int grp = lane >> 4;
  const int lk = cfrag_lane_off(ldt);
  const float *dRow = sDecay + 4 * grp;
#pragma unroll
  for (int t = 0; t < DT; ++t) {
    const f32x4_t dec = *reinterpret_cast<const f32x4_t *>(dRow + 16 * t);
#pragma unroll
    for (int v = 0; v < NVW; ++v) h[t][v] = h[t][v] * dec;
  }
#pragma unroll
  for (int s = 0; s < SC; ++s) {
#pragma unroll
    for (int t = 0; t < DT; ++t) {
      const bf16x8_t fk = load_frag32_at(sKt + 32 * s * ldt + 16 * t, ldt, lk);
#pragma unroll
      for (int v = 0; v < NVW; ++v) h[t][v] = M::mma(fk, fv[s][v], h[t][v]);
    }
  }
}

}  // namespace kda

namespace kda {

// ---------------------------------------------------------------------------------------------
// (2) grams for the fused kernel. Each wave owns one row block i of both grams
// and a 1/HS share of the channels (HS = 1 or 2 waves per row block): it builds
// the row operands of block i once -- q, k scaled by 2^(b_r - m_i) (midpoint
// anchor, diagonal block) and by 2^(b_r - a_i) (first-row anchor a_i,
// off-diagonal blocks) -- and the column operands k_s 2^(m_i - b_s)
// (diagonal) and k_s 2^(a_i - b_s) (blocks j < i), so every exponent is a
// midpoint or paired non-positive offset ("FLA KDA Skill", section "Safe gate
// numerical note"). One exponential pair per element serves the diagonal; the
// off-diagonal row operands are those times the table 2^(m_i - a_i). Non-safe
// gates, unbounded, take the diagonal block per pair (section "Safe vs
// non-safe intra path").
// Only causal blocks are formed ("[examples] Read only the causal columns in
// chunk_fwd_A_diag_anchored", description). With HS = 2 each half stores its
// scaled, masked partial sums of one matrix, and after a barrier adds its own
// partial sums of the other and writes it; the half that completes A_kk then
// inverts the diagonal block T_ii from its own rows, with no further barrier.
// ---------------------------------------------------------------------------------------------
// Row block I of the grams over channels [c0, c0 + 32 NS), plus the chunk's
// other operand tiles for the same (token, channel) elements:
//   q~  = scale q 2^b      written over q (this wave alone reads these q), with
//                          the channels of each 32-block in operand order
//   k~  = k 2^(b_L - b)    written to sKt
//   X_w = beta k 2^b       returned in xw (written after the grams' barrier)
// For the safe gate these reuse the midpoint exponentials: scale 2^b =
// 2^(b - m_I) T1 and 2^(b_L - b) = 2^(m_I - b) T2 with the per-channel tables
// T1 = scale 2^m_I, T2 = 2^(b_L - m_I); other gates take them directly.
//
// XP = 1 (row block 0 of a 32-row chunk): the wave also forms the column operand
// of block pair (1, 0), k_s 2^(a_1 - b_s) for its own rows s, and stores it in
// operand order to sXc at step slot xs + s. XP = 2 (row block 1): the
// off-diagonal products are left out; the row operands come back in fo for
// the caller to multiply with sXc once the other wave has written it.
template <int I, int NC, int NS, bool SAFE, int XP = 0>
__device__ __forceinline__ void gram_row_partial(bf16_t *sQ, const bf16_t *sK, int ldt, const float *sB, int ldb,
                                                 int c0, const float *sT0, const float *sT1, const float *sT2,
                                                 const float *sBL, int D,
                                                 float scale, float beta_r, bf16_t *sKt, f32x4_t (&accQ)[NC],
                                                 f32x4_t (&accK)[NC], bf16x4_t (&xw)[NS][2],
                                                 bf16x8_t *sXc = nullptr, int xs = 0,
                                                 bf16x8_t (*fo)[2] = nullptr) {
  using M = Mma<bf16_t>;
  const int lane = tid_opaque() & 63;
  const int n16 = lane & 15, grp = lane >> 4;
  const int rr = 16 * I + n16;
  const float beta_over_scale = SAFE ? beta_r * __builtin_amdgcn_rcpf(scale) : 0.f;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int kb = c0 + 32 * s + 4 * grp;  // slots e < 4: channel kb + e; e >= 4: kb + 16 + (e - 4)
    f32x4_t br[2], ba[2], bm[2], t0[2], t1[2], t2[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      br[hh] = *reinterpret_cast<const f32x4_t *>(sB + rr * ldb + kb + 16 * hh);
      ba[hh] = *reinterpret_cast<const f32x4_t *>(sB + (16 * I) * ldb + kb + 16 * hh);
      if (SAFE) {
        bm[hh] = *reinterpret_cast<const f32x4_t *>(sB + (16 * I + 8) * ldb + kb + 16 * hh);
        if (I > 0) t0[hh] = *reinterpret_cast<const f32x4_t *>(sT0 + I * D + kb + 16 * hh);
        t1[hh] = *reinterpret_cast<const f32x4_t *>(sT1 + I * D + kb + 16 * hh);
        t2[hh] = *reinterpret_cast<const f32x4_t *>(sT2 + I * D + kb + 16 * hh);
      } else {
        t2[hh] = *reinterpret_cast<const f32x4_t *>(sBL + kb + 16 * hh);
      }
    }
    const bf16x4_t q0 = *reinterpret_cast<const bf16x4_t *>(sQ + rr * ldt + kb);
    const bf16x4_t q1 = *reinterpret_cast<const bf16x4_t *>(sQ + rr * ldt + kb + 16);
    const bf16x4_t k0 = *reinterpret_cast<const bf16x4_t *>(sK + rr * ldt + kb);
    const bf16x4_t k1 = *reinterpret_cast<const bf16x4_t *>(sK + rr * ldt + kb + 16);
    float vqd[8], vkd[8], vqo[8], vko[8], vkc[8], vqt[8], vxw[8], vkt[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int hh = e >> 2, ee = e & 3;
      const float qf = static_cast<float>(hh ? q1[ee] : q0[ee]);
      const float kf = static_cast<float>(hh ? k1[ee] : k0[ee]);
      if (SAFE) {
        // one pair of exponentials per element: 2^(b - m_I) for the diagonal
        // block's row operands, its inverse for the column operand; the
        // off-diagonal row operands 2^(b - a_I) and the other tiles are
        // products with per-channel tables
        const float d = br[hh][ee] - bm[hh][ee];
        const float ed = fast_exp2(d), ec = fast_exp2(-d);
        vqd[e] = qf * ed;
        vkd[e] = kf * ed;
        vkc[e] = kf * ec;
        if (I > 0) {
          vqo[e] = vqd[e] * t0[hh][ee];
          vko[e] = vkd[e] * t0[hh][ee];
        } else {
          vqo[e] = vko[e] = 0.f;
        }
        vqt[e] = vqd[e] * t1[hh][ee];                        // scale q 2^b
        vxw[e] = vkd[e] * (t1[hh][ee] * beta_over_scale);   // beta k 2^b
        vkt[e] = vkc[e] * t2[hh][ee];                        // k 2^(b_L - b)
      } else {
        const float E = fast_exp2(br[hh][ee]), El = fast_exp2(t2[hh][ee] - br[hh][ee]);
        vqt[e] = scale * qf * E;
        vxw[e] = beta_r * kf * E;
        vkt[e] = kf * El;
        if (I > 0) {
          const float eo = fast_exp2(br[hh][ee] - ba[hh][ee]);
          vqo[e] = qf * eo;
          vko[e] = kf * eo;
        } else {
          vqo[e] = vko[e] = 0.f;
        }
        vkc[e] = 0.f;
      }
    }
    bf16x8_t fqo, fko, fqd, fkd, fcd;
    if (I > 0) {
      fqo = pack_bf16x8(vqo);
      fko = pack_bf16x8(vko);
      if constexpr (XP == 2) {
        fo[s][0] = fqo;
        fo[s][1] = fko;
      }
    }
    if constexpr (XP == 1) {
      // k_s 2^(a_1 - b_s) for this lane's row s = n16 of block 0 (a_1 = b at row 16)
      float vx[8];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const f32x4_t a1 = *reinterpret_cast<const f32x4_t *>(sB + 16 * ldb + kb + 16 * hh);
#pragma unroll
        for (int ee = 0; ee < 4; ++ee) {
          const float kf = static_cast<float>(hh ? k1[ee] : k0[ee]);
          vx[4 * hh + ee] = kf * fast_exp2(a1[ee] - br[hh][ee]);
        }
      }
      sXc[(xs + s) * 64 + lane] = pack_bf16x8(vx);
    }
    if (SAFE) {
      fqd = pack_bf16x8(vqd);
      fkd = pack_bf16x8(vkd);
      fcd = pack_bf16x8(vkc);
    }
    bf16x4_t qt[2], kt[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      qt[hh] = pack_bf16x4(vqt[4 * hh], vqt[4 * hh + 1], vqt[4 * hh + 2], vqt[4 * hh + 3]);
      kt[hh] = pack_bf16x4(vkt[4 * hh], vkt[4 * hh + 1], vkt[4 * hh + 2], vkt[4 * hh + 3]);
      xw[s][hh] = pack_bf16x4(vxw[4 * hh], vxw[4 * hh + 1], vxw[4 * hh + 2], vxw[4 * hh + 3]);
    }
    // q~ goes back in the operand order of the 16x16x32 product (the lane's
    // channels kb..kb+3, kb+16..kb+19 side by side at c0 + 32 s + 8 grp), so
    // the product with h reads it as one 16-byte vector; the raw q of this
    // 32-channel block was read above by the same lanes
    *reinterpret_cast<bf16x8_t *>(sQ + rr * ldt + c0 + 32 * s + 8 * grp) =
        __builtin_shufflevector(qt[0], qt[1], 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) *reinterpret_cast<bf16x4_t *>(sKt + rr * ldt + kb + 16 * hh) = kt[hh];
    if (SAFE) {
      accQ[I] = M::mma(fcd, fqd, accQ[I]);
      accK[I] = M::mma(fcd, fkd, accK[I]);
    }
#pragma unroll
    for (int j = 0; j < (XP == 2 ? 0 : I); ++j) {
      const int cs = 16 * j + n16;
      const bf16x4_t c0v = *reinterpret_cast<const bf16x4_t *>(sK + cs * ldt + kb);
      const bf16x4_t c1v = *reinterpret_cast<const bf16x4_t *>(sK + cs * ldt + kb + 16);
      float vc[8];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const f32x4_t bc = *reinterpret_cast<const f32x4_t *>(sB + cs * ldb + kb + 16 * hh);
#pragma unroll
        for (int ee = 0; ee < 4; ++ee) {
          const float kf = static_cast<float>(hh ? c1v[ee] : c0v[ee]);
          vc[4 * hh + ee] = kf * fast_exp2(ba[hh][ee] - bc[ee]);
        }
      }
      const bf16x8_t fc = pack_bf16x8(vc);
      // column operand first: the accumulator holds the block transposed, so
      // lane (row n16, group g) gets A[16I + n16][16j + 4g .. 16j + 4g + 3]
      accQ[j] = M::mma(fc, fqo, accQ[j]);
      accK[j] = M::mma(fc, fko, accK[j]);
    }
  }
}

// Scale, beta and masks of row block I, then one 16-byte store per block:
// lane holds A[r = 16I + n16][16j + 4g .. 16j + 4g + 3]. doQ / doK select
// A_qk / A_kk. With add, the other channel half's partial sums (A_qk in sAqk,
// A_kk in sAkk) are added first. Final A_qk goes to sAqh as bf16, partial
// A_qk to sAqk; -A_kk (partial or final) always to sAkk.
// With four channel quarters, xq0/xq1 and xk0/xk1 hold two more partial sums of
// A_qk and -A_kk (same layout), added with the one in sAqk / sAkk.
template <int I, int NC>
__device__ __forceinline__ void gram_finish(f32x4_t (&accQ)[NC], f32x4_t (&accK)[NC], bool doQ, bool doK, bool add,
                                            bool final, int r, int L, float scale, float beta_r, float *sAkk,
                                            float *sAqk, int lda, bf16_t *sAqh, int ldh,
                                            const float *xq0 = nullptr, const float *xq1 = nullptr,
                                            const float *xk0 = nullptr, const float *xk1 = nullptr) {
  const int grp = (tid_opaque() & 63) >> 4;
  f32x4_t prevQ[I + 1], prevK[I + 1];
  if (add) {
#pragma unroll
    for (int j = 0; j <= I; ++j) {
      const int o = r * lda + 16 * j + 4 * grp;
      if (doQ) {
        prevQ[j] = *reinterpret_cast<const f32x4_t *>(sAqk + o);
        if (xq0) prevQ[j] = prevQ[j] + *reinterpret_cast<const f32x4_t *>(xq0 + o) + *reinterpret_cast<const f32x4_t *>(xq1 + o);
      }
      if (doK) {
        prevK[j] = *reinterpret_cast<const f32x4_t *>(sAkk + o);
        if (xk0) prevK[j] = prevK[j] + *reinterpret_cast<const f32x4_t *>(xk0 + o) + *reinterpret_cast<const f32x4_t *>(xk1 + o);
      }
    }
  }
  const bool row_ok = r < L;
#pragma unroll
  for (int j = 0; j <= I; ++j) {
    f32x4_t aq = accQ[j] * scale, ak = accK[j] * (-beta_r);
    if (j == I) {  // diagonal block: causal masks inside the block
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int sj = 16 * j + 4 * grp + e;
        aq[e] = (sj <= r) ? aq[e] : 0.f;
        ak[e] = (sj < r) ? ak[e] : 0.f;
      }
    }
    if (L < 16 * NC && !row_ok) {
      aq = zero4();
      ak = zero4();
    }
    if (doQ) {
      if (add) aq = aq + prevQ[j];
      if (final)
        *reinterpret_cast<bf16x4_t *>(sAqh + r * ldh + 16 * j + 4 * grp) = to_bf16x4(aq);
      else
        *reinterpret_cast<f32x4_t *>(sAqk + r * lda + 16 * j + 4 * grp) = aq;
    }
    if (doK) {
      if (add) ak = ak + prevK[j];
      *reinterpret_cast<f32x4_t *>(sAkk + r * lda + 16 * j + 4 * grp) = ak;
    }
  }
  // the product with A_qk reads 32 columns at a time: zero the block right of
  // an even diagonal block
  if constexpr ((I & 1) == 0 && I + 1 < NC) {
    if (doQ && final) *reinterpret_cast<bf16x4_t *>(sAqh + r * ldh + 16 * (I + 1) + 4 * grp) = to_bf16x4(zero4());
  }
}

// -A_kk comes out fp32 in sAkk (negated: the substitution subtracts it);
// A_qk comes out bf16 in sAqh (row stride ldh), with sAqk (fp32) holding the
// second channel half's partial sums meanwhile.
// Besides the grams, writes q~ over q, k~ into sKt and X_w = beta k 2^b into
// sXw (which may overlap sB: it is written after a barrier). With two waves per
// row block, the first of each pair calls idle() once its share is done; every
// wave calls pre() when its first-phase share is done, before the grams' barrier.
// The channel half of its row block that wave w takes in the grams. With 8
// waves and 4 row blocks, the halves alternate so that each SIMD (waves w and
// w + 4) holds one wave of either half.
// Channel shares per row block: 4 when there are at least four waves per row
// block (eight waves on 32-row chunks), else 2 or 1.
template <int NW, int NC>
constexpr int gram_shares() {
  return (NW / NC >= 4) ? 4 : ((NW / NC >= 2) ? 2 : 1);
}

template <int NW, int NC>
__device__ __forceinline__ int gram_half(int w) {
  if constexpr (NW == 8 && NC == 4) return (w & 1) ^ (w >> 2);
  else return w % gram_shares<NW, NC>();
}

// The waves that load the next chunk's q, k, v during the grams: with two
// shares one of each pair 2m, 2m + 1 (share 0, after the barrier); with four
// the waves of row block 0 (the first half), whose pass is the shorter, before
// the barrier.
template <int NW, int NC>
__device__ __forceinline__ bool gram_loader(int w) {
  if constexpr (gram_shares<NW, NC>() == 4) return w < NW / 2;
  else return gram_half<NW, NC>(w) == 0;
}

// With four shares (32-row chunks, eight waves), sPart holds four more [C][lda]
// fp32 partial-sum tiles (A_qk of shares 2 and 3, then -A_kk of shares 2 and 3);
// share 0 completes A_qk, share 1 -A_kk and its diagonal inverse. Row block 0's
// waves also form block pair (1, 0)'s column operand into sXc before a barrier;
// row block 1's waves, whose pass is the longer, multiply it after the barrier.
// Row block 0's waves also issue the next chunk's loads (idle) before it.
template <int NT, int C, int D, bool SAFE, typename Idle, typename Pre>
__device__ __forceinline__ void grams_fused(bf16_t *sQ, const bf16_t *sK, int ldt, const float *sB, int ldb,
                                            const float *sBeta, float scale, float *sAkk, float *sAqk, int lda,
                                            bf16_t *sAqh, int ldh, int L, const float *sT0, const float *sT1,
                                            const float *sT2, const float *sBL, bf16_t *sKt, bf16_t *sXw,
                                            bf16_t *sTd, int ldtd, float *sPart, bf16x8_t *sXc, Idle &&idle,
                                            Pre &&pre) {
  constexpr int NW = NT / 64, NC = C / 16;
  constexpr int HS = gram_shares<NW, NC>(), CW = D / HS, NS = CW / 32;
  static_assert(NW >= NC && CW % 32 == 0, "wave split of the grams");
  const int lane = tid_opaque() & 63, w = wave_id();
  const int n16 = lane & 15, grp = lane >> 4;
  // row block per wave; with 8 waves and 4 row blocks, blocks 0 and 3 (and 1
  // and 2) share a SIMD (waves w and w + 4), which evens out the per-SIMD work
  const int i = (NW == 8 && NC == 4) ? ((w < 4) ? (w >> 1) : (3 - ((w - 4) >> 1))) : w / HS;
  const int hsel = gram_half<NW, NC>(w);
  const bool active = i < NC;
  const int c0 = hsel * CW;
  const int r = 16 * i + n16;
  const float beta_r = active ? sBeta[r] : 0.f;
  bf16x4_t xw[NS][2];
  bf16x8_t fo[NS][2];  // row block 1's off-diagonal row operands (four shares, 32-row chunks)

  f32x4_t accQ[NC], accK[NC];
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    accQ[j] = zero4();
    accK[j] = zero4();
  }
  // the row blocks with more causal blocks have the longer dependency chains:
  // they take the issue slots first, the short ones fill the gaps
  if (NW == 8 && NC == 4) {
    if (i == 3) __builtin_amdgcn_s_setprio(3);
    else if (i == 2) __builtin_amdgcn_s_setprio(2);
  }
  if (active) {
    if constexpr (!SAFE) {
      // token-parallel diagonal block over this wave's channels (before q is
      // overwritten), in the transposed layout: lane owns row r = 16i + n16 and
      // columns 16i + 4*grp + e
      // columns, four channels per step (vector LDS reads; the sums keep the
      // channel order)
      for (int kk = c0; kk < c0 + CW; kk += 4) {
        const bf16x4_t q4 = *reinterpret_cast<const bf16x4_t *>(sQ + r * ldt + kk);
        const bf16x4_t k4 = *reinterpret_cast<const bf16x4_t *>(sK + r * ldt + kk);
        const f32x4_t b4 = *reinterpret_cast<const f32x4_t *>(sB + r * ldb + kk);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int sc = 16 * i + 4 * grp + e;
          const f32x4_t bc = *reinterpret_cast<const f32x4_t *>(sB + sc * ldb + kk);
          const bf16x4_t kc = *reinterpret_cast<const bf16x4_t *>(sK + sc * ldt + kk);
          const bool on = r >= sc;
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const float f = on ? fast_exp2(b4[u] - bc[u]) : 0.f;
            const float kf = static_cast<float>(kc[u]) * f;
            accQ[i][e] += static_cast<float>(q4[u]) * kf;
            accK[i][e] += static_cast<float>(k4[u]) * kf;
          }
        }
      }
    }
#define KDA_GRAM_ROW(II)                                                                                     \
  gram_row_partial<II, NC, NS, SAFE>(sQ, sK, ldt, sB, ldb, c0, sT0, sT1, sT2, sBL, D, scale, beta_r, sKt, accQ, accK, \
                                     xw)
    if constexpr (HS == 4) {
      // row block 0 forms block pair (1, 0)'s column operand for block 1's
      // waves, whose own pass is the longer; they multiply it after the barrier below
      if (i == 0) {
        gram_row_partial<0, NC, NS, SAFE, 1>(sQ, sK, ldt, sB, ldb, c0, sT0, sT1, sT2, sBL, D, scale, beta_r, sKt, accQ,
                                             accK, xw, sXc, hsel * NS);
        // this block's pass is the shorter: its waves issue the next chunk's loads
        idle();
      } else
        gram_row_partial<1, NC, NS, SAFE, 2>(sQ, sK, ldt, sB, ldb, c0, sT0, sT1, sT2, sBL, D, scale, beta_r, sKt, accQ,
                                             accK, xw, nullptr, 0, fo);
    } else
    switch (i) {
      case 0: KDA_GRAM_ROW(0); break;
      case 1: KDA_GRAM_ROW(1); break;
      case 2:
        if constexpr (NC > 2) KDA_GRAM_ROW(2);
        break;
      case 3:
        if constexpr (NC > 3) KDA_GRAM_ROW(3);
        break;
    }
#undef KDA_GRAM_ROW
  }
  static_assert(HS != 4 || NC == 2, "four shares on 32-row chunks only");
  if constexpr (HS == 4) {
    __syncthreads();  // block pair (1, 0)'s column operand is in sXc
    if (i == 1) {
      using M = Mma<bf16_t>;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const bf16x8_t fc = sXc[(hsel * NS + s) * 64 + lane];
        accQ[0] = M::mma(fc, fo[s][0], accQ[0]);
        accK[0] = M::mma(fc, fo[s][1], accK[0]);
      }
    }
  }
  // X_w over b once every wave is past its reads of b
  auto store_xw = [&]() {
    if (active) {
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
          *reinterpret_cast<bf16x4_t *>(sXw + r * ldt + c0 + 32 * s + 4 * grp + 16 * hh) = xw[s][hh];
    }
  };
  auto finish_at = [&](bool doQ, bool doK, bool add, bool final, float *dK, float *dQ, const float *xq0,
                       const float *xq1, const float *xk0, const float *xk1) {
    switch (i) {
      case 0: gram_finish<0, NC>(accQ, accK, doQ, doK, add, final, r, L, scale, beta_r, dK, dQ, lda, sAqh, ldh, xq0, xq1, xk0, xk1); break;
      case 1: gram_finish<1, NC>(accQ, accK, doQ, doK, add, final, r, L, scale, beta_r, dK, dQ, lda, sAqh, ldh, xq0, xq1, xk0, xk1); break;
      case 2:
        if constexpr (NC > 2) gram_finish<2, NC>(accQ, accK, doQ, doK, add, final, r, L, scale, beta_r, dK, dQ, lda, sAqh, ldh, xq0, xq1, xk0, xk1);
        break;
      case 3:
        if constexpr (NC > 3) gram_finish<3, NC>(accQ, accK, doQ, doK, add, final, r, L, scale, beta_r, dK, dQ, lda, sAqh, ldh, xq0, xq1, xk0, xk1);
        break;
    }
  };
  auto finish = [&](bool doQ, bool doK, bool add, bool final) {
    finish_at(doQ, doK, add, final, sAkk, sAqk, nullptr, nullptr, nullptr, nullptr);
  };
  if (NW == 8 && NC == 4) __builtin_amdgcn_s_setprio(0);
  if constexpr (HS == 4) {
    // each share stores the partial sums of the matrices it does not complete:
    // share 0 -A_kk (to sAkk), share 1 A_qk (to sAqk), shares 2 and 3 both (to sPart)
    const int tile = C * lda;
    if (active) {
      if (hsel == 0) finish(false, true, false, false);
      else if (hsel == 1) finish(true, false, false, false);
      else finish_at(true, true, false, false, sPart + (hsel == 2 ? 2 : 3) * tile, sPart + (hsel == 2 ? 0 : 1) * tile,
                     nullptr, nullptr, nullptr, nullptr);
    }
    pre();
    __syncthreads();
    store_xw();
    if (hsel == 0) {
      if (active) finish_at(true, false, true, true, sAkk, sAqk, sPart, sPart + tile, nullptr, nullptr);
    } else if (hsel == 1) {
      if (active) {
        __builtin_amdgcn_s_setprio(2);
        finish_at(false, true, true, true, sAkk, sAqk, nullptr, nullptr, sPart + 2 * tile, sPart + 3 * tile);
        lds_wave_order();
        diag_inverse_block(sAkk, lda, sTd, ldtd, i);
        __builtin_amdgcn_s_setprio(0);
      }
    }
  } else if constexpr (HS == 2) {
    // the two halves split the merge: half 1 finishes A_qk's partner and half 0
    // A_kk's, so each wave stores one partial and completes the other matrix
    if (active) {
      if (hsel == 1) finish(true, false, false, false);
      else finish(false, true, false, false);
    }
    pre();  // each wave as it finishes its share: the waves reach this point at different times
    __syncthreads();
    store_xw();
    if (hsel == 0) {
      if (active) finish(true, false, true, true);
      idle();  // while the other half inverts the diagonal blocks
    } else if (active) {
      // the inverse is a chain of cross-lane steps: it takes the issue slots first
      __builtin_amdgcn_s_setprio(2);
      finish(false, true, true, true);
      lds_wave_order();  // this wave's A_kk rows are read back across lanes
      diag_inverse_block(sAkk, lda, sTd, ldtd, i);
      __builtin_amdgcn_s_setprio(0);
    }
  } else {
    if (active) {
      finish(true, true, false, true);
      lds_wave_order();
      diag_inverse_block(sAkk, lda, sTd, ldtd, i);
    }
    pre();
    __syncthreads();
    store_xw();
  }
}

}  // namespace kda
