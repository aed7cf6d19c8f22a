// Building blocks of the fused chunk kernel (bf16 operands, gfx950).
//
// Beyond the shared steps in chunk_tiles.h, the fused kernel
//  - solves (I + A_kk) [w | u] = [beta k 2^b | beta v] by blocked forward
//    substitution per 16-column tile, so no wave waits for another's columns
//    and only the four 16x16 diagonal inverses are formed explicitly;
//  - keeps w^T and k~ = k 2^(b_L - b) in LDS in the layouts their producers
//    write with wide stores, and reads the transposed MFMA operands with
//    ds_read_b64_tr_b16.
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

// Lane l of M (row-major bf16, row stride ld elements; ld % 4 == 0, n0 % 4 == 0):
// {M[k0 + 4g + e][n0 + l%16]}, e = 0..3, g = (l%64)/16.
__device__ __forceinline__ bf16x4_t load_cfrag(const bf16_t *M, int ld, int k0, int n0) {
  const int lane = tid_opaque() & 63;
  const int g = lane >> 4, s = lane & 15;
  const bf16_t *p = M + (k0 + 4 * g + (s >> 2)) * ld + n0 + 4 * (s & 3);
  const i16x4_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (i16x4_t __attribute__((address_space(3))) *)(p));
  return __builtin_bit_cast(bf16x4_t, r);
}

__device__ __forceinline__ f32x4_t mma16(const bf16x4_t &a, const bf16x4_t &b, const f32x4_t &c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4_t, a), __builtin_bit_cast(i16x4_t, b), c,
                                                    0, 0, 0);
}

__device__ __forceinline__ bf16x4_t to_bf16x4(const f32x4_t &x) {
  bf16x4_t r;
#pragma unroll
  for (int e = 0; e < 4; ++e) r[e] = static_cast<bf16_t>(x[e]);
  return r;
}

__device__ __forceinline__ f32x4_t to_f32x4(const bf16x4_t &x) {
  f32x4_t r;
#pragma unroll
  for (int e = 0; e < 4; ++e) r[e] = static_cast<float>(x[e]);
  return r;
}

// Two C-layout fragments (contraction rows k0.. and k0+16..) as the 8-slot
// operand of a 16x16x32 product under the kidx map of Mma<bf16_t>.
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

// ---------------------------------------------------------------------------------------------
// (3) the diagonal blocks T_ii = (I + A_ii)^-1, i < C/16, by forward
// substitution in FP32 on one wave (lane = block i, column c), stored as
// bf16 T_ii[r][c] with row stride ldt.
// ---------------------------------------------------------------------------------------------
template <int C>
__device__ __forceinline__ void diag_inverse(const float *sAkk, int lda, bf16_t *sTd, int ldt) {
  constexpr int NC = C / 16;
  const int lane = tid_opaque() & 63;
  if (lane >= 16 * NC) return;
  const int i = lane >> 4, c = lane & 15;
  const float *A = sAkk + 16 * i * lda + 16 * i;
  float x[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) x[r] = (r == c) ? 1.f : 0.f;
#pragma unroll
  for (int s = 0; s < 16; ++s) {
#pragma unroll
    for (int r = s + 1; r < 16; ++r) x[r] -= A[r * lda + s] * x[s];
  }
  bf16_t *T = sTd + i * 16 * ldt;
#pragma unroll
  for (int r = 0; r < 16; ++r) T[r * ldt + c] = static_cast<bf16_t>(x[r]);
}

// ---------------------------------------------------------------------------------------------
// Elementwise operand pass over the chunk, 8 channels per item, on threads
// [0, nthr): with E = 2^b,
//   q~  = scale q E            in place of q
//   X_w = beta k E             in place of k
//   k~  = k 2^(b_L - b)        into sKt
// Rows past the chunk's end hold q = k = 0 and carry the last valid b, so
// they give zeros.
// ---------------------------------------------------------------------------------------------
template <int C, int D>
__device__ __forceinline__ void operand_pass(bf16_t *sQ, bf16_t *sK, bf16_t *sKt, int ldt, const float *sB, int ldb,
                                             const float *sBL, const float *sBeta, float scale, int nthr) {
  constexpr int G = C * D / 8, GPR = D / 8;
  for (int g = tid_opaque(); g < G; g += nthr) {
    const int r = g / GPR, c = (g % GPR) * 8;
    const bf16x8_t q = *reinterpret_cast<const bf16x8_t *>(sQ + r * ldt + c);
    const bf16x8_t k = *reinterpret_cast<const bf16x8_t *>(sK + r * ldt + c);
    const f32x4_t b0 = *reinterpret_cast<const f32x4_t *>(sB + r * ldb + c);
    const f32x4_t b1 = *reinterpret_cast<const f32x4_t *>(sB + r * ldb + c + 4);
    const f32x4_t l0 = *reinterpret_cast<const f32x4_t *>(sBL + c);
    const f32x4_t l1 = *reinterpret_cast<const f32x4_t *>(sBL + c + 4);
    const float beta = sBeta[r];
    bf16x8_t qt, xw, kt;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float b = e < 4 ? b0[e] : b1[e - 4];
      const float bl = e < 4 ? l0[e] : l1[e - 4];
      const float E = fast_exp2(b);
      const float kf = static_cast<float>(k[e]);
      qt[e] = static_cast<bf16_t>(scale * static_cast<float>(q[e]) * E);
      xw[e] = static_cast<bf16_t>(beta * kf * E);
      kt[e] = static_cast<bf16_t>(kf * fast_exp2(bl - b));
    }
    *reinterpret_cast<bf16x8_t *>(sQ + r * ldt + c) = qt;
    *reinterpret_cast<bf16x8_t *>(sK + r * ldt + c) = xw;
    *reinterpret_cast<bf16x8_t *>(sKt + r * ldt + c) = kt;
  }
}

// ---------------------------------------------------------------------------------------------
// (4) One 16-column tile ct of W = (I + A_kk)^-1 X by blocked forward
// substitution: R_i = X_i - sum_{j<i} A_ij W_j, W_i = T_ii R_i. X is a
// row-major bf16 tile; rows are scaled by rowscale[r] when given. W comes
// back as C-layout accumulators, one per row block.
// ---------------------------------------------------------------------------------------------
template <int C>
__device__ __forceinline__ void wy_subst(const bf16_t *sX, int ldx, int ct, const float *rowscale, const float *sAkk,
                                         int lda, const bf16_t *sTd, int ldt, f32x4_t (&W)[C / 16]) {
  constexpr int NC = C / 16;
  const int lane = tid_opaque() & 63;
  const int n16 = lane & 15, grp = lane >> 4;
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    f32x4_t R = to_f32x4(load_cfrag(sX, ldx, 16 * i, 16 * ct));
    if (rowscale) {
      const f32x4_t rs = *reinterpret_cast<const f32x4_t *>(rowscale + 16 * i + 4 * grp);
      R = R * rs;
    }
#pragma unroll
    for (int j = 0; j < i; ++j) {
      const f32x4_t a = *reinterpret_cast<const f32x4_t *>(sAkk + (16 * i + n16) * lda + 16 * j + 4 * grp);
      R = mma16(to_bf16x4(-a), to_bf16x4(W[j]), R);
    }
    const bf16x4_t t = *reinterpret_cast<const bf16x4_t *>(sTd + (16 * i + n16) * ldt + 4 * grp);
    W[i] = mma16(t, to_bf16x4(R), zero4());
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
// p1 = w h with w read from w^T, o = q~ h with q~ row-major.
// ---------------------------------------------------------------------------------------------
template <int C, int D, int NVW>
__device__ __forceinline__ void wq_times_state(f32x4_t (&p1)[C / 16][NVW], f32x4_t (&o)[C / 16][NVW],
                                               const bf16_t *sWT, int ldw, const bf16_t *sQ, int ldt,
                                               const f32x4_t (&h)[D / 16][NVW]) {
  using M = Mma<bf16_t>;
  constexpr int NC = C / 16, DT = D / 16, SD = D / 32;
  const int lane = tid_opaque() & 63;
  const int n16 = lane & 15, grp = lane >> 4;
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
      const bf16x8_t fw = load_frag32(sWT, ldw, 32 * s, 16 * i);
      bf16x8_t fq;
      const bf16x4_t q0 = *reinterpret_cast<const bf16x4_t *>(sQ + (16 * i + n16) * ldt + 32 * s + 4 * grp);
      const bf16x4_t q1 = *reinterpret_cast<const bf16x4_t *>(sQ + (16 * i + n16) * ldt + 32 * s + 16 + 4 * grp);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        fq[e] = q0[e];
        fq[e + 4] = q1[e];
      }
#pragma unroll
      for (int v = 0; v < NVW; ++v) {
        p1[i][v] = M::mma(fw, fh[v], p1[i][v]);
        o[i][v] = M::mma(fq, fh[v], o[i][v]);
      }
    }
  }
}

// h <- Diag(2^b_L) h + k~^T v_new with k~ row-major [C][ldt].
template <int C, int D, int NVW>
__device__ __forceinline__ void state_update_kt(f32x4_t (&h)[D / 16][NVW], const bf16_t *sKt, int ldt,
                                                const f32x4_t (&vn)[C / 16][NVW], const float *sDecay) {
  using M = Mma<bf16_t>;
  constexpr int NC = C / 16, DT = D / 16, SC = C / 32;
  const int lane = tid_opaque() & 63;
  const int grp = lane >> 4;
#pragma unroll
  for (int t = 0; t < DT; ++t) {
    const f32x4_t dec = *reinterpret_cast<const f32x4_t *>(sDecay + 16 * t + 4 * grp);
#pragma unroll
    for (int v = 0; v < NVW; ++v) h[t][v] = h[t][v] * dec;
  }
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
    for (int t = 0; t < DT; ++t) {
      const bf16x8_t fk = load_frag32(sKt, ldt, 32 * s, 16 * t);
#pragma unroll
      for (int v = 0; v < NVW; ++v) h[t][v] = M::mma(fk, fv[v], h[t][v]);
    }
  }
}

}  // namespace kda
