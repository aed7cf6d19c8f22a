// The pipelined fused schedule of the chunked KDA forward (bf16, C = 64,
// D = 128, safe gate): one persistent workgroup per (sequence, head), whose
// eight waves take two roles and run two chunks at once.
//
//   key waves 0..3    steps (1)-(4) of chunk c: the gate activation and its
//                     chunk-local cumsum, the row operands and products of the
//                     grams (wave i owns row block i), the diagonal inverses
//                     and the w tiles of the substitution
//   state waves 4..7  steps (5)-(6) of chunk c-1 (w h, v_new, o, the state
//                     update), the column operands of the grams of chunk c
//                     (wave 4+i: block i), q~ h and the u tiles of the
//                     substitution; wave 4+s owns value columns 32s..32s+31 of
//                     the FP32 state, which lives in its accumulators for the
//                     whole sequence
//
// Each chunk takes four periods separated by workgroup barriers; in each, the
// two roles work on different data, so the VALU-heavy key side and the
// MFMA-heavy state side share every SIMD (one wave of each per SIMD):
//
//   P1  key: gate activation, cumsum, anchors   state: w h, v_new, o of c-1
//   P2  key: row operands, q~, k 2^b            state: column operands, k~
//   P3  key: gram products, A, T_ii             state: h <- 2^b_L h + k~^T v_new
//                                                      (c-1), then q~ h of c
//   P4  key: w tiles of the substitution        state: u tiles of the substitution
//
// Each role runs its own loop with the same barriers, so the register
// allocator sees their lifetimes apart. LDS regions are reused by lifetime
// (about 154 KB).
//
// Numerics ("FLA KDA Skill", section "Safe gate numerical note"; "[examples]
// Read only the causal columns in chunk_fwd_A_diag_anchored", description):
// only the ten causal 16x16 blocks of each gram are formed; a diagonal block
// pairs 2^(b_r - m_i) with 2^(m_i - b_s) (midpoint anchor m_i = b at row
// 16i + 8); an off-diagonal block (i, j < i) pairs 2^(b_r - a_i) with
// 2^(a_i - b_s) (first-row anchor a_i), both exponents non-positive. The gate
// step leaves d = b - m_i per element, so one exponential per element serves
// each side: the off-diagonal operands are the diagonal ones times per-channel
// tables 2^(m_i - a_i) (rows) and 2^(a_i - m_j) (columns, formed by the wave
// of block j), and q 2^b, k 2^b, k 2^(b_L - b) are the same products with
// 2^m_i and 2^(b_L - m_i). The output scale and the q row norms are applied to
// o at the store, beta to the right-hand sides of the substitution.
#include "chunk_fused_tiles.h"
#include "kda_launch.h"

namespace kda {
namespace {

typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef unsigned u32x2v_t __attribute__((ext_vector_type(2)));

// Raw buffer resources: loads at offsets past `bytes` return zeros and
// stores there are dropped, so rows past a partial chunk need no masks
// (the row is always part of the checked vector offset).
__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ float bload_f32(rsrc_t r, uint32_t voff) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, 0, 0));
}
__device__ __forceinline__ u32x4_t bload_b128(rsrc_t r, uint32_t voff) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, 0, 0));
}
__device__ __forceinline__ void bstore_b64(rsrc_t r, uint32_t voff, bf16x4_t x) {
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2v_t, x), r, (int)voff, 0, 0);
}

constexpr int kC = 64, kD = 128, kNT = 512, kNC = 4;
constexpr int kLDB = kD + 4;   // fp32 d [C][LDB]
constexpr int kLDT = kD + 8;   // bf16 [C][LDT] tiles
constexpr int kLDA = kC + 8;   // bf16 -A_kk [C][LDA]
constexpr int kLDW = kC + 8;   // bf16 w^T [D][LDW]
constexpr int kLDTD = 16 + 8;  // bf16 diagonal inverses [C][LDTD]
constexpr int kLDF = kLDT / 2; // fp32 diagonal blocks of -A_kk, row stride (floats) of the Cd rows they sit in

// Index of the column-operand table of block pair (row block ip, column block i), ip > i.
__host__ __device__ constexpr int pair_index(int ip, int i) { return i == 0 ? ip - 1 : (i == 1 ? ip + 1 : 5); }

struct PipeSmem {
  // R1, live P1-P2: d = b - m_i and the anchor tables
  static constexpr size_t d = 0;                         // fp32 [C][LDB]
  static constexpr size_t t1 = d + 4 * kC * kLDB;        // fp32 [4][D]  2^m_i
  static constexpr size_t t2 = t1 + 4 * kNC * kD;        // 2^(b_L - m_i)
  static constexpr size_t t0 = t2 + 4 * kNC * kD;        // 2^(m_i - a_i)
  static constexpr size_t te = t0 + 4 * kNC * kD;        // fp32 [6][D]  2^(a_ip - m_i)
  static constexpr size_t r1_end = te + 4 * 6 * kD;
  //   reused P3-P4: -A_kk, T_ii, v
  static constexpr size_t akk = 0;                       // bf16 [C][LDA]
  static constexpr size_t td = akk + 2 * kC * kLDA;      // bf16 [C][LDTD]
  static constexpr size_t v = td + 2 * kC * kLDTD;       // bf16 [C][LDT]
  static_assert(v + 2 * kC * kLDT <= r1_end, "R1 reuse");
  // R2, live P2-P3: the column operands of the diagonal blocks, the exported
  // column operands of the off-diagonal blocks, q~ (operand order)
  static constexpr size_t r2 = r1_end;
  static constexpr size_t cd = r2;                       // bf16 [C][LDT]
  static constexpr size_t ex = cd + 2 * kC * kLDT;       // bf16 [6][16][LDT]
  static constexpr size_t qt = ex + 2 * 6 * 16 * kLDT;   // bf16 [C][LDT]
  static constexpr size_t r2_end = qt + 2 * kC * kLDT;
  //   each Cd row r, once the wave of its block has read it (P3), holds A_qk row r
  //   (bf16, first 64 elements; read in P1') and the fp32 row of the diagonal
  //   block of -A_kk (16 floats at element 64)
  static constexpr size_t aqk = cd;                      // bf16 [C][LDT]
  static constexpr size_t dsc = cd + 2 * kC;             // fp32, row stride LDF
  //   the export region holds w^T from P4 to P1'
  static constexpr size_t wt = ex;                       // bf16 [D][LDW]
  static_assert(2 * kD * kLDW <= 2 * 6 * 16 * kLDT, "w^T in the export region");
  // R3, live P2-P4: k 2^b (beta joins in the substitution)
  static constexpr size_t xw = r2_end;                   // bf16 [C][LDT]
  // R4: k~ = k 2^(b_L - b) by chunk parity (written P2, read P3 of the next chunk)
  static constexpr size_t kt = xw + 2 * kC * kLDT;       // bf16 [2][C][LDT]
  static constexpr size_t lam = kt + 2 * 2 * kC * kLDT;  // fp32 [2][D]  2^b_L by chunk parity
  static constexpr size_t beta = lam + 4 * 2 * kD;       // fp32 [C]
  static constexpr size_t qn = beta + 4 * kC;            // fp32 [C]  output row scales
  static constexpr size_t total = qn + 4 * kC;
  static_assert(total <= 160 * 1024, "LDS");
  static_assert(d % 16 == 0 && t1 % 16 == 0 && t2 % 16 == 0 && t0 % 16 == 0 && te % 16 == 0 && akk % 16 == 0 &&
                    td % 16 == 0 && v % 16 == 0 && cd % 16 == 0 && ex % 16 == 0 && qt % 16 == 0 &&
                    dsc % 16 == 0 && wt % 16 == 0 && xw % 16 == 0 && kt % 16 == 0 && lam % 16 == 0 &&
                    beta % 16 == 0 && qn % 16 == 0 && (kLDT * 2) % 16 == 0,
                "16-byte aligned buffers");
};

__device__ __forceinline__ bf16x8_t bf8(const float (&x)[8]) { return pack_bf16x8(x); }

// (4) Two 16-column tiles ca, cb of W = (I + A_kk)^-1 Diag(beta) X by blocked
// forward substitution: R_i = beta_i X_i - sum_{j<i} A_ij W_j, W_i = T_ii R_i.
// X row-major bf16 [C][ldx]; sA holds -A_kk (bf16, strictly lower blocks);
// sTd the diagonal inverses. W comes back as C-layout tiles per row block.
__device__ __forceinline__ void subst_pair(const bf16_t *sX, int ca, int cb, int ldx, const float *sBeta,
                                           const bf16_t *sA, int lda, const bf16_t *sTd, int ldt,
                                           f32x4_t (&Wa)[kNC], f32x4_t (&Wb)[kNC]) {
  const int lane = tid_opaque() & 63;
  const int n16 = lane & 15, grp = lane >> 4;
  const int lx = cfrag_lane_off(ldx);
  const bf16_t *aRow = sA + n16 * lda + 4 * grp;
  const bf16_t *tRow = sTd + n16 * ldt + 4 * grp;
  const float *bRow = sBeta + 4 * grp;
  bf16x4_t wa[kNC], wb[kNC];
#pragma unroll
  for (int i = 0; i < kNC; ++i) {
    const f32x4_t bet = *reinterpret_cast<const f32x4_t *>(bRow + 16 * i);
    f32x4_t Ra = to_f32x4(load_cfrag_at(sX + 16 * i * ldx + 16 * ca, lx)) * bet;
    f32x4_t Rb = to_f32x4(load_cfrag_at(sX + 16 * i * ldx + 16 * cb, lx)) * bet;
#pragma unroll
    for (int j = 0; j < i; ++j) {
      const bf16x4_t a = *reinterpret_cast<const bf16x4_t *>(aRow + 16 * i * lda + 16 * j);
      Ra = mma16(a, wa[j], Ra);
      Rb = mma16(a, wb[j], Rb);
    }
    const bf16x4_t t = *reinterpret_cast<const bf16x4_t *>(tRow + 16 * i * ldt);
    Wa[i] = mma16(t, to_bf16x4(Ra), zero4());
    Wb[i] = mma16(t, to_bf16x4(Rb), zero4());
    wa[i] = to_bf16x4(Wa[i]);
    wb[i] = to_bf16x4(Wb[i]);
  }
}

// ---------------------------------------------------------------------------------------------
// Key side, P1: the gate of this thread's two channels (ch0, ch0 + 1) over row
// block blk = lane / 16 (rows 16 blk .. 16 blk + 15): activation (log2 units),
// the cumsum over the chunk (sequential over the 16 rows, then an exclusive
// scan over the four blocks of the same channels, which sit in the same wave),
// d = b - m_blk to LDS, and the anchor tables of block blk.
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ void key_gate(const f32x2_t (&xr)[16], const float (&dtc)[2], float c1, float c2, int L,
                                         int cpar, int w, char *smem) {
  using S = PipeSmem;
  const int lane = tid_opaque() & 63;
  const int pr = lane & 15, blk = lane >> 4, ch0 = 2 * (16 * w + pr);
  // the sigmoids' cumsum over this block's rows; b = c2 * (the chunk's cumsum),
  // c2 = lower_bound * log2(e). Rows past the slot end do not exist: the masked
  // copy runs only for a partial chunk (a uniform branch).
  float P[16][2];
  if (L == kC) {
#pragma unroll
    for (int r = 0; r < 16; ++r)
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const float sg = fast_rcp(1.0f + fast_exp2(fmaf(xr[r][e], c1, dtc[e])));
        P[r][e] = (r == 0) ? sg : P[r - 1][e] + sg;
      }
  } else {
#pragma unroll
    for (int r = 0; r < 16; ++r)
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        float sg = fast_rcp(1.0f + fast_exp2(fmaf(xr[r][e], c1, dtc[e])));
        sg = (16 * blk + r < L) ? sg : 0.f;
        P[r][e] = (r == 0) ? sg : P[r - 1][e] + sg;
      }
  }
  // inclusive scan of the block totals over blk, the exclusive offset, b_L
  float inc[2], off[2], bL[2], m[2], a[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    inc[e] = P[15][e];
    float y = __shfl_up(inc[e], 16);
    if (blk >= 1) inc[e] += y;
    y = __shfl_up(inc[e], 32);
    if (blk >= 2) inc[e] += y;
    y = __shfl_up(inc[e], 16);
    off[e] = (blk >= 1) ? y : 0.f;
    bL[e] = c2 * __shfl(inc[e], pr + 48);
    a[e] = c2 * (P[0][e] + off[e]);  // b at the block's first row
    m[e] = c2 * (P[8][e] + off[e]);  // b at its midpoint row
  }
  // d = b - m = c2 * P + (c2 * off - m): one fma per element
  float *dRow = reinterpret_cast<float *>(smem + S::d) + (16 * blk) * kLDB + ch0;
  float k0[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) k0[e] = fmaf(c2, off[e], -m[e]);
#pragma unroll
  for (int r = 0; r < 16; ++r)
    *reinterpret_cast<f32x2_t *>(dRow + r * kLDB) = f32x2_t{fmaf(c2, P[r][0], k0[0]), fmaf(c2, P[r][1], k0[1])};
  // tables of block blk: 2^m, 2^(b_L - m), 2^(m - a); and its column tables for
  // every later row block ip, 2^(a_ip - m) (a_ip from the lanes of block ip)
  auto put = [&](size_t base, int row, float x0, float x1) {
    *reinterpret_cast<f32x2_t *>(reinterpret_cast<float *>(smem + base) + row * kD + ch0) = f32x2_t{x0, x1};
  };
  put(S::t1, blk, fast_exp2(m[0]), fast_exp2(m[1]));
  put(S::t2, blk, fast_exp2(bL[0] - m[0]), fast_exp2(bL[1] - m[1]));
  put(S::t0, blk, fast_exp2(m[0] - a[0]), fast_exp2(m[1] - a[1]));
#pragma unroll
  for (int ip = 1; ip < kNC; ++ip) {
    const float ap0 = __shfl(a[0], pr + 16 * ip), ap1 = __shfl(a[1], pr + 16 * ip);
    if (ip > blk) put(S::te, pair_index(ip, blk), fast_exp2(ap0 - m[0]), fast_exp2(ap1 - m[1]));
  }
  if (blk == kNC - 1) put(S::lam, cpar, fast_exp2(bL[0]), fast_exp2(bL[1]));
}

// ---------------------------------------------------------------------------------------------
// Key side, P2: the row operands of block I over all D channels, from q, k
// (registers, loaded from HBM in operand layout: lane (row n16, group g) holds
// channels 32s + 8g .. 32s + 8g + 7 of slice s) and d = b - m_I:
//   diagonal  Qd = q 2^d, Kd = k 2^d
//   off-diag  Qo = Qd 2^(m_I - a_I), Ko = Kd 2^(m_I - a_I)      (I > 0)
//   q~ = Qd 2^m_I to LDS in the operand order of the state side's q~ h,
//   k 2^b = Kd 2^m_I to LDS (row-major), and the raw q's row sums of squares.
// ---------------------------------------------------------------------------------------------
template <int I, bool QN>
__device__ __forceinline__ void key_row_operands(const u32x4_t (&qr)[4], const u32x4_t (&kr)[4], char *smem,
                                                 bf16x8_t (&fQd)[4], bf16x8_t (&fKd)[4], bf16x8_t (&fQo)[4],
                                                 bf16x8_t (&fKo)[4], float &ss) {
  using S = PipeSmem;
  const int lane = tid_opaque() & 63;
  const int n16 = lane & 15, grp = lane >> 4;
  const int r = 16 * I + n16;
  const float *dRow = reinterpret_cast<const float *>(smem + S::d) + r * kLDB + 8 * grp;
  const float *tt1 = reinterpret_cast<const float *>(smem + S::t1) + I * kD + 8 * grp;
  const float *tt0 = reinterpret_cast<const float *>(smem + S::t0) + I * kD + 8 * grp;
  // q~ store positions of the lane's two channel quads under the state side's
  // operand order (see q_times_state): quad e/4 of group g lands at p0 or p0 + 8
  const int p0 = (grp < 2) ? 16 * grp : 16 * (grp - 2) + 4;
  bf16_t *qtRow = reinterpret_cast<bf16_t *>(smem + S::qt) + r * kLDT + p0;
  bf16_t *xwRow = reinterpret_cast<bf16_t *>(smem + S::xw) + r * kLDT + 8 * grp;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const bf16x8_t q8 = __builtin_bit_cast(bf16x8_t, qr[s]);
    const bf16x8_t k8 = __builtin_bit_cast(bf16x8_t, kr[s]);
    float dd[8], e1[8], e0[8];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const f32x4_t d4 = *reinterpret_cast<const f32x4_t *>(dRow + 32 * s + 4 * hh);
      const f32x4_t a4 = *reinterpret_cast<const f32x4_t *>(tt1 + 32 * s + 4 * hh);
      f32x4_t z4 = zero4();
      if (I > 0) z4 = *reinterpret_cast<const f32x4_t *>(tt0 + 32 * s + 4 * hh);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        dd[4 * hh + e] = d4[e];
        e1[4 * hh + e] = a4[e];
        e0[4 * hh + e] = z4[e];
      }
    }
    float Qd[8], Kd[8], Qo[8], Ko[8], qt[8], xw[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float qf = static_cast<float>(q8[e]), kf = static_cast<float>(k8[e]);
      const float ed = fast_exp2(dd[e]);
      Qd[e] = qf * ed;
      Kd[e] = kf * ed;
      if (I > 0) {
        Qo[e] = Qd[e] * e0[e];
        Ko[e] = Kd[e] * e0[e];
      }
      qt[e] = Qd[e] * e1[e];
      xw[e] = Kd[e] * e1[e];
    }
    if constexpr (QN) {
#pragma unroll
      for (int e = 0; e < 8; ++e) ss = fmaf(static_cast<float>(q8[e]), static_cast<float>(q8[e]), ss);
    }
    fQd[s] = bf8(Qd);
    fKd[s] = bf8(Kd);
    if (I > 0) {
      fQo[s] = bf8(Qo);
      fKo[s] = bf8(Ko);
    }
    *reinterpret_cast<bf16x4_t *>(qtRow + 32 * s) = pack_bf16x4(qt[0], qt[1], qt[2], qt[3]);
    *reinterpret_cast<bf16x4_t *>(qtRow + 32 * s + 8) = pack_bf16x4(qt[4], qt[5], qt[6], qt[7]);
    *reinterpret_cast<bf16x8_t *>(xwRow + 32 * s) = bf8(xw);
  }
}

// Key side, P3: the gram products of row block I, A_qk and -A_kk (beta folded)
// to LDS, and T_II = (I + A_II)^-1 from the fp32 diagonal block. A_qk and the
// diagonal block take the place of this block's Cd rows once they are read.
template <int I>
__device__ __forceinline__ void key_grams(const bf16x8_t (&fQd)[4], const bf16x8_t (&fKd)[4],
                                          const bf16x8_t (&fQo)[4], const bf16x8_t (&fKo)[4], char *smem) {
  using S = PipeSmem;
  using M = Mma<bf16_t>;
  const int lane = tid_opaque() & 63;
  const int n16 = lane & 15, grp = lane >> 4;
  const int r = 16 * I + n16;
  f32x4_t accQ[I + 1], accK[I + 1];
#pragma unroll
  for (int j = 0; j <= I; ++j) {
    accQ[j] = zero4();
    accK[j] = zero4();
  }
  // column operand first: lane (row n16, group g) gets A[16I + n16][16j + 4g .. 16j + 4g + 3]
  const bf16_t *cRow = reinterpret_cast<const bf16_t *>(smem + S::cd) + r * kLDT + 8 * grp;
  bf16x8_t fc[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) fc[s] = *reinterpret_cast<const bf16x8_t *>(cRow + 32 * s);
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    accQ[I] = M::mma(fc[s], fQd[s], accQ[I]);
    accK[I] = M::mma(fc[s], fKd[s], accK[I]);
  }
#pragma unroll
  for (int j = 0; j < I; ++j) {
    const bf16_t *eRow = reinterpret_cast<const bf16_t *>(smem + S::ex) + (pair_index(I, j) * 16 + n16) * kLDT + 8 * grp;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const bf16x8_t fe = *reinterpret_cast<const bf16x8_t *>(eRow + 32 * s);
      accQ[j] = M::mma(fe, fQo[s], accQ[j]);
      accK[j] = M::mma(fe, fKo[s], accK[j]);
    }
  }
  const float nbeta = -reinterpret_cast<const float *>(smem + S::beta)[r];
  bf16_t *aqRow = reinterpret_cast<bf16_t *>(smem + S::aqk) + r * kLDT + 4 * grp;
  bf16_t *akRow = reinterpret_cast<bf16_t *>(smem + S::akk) + r * kLDA + 4 * grp;
  float *dsRow = reinterpret_cast<float *>(smem + S::dsc) + r * kLDF + 4 * grp;
  lds_wave_order();  // the Cd rows of this block are read before A_qk and -A_ii replace them
#pragma unroll
  for (int j = 0; j <= I; ++j) {
    f32x4_t aq = accQ[j], ak = accK[j] * nbeta;
    if (j == I) {  // diagonal block: causal masks inside the block
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int col = 4 * grp + e;
        aq[e] = (col <= n16) ? aq[e] : 0.f;
        ak[e] = (col < n16) ? ak[e] : 0.f;
      }
      *reinterpret_cast<f32x4_t *>(dsRow) = ak;
    } else {
      *reinterpret_cast<bf16x4_t *>(akRow + 16 * j) = to_bf16x4(ak);
    }
    *reinterpret_cast<bf16x4_t *>(aqRow + 16 * j) = to_bf16x4(aq);
  }
  // the causal product reads A_qk 32 columns at a time: zero the block right of an even diagonal block
  if constexpr ((I & 1) == 0) *reinterpret_cast<bf16x4_t *>(aqRow + 16 * (I + 1)) = to_bf16x4(zero4());
  lds_wave_order();  // this wave's diagonal rows are read back across lanes
  diag_inverse16(reinterpret_cast<const float *>(smem + S::dsc) + 16 * I * kLDF, kLDF,
                 reinterpret_cast<bf16_t *>(smem + S::td) + 16 * I * kLDTD, kLDTD);
}

// State side, P2: the column operands of block I: Cd = k 2^(-d) = k 2^(m_I - b)
// (its diagonal block), k~ = Cd 2^(b_L - m_I), and for every later row block ip
// the exported column operand Cd 2^(a_ip - m_I) = k 2^(a_ip - b).
template <int I>
__device__ __forceinline__ void state_col_operands(const u32x4_t (&kr)[4], char *smem, int cpar) {
  using S = PipeSmem;
  const int lane = tid_opaque() & 63;
  const int n16 = lane & 15, grp = lane >> 4;
  const int r = 16 * I + n16;
  const float *dRow = reinterpret_cast<const float *>(smem + S::d) + r * kLDB + 8 * grp;
  const float *tt2 = reinterpret_cast<const float *>(smem + S::t2) + I * kD + 8 * grp;
  const float *te = reinterpret_cast<const float *>(smem + S::te) + 8 * grp;
  bf16_t *cdRow = reinterpret_cast<bf16_t *>(smem + S::cd) + r * kLDT + 8 * grp;
  bf16_t *ktRow = reinterpret_cast<bf16_t *>(smem + S::kt) + (cpar * kC + r) * kLDT + 8 * grp;
  bf16_t *exRow = reinterpret_cast<bf16_t *>(smem + S::ex) + n16 * kLDT + 8 * grp;
  constexpr int NE = kNC - 1 - I;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const bf16x8_t k8 = __builtin_bit_cast(bf16x8_t, kr[s]);
    float dd[8], e2[8], ee[NE > 0 ? NE : 1][8];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const f32x4_t d4 = *reinterpret_cast<const f32x4_t *>(dRow + 32 * s + 4 * hh);
      const f32x4_t a4 = *reinterpret_cast<const f32x4_t *>(tt2 + 32 * s + 4 * hh);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        dd[4 * hh + e] = d4[e];
        e2[4 * hh + e] = a4[e];
      }
#pragma unroll
      for (int x = 0; x < NE; ++x) {
        const f32x4_t t4 = *reinterpret_cast<const f32x4_t *>(te + pair_index(I + 1 + x, I) * kD + 32 * s + 4 * hh);
#pragma unroll
        for (int e = 0; e < 4; ++e) ee[x][4 * hh + e] = t4[e];
      }
    }
    float cd[8], kt[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      cd[e] = static_cast<float>(k8[e]) * fast_exp2(-dd[e]);
      kt[e] = cd[e] * e2[e];
    }
    *reinterpret_cast<bf16x8_t *>(cdRow + 32 * s) = bf8(cd);
    *reinterpret_cast<bf16x8_t *>(ktRow + 32 * s) = bf8(kt);
#pragma unroll
    for (int x = 0; x < NE; ++x) {
      float co[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) co[e] = cd[e] * ee[x][e];
      *reinterpret_cast<bf16x8_t *>(exRow + pair_index(I + 1 + x, I) * 16 * kLDT + 32 * s) = bf8(co);
    }
  }
}

// ---------------------------------------------------------------------------------------------
// The key side's loop (waves 0..3).
// ---------------------------------------------------------------------------------------------
template <bool QN>
__device__ __forceinline__ void key_side(const ChunkParams &p, char *smem, int i, int h, const SlotRange &sr,
                                         int nch) {
  using S = PipeSmem;
  const int t = tid_opaque();  // 0..255
  const int n16 = t & 15, grp = (t & 63) >> 4;
  const int Kr = p.Kr, H = p.H;
  const int hk = h / (H / p.Hk);
  const uint32_t ldx = (uint32_t)H * Kr, ldq = (uint32_t)p.Hk * Kr;
  const float expA = fast_exp2(p.A_log[h] * kLog2e);
  const float c1 = -expA * kLog2e, c2 = p.lower_bound * kLog2e;
  // gate lanes: channels ch0, ch0 + 1 of row block lane / 16
  const int ch0 = 2 * (16 * i + (t & 15)), gb = (t & 63) >> 4;
  float dtc[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) dtc[e] = (p.dt_bias && ch0 + e < Kr) ? p.dt_bias[h * Kr + ch0 + e] * c1 : 0.f;
  // lane offsets: the first gate row of this lane's block, and the q/k row
  // 16i + n16 at channel 8 g (+ 64 bytes per 32-channel slice)
  const uint32_t xoff = ch0 < Kr ? ((16u * gb) * ldx + ch0) * 4u : 0x40000000u;
  const uint32_t qoff = ((16u * i + n16) * ldq + 8u * grp) * 2u;
  bool qk_ok[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) qk_ok[s] = 32 * s + 8 * grp < Kr;

  f32x2_t xr[16];
  float br = 0.f;
  u32x4_t qr[4], kr[4];
  auto load_gate = [&](int64_t t0, int L) {
    const rsrc_t rx = make_rsrc(p.g + (t0 * H + h) * Kr, (uint32_t)((L - 1) * ldx + Kr) * 4u);
    if (L == kC) {  // every row exists: the row offset rides in the scalar offset
#pragma unroll
      for (int r = 0; r < 16; ++r)
        xr[r] = __builtin_bit_cast(f32x2_t, __builtin_amdgcn_raw_buffer_load_b64(rx, (int)xoff, (int)(r * ldx * 4u), 0));
    } else {  // the row is part of the checked offset: rows past the slot end read zeros
#pragma unroll
      for (int r = 0; r < 16; ++r)
        xr[r] = __builtin_bit_cast(f32x2_t, __builtin_amdgcn_raw_buffer_load_b64(rx, (int)(xoff + r * ldx * 4u), 0, 0));
    }
    if (t < kC) {
      const rsrc_t rb = make_rsrc(p.beta + t0 * H + h, (uint32_t)((L - 1) * H + 1) * 4u);
      br = bload_f32(rb, (uint32_t)t * H * 4u);
    }
  };
  auto load_qk = [&](int64_t t0, int L) {
    const size_t e0 = (size_t)(t0 * p.Hk + hk) * Kr;
    const uint32_t bytes = (uint32_t)((L - 1) * ldq + Kr) * 2u;
    const rsrc_t rq = make_rsrc(reinterpret_cast<const bf16_t *>(p.q) + e0, bytes);
    const rsrc_t rk = make_rsrc(reinterpret_cast<const bf16_t *>(p.k) + e0, bytes);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint32_t off = qk_ok[s] ? qoff + 64u * s : 0x40000000u;
      qr[s] = bload_b128(rq, off);
      kr[s] = bload_b128(rk, off);
    }
  };
  if (nch > 0) {
    load_gate(sr.t0, min(kC, sr.len));
    load_qk(sr.t0, min(kC, sr.len));
  }
  bf16x8_t fQd[4], fKd[4], fQo[4], fKo[4];
  for (int c = 0; c < nch; ++c) {
    const int64_t t0 = sr.t0 + (int64_t)c * kC;
    const int L = min(kC, sr.len - c * kC);
    const bool more = c + 1 < nch;
    const int Ln = more ? min(kC, sr.len - (c + 1) * kC) : 0;
    // ---- P1: gate activation, cumsum, d = b - m_i and the anchor tables; beta.
    // This chunk's gate and beta loads were issued before its eight q and k
    // loads, which are needed only in P2: wait for all but those eight.
    __builtin_amdgcn_s_waitcnt(0x0F78);  // vmcnt(8)
    key_gate(xr, dtc, c1, c2, L, c & 1, i, smem);
    {
      const int tt = tid_opaque();
      if (tt < kC) reinterpret_cast<float *>(smem + S::beta)[tt] = (p.beta_logits && tt < L) ? sigmoid_f32(br) : br;
    }
    __syncthreads();
    // ---- P2: row operands of block i (the state waves' column operands take
    // the issue slots first: the key side's grams wait on them)
    wait_vmem();
    float ss = 0.f;
    switch (i) {
      case 0: key_row_operands<0, QN>(qr, kr, smem, fQd, fKd, fQo, fKo, ss); break;
      case 1: key_row_operands<1, QN>(qr, kr, smem, fQd, fKd, fQo, fKo, ss); break;
      case 2: key_row_operands<2, QN>(qr, kr, smem, fQd, fKd, fQo, fKo, ss); break;
      default: key_row_operands<3, QN>(qr, kr, smem, fQd, fKd, fQo, fKo, ss); break;
    }
    {
      // output row scale: the query scale, times 1/|q_r| for raw q
      const int lane = tid_opaque() & 63, n16 = lane & 15, grp = lane >> 4;
      ss += __shfl_xor(ss, 16);
      ss += __shfl_xor(ss, 32);
      float sc = p.scale;
      if constexpr (QN) sc *= rsqrtf(ss + kQNormEps);
      if (grp == 0) reinterpret_cast<float *>(smem + S::qn)[16 * i + n16] = sc;
    }
    __syncthreads();
    // ---- P3: gram products, A_qk and -A_kk to LDS, diagonal inverse of block i;
    // the next chunk's gate input streams in from here, its q and k from P4
    if (more) load_gate(t0 + kC, Ln);
    switch (i) {
      case 0: key_grams<0>(fQd, fKd, fQo, fKo, smem); break;
      case 1: key_grams<1>(fQd, fKd, fQo, fKo, smem); break;
      case 2: key_grams<2>(fQd, fKd, fQo, fKo, smem); break;
      default: key_grams<3>(fQd, fKd, fQo, fKo, smem); break;
    }
    __syncthreads();
    // ---- P4: w tiles 2i, 2i+1 of the substitution, to w^T
    if (more) load_qk(t0 + kC, Ln);
    {
      f32x4_t Wa[kNC], Wb[kNC];
      subst_pair(reinterpret_cast<const bf16_t *>(smem + S::xw), 2 * i, 2 * i + 1, kLDT,
                 reinterpret_cast<const float *>(smem + S::beta), reinterpret_cast<const bf16_t *>(smem + S::akk),
                 kLDA, reinterpret_cast<const bf16_t *>(smem + S::td), kLDTD, Wa, Wb);
      bf16_t *sWT = reinterpret_cast<bf16_t *>(smem + S::wt);
      store_wT<kC>(sWT, kLDW, 2 * i, Wa);
      store_wT<kC>(sWT, kLDW, 2 * i + 1, Wb);
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------------------------
// The state side's loop (waves 4..7; wave 4 + sidx owns value columns 32 sidx..).
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ void state_side(const ChunkParams &p, char *smem, int sidx, int n, int h, int nh,
                                           const SlotRange &sr, int nch) {
  using S = PipeSmem;
  constexpr int NVW = 2;
  const int lane = tid_opaque() & 63, n16 = lane & 15, grp = lane >> 4;
  const int Kr = p.Kr, Vr = p.Vr, H = p.H;
  const int hk = h / (H / p.Hk);
  const int col0 = 32 * sidx;
  const uint32_t ldq = (uint32_t)p.Hk * Kr, ldv = (uint32_t)H * Vr;
  const int64_t sbase = (int64_t)nh * Kr * Vr;
  float *hcs = p.hc ? p.hc + ((int64_t)(p.cu ? p.chunk_off[n] : n * ((p.T + kC - 1) / kC)) * H + h) * Kr * Vr
                    : nullptr;
  // this wave's row block of k (column operands) and v (the substitution's right-hand side)
  const uint32_t koff = ((16u * sidx + n16) * ldq + 8u * grp) * 2u;
  const uint32_t voff = ((16u * sidx + n16) * ldv + 8u * grp) * 2u;
  bool k_ok[4], v_ok[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    k_ok[s] = 32 * s + 8 * grp < Kr;
    v_ok[s] = 32 * s + 8 * grp < Vr;
  }
  u32x4_t kr[4], vr[4];
  auto load_k = [&](int64_t t0, int L) {
    const rsrc_t rk = make_rsrc(reinterpret_cast<const bf16_t *>(p.k) + (size_t)(t0 * p.Hk + hk) * Kr,
                                (uint32_t)((L - 1) * ldq + Kr) * 2u);
#pragma unroll
    for (int s = 0; s < 4; ++s) kr[s] = bload_b128(rk, k_ok[s] ? koff + 64u * s : 0x40000000u);
  };
  auto load_v = [&](int64_t t0, int L) {
    const rsrc_t rv = make_rsrc(reinterpret_cast<const bf16_t *>(p.v) + (size_t)(t0 * H + h) * Vr,
                                (uint32_t)((L - 1) * ldv + Vr) * 2u);
#pragma unroll
    for (int s = 0; s < 4; ++s) vr[s] = bload_b128(rv, v_ok[s] ? voff + 64u * s : 0x40000000u);
  };

  f32x4_t hs[kD / 16][NVW];
  if (p.h0) {
    load_strip<kD / 16, NVW>(hs, p.h0 + sbase, Vr, col0, Kr, Vr);
  } else {
#pragma unroll
    for (int tt = 0; tt < kD / 16; ++tt)
#pragma unroll
      for (int v = 0; v < NVW; ++v) hs[tt][v] = zero4();
  }
  if (nch > 0) {
    load_k(sr.t0, min(kC, sr.len));
    load_v(sr.t0, min(kC, sr.len));
  }
  f32x4_t oT[kNC][NVW], uv[kNC][NVW];
  bf16x8_t vprev[kC / 32][NVW];
  const float *sQn = reinterpret_cast<const float *>(smem + S::qn);

  // steps (5)-(6) of the chunk at t0 with L rows: v_new = u - w h, o = q~ h + A_qk v_new (scaled), stored;
  // v_new kept as the operand fragments of its state update
  auto tail = [&](int64_t t0, int L) {
    f32x4_t p1[kNC][NVW];
#pragma unroll
    for (int ii = 0; ii < kNC; ++ii)
#pragma unroll
      for (int v = 0; v < NVW; ++v) p1[ii][v] = zero4();
    w_times_state<kC, kD, NVW>(p1, reinterpret_cast<const bf16_t *>(smem + S::wt), kLDW, hs);
#pragma unroll
    for (int ii = 0; ii < kNC; ++ii)
#pragma unroll
      for (int v = 0; v < NVW; ++v) uv[ii][v] = uv[ii][v] - p1[ii][v];
    causal_times_h<kC, NVW>(oT, reinterpret_cast<const bf16_t *>(smem + S::aqk), kLDT, uv);
    vnew_frags<kC, NVW>(vprev, uv);
    const rsrc_t ro = make_rsrc(reinterpret_cast<bf16_t *>(p.o) + (size_t)(t0 * H + h) * Vr,
                                (uint32_t)((L - 1) * ldv + Vr) * 2u);
#pragma unroll
    for (int ii = 0; ii < kNC; ++ii) {
      const float sc = sQn[16 * ii + n16];
#pragma unroll
      for (int v = 0; v < NVW; ++v) {
        const int cc = col0 + 16 * v + 4 * grp;  // four columns, all below Vr or none
        const uint32_t off = cc < Vr ? ((16u * ii + n16) * ldv + cc) * 2u : 0x40000000u;
        bstore_b64(ro, off, to_bf16x4(oT[ii][v] * sc));
      }
    }
  };
  auto update = [&](int c) {
    state_update_kt<kC, kD, NVW>(hs, reinterpret_cast<const bf16_t *>(smem + S::kt) + (c & 1) * kC * kLDT, kLDT,
                                 vprev, reinterpret_cast<const float *>(smem + S::lam) + (c & 1) * kD);
  };

  int64_t t0p = 0;
  int Lp = 0;
  for (int c = 0; c < nch; ++c) {
    const int64_t t0 = sr.t0 + (int64_t)c * kC;
    const int L = min(kC, sr.len - c * kC);
    const bool more = c + 1 < nch;
    const int Ln = more ? min(kC, sr.len - (c + 1) * kC) : 0;
    // ---- P1: the previous chunk's products and output
    if (c > 0) tail(t0p, Lp);
    __syncthreads();
    // ---- P2: column operands of block sidx (k~ into this chunk's parity buffer);
    // the state waves issue first in this period (measured: 1.5% shorter chunks
    // than giving the first slots to the heavier wave of each role).
    // This chunk's k and v loads came before the previous chunk's eight o stores
    // (P1), and vector memory operations retire in order: wait for all but those.
    __builtin_amdgcn_s_waitcnt(0x0F78);  // vmcnt(8)
    __builtin_amdgcn_s_setprio(2);
    switch (sidx) {
      case 0: state_col_operands<0>(kr, smem, c & 1); break;
      case 1: state_col_operands<1>(kr, smem, c & 1); break;
      case 2: state_col_operands<2>(kr, smem, c & 1); break;
      default: state_col_operands<3>(kr, smem, c & 1); break;
    }
    __builtin_amdgcn_s_setprio(0);
    if (more) load_k(t0 + kC, Ln);
    __syncthreads();
    // ---- P3: the previous chunk's state update, the state entering this chunk,
    // q~ h of this chunk; v rows of block sidx to LDS
    if (c > 0) update(c - 1);
    if (hcs) store_strip<float, kD / 16, NVW>(hcs + (int64_t)c * H * Kr * Vr, Vr, col0, Kr, hs, Vr);
#pragma unroll
    for (int ii = 0; ii < kNC; ++ii)
#pragma unroll
      for (int v = 0; v < NVW; ++v) oT[ii][v] = zero4();
    q_times_state<kC, kD, NVW>(oT, reinterpret_cast<const bf16_t *>(smem + S::qt), kLDT, hs);
    {
      bf16_t *vRow = reinterpret_cast<bf16_t *>(smem + S::v) + (16 * sidx + n16) * kLDT + 8 * grp;
#pragma unroll
      for (int s = 0; s < 4; ++s) *reinterpret_cast<u32x4_t *>(vRow + 32 * s) = vr[s];
    }
    if (more) load_v(t0 + kC, Ln);
    __syncthreads();
    // ---- P4: u tiles of this wave's value columns
    {
      f32x4_t Ua[kNC], Ub[kNC];
      subst_pair(reinterpret_cast<const bf16_t *>(smem + S::v), 2 * sidx, 2 * sidx + 1, kLDT,
                 reinterpret_cast<const float *>(smem + S::beta), reinterpret_cast<const bf16_t *>(smem + S::akk),
                 kLDA, reinterpret_cast<const bf16_t *>(smem + S::td), kLDTD, Ua, Ub);
#pragma unroll
      for (int ii = 0; ii < kNC; ++ii) {
        uv[ii][0] = Ua[ii];
        uv[ii][1] = Ub[ii];
      }
    }
    __syncthreads();
    t0p = t0;
    Lp = L;
  }
  if (nch > 0) {
    // the last chunk's products, output and state update (the key side is done)
    tail(t0p, Lp);
    update(nch - 1);
  }
  if (p.ht && !(sr.len == 0 && p.ht == p.h0)) store_strip<float, kD / 16, NVW>(p.ht + sbase, Vr, col0, Kr, hs, Vr);
}

template <bool QN>
__global__ __launch_bounds__(kNT) void pipe_chunk_kernel(ChunkParams p) {
  extern __shared__ __align__(16) char smem[];
  const int w = wave_id();
  const int nh = blockIdx.x, n = nh / p.H, h = nh % p.H;
  const SlotRange sr = slot_range(p.cu, n, p.T);
  const int nch = (sr.len + kC - 1) / kC;
  if (w < 4) key_side<QN>(p, smem, w, h, sr, nch);
  else state_side(p, smem, w - 4, n, h, nh, sr, nch);
}

}  // namespace

// The pipelined kernel takes bf16, C = 64, D = 128, the safe gate, and one
// workgroup per (sequence, head).
bool pipe_supported(const ChunkParams &p) {
  return p.is_bf16 && p.C == kC && p.D == kD && p.gate_kind == kGateSafe;
}

hipError_t launch_pipe(const ChunkParams &p, hipStream_t st) {
  if (!pipe_supported(p)) return hipErrorInvalidValue;
  if (p.N * p.H == 0) return hipSuccess;
  const size_t smem = PipeSmem::total;
  auto kern = p.q_l2norm ? pipe_chunk_kernel<true> : pipe_chunk_kernel<false>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)smem);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return e;
  }
  hipLaunchKernelGGL(kern, dim3(p.N * p.H), dim3(kNT), smem, st, p);
  return hipGetLastError();
}

}  // namespace kda
