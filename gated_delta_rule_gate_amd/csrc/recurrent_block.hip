// Blocked form of the fused recurrence (bf16 inputs, K = V = 128).
//
// The recurrence of "Add fused recurrent_kda for decode and inference prefill"
// (section "Agent note": FP32 state per (sequence, head), token order) costs
// four FP32 operations per state element and token when it is evaluated token
// by token, all of them on the vector ALUs. This kernel keeps the same state,
// the same token order and the same inputs, but scans the tokens of a sequence
// in blocks of 16 and writes each block's effect on the state in the WY form of
// the chunked path (the WY recompute of "FLA KDA Skill", section "Public code
// map", with a chunk of one 16-token sub-chunk, whose grams take the midpoint
// offset of section "Safe gate numerical note"): with b the in-block cumsum of
// the log2 gate and m its value at the anchor row,
//
//   A_kk = beta_r sum_c k_r k_s 2^(b_r - b_s)  (s < r),  A_qk = scale sum_c q_r k_s 2^(b_r - b_s)  (s <= r)
//          both from the anchored operands k 2^(b - m), q 2^(b - m), k 2^(m - b)
//   T    = (I + A_kk)^-1                        (16 x 16, forward substitution)
//   W    = T (beta k 2^b),   U = T (beta v)
//   vnew = U - W S,   o = scale (q 2^b) S + A_qk vnew,   S <- Diag(2^b_L) S + (k 2^(b_L - b))^T vnew
//
// Every product runs on the matrix cores (v_mfma_f32_16x16x32_bf16 and
// _16x16x16_bf16) with FP32 accumulation, as in the chunked kernels; the state
// S stays in accumulator registers for the whole sequence (wave w owns value
// columns 32w .. 32w + 31), so it is read from and written to HBM once.
//
// The anchored operands are finite only while every exponent stays in range.
// Each block checks, per channel, that |b_r - m|, b_r and b_L - b_r are at most
// 100 (log2 units); if any channel fails, the whole block is evaluated one
// token at a time by the same code (a block of one token has every exponent 0
// except 2^b itself), which is exact for any gate.
#include "chunk_fused_tiles.h"
#include "kda_launch.h"

namespace kda {
namespace {

constexpr int kBT = 16;         // tokens per block
constexpr int kBD = 128;        // K = V
constexpr int kBThreads = 256;  // four waves
constexpr int kLR = kBD + 8;    // row stride of row-major [token][channel] bf16 tiles
constexpr int kLC = kBT + 8;    // row stride of channel-major [channel][token] bf16 tiles
constexpr int kLA = 20;         // row stride of the fp32 [16][16] block of -beta A_kk
constexpr float kExpLimit = 100.f;

struct BlkSmem {
  static constexpr size_t rq = 0;                   // raw q [16][128] bf16
  static constexpr size_t rk = rq + 2 * kBT * kBD;  // raw k
  static constexpr size_t rv = rk + 2 * kBT * kBD;  // raw v
  static constexpr size_t qd = rv + 2 * kBT * kBD;  // scale q 2^(b - m) [16][kLR]
  static constexpr size_t kd = qd + 2 * kBT * kLR;  // k 2^(b - m)
  static constexpr size_t cd = kd + 2 * kBT * kLR;  // k 2^(m - b)
  static constexpr size_t qt = cd + 2 * kBT * kLR;  // scale q 2^b
  static constexpr size_t wm = qt + 2 * kBT * kLR;  // W [16][kLR]
  static constexpr size_t xT = wm + 2 * kBT * kLR;  // (beta k 2^b)^T [128][kLC]
  static constexpr size_t kT = xT + 2 * kBD * kLC;  // (k 2^(b_L - b))^T [128][kLC]
  static constexpr size_t vT = kT + 2 * kBD * kLC;  // (beta v)^T [128][kLC]
  static constexpr size_t aq = vT + 2 * kBD * kLC;  // A_qk [16][kLC] bf16
  static constexpr size_t td = aq + 2 * kBT * kLC;  // T [16][kLC] bf16
  static constexpr size_t ak = td + 2 * kBT * kLC;  // -beta A_kk [16][kLA] fp32
  static constexpr size_t lam = ak + 4 * kBT * kLA;  // 2^b_L [128]
  static constexpr size_t beta = lam + 4 * kBD;      // beta per block row [16]
  static constexpr size_t qn = beta + 4 * kBT;       // 1/sqrt(|q|^2 + eps) per block row [16]
  static constexpr size_t flag = qn + 4 * kBT;       // out-of-range flag per block parity [2] (int)
  static constexpr size_t total = flag + 16;
};

typedef short s16x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ s16x4_t pack4(float a, float b, float c, float d) {
  return __builtin_bit_cast(s16x4_t, u32x2_t{pack_bf16x2(a, b), pack_bf16x2(c, d)});
}

__device__ __forceinline__ s16x4_t lds4(const char *smem, size_t base, int row, int ld, int col) {
  return *reinterpret_cast<const s16x4_t *>(smem + base + 2 * (row * ld + col));
}

// 16x16x32 operand of a row-major [row][channel] bf16 tile: row `row`, the
// channels of contraction step s and lane group grp in the kidx order.
__device__ __forceinline__ bf16x8_t lds_kidx(const char *smem, size_t base, int row, int s, int grp) {
  const bf16_t *p = reinterpret_cast<const bf16_t *>(smem + base) + row * kLR + 32 * s + 4 * grp;
  const u32x2_t lo = *reinterpret_cast<const u32x2_t *>(p);
  const u32x2_t hi = *reinterpret_cast<const u32x2_t *>(p + 16);
  return __builtin_bit_cast(bf16x8_t, u32x4_t{lo[0], lo[1], hi[0], hi[1]});
}

// Raw buffer resources: loads past `bytes` return zeros, stores there are
// dropped; the row is always part of the checked vector offset.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ f32x4_t mma16(s16x4_t a, s16x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

template <bool QN, int GK>
__global__ __launch_bounds__(kBThreads, 2) void recurrent_block_kernel(RecurrentParams p) {
  using M = Mma<bf16_t>;
  using S = BlkSmem;
  extern __shared__ __align__(16) char smem[];
  const int nh = blockIdx.x;
  const int n = nh / p.H, h = nh % p.H;
  const int hk = h / (p.H / p.Hk);
  // lane-derived values are re-read from tid_opaque() where they are used, so
  // the block loop does not keep per-lane addresses live in registers
  const int w = wave_id();
  const int col0 = 32 * w;  // value columns of this wave
  const SlotRange sr = slot_range(p.cu, n, p.T);
  const int64_t sbase = (int64_t)nh * kBD * kBD;
  const int ldq = p.Hk * kBD, ldv = p.H * kBD;  // row strides (elements) of q/k and of v, g, o
  const bf16_t *qg = reinterpret_cast<const bf16_t *>(p.q) + (int64_t)hk * kBD;
  const bf16_t *kg = reinterpret_cast<const bf16_t *>(p.k) + (int64_t)hk * kBD;
  const bf16_t *vg = reinterpret_cast<const bf16_t *>(p.v) + (int64_t)h * kBD;
  const float *gg = p.g + (int64_t)h * kBD;
  bf16_t *og = reinterpret_cast<bf16_t *>(p.o) + (int64_t)h * kBD;

  // ---- state: Sx[ct][t] holds rows (channels) 16 t .. of value columns col0 + 16 ct .. (C layout)
  f32x4_t Sx[2][8];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct)
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      if (p.h0) {
        const int ln = tid_opaque() & 63;
        const float *src = p.h0 + sbase + (int64_t)(16 * t + 4 * (ln >> 4)) * kBD + col0 + 16 * ct + (ln & 15);
        Sx[ct][t] = f32x4_t{src[0], src[kBD], src[2 * kBD], src[3 * kBD]};
      } else {
        Sx[ct][t] = zero4();
      }
    }

  constexpr bool gated = GK == kGateSafe || GK == kGateSoftplus;
  const float expA = gated ? fast_exp2(p.A_log[h] * kLog2e) : 0.f;
  const float dtc = p.dt_bias ? p.dt_bias[h * kBD + 64 * (w & 1) + (tid_opaque() & 63)] : 0.f;

  // next block's raw inputs: 16 bytes of q, k, v (row tid / 16), the gate input of
  // channel c for all 16 rows, beta of row tid (tid < 16)
  u32x4_t pq, pk, pv;
  float pg[kBT], pb = 0.f;
  auto fetch = [&](int blk) {
    const int64_t t0 = sr.t0 + (int64_t)kBT * blk;
    const int L = min(kBT, sr.len - kBT * blk);  // >= 1
    const int t = tid_opaque();
    const rsrc_t rq = make_rsrc(qg + t0 * ldq, (uint32_t)((L - 1) * ldq + kBD) * 2u);
    const rsrc_t rk = make_rsrc(kg + t0 * ldq, (uint32_t)((L - 1) * ldq + kBD) * 2u);
    const rsrc_t rv = make_rsrc(vg + t0 * ldv, (uint32_t)((L - 1) * ldv + kBD) * 2u);
    const rsrc_t rg = make_rsrc(gg + t0 * ldv, (uint32_t)((L - 1) * ldv + kBD) * 4u);
    const uint32_t oq = (uint32_t)((t >> 4) * ldq + (t & 15) * 8) * 2u;
    const uint32_t ov = (uint32_t)((t >> 4) * ldv + (t & 15) * 8) * 2u;
    pq = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rq, (int)oq, 0, 0));
    pk = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rk, (int)oq, 0, 0));
    pv = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rv, (int)ov, 0, 0));
#pragma unroll
    for (int rr = 0; rr < kBT; ++rr)
      pg[rr] = __uint_as_float(
          __builtin_amdgcn_raw_buffer_load_b32(rg, (int)((uint32_t)(rr * ldv + 64 * (w & 1) + (t & 63)) * 4u), 0, 0));
    if (t < kBT) {
      const rsrc_t rb = make_rsrc(p.beta + t0 * p.H + h, (uint32_t)((L - 1) * p.H + 1) * 4u);
      pb = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rb, (int)((uint32_t)(t * p.H) * 4u), 0, 0));
    }
  };

  // Phase 1 of a (sub-)block of Ls rows starting at block row r0, for channel
  // c = 64 (w & 1) + lane and LDS rows 8 HR .. 8 HR + 7 (HR = w / 2): operand
  // row rr comes from block row r0 + rr. FAST: r0 = 0, Ls = L, b is the cumsum
  // over the block; otherwise Ls = 1 and the single row's b is its own gate.
  auto operands = [&](auto hr_tag, const float (&gl)[kBT], bool fast, int r0, int Ls) {
    constexpr int HR = decltype(hr_tag)::value;
    const int c = 64 * (w & 1) + (tid_opaque() & 63);
    float b[8];
    float m, bL;
    if (fast) {
      float acc = 0.f, b8 = 0.f;
#pragma unroll
      for (int r = 0; r < kBT; ++r) {
        acc += gl[r];
        if (r == 8) b8 = acc;
        if (r >= 8 * HR && r < 8 * HR + 8) b[r - 8 * HR] = acc;
      }
      m = (Ls > 8) ? b8 : acc;  // anchor row min(8, Ls - 1); rows past Ls keep b_L
      bL = acc;
    } else {
      float g0 = 0.f;
#pragma unroll
      for (int r = 0; r < kBT; ++r) g0 = (r == r0) ? gl[r] : g0;
#pragma unroll
      for (int j = 0; j < 8; ++j) b[j] = g0;
      m = g0;
      bL = g0;
    }
    const float tm = fast_exp2(m), tl = fast_exp2(bL - m);
    const bf16_t *rq = reinterpret_cast<const bf16_t *>(smem + S::rq);
    const bf16_t *rk = reinterpret_cast<const bf16_t *>(smem + S::rk);
    const bf16_t *rv = reinterpret_cast<const bf16_t *>(smem + S::rv);
    const float *sb = reinterpret_cast<const float *>(smem + S::beta);
    bf16_t *qd = reinterpret_cast<bf16_t *>(smem + S::qd);
    bf16_t *kd = reinterpret_cast<bf16_t *>(smem + S::kd);
    bf16_t *cd = reinterpret_cast<bf16_t *>(smem + S::cd);
    bf16_t *qt = reinterpret_cast<bf16_t *>(smem + S::qt);
    float xw[8], kt[8], bv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int rr = 8 * HR + j;
      const bool valid = rr < Ls;
      const int row = min(r0 + rr, kBT - 1);
      const float q = valid ? static_cast<float>(rq[row * kBD + c]) * p.scale : 0.f;
      const float k = valid ? static_cast<float>(rk[row * kBD + c]) : 0.f;
      const float v = valid ? static_cast<float>(rv[row * kBD + c]) : 0.f;
      const float be = valid ? sb[row] : 0.f;
      // a block of one token has b = m = b_L: its only exponential is 2^b
      // (0 for a gate of -inf), the others are exactly 1
      // with the range check passed, 2^b = 2^(b - m) 2^m and 2^(b_L - b) = 2^(m - b) 2^(b_L - m)
      // with both factors finite
      const float br = b[j];
      const float e1 = fast ? fast_exp2(br - m) : 1.f, e2 = fast ? fast_exp2(m - br) : 1.f;
      const float eb = fast ? e1 * tm : fast_exp2(br);
      const float el = fast ? e2 * tl : 1.f;
      qd[rr * kLR + c] = static_cast<bf16_t>(valid ? q * e1 : 0.f);
      kd[rr * kLR + c] = static_cast<bf16_t>(valid ? k * e1 : 0.f);
      cd[rr * kLR + c] = static_cast<bf16_t>(valid ? k * e2 : 0.f);
      qt[rr * kLR + c] = static_cast<bf16_t>(valid ? q * eb : 0.f);
      xw[j] = valid ? be * k * eb : 0.f;
      kt[j] = valid ? k * el : 0.f;
      bv[j] = be * v;
    }
    auto put8 = [&](size_t base, const float (&x)[8]) {
      *reinterpret_cast<u32x4_t *>(smem + base + 2 * (c * kLC + 8 * HR)) =
          u32x4_t{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                  pack_bf16x2(x[6], x[7])};
    };
    put8(S::xT, xw);
    put8(S::kT, kt);
    put8(S::vT, bv);
    if (HR == 0) reinterpret_cast<float *>(smem + S::lam)[c] = fast_exp2(bL);
  };

  // Phases 2-4 of a (sub-)block: grams and T, W and U, then vnew, o and the state.
  auto products = [&](int64_t trow, int r0, int Ls) {
    const int lane = tid_opaque() & 63, n16 = lane & 15, grp = lane >> 4;
    // ---- phase 2: wave 0 forms A_qk, -beta A_kk and T; every wave q~ S
    f32x4_t O[2] = {zero4(), zero4()};
    auto q_times_state = [&]() {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const bf16x8_t a = lds_kidx(smem, S::qt, n16, s, grp);
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) O[ct] = M::mma(a, acc_frag<bf16_t>(Sx[ct], s), O[ct]);
      }
    };
    if (w == 0) {
      f32x4_t aqa = zero4(), aka = zero4();
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const bf16x8_t bc = lds_kidx(smem, S::cd, n16, s, grp);
        aqa = M::mma(lds_kidx(smem, S::qd, n16, s, grp), bc, aqa);
        aka = M::mma(lds_kidx(smem, S::kd, n16, s, grp), bc, aka);
      }
      const float *sb = reinterpret_cast<const float *>(smem + S::beta);
      bf16_t *aqs = reinterpret_cast<bf16_t *>(smem + S::aq);
      float *aks = reinterpret_cast<float *>(smem + S::ak);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * grp + i;
        const float be = (r < Ls) ? sb[min(r0 + r, kBT - 1)] : 0.f;
        aqs[r * kLC + n16] = static_cast<bf16_t>(n16 <= r ? aqa[i] : 0.f);
        aks[r * kLA + n16] = (n16 < r) ? -be * aka[i] : 0.f;
      }
      if constexpr (QN) {
        // 1/sqrt(|q|^2 + eps) of LDS row n16 (block row r0 + n16)
        const bf16_t *rq = reinterpret_cast<const bf16_t *>(smem + S::rq) + ((r0 + n16) & (kBT - 1)) * kBD + 32 * grp;
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < 32; e += 8) {
          const bf16x8_t q8 = *reinterpret_cast<const bf16x8_t *>(rq + e);
#pragma unroll
          for (int u = 0; u < 8; ++u) ss = fmaf(static_cast<float>(q8[u]), static_cast<float>(q8[u]), ss);
        }
        ss += __shfl_xor(ss, 16);
        ss += __shfl_xor(ss, 32);
        if (grp == 0) reinterpret_cast<float *>(smem + S::qn)[n16] = rsqrtf(ss + kQNormEps);
      }
      lds_wave_order();
      diag_inverse16(aks, kLA, reinterpret_cast<bf16_t *>(smem + S::td), kLC);
    }
    q_times_state();
    __syncthreads();
    // ---- phase 3: W for channels col0 .. col0 + 31 (to LDS), U for this wave's value columns
    const s16x4_t tA = lds4(smem, S::td, n16, kLC, 4 * grp);
    f32x4_t U[2];
    bf16_t *wms = reinterpret_cast<bf16_t *>(smem + S::wm);
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      const int ch = col0 + 16 * ct + n16;
      const f32x4_t wv = mma16(tA, lds4(smem, S::xT, ch, kLC, 4 * grp), zero4());
#pragma unroll
      for (int i = 0; i < 4; ++i) wms[(4 * grp + i) * kLR + ch] = static_cast<bf16_t>(wv[i]);
      U[ct] = mma16(tA, lds4(smem, S::vT, ch, kLC, 4 * grp), zero4());
    }
    __syncthreads();
    // ---- phase 4: vnew = U - W S, o = q~ S + A_qk vnew, S <- Diag(2^b_L) S + k~^T vnew
    s16x4_t vb[2];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      f32x4_t P = zero4();
#pragma unroll
      for (int s = 0; s < 4; ++s) P = M::mma(lds_kidx(smem, S::wm, n16, s, grp), acc_frag<bf16_t>(Sx[ct], s), P);
      const f32x4_t vn = U[ct] - P;
      vb[ct] = pack4(vn[0], vn[1], vn[2], vn[3]);
    }
    const s16x4_t aA = lds4(smem, S::aq, n16, kLC, 4 * grp);
    const float *qns = reinterpret_cast<const float *>(smem + S::qn);
    const rsrc_t ro = make_rsrc(og + trow * ldv, (uint32_t)((Ls - 1) * ldv + kBD) * 2u);
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      O[ct] = mma16(aA, vb[ct], O[ct]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * grp + i;
        const float ov = QN ? O[ct][i] * qns[r] : O[ct][i];
        // rows past Ls fall outside the resource: the store is dropped
        const uint32_t off = (uint32_t)((r < Ls ? r : kBT) * ldv + col0 + 16 * ct + n16) * 2u;
        __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, static_cast<bf16_t>(ov)), ro,
                                              (int)off, 0, 0);
      }
    }
    const float *lam = reinterpret_cast<const float *>(smem + S::lam);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const f32x4_t l4 = *reinterpret_cast<const f32x4_t *>(lam + 16 * t + 4 * grp);
      const s16x4_t kA = lds4(smem, S::kT, 16 * t + n16, kLC, 4 * grp);
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) Sx[ct][t] = mma16(kA, vb[ct], Sx[ct][t] * l4);
    }
    __syncthreads();
  };

  const int nb = (sr.len + kBT - 1) / kBT;
  int *flags = reinterpret_cast<int *>(smem + S::flag);
  // the next block's activated gate of channel c (log2 units), and whether any
  // exponent of its anchored operands could leave range; the flag of block j
  // is ORed into flags[j & 1] before a barrier that precedes its use
  float gl[kBT];
  auto gate_and_check = [&](int blk) {
    const int L = min(kBT, sr.len - kBT * blk);
#pragma unroll
    for (int r = 0; r < kBT; ++r) gl[r] = (r < L) ? gate_log2(GK, pg[r], dtc, expA, p.lower_bound) : 0.f;
    float acc = 0.f, b8 = 0.f, bmin = 0.f, bmax = 0.f;
#pragma unroll
    for (int r = 0; r < kBT; ++r) {
      acc += gl[r];
      if (r == 8) b8 = acc;
      bmin = (r == 0) ? acc : fminf(bmin, acc);
      bmax = (r == 0) ? acc : fmaxf(bmax, acc);
    }
    const float m = (L > 8) ? b8 : acc;
    const bool bad = !(bmax - m <= kExpLimit && m - bmin <= kExpLimit && bmax <= kExpLimit &&
                       acc - bmin <= kExpLimit && acc - m <= kExpLimit);
    if (bad) atomicOr(flags + (blk & 1), 1);
  };
  if (tid_opaque() < 2) flags[tid_opaque()] = 0;
  __syncthreads();
  if (nb > 0) {
    fetch(0);
    wait_vmem();
    gate_and_check(0);
  }
  for (int blk = 0; blk < nb; ++blk) {
    const int64_t t0 = sr.t0 + (int64_t)kBT * blk;
    const int L = min(kBT, sr.len - kBT * blk);
    // stage the raw block, start the next block's loads
    {
      const int t = tid_opaque();
      const int off = 2 * ((t >> 4) * kBD + (t & 15) * 8);
      *reinterpret_cast<u32x4_t *>(smem + S::rq + off) = pq;
      *reinterpret_cast<u32x4_t *>(smem + S::rk + off) = pk;
      *reinterpret_cast<u32x4_t *>(smem + S::rv + off) = pv;
      if (t < kBT) reinterpret_cast<float *>(smem + S::beta)[t] = (p.beta_logits && t < L) ? sigmoid_f32(pb) : pb;
    }
    float glc[kBT];
#pragma unroll
    for (int r = 0; r < kBT; ++r) glc[r] = gl[r];
    if (blk + 1 < nb) fetch(blk + 1);
    __syncthreads();  // the raw block and this block's flag are visible
    // the whole block at once, or (any exponent out of range) one token at a time
    const bool fast = flags[blk & 1] == 0;
    const int Ls = fast ? L : 1;
    for (int r0 = 0; r0 < L; r0 += Ls) {
      if (w < 2)
        operands(std::integral_constant<int, 0>{}, glc, fast, r0, Ls);
      else
        operands(std::integral_constant<int, 1>{}, glc, fast, r0, Ls);
      __syncthreads();
      if (r0 + Ls >= L) {
        // last pass of the block: clear this block's flag for block + 2 and check
        // the next block, both before the products' final barrier
        if (tid_opaque() == 0) flags[blk & 1] = 0;
        if (blk + 1 < nb) {
          wait_vmem();
          gate_and_check(blk + 1);
        }
      }
      products(t0 + r0, r0, Ls);
    }
  }

  // ---- state store (an empty slot updated in place keeps its bits)
  if (p.ht && !(sr.len == 0 && p.ht == p.h0)) {
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int ln = tid_opaque() & 63;
        float *dst = p.ht + sbase + (int64_t)(16 * t + 4 * (ln >> 4)) * kBD + col0 + 16 * ct + (ln & 15);
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[i * kBD] = Sx[ct][t][i];
      }
  }
}

}  // namespace

bool recurrent_block_supported(const RecurrentParams &p) {
  return p.is_bf16 && p.K == kBD && p.V == kBD && p.gate_kind != kGateLog2Cumsum && p.T > 1 &&
         (p.cu == nullptr || p.T > p.N);
}

hipError_t launch_recurrent_block(const RecurrentParams &p, hipStream_t st) {
  const int grid = p.N * p.H;
  if (grid == 0) return hipSuccess;
  constexpr size_t smem = BlkSmem::total;
  auto pick = [&](auto gk) {
    constexpr int GK = decltype(gk)::value;
    return p.q_l2norm ? recurrent_block_kernel<true, GK> : recurrent_block_kernel<false, GK>;
  };
  decltype(pick(std::integral_constant<int, kGateLog2>{})) kern;
  switch (p.gate_kind) {
    case kGateLog2: kern = pick(std::integral_constant<int, kGateLog2>{}); break;
    case kGateLogE: kern = pick(std::integral_constant<int, kGateLogE>{}); break;
    case kGateSafe: kern = pick(std::integral_constant<int, kGateSafe>{}); break;
    case kGateSoftplus: kern = pick(std::integral_constant<int, kGateSoftplus>{}); break;
    default: return hipErrorInvalidValue;
  }
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kBThreads), smem, st, p);
  return hipGetLastError();
}

}  // namespace kda
