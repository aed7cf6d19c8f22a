// LDS layout of the fused chunk kernel, and the register-staged loader of one
// chunk's raw inputs; the split schedule's key side shares both.
#pragma once

#include "chunk_fused_tiles.h"
#include "kda_launch.h"

namespace kda {

template <int C, int D, int NT>
struct FusedSmem {
  using TL = Tile<bf16_t, C, D>;
  static constexpr int LDT = TL::LDT;   // q, k, v, k~ [C][LDT] bf16
  static constexpr int LDB = TL::LDB;   // gate / b [C][LDB] fp32; o staging [C][LDB] fp32
  static constexpr int LDA = TL::LDA;   // A_kk, A_qk [C][LDA] fp32
  static constexpr int LDW = C + 8;     // w^T [D][LDW] bf16
  static constexpr int LDTD = 16 + 8;   // diagonal inverses [C][LDTD] bf16
  static constexpr size_t tile = 2 * C * LDT;
  static constexpr size_t q = 0;
  static constexpr size_t k = q + tile;
  static constexpr size_t v = k + tile;
  // the b region later holds X_w = beta k 2^b ([C][LDT] bf16) and w^T after it
  static constexpr size_t xw_off = 0, wt_off = tile;
  static constexpr size_t breg = (4 * C * LDB > tile + 2 * D * LDW) ? 4 * C * LDB : tile + 2 * D * LDW;
  static constexpr size_t b = v + tile;
  static constexpr size_t akk = b + breg;
  static constexpr size_t kt = akk + 4 * C * LDA;
  static constexpr size_t aqk = kt + tile;
  static constexpr int LDAH = C + 8;    // A_qk [C][LDAH] bf16
  static constexpr size_t aqh = aqk + 4 * C * LDA;
  static constexpr size_t td = aqh + 2 * C * LDAH;
  static constexpr size_t t1 = td + 2 * C * LDTD;     // scale 2^m_i per row block and channel, fp32 [C/16][D]
  static constexpr size_t t2 = t1 + 4 * (C / 16) * D;  // 2^(b_L - m_i)
  static constexpr size_t t0 = t2 + 4 * (C / 16) * D;  // 2^(m_i - a_i)
  static constexpr size_t beta = t0 + 4 * (C / 16) * D;
  static constexpr size_t bl = beta + 4 * C;
  static constexpr size_t decay = bl + 4 * D;
  static constexpr size_t dt = decay + 2 * 4 * D;  // decay: two chunks (the state update trails by one)
  static constexpr size_t seg = dt + 4 * D;
  static constexpr size_t qn = seg + 4 * NT;  // per chunk row: 1/sqrt(|q|^2 + eps) (q_l2norm)
  // with four channel shares in the grams, their extra partial sums: fp32 [4][C][LDA];
  // and on 32-row chunks block pair (1, 0)'s column operand, 16-byte fragments
  // [4 shares][D / 128 steps][64 lanes]
  static constexpr bool SHARES4 = gram_shares<NT / 64, C / 16>() == 4;
  static constexpr size_t part = qn + 4 * C;
  static constexpr size_t xc = part + (SHARES4 ? 4 * 4 * C * LDA : 0);
  static constexpr size_t total = xc + ((SHARES4 && C == 32) ? 4 * (D / 128) * 64 * 16 : 0);
  static_assert(total <= 160 * 1024, "LDS");
};

// One chunk's raw inputs held in registers between the HBM load and the LDS store.
// q, k and v are loaded and stored by NL threads (loader index in [0, NL)):
// all of them, one wave of each pair 2m, 2m + 1 (the pair's first half of the
// grams), which issues those loads while the other inverts a diagonal block,
// or (LOW) the first NT / 2 threads. The gate input and beta use every thread.
template <typename Tin, int C, int D, int NT, int NL, bool LOW = false>
struct ChunkRegs {
  static constexpr int EPV = 16 / (int)sizeof(Tin);
  static constexpr int VPR = D / EPV, NVT = C * VPR, IT = (NVT + NL - 1) / NL;  // q, k, v tiles
  static constexpr int XPR = D / 4, NVX = C * XPR, IX = (NVX + NT - 1) / NT;    // gate tile (fp32)
  // the q/k/v loader index of this thread (valid on loader waves)
  static __device__ __forceinline__ unsigned loader_index() {
    const unsigned t = (unsigned)tid_opaque();
    return (NL == NT || LOW) ? t : (((t >> 7) << 6) | (t & 63));
  }
  u32x4_t q[IT], k[IT], v[IT];
  f32x4_t x[IX];
  float beta;

  // The chunk's first element is a uniform base pointer; each vector is a
  // 32-bit unsigned element offset from it, so the loads take the
  // scalar-base + vector-offset form.
  // q, k, v of the chunk at t0
  __device__ __forceinline__ void load_qkv(const ChunkParams &p, int64_t t0, int L, int h) {
    const unsigned ld = (unsigned)p.H * p.Vr, ldk = (unsigned)p.Hk * p.Kr;
    const int64_t base = t0 * (int64_t)ld + (int64_t)h * p.Vr;
    const int64_t basek = t0 * (int64_t)ldk + (int64_t)(h / (p.H / p.Hk)) * p.Kr;  // q/k head of value head h
    const Tin *gq = reinterpret_cast<const Tin *>(p.q) + basek;
    const Tin *gk = reinterpret_cast<const Tin *>(p.k) + basek;
    const Tin *gv = reinterpret_cast<const Tin *>(p.v) + base;
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const unsigned idx = it * NL + loader_index();
      const int r = idx / VPR, c = (idx % VPR) * EPV;
      const bool ok = (NVT % NL == 0 || idx < NVT) && r < L;
      const unsigned off = (unsigned)r * ld + (unsigned)c, offk = (unsigned)r * ldk + (unsigned)c;
      const u32x4_t z = {0u, 0u, 0u, 0u};
      // channels >= Kr and value columns >= Vr are zeros (whole vectors: widths are multiples of 8)
      q[it] = ok && c < p.Kr ? *reinterpret_cast<const u32x4_t *>(gq + offk) : z;
      k[it] = ok && c < p.Kr ? *reinterpret_cast<const u32x4_t *>(gk + offk) : z;
      v[it] = ok && c < p.Vr ? *reinterpret_cast<const u32x4_t *>(gv + off) : z;
    }
  }

  // gate input and beta of the chunk at t0
  __device__ __forceinline__ void load_gate(const ChunkParams &p, int64_t t0, int L, int h) {
    const unsigned ld = (unsigned)p.H * p.Kr;
    const int64_t base = t0 * (int64_t)ld + (int64_t)h * p.Kr;
    const float *gx = p.g + base;
#pragma unroll
    for (int it = 0; it < IX; ++it) {
      const unsigned idx = it * NT + (unsigned)tid_opaque();
      const int r = idx / XPR, c = (idx % XPR) * 4;
      const bool ok = (NVX % NT == 0 || idx < NVX) && r < L && c < p.Kr;
      const unsigned off = (unsigned)r * ld + (unsigned)c;
      x[it] = ok ? *reinterpret_cast<const f32x4_t *>(gx + off) : zero4();
    }
    const int r = tid_opaque();
    beta = (r < C && r < L) ? p.beta[(t0 + r) * p.H + h] : 0.f;
  }

  // q, k, v to their tiles; the gate input, activated, to sB (rows >= L: 0).
  // For the safe gate sDt holds dt_bias * c1 with c1 = -exp(A_log) log2(e),
  // so the sigmoid's exponent is one fma.
  template <int GK>
  __device__ __forceinline__ void store(bool loader, Tin *sQ, Tin *sK, Tin *sV, float *sB, float *sBeta,
                                        const float *sDt, int L, float expA, float lower_bound, bool qnorm,
                                        float *sQn, bool blogit) const {
    using TL = Tile<Tin, C, D>;
    wait_vmem();
    if (loader && qnorm) {
      // 1/sqrt(|q_r|^2 + eps) per row: a row's VPR vectors sit on VPR adjacent lanes
      static_assert((VPR & (VPR - 1)) == 0 && VPR <= 64 && (NL % VPR) == 0, "rows within a wave");
#pragma unroll
      for (int it = 0; it < IT; ++it) {
        const unsigned idx = it * NL + loader_index();
        float ss = 0.f;
        if (NVT % NL == 0 || idx < NVT) {
          const bf16x8_t x = __builtin_bit_cast(bf16x8_t, q[it]);
#pragma unroll
          for (int e = 0; e < 8; ++e) ss = fmaf(static_cast<float>(x[e]), static_cast<float>(x[e]), ss);
        }
#pragma unroll
        for (int m = 1; m < VPR; m <<= 1) ss += __shfl_xor(ss, m);
        if ((NVT % NL == 0 || idx < NVT) && idx % VPR == 0) sQn[idx / VPR] = rsqrtf(ss + kQNormEps);
      }
    }
    if (loader)
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const unsigned idx = it * NL + loader_index();
      const unsigned r = idx / VPR, c = (idx % VPR) * EPV;
      if (NVT % NL == 0 || idx < NVT) {
        *reinterpret_cast<u32x4_t *>(sQ + r * TL::LDT + c) = q[it];
        *reinterpret_cast<u32x4_t *>(sK + r * TL::LDT + c) = k[it];
        *reinterpret_cast<u32x4_t *>(sV + r * TL::LDT + c) = v[it];
      }
    }
    const float c1 = -expA * kLog2e, c2 = lower_bound * kLog2e;
#pragma unroll
    for (int it = 0; it < IX; ++it) {
      const unsigned idx = it * NT + (unsigned)tid_opaque();
      const unsigned r = idx / XPR, c = (idx % XPR) * 4;
      if (NVX % NT == 0 || idx < NVX) {
        const f32x4_t dt = *reinterpret_cast<const f32x4_t *>(sDt + c);
        f32x4_t la;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if constexpr (GK == kGateSafe)
            la[e] = c2 * fast_rcp(1.0f + fast_exp2(fmaf(x[it][e], c1, dt[e])));
          else
            la[e] = gate_log2(GK, x[it][e], dt[e], expA, lower_bound);
        }
        // rows >= L were loaded as zeros, so the activation is finite there
        if (L < C && (int)r >= L) la = zero4();
        *reinterpret_cast<f32x4_t *>(sB + r * TL::LDB + c) = la;
      }
    }
    if (tid_opaque() < C) sBeta[tid_opaque()] = (blogit && tid_opaque() < L) ? sigmoid_f32(beta) : beta;
  }
};

}  // namespace kda
