// Backward of the chunked KDA forward, staged. The forward's steps (1)-(5)
// are recomputed first by the staged forward kernels (gate cumsum b, A_kk,
// A_qk, T, w, u, v_new and the chunk-start states h_c in the workspace); then,
// per chunk of L <= C rows with state h at its start and h' after it, and
// with q~ = scale q 2^b, k~ = k 2^(b_L - b), lambda = 2^b_L, X_w = beta k 2^b,
// X_u = beta v:
//
//   scan   (reverse over chunks, per (sequence, head, 64 value columns)):
//            dv_new = A_qk^T do + k~ dh'
//            dh     = lambda dh' + q~^T do - w^T dv_new
//   V contractions (per chunk and head):
//            dq~ = do h^T, dk~ = v_new dh'^T, dw = -dv_new h^T,
//            dA_qk = lower(do v_new^T), dT_u = dv_new X_u^T, dlambda = rowsum(h * dh')
//   WY     (per chunk and head): dT = dw X_w^T + dT_u, dX_w = T^T dw, dX_u = T^T dv_new,
//            dA_kk = -strict_lower(T^T dT T^T), dv = beta dX_u
//   grams  (per chunk and head): the decay factors 2^(b_r - b_s) per pair give
//            dq, dk and the gradient dB of the natural-log cumsum; dg is its
//            reverse cumsum within the chunk, carried through the gate activation
//   params reduce the per-chunk sums of dA_log and ddt_bias.
//
// Every product runs on the fp32 matrix cores (v_mfma_f32_16x16x4_f32) from
// LDS operands; the pair sums of the grams step run on the vector units. The
// method's backward is named, not printed, on the pages ("FLA KDA Skill",
// "Public code map": chunk_kda_bwd, chunk_kda_bwd_intra,
// chunk_kda_bwd_wy_dqkg_fused); the steps above are the reverse mode of the
// forward steps as the chunked forward computes them.
#include "chunk_loc.h"
#include "chunk_fused_tiles.h"
#include "chunk_tiles.h"
#include "kda_launch.h"

namespace kda {

namespace {

constexpr int kBT = 256;  // threads per workgroup (4 waves)

// One 16x16 tile of a product of fp32 LDS operands:
//   acc += sum over k < KN of A(m0 + m, k) B(k, n0 + n),
// A(m, k) = A[m * am + k * ak], B(k, n) = B[k * bk + n * bn]. Lane l feeds
// A(m0 + l % 16, k0 + l / 16) and B(k0 + l / 16, n0 + l % 16); the result gives
// lane l rows m0 + 4 (l / 16) + e, e = 0..3, of column n0 + l % 16.
template <int KN>
__device__ __forceinline__ f32x4_t mm16(f32x4_t acc, const float *A, int am, int ak, const float *B, int bk, int bn,
                                       int m0, int n0) {
  const int lane = tid_opaque() & 63, r = lane & 15, g = lane >> 4;  // recomputed per use, never hoisted
  const float *pa = A + (m0 + r) * am + g * ak;
  const float *pb = B + g * bk + (n0 + r) * bn;
#pragma unroll 8
  for (int k0 = 0; k0 < KN; k0 += 4) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(pa[k0 * ak], pb[k0 * bk], acc, 0, 0, 0);
  return acc;
}

// A [ROWS][COLS] fp32 LDS tile (row stride lds, a multiple of 4) from global rows
// of T (row stride ldg elements) with 16-byte loads: 4 fp32 or 8 bf16 columns
// per load. Rows >= L and columns >= ncol read as 0 (ncol, ldg and the base
// are multiples of the vector width). fn(r, c, v) may then rewrite the EPV
// values of row r, columns c.. before they are stored.
template <typename T, int ROWS, int COLS, typename Fn>
__device__ __forceinline__ void tile_f32(float *s, int lds, const T *g, int64_t ldg, int L, int ncol, Fn &&fn) {
  constexpr int EPV = 16 / (int)sizeof(T);
  constexpr int VPR = COLS / EPV, NV = ROWS * VPR;
  static_assert(COLS % EPV == 0, "whole vectors per row");
#pragma unroll 4
  for (int idx = threadIdx.x; idx < NV; idx += kBT) {
    const int r = idx / VPR, c = (idx % VPR) * EPV;
    float v[EPV];
    if (r < L && c < ncol) {
      const u32x4_t raw = *reinterpret_cast<const u32x4_t *>(g + (int64_t)r * ldg + c);
      if constexpr (sizeof(T) == 4) {
        const f32x4_t f = __builtin_bit_cast(f32x4_t, raw);
#pragma unroll
        for (int e = 0; e < EPV; ++e) v[e] = f[e];
      } else {
        const bf16x8_t f = __builtin_bit_cast(bf16x8_t, raw);
#pragma unroll
        for (int e = 0; e < EPV; ++e) v[e] = static_cast<float>(f[e]);
      }
    } else {
#pragma unroll
      for (int e = 0; e < EPV; ++e) v[e] = 0.f;
    }
    fn(r, c, v);
#pragma unroll
    for (int e = 0; e < EPV; e += 4)
      *reinterpret_cast<f32x4_t *>(s + r * lds + c + e) = f32x4_t{v[e], v[e + 1], v[e + 2], v[e + 3]};
  }
}

template <typename T, int ROWS, int COLS>
__device__ __forceinline__ void tile_f32(float *s, int lds, const T *g, int64_t ldg, int L, int ncol) {
  tile_f32<T, ROWS, COLS>(s, lds, g, ldg, L, ncol, [](int, int, float *) {});
}

// 4 fp32 values at p (16-byte aligned)
__device__ __forceinline__ f32x4_t ld4(const float *p) { return *reinterpret_cast<const f32x4_t *>(p); }

__device__ __forceinline__ int tile_row(int e) { return 4 * ((tid_opaque() & 63) >> 4) + e; }
__device__ __forceinline__ int tile_col() { return tid_opaque() & 15; }

__device__ __forceinline__ float beta_at(const ChunkParams &p, int64_t row, int h) {
  const float b = p.beta[row * p.H + h];
  return p.beta_logits ? sigmoid_f32(b) : b;
}

// Sums over aligned groups of 8 or 16 lanes through DPP (two quad permutes,
// then the half-row and the row mirror), every lane of a group left with the
// group's sum. Each step adds the same pair of partial sums as a lane shuffle by
// xor 1, 2, 4, 8 would, so the results are the same; the operands move on the
// VALU's own crossbar instead of the LDS permute network.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float lanes8_sum(float x) {
  x += dpp_mov<0xB1>(x);   // quad_perm [1, 0, 3, 2]
  x += dpp_mov<0x4E>(x);   // quad_perm [2, 3, 0, 1]
  x += dpp_mov<0x141>(x);  // row_half_mirror: lane i and 7 - i of each half-row
  return x;
}
__device__ __forceinline__ float lanes16_sum(float x) {
  x = lanes8_sum(x);
  return x + dpp_mov<0x140>(x);  // row_mirror: lane i and 15 - i of each row
}

// Raw buffer stores: offsets at or past `bytes` are dropped, so the masked rows
// and channels of a tile need no branches.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t store_rsrc(void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(base, (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ void bstore_f32(rsrc_t r, uint32_t voff, float x) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), r, (int)voff, 0, 0);
}

// ---- scan: dv_new and the state gradients, reverse over the chunks ----
// One workgroup per (sequence, head), D / 16 waves; wave w keeps the state
// gradient of value columns 16w .. 16w + 15 in accumulator registers (C layout:
// tile t holds channels 16t + 4(l/16) + e of column l % 16), which serve
// unchanged as the B operand of the product with k~ under the contraction map
// of Mma<float>. A chunk's operands (A_qk, do, k~, q~, w, b_L) each have an
// LDS buffer, written from registers when the chunk starts; the loads of the
// chunk before it (the next in the reverse walk) are issued right after, so
// they are in flight while this chunk's products run.
template <int C, int D>
struct ScanSmem {
  static constexpr int LA = C + 4, LX = D + 4;
  static constexpr size_t a = 0;                // fp32 [C][LA] A_qk, causal
  static constexpr size_t dO = a + 4 * C * LA;  // fp32 [C][LX] do (value columns)
  static constexpr size_t k = dO + 4 * C * LX;  // fp32 [C][LX] k~ = k 2^(b_L - b)
  static constexpr size_t q = k + 4 * C * LX;   // q~ = scale q 2^b
  static constexpr size_t w = q + 4 * C * LX;   // w
  static constexpr size_t bl = w + 4 * C * LX;  // fp32 [D] b_L
  static constexpr size_t total = bl + 4 * D;
  static_assert(total <= 160 * 1024, "LDS");
};

// One chunk's scan operands in registers, between their global loads and the
// LDS stores. Thread t covers the same channel vector (t % VPR) in every row it
// loads, so one b_L vector pair serves all of its k rows.
template <typename Tin, int C, int D, int NT>
struct ScanRegs {
  static constexpr int EPV = 16 / (int)sizeof(Tin), NB = EPV / 4;  // inputs per vector; b vectors per input vector
  static constexpr int NA = C * C / 4, IA = (NA + NT - 1) / NT;     // A_qk vectors
  static constexpr int VPR = D / EPV, NI = C * VPR, II = (NI + NT - 1) / NT;  // do, k, q vectors
  static constexpr int NF = C * D / 4, IF = (NF + NT - 1) / NT;     // w vectors
  static_assert(NT % VPR == 0, "one channel vector per thread");
  u32x4_t a[IA], dO[II], k[II], q[II], w[IF];
  f32x4_t b[II][NB], bl[NB];

  __device__ __forceinline__ void load(const ChunkParams &p, const BwdParams &bw, int64_t t0, int L, int h) {
    const int t = threadIdx.x;
    const int64_t ld = (int64_t)p.H * D, ldc = (int64_t)p.H * C, ldk = (int64_t)p.H * p.Kr, ldv = (int64_t)p.H * p.Vr;
    const u32x4_t z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int it = 0; it < IA; ++it) {
      const int idx = it * NT + t, r = idx / (C / 4), c = (idx % (C / 4)) * 4;
      a[it] = ((NA % NT == 0 || idx < NA) && r < L)
                  ? *reinterpret_cast<const u32x4_t *>(p.Aqk + (t0 + r) * ldc + h * C + c) : z;
    }
    const Tin *gdo = reinterpret_cast<const Tin *>(bw.dout) + t0 * ldv + h * p.Vr;
    const Tin *gk = reinterpret_cast<const Tin *>(p.k) + t0 * ldk + h * p.Kr;
    const Tin *gq = reinterpret_cast<const Tin *>(p.q) + t0 * ldk + h * p.Kr;
    const float *gb = p.b + t0 * ld + h * D;
#pragma unroll
    for (int it = 0; it < II; ++it) {
      const int idx = it * NT + t, r = idx / VPR, c = (idx % VPR) * EPV;
      const bool ok = (NI % NT == 0 || idx < NI) && r < L;
      dO[it] = ok && c < p.Vr ? *reinterpret_cast<const u32x4_t *>(gdo + r * ldv + c) : z;
      k[it] = ok && c < p.Kr ? *reinterpret_cast<const u32x4_t *>(gk + r * ldk + c) : z;
      q[it] = ok && c < p.Kr ? *reinterpret_cast<const u32x4_t *>(gq + r * ldk + c) : z;
#pragma unroll
      for (int j = 0; j < NB; ++j) b[it][j] = ok ? ld4(gb + r * ld + c + 4 * j) : zero4();
    }
    const int c0 = (t % VPR) * EPV;
#pragma unroll
    for (int j = 0; j < NB; ++j) bl[j] = L > 0 ? ld4(gb + (int64_t)(L - 1) * ld + c0 + 4 * j) : zero4();
  }

  // w, loaded apart from the rest (later in the chunk before, where fewer registers are live)
  __device__ __forceinline__ void load_w(const ChunkParams &p, int64_t t0, int L, int h) {
    const int t = threadIdx.x;
    const int64_t ld = (int64_t)p.H * D;
    const u32x4_t z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int it = 0; it < IF; ++it) {
      const int idx = it * NT + t, r = idx / (D / 4), c = (idx % (D / 4)) * 4;
      w[it] = ((NF % NT == 0 || idx < NF) && r < L)
                  ? *reinterpret_cast<const u32x4_t *>(p.w + (t0 + r) * ld + h * D + c) : z;
    }
  }

  // the EPV inputs of a vector as floats
  static __device__ __forceinline__ void unpack(u32x4_t raw, float (&v)[EPV]) {
    if constexpr (sizeof(Tin) == 4) {
      const f32x4_t f = __builtin_bit_cast(f32x4_t, raw);
#pragma unroll
      for (int e = 0; e < EPV; ++e) v[e] = f[e];
    } else {
      const bf16x8_t f = __builtin_bit_cast(bf16x8_t, raw);
#pragma unroll
      for (int e = 0; e < EPV; ++e) v[e] = static_cast<float>(f[e]);
    }
  }

  __device__ __forceinline__ void store(char *smem, float scale) const {
    using S = ScanSmem<C, D>;
    const int t = threadIdx.x;
    float *sA = reinterpret_cast<float *>(smem + S::a), *sDo = reinterpret_cast<float *>(smem + S::dO);
    float *sK = reinterpret_cast<float *>(smem + S::k), *sQ = reinterpret_cast<float *>(smem + S::q);
    float *sW = reinterpret_cast<float *>(smem + S::w), *sBL = reinterpret_cast<float *>(smem + S::bl);
#pragma unroll
    for (int it = 0; it < IA; ++it) {
      const int idx = it * NT + t, r = idx / (C / 4), c = (idx % (C / 4)) * 4;
      if (NA % NT == 0 || idx < NA) {
        f32x4_t v = __builtin_bit_cast(f32x4_t, a[it]);
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (c + e <= r) ? v[e] : 0.f;
        *reinterpret_cast<f32x4_t *>(sA + r * S::LA + c) = v;
      }
    }
#pragma unroll
    for (int it = 0; it < II; ++it) {
      const int idx = it * NT + t, r = idx / VPR, c = (idx % VPR) * EPV;
      if (NI % NT == 0 || idx < NI) {
        float fo[EPV], fk[EPV], fq[EPV];
        unpack(dO[it], fo);
        unpack(k[it], fk);
        unpack(q[it], fq);
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          f32x4_t ko, qo;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            ko[e] = fk[4 * j + e] * fast_exp2(bl[j][e] - b[it][j][e]);
            qo[e] = fq[4 * j + e] * (scale * fast_exp2(b[it][j][e]));
          }
          *reinterpret_cast<f32x4_t *>(sDo + r * S::LX + c + 4 * j) =
              f32x4_t{fo[4 * j], fo[4 * j + 1], fo[4 * j + 2], fo[4 * j + 3]};
          *reinterpret_cast<f32x4_t *>(sK + r * S::LX + c + 4 * j) = ko;
          *reinterpret_cast<f32x4_t *>(sQ + r * S::LX + c + 4 * j) = qo;
        }
      }
    }
#pragma unroll
    for (int it = 0; it < IF; ++it) {
      const int idx = it * NT + t, r = idx / (D / 4), c = (idx % (D / 4)) * 4;
      if (NF % NT == 0 || idx < NF) *reinterpret_cast<u32x4_t *>(sW + r * S::LX + c) = w[it];
    }
    if (t < VPR) {
#pragma unroll
      for (int j = 0; j < NB; ++j) *reinterpret_cast<f32x4_t *>(sBL + t * EPV + 4 * j) = bl[j];
    }
  }
};

template <typename Tin, int C, int D>
__global__ __launch_bounds__(4 * D) void bwd_scan_kernel(ChunkParams p, BwdParams bw) {
  using M = Mma<float>;
  using S = ScanSmem<C, D>;
  constexpr int NT = 4 * D, NC = C / 16, DT = D / 16, LA = S::LA, LX = S::LX;
  const int nh = blockIdx.x;
  const int n = nh / p.H, h = nh % p.H;
  const int wid = wave_id();
  const int n16 = tid_opaque() & 15, grp = (tid_opaque() & 63) >> 4;
  const int jc = 16 * wid + n16;  // this lane's value column
  const int Kr = p.Kr, Vr = p.Vr;
  const SlotRange sr = slot_range(p.cu, n, p.T);
  const int nch = (sr.len + C - 1) / C;
  const int cbase = p.cu ? p.chunk_off[n] : n * ((p.T + C - 1) / C);
  const int64_t sbase = (int64_t)nh * Kr * Vr;
  const int64_t ld = (int64_t)p.H * D;
  extern __shared__ __align__(16) char smem[];
  const float *sA = reinterpret_cast<const float *>(smem + S::a), *sDo = reinterpret_cast<const float *>(smem + S::dO);
  const float *sK = reinterpret_cast<const float *>(smem + S::k), *sQ = reinterpret_cast<const float *>(smem + S::q);
  const float *sW = reinterpret_cast<const float *>(smem + S::w), *sBL = reinterpret_cast<const float *>(smem + S::bl);

  f32x4_t dh[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = 16 * t + tile_row(e);
      dh[t][e] = (bw.dht && i < Kr && jc < Vr) ? bw.dht[sbase + (int64_t)i * Vr + jc] : 0.f;
    }
  ScanRegs<Tin, C, D, NT> R;
  if (nch > 0) {
    const int c = nch - 1;
    R.load(p, bw, sr.t0 + (int64_t)c * C, min(C, sr.len - c * C), h);
    R.load_w(p, sr.t0 + (int64_t)c * C, min(C, sr.len - c * C), h);
  }
  for (int c = nch - 1; c >= 0; --c) {
    const int64_t t0 = sr.t0 + (int64_t)c * C;
    const int L = min(C, sr.len - c * C);
    const int64_t gc = cbase + c;
    R.store(smem, p.scale);
    // gradient of the state after this chunk (channels past Kr fall outside the range)
    if (jc < Vr) {
      const rsrc_t rdh = store_rsrc(bw.dhn + (gc * p.H + h) * Kr * Vr, (uint32_t)(Kr * Vr) * 4u);
#pragma unroll
      for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) bstore_f32(rdh, (uint32_t)((16 * t + tile_row(e)) * Vr + jc) * 4u, dh[t][e]);
    }
    __syncthreads();
    if (c > 0) R.load(p, bw, t0 - C, C, h);  // every chunk but a slot's last has C rows
    // dv_new = A_qk^T do + k~ dh (rows past L fall outside the range)
    const rsrc_t rdv = store_rsrc(bw.dvn + t0 * ld + h * D, (uint32_t)((L - 1) * ld + D) * 4u);
    f32x4_t dv[NC];
#pragma unroll
    for (int rt = 0; rt < NC; ++rt) {
      f32x4_t acc = mm16<C>(zero4(), sA, 1, LA, sDo, LX, 1, 16 * rt, 16 * wid);
#pragma unroll
      for (int st = 0; st < D / 4; ++st)
        acc = M::mma(sK[(16 * rt + n16) * LX + M::kidx(st, grp, 0)], dh[st >> 2][st & 3], acc);  // dh: registers
      dv[rt] = acc;
#pragma unroll
      for (int e = 0; e < 4; ++e) bstore_f32(rdv, (uint32_t)((16 * rt + tile_row(e)) * ld + jc) * 4u, acc[e]);
    }
    if (c > 0) R.load_w(p, t0 - C, C, h);
    // dh <- 2^b_L dh + q~^T do - w^T dv_new (dv_new from registers, under the same contraction map)
#pragma unroll
    for (int t = 0; t < DT; ++t) {
      f32x4_t acc = mm16<C>(zero4(), sQ, 1, LX, sDo, LX, 1, 16 * t, 16 * wid);
      f32x4_t wv = zero4();
#pragma unroll
      for (int st = 0; st < C / 4; ++st)
        wv = M::mma(sW[M::kidx(st, grp, 0) * LX + 16 * t + n16], dv[st >> 2][st & 3], wv);
#pragma unroll
      for (int e = 0; e < 4; ++e) dh[t][e] = fast_exp2(sBL[16 * t + tile_row(e)]) * dh[t][e] + acc[e] - wv[e];
    }
    __syncthreads();  // every buffer is rewritten by the next chunk
  }
  if (bw.dh0 && jc < Vr) {
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 16 * t + tile_row(e);
        if (i < Kr) bw.dh0[sbase + (int64_t)i * Vr + jc] = dh[t][e];
      }
  }
}

// x = hi + lo + (about 2^-16 |x|), both rounded to nearest-even bf16; two dwords each
__device__ __forceinline__ void split_bf16x4(const f32x4_t &x, u32x2_t &hi, u32x2_t &lo) {
  hi = u32x2_t{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
  const float h0 = __uint_as_float(hi[0] << 16), h1 = __uint_as_float(hi[0] & 0xFFFF0000u);
  const float h2 = __uint_as_float(hi[1] << 16), h3 = __uint_as_float(hi[1] & 0xFFFF0000u);
  lo = u32x2_t{pack_bf16x2(x[0] - h0, x[1] - h1), pack_bf16x2(x[2] - h2, x[3] - h3)};
}

// ---- the scan for bf16 inputs: the same steps on the bf16 matrix cores ----
// Every product runs as 16x16x16 bf16 matrix products with fp32 operands split
// into bf16 high and low parts (x = hi + lo + about 2^-16 |x|; A B is taken as
// A_hi B_hi + A_hi B_lo + A_lo B_hi). LDS holds the chunk's tiles row-major as
// the loads deliver them (A_qk, do, k~, q~, w by token), written with wide
// stores; the products that contract over tokens read their operands with the
// transposing LDS load (load_cfrag), whose four K elements per lane are the
// rows 4g .. 4g + 3 of a 16-row block -- the layout in which dh (channels) and
// dv_new (tokens) already sit in their accumulators.
template <int C, int D>
struct ScanSplitSmem {
  static constexpr int LA = C + 8, LT = D + 8;  // bf16 row strides
  static constexpr size_t atH = 0, atL = atH + 2 * C * LA;  // [C][LA] A_qk (token k, column m), causal
  static constexpr size_t dO = atL + 2 * C * LA;            // [C][LT] do
  static constexpr size_t kH = dO + 2 * C * LT, kL = kH + 2 * C * LT;  // k~ = k 2^(b_L - b)
  static constexpr size_t qH = kL + 2 * C * LT, qL = qH + 2 * C * LT;  // q~ = scale q 2^b
  static constexpr size_t wH = qL + 2 * C * LT, wL = wH + 2 * C * LT;  // w
  static constexpr size_t bl = wL + 2 * C * LT;                        // fp32 [D] b_L
  static constexpr size_t total = bl + 4 * D;
  static_assert(total <= 160 * 1024, "LDS");
};

template <int C, int D>
__device__ __forceinline__ void scan_split_store(const ScanRegs<bf16_t, C, D, 4 * D> &R, char *smem, float scale) {
  using S = ScanSplitSmem<C, D>;
  using Rg = ScanRegs<bf16_t, C, D, 4 * D>;
  constexpr int NT = 4 * D;
  const int t = threadIdx.x;
#pragma unroll
  for (int it = 0; it < Rg::IA; ++it) {
    const int idx = it * NT + t, k = idx / (C / 4), m0 = (idx % (C / 4)) * 4;
    if (Rg::NA % NT == 0 || idx < Rg::NA) {
      f32x4_t a = __builtin_bit_cast(f32x4_t, R.a[it]);
#pragma unroll
      for (int e = 0; e < 4; ++e) a[e] = (m0 + e <= k) ? a[e] : 0.f;
      u32x2_t hi, lo;
      split_bf16x4(a, hi, lo);
      const int o = 2 * (k * S::LA + m0);
      *reinterpret_cast<u32x2_t *>(smem + S::atH + o) = hi;
      *reinterpret_cast<u32x2_t *>(smem + S::atL + o) = lo;
    }
  }
#pragma unroll
  for (int it = 0; it < Rg::II; ++it) {
    const int idx = it * NT + t, r = idx / Rg::VPR, c = (idx % Rg::VPR) * 8;
    if (Rg::NI % NT == 0 || idx < Rg::NI) {
      const int o = 2 * (r * S::LT + c);
      *reinterpret_cast<u32x4_t *>(smem + S::dO + o) = R.dO[it];
      const bf16x8_t k8 = __builtin_bit_cast(bf16x8_t, R.k[it]), q8 = __builtin_bit_cast(bf16x8_t, R.q[it]);
      u32x2_t kh[2], kl[2], qh[2], ql[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        f32x4_t kt, qt;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float bb = R.b[it][j][e];
          kt[e] = static_cast<float>(k8[4 * j + e]) * fast_exp2(R.bl[j][e] - bb);
          qt[e] = static_cast<float>(q8[4 * j + e]) * (scale * fast_exp2(bb));
        }
        split_bf16x4(kt, kh[j], kl[j]);
        split_bf16x4(qt, qh[j], ql[j]);
      }
      *reinterpret_cast<u32x4_t *>(smem + S::kH + o) = u32x4_t{kh[0][0], kh[0][1], kh[1][0], kh[1][1]};
      *reinterpret_cast<u32x4_t *>(smem + S::kL + o) = u32x4_t{kl[0][0], kl[0][1], kl[1][0], kl[1][1]};
      *reinterpret_cast<u32x4_t *>(smem + S::qH + o) = u32x4_t{qh[0][0], qh[0][1], qh[1][0], qh[1][1]};
      *reinterpret_cast<u32x4_t *>(smem + S::qL + o) = u32x4_t{ql[0][0], ql[0][1], ql[1][0], ql[1][1]};
    }
  }
#pragma unroll
  for (int it = 0; it < Rg::IF; ++it) {
    const int idx = it * NT + t, r = idx / (D / 4), c = (idx % (D / 4)) * 4;
    if (Rg::NF % NT == 0 || idx < Rg::NF) {
      u32x2_t hi, lo;
      split_bf16x4(__builtin_bit_cast(f32x4_t, R.w[it]), hi, lo);
      const int o = 2 * (r * S::LT + c);
      *reinterpret_cast<u32x2_t *>(smem + S::wH + o) = hi;
      *reinterpret_cast<u32x2_t *>(smem + S::wL + o) = lo;
    }
  }
  if (t < Rg::VPR) {
#pragma unroll
    for (int j = 0; j < Rg::NB; ++j)
      *reinterpret_cast<f32x4_t *>(reinterpret_cast<float *>(smem + S::bl) + t * 8 + 4 * j) = R.bl[j];
  }
}

// hi / lo bf16 halves of four floats, as 16x16x16 operand fragments
__device__ __forceinline__ void split4(const f32x4_t &x, bf16x4_t &hi, bf16x4_t &lo) {
  u32x2_t h, l;
  split_bf16x4(x, h, l);
  hi = __builtin_bit_cast(bf16x4_t, h);
  lo = __builtin_bit_cast(bf16x4_t, l);
}

template <int C, int D>
__global__ __launch_bounds__(4 * D) void bwd_scan_split_kernel(ChunkParams p, BwdParams bw) {
  using S = ScanSplitSmem<C, D>;
  constexpr int NT = 4 * D, NC = C / 16, DT = D / 16, LA = S::LA, LT = S::LT;
  const int nh = blockIdx.x;
  const int n = nh / p.H, h = nh % p.H;
  const int wid = wave_id();
  const int n16 = tid_opaque() & 15, grp = (tid_opaque() & 63) >> 4;
  const int jc = 16 * wid + n16;  // this lane's value column
  const int Kr = p.Kr, Vr = p.Vr;
  const SlotRange sr = slot_range(p.cu, n, p.T);
  const int nch = (sr.len + C - 1) / C;
  const int cbase = p.cu ? p.chunk_off[n] : n * ((p.T + C - 1) / C);
  const int64_t sbase = (int64_t)nh * Kr * Vr;
  const int64_t ld = (int64_t)p.H * D;
  extern __shared__ __align__(16) char smem[];
  const float *sBL = reinterpret_cast<const float *>(smem + S::bl);
  const bf16_t *atH = reinterpret_cast<const bf16_t *>(smem + S::atH), *atL = reinterpret_cast<const bf16_t *>(smem + S::atL);
  const bf16_t *dO = reinterpret_cast<const bf16_t *>(smem + S::dO);
  const bf16_t *kH = reinterpret_cast<const bf16_t *>(smem + S::kH), *kL = reinterpret_cast<const bf16_t *>(smem + S::kL);
  const bf16_t *qH = reinterpret_cast<const bf16_t *>(smem + S::qH), *qL = reinterpret_cast<const bf16_t *>(smem + S::qL);
  const bf16_t *wH = reinterpret_cast<const bf16_t *>(smem + S::wH), *wL = reinterpret_cast<const bf16_t *>(smem + S::wL);

  f32x4_t dh[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = 16 * t + tile_row(e);
      dh[t][e] = (bw.dht && i < Kr && jc < Vr) ? bw.dht[sbase + (int64_t)i * Vr + jc] : 0.f;
    }
  ScanRegs<bf16_t, C, D, NT> R;
  if (nch > 0) {
    const int c = nch - 1;
    R.load(p, bw, sr.t0 + (int64_t)c * C, min(C, sr.len - c * C), h);
    R.load_w(p, sr.t0 + (int64_t)c * C, min(C, sr.len - c * C), h);
  }
  for (int c = nch - 1; c >= 0; --c) {
    const int64_t t0 = sr.t0 + (int64_t)c * C;
    const int L = min(C, sr.len - c * C);
    const int64_t gc = cbase + c;
    scan_split_store<C, D>(R, smem, p.scale);
    // gradient of the state after this chunk (channels past Kr fall outside the range)
    if (jc < Vr) {
      const rsrc_t rdh = store_rsrc(bw.dhn + (gc * p.H + h) * Kr * Vr, (uint32_t)(Kr * Vr) * 4u);
#pragma unroll
      for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) bstore_f32(rdh, (uint32_t)((16 * t + tile_row(e)) * Vr + jc) * 4u, dh[t][e]);
    }
    __syncthreads();
    if (c > 0) R.load(p, bw, t0 - C, C, h);  // every chunk but a slot's last has C rows
    const int loA = cfrag_lane_off(LA), loT = cfrag_lane_off(LT);
    // dv_new = A_qk^T do + k~ dh (rows past L fall outside the range)
    const rsrc_t rdv = store_rsrc(bw.dvn + t0 * ld + h * D, (uint32_t)((L - 1) * ld + D) * 4u);
    bf16x4_t dhH[DT], dhL[DT];
#pragma unroll
    for (int t = 0; t < DT; ++t) split4(dh[t], dhH[t], dhL[t]);
    f32x4_t dv[NC];
#pragma unroll
    for (int rt = 0; rt < NC; ++rt) {
      f32x4_t acc = zero4();
#pragma unroll
      for (int kb = 0; kb < NC; ++kb) {
        const bf16x4_t o = load_cfrag_at(dO + 16 * kb * LT + 16 * wid, loT);
        acc = mma16(load_cfrag_at(atH + 16 * kb * LA + 16 * rt, loA), o, acc);
        acc = mma16(load_cfrag_at(atL + 16 * kb * LA + 16 * rt, loA), o, acc);
      }
      const int ko = (16 * rt + n16) * LT + 4 * grp;  // k~ row of this lane, channels 16 ib + 4 g ..
#pragma unroll
      for (int ib = 0; ib < DT; ++ib) {
        const bf16x4_t ah = *reinterpret_cast<const bf16x4_t *>(kH + ko + 16 * ib);
        const bf16x4_t al = *reinterpret_cast<const bf16x4_t *>(kL + ko + 16 * ib);
        acc = mma16(ah, dhH[ib], acc);
        acc = mma16(ah, dhL[ib], acc);
        acc = mma16(al, dhH[ib], acc);
      }
      dv[rt] = acc;
#pragma unroll
      for (int e = 0; e < 4; ++e) bstore_f32(rdv, (uint32_t)((16 * rt + tile_row(e)) * ld + jc) * 4u, acc[e]);
    }
    if (c > 0) R.load_w(p, t0 - C, C, h);
    // dh <- 2^b_L dh + q~^T do - w^T dv_new
    bf16x4_t vh[NC], vl[NC];
#pragma unroll
    for (int kb = 0; kb < NC; ++kb) split4(dv[kb], vh[kb], vl[kb]);
#pragma unroll
    for (int t = 0; t < DT; ++t) {
      f32x4_t acc = zero4(), wv = zero4();
#pragma unroll
      for (int kb = 0; kb < NC; ++kb) {
        const bf16x4_t o = load_cfrag_at(dO + 16 * kb * LT + 16 * wid, loT);
        acc = mma16(load_cfrag_at(qH + 16 * kb * LT + 16 * t, loT), o, acc);
        acc = mma16(load_cfrag_at(qL + 16 * kb * LT + 16 * t, loT), o, acc);
        const bf16x4_t ah = load_cfrag_at(wH + 16 * kb * LT + 16 * t, loT);
        wv = mma16(ah, vh[kb], wv);
        wv = mma16(ah, vl[kb], wv);
        wv = mma16(load_cfrag_at(wL + 16 * kb * LT + 16 * t, loT), vh[kb], wv);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) dh[t][e] = fast_exp2(sBL[16 * t + tile_row(e)]) * dh[t][e] + acc[e] - wv[e];
    }
    __syncthreads();  // every buffer is rewritten by the next chunk
  }
  if (bw.dh0 && jc < Vr) {
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 16 * t + tile_row(e);
        if (i < Kr) bw.dh0[sbase + (int64_t)i * Vr + jc] = dh[t][e];
      }
  }
}

// ---- contractions over the value columns ----
// Persistent workgroups of eight waves walk (chunk, head) items, each in slabs
// of SJ value columns; the next two slabs' tiles (of the same item or the next
// ones) are in flight in registers while the current slab's products run. Wave
// w accumulates its share of the output tiles over the item's slabs.
//
// The products contract over the slab's value columns on the bf16 matrix cores
// with fp32 accuracy: each fp32 operand x is held as hi = bf16(x) and
// lo = bf16(x - hi), and A B ~ A_hi B_hi + A_hi B_lo + A_lo B_hi (the dropped
// A_lo B_lo and the rounding of lo are about 2^-16 of each term); operands that
// arrive in bf16 (do, for bf16 inputs) are exact and take no lo part.

template <int C, int D>
struct ContractSmem {
  static constexpr int SJ = 32, LB = SJ + 8;  // bf16 row stride of every tile (80 bytes)
  // hi and lo tiles: do, beta v, v_new, dv_new [C][LB]; h, dh' [D][LB]
  static constexpr size_t tc = 2 * C * LB, td = 2 * D * LB;
  static constexpr size_t doH = 0, doL = doH + tc, bvH = doL + tc, bvL = bvH + tc, vnH = bvL + tc, vnL = vnH + tc;
  static constexpr size_t dvH = vnL + tc, dvL = dvH + tc, hH = dvL + tc, hL = hH + td, dhH = hL + td, dhL = dhH + td;
  static constexpr size_t beta = dhL + td;  // fp32 [C]
  static constexpr size_t total = beta + 4 * C;
  static_assert(total <= 160 * 1024, "LDS");
};

template <typename Tin, int C, int D, int NT>
struct ContractRegs {
  using S = ContractSmem<C, D>;
  static constexpr int SJ = S::SJ, EPV = 16 / (int)sizeof(Tin);
  static constexpr int VI = C * SJ / EPV, II = (VI + NT - 1) / NT;  // do, v vectors of a slab
  static constexpr int VF = C * SJ / 4, IF = (VF + NT - 1) / NT;    // v_new, dv_new
  static constexpr int VH = D * SJ / 4, IH = (VH + NT - 1) / NT;    // h, dh'
  static_assert(NT % (SJ / 4) == 0, "whole rows of h per group of threads");
  u32x4_t dO[II], v[II], vn[IF], dvn[IF], hh[IH], dh[IH];
  float beta;

  // slab j0 of the chunk at t0 (L rows, global index gci) and head h
  __device__ __forceinline__ void load(const ChunkParams &p, const BwdParams &bw, int64_t t0, int L, int gci, int h,
                                       int j0) {
    const int t = threadIdx.x;
    const int Kr = p.Kr, Vr = p.Vr, nj = Vr - j0;
    const int64_t ld = (int64_t)p.H * D, ldv = (int64_t)p.H * Vr;
    const int64_t hbase = ((int64_t)gci * p.H + h) * Kr * Vr + j0;
    const Tin *gdo = reinterpret_cast<const Tin *>(bw.dout) + t0 * ldv + h * Vr + j0;
    const Tin *gv = reinterpret_cast<const Tin *>(p.v) + t0 * ldv + h * Vr + j0;
    const u32x4_t z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int it = 0; it < II; ++it) {
      const int idx = it * NT + t, r = idx / (SJ / EPV), c = (idx % (SJ / EPV)) * EPV;
      const bool ok = (VI % NT == 0 || idx < VI) && r < L && c < nj;
      dO[it] = ok ? *reinterpret_cast<const u32x4_t *>(gdo + r * ldv + c) : z;
      v[it] = ok ? *reinterpret_cast<const u32x4_t *>(gv + r * ldv + c) : z;
    }
#pragma unroll
    for (int it = 0; it < IF; ++it) {
      const int idx = it * NT + t, r = idx / (SJ / 4), c = (idx % (SJ / 4)) * 4;
      const bool ok = (VF % NT == 0 || idx < VF) && r < L && c < nj;
      const int64_t o = (t0 + r) * ld + h * D + j0 + c;
      vn[it] = ok ? *reinterpret_cast<const u32x4_t *>(p.vnew + o) : z;
      dvn[it] = ok ? *reinterpret_cast<const u32x4_t *>(bw.dvn + o) : z;
    }
#pragma unroll
    for (int it = 0; it < IH; ++it) {
      const int idx = it * NT + t, i = idx / (SJ / 4), c = (idx % (SJ / 4)) * 4;
      const bool ok = (VH % NT == 0 || idx < VH) && i < Kr && c < nj;
      const int64_t o = hbase + (int64_t)i * Vr + c;
      hh[it] = ok ? *reinterpret_cast<const u32x4_t *>(p.hc + o) : z;
      dh[it] = ok ? *reinterpret_cast<const u32x4_t *>(bw.dhn + o) : z;
    }
    if (t < C) beta = t < L ? beta_at(p, t0 + t, h) : 0.f;
  }

  static __device__ __forceinline__ void put(char *smem, size_t hiOff, size_t loOff, int r, int c, const f32x4_t &x) {
    u32x2_t hi, lo;
    split_bf16x4(x, hi, lo);
    *reinterpret_cast<u32x2_t *>(smem + hiOff + 2 * (r * S::LB + c)) = hi;
    *reinterpret_cast<u32x2_t *>(smem + loOff + 2 * (r * S::LB + c)) = lo;
  }

  // the slab's tiles to LDS as hi / lo pairs (beta of a new item first: v's rows
  // are scaled by it); adds this slab's h dh' row sums to dlam (threads that
  // lead a row group of h)
  __device__ __forceinline__ void store(char *smem, bool item_start, float (&dlam)[IH]) const {
    const int t = threadIdx.x;
    float *sBeta = reinterpret_cast<float *>(smem + S::beta);
    if (item_start) {
      if (t < C) sBeta[t] = beta;
      __syncthreads();
    }
#pragma unroll
    for (int it = 0; it < II; ++it) {
      const int idx = it * NT + t, r = idx / (SJ / EPV), c = (idx % (SJ / EPV)) * EPV;
      if (VI % NT == 0 || idx < VI) {
        const float be = sBeta[r];
        if constexpr (sizeof(Tin) == 4) {
          const f32x4_t x = __builtin_bit_cast(f32x4_t, dO[it]), y = __builtin_bit_cast(f32x4_t, v[it]);
          put(smem, S::doH, S::doL, r, c, x);
          put(smem, S::bvH, S::bvL, r, c, y * be);
        } else {
          // bf16 do is exact: its lo tile stays unused
          *reinterpret_cast<u32x4_t *>(smem + S::doH + 2 * (r * S::LB + c)) = dO[it];
          const bf16x8_t y = __builtin_bit_cast(bf16x8_t, v[it]);
          put(smem, S::bvH, S::bvL, r, c, f32x4_t{(float)y[0], (float)y[1], (float)y[2], (float)y[3]} * be);
          put(smem, S::bvH, S::bvL, r, c + 4, f32x4_t{(float)y[4], (float)y[5], (float)y[6], (float)y[7]} * be);
        }
      }
    }
#pragma unroll
    for (int it = 0; it < IF; ++it) {
      const int idx = it * NT + t, r = idx / (SJ / 4), c = (idx % (SJ / 4)) * 4;
      if (VF % NT == 0 || idx < VF) {
        put(smem, S::vnH, S::vnL, r, c, __builtin_bit_cast(f32x4_t, vn[it]));
        put(smem, S::dvH, S::dvL, r, c, __builtin_bit_cast(f32x4_t, dvn[it]));
      }
    }
#pragma unroll
    for (int it = 0; it < IH; ++it) {
      const int idx = it * NT + t, i = idx / (SJ / 4), c = (idx % (SJ / 4)) * 4;
      const f32x4_t x = __builtin_bit_cast(f32x4_t, hh[it]), y = __builtin_bit_cast(f32x4_t, dh[it]);
      float part = 0.f;
      if (VH % NT == 0 || idx < VH) {
        put(smem, S::hH, S::hL, i, c, x);
        put(smem, S::dhH, S::dhL, i, c, y);
        part = x[0] * y[0] + x[1] * y[1] + x[2] * y[2] + x[3] * y[3];
      }
      static_assert(SJ / 4 == 8, "a row's partial products on 8 adjacent lanes");
      dlam[it] += lanes8_sum(part);
    }
  }
};

// One 16x16 output tile over the slab: acc += A B^T with A rows a0.. of (aH, aL)
// and B rows b0.. of (bH, bL), both [rows][LB] bf16 with the slab's columns
// contiguous; A_lo is skipped when A is exact.
template <int LB, bool A_EXACT>
__device__ __forceinline__ f32x4_t mma_split(f32x4_t acc, const char *smem, size_t aH, size_t aL, int a0, size_t bH,
                                             size_t bL, int b0) {
  using M = Mma<bf16_t>;
  const int lane = tid_opaque() & 63, r = lane & 15, g = lane >> 4;
  const int ao = 2 * ((a0 + r) * LB + 8 * g), bo = 2 * ((b0 + r) * LB + 8 * g);
  const bf16x8_t ah = *reinterpret_cast<const bf16x8_t *>(smem + aH + ao);
  const bf16x8_t bh = *reinterpret_cast<const bf16x8_t *>(smem + bH + bo);
  const bf16x8_t bl = *reinterpret_cast<const bf16x8_t *>(smem + bL + bo);
  acc = M::mma(ah, bh, acc);
  acc = M::mma(ah, bl, acc);
  if constexpr (!A_EXACT) {
    const bf16x8_t al = *reinterpret_cast<const bf16x8_t *>(smem + aL + ao);
    acc = M::mma(al, bh, acc);
  }
  return acc;
}

constexpr int kContractThreads = 512;

template <typename Tin, int C, int D>
__global__ __launch_bounds__(kContractThreads) void bwd_contract_kernel(ChunkParams p, BwdParams bw) {
  constexpr int NT = kContractThreads, NW = NT / 64;
  using R = ContractRegs<Tin, C, D, NT>;
  using S = ContractSmem<C, D>;
  constexpr int SJ = S::SJ, LB = S::LB, NC = C / 16, DT = D / 16;
  constexpr int NTW = (NC * DT + NW - 1) / NW, NCW = (NC * NC + NW - 1) / NW;  // tiles per wave
  constexpr bool DO_EXACT = sizeof(Tin) == 2;
  static_assert(SJ == Mma<bf16_t>::KS, "one contraction step per slab");
  const int wid = threadIdx.x >> 6;
  const int total = p.cu ? p.chunk_off[p.N] : p.B * ((p.T + C - 1) / C);
  const int64_t items = (int64_t)total * p.H;
  const int nsl = (p.Vr + SJ - 1) / SJ;
  const int64_t steps = items > blockIdx.x ? ((items - 1 - blockIdx.x) / gridDim.x + 1) * nsl : 0;
  const int64_t ld = (int64_t)p.H * D, ldc = (int64_t)p.H * C;
  extern __shared__ __align__(16) char smem[];

  // step s -> item (chunk, head) and slab
  auto at = [&](int64_t st, ChunkLoc &lc, int &h, int &j0) {
    const int64_t it = blockIdx.x + (st / nsl) * gridDim.x;
    h = (int)(it % p.H);
    locate_chunk(p, (int)(it / p.H), lc);
    j0 = (int)(st % nsl) * SJ;
  };
  // two slabs' loads in flight: a slab's registers are refilled with the slab two steps on
  R regs0, regs1;
  if (steps > 0) {
    ChunkLoc lc;
    int h, j0;
    at(0, lc, h, j0);
    regs0.load(p, bw, lc.t0, lc.L, lc.gci, h, j0);
  }
  if (steps > 1) {
    ChunkLoc lc;
    int h, j0;
    at(1, lc, h, j0);
    regs1.load(p, bw, lc.t0, lc.L, lc.gci, h, j0);
  }
  float dlam[R::IH];  // row sums of h dh' for the rows this thread leads
#pragma unroll
  for (int q = 0; q < R::IH; ++q) dlam[q] = 0.f;
  f32x4_t aq[NTW], ak[NTW], aw[NTW], aa[NCW], at2[NCW];
#pragma unroll
  for (int t = 0; t < NTW; ++t) aq[t] = ak[t] = aw[t] = zero4();
#pragma unroll
  for (int t = 0; t < NCW; ++t) aa[t] = at2[t] = zero4();

  auto step = [&](int64_t st, R &regs) {
    ChunkLoc lc;
    int h, j0;
    at(st, lc, h, j0);
    regs.store(smem, j0 == 0, dlam);
    __syncthreads();
    if (st + 2 < steps) {
      ChunkLoc ln;
      int hn, jn;
      at(st + 2, ln, hn, jn);
      regs.load(p, bw, ln.t0, ln.L, ln.gci, hn, jn);
    }
#pragma unroll
    for (int t = 0; t < NTW; ++t) {
      const int tile = wid * NTW + t, rt = tile / DT, ct = tile % DT;
      if (NC * DT % NW == 0 || tile < NC * DT) {
        aq[t] = mma_split<LB, DO_EXACT>(aq[t], smem, S::doH, S::doL, 16 * rt, S::hH, S::hL, 16 * ct);    // do h^T
        ak[t] = mma_split<LB, false>(ak[t], smem, S::vnH, S::vnL, 16 * rt, S::dhH, S::dhL, 16 * ct);     // v_new dh'^T
        aw[t] = mma_split<LB, false>(aw[t], smem, S::dvH, S::dvL, 16 * rt, S::hH, S::hL, 16 * ct);       // dv_new h^T
      }
    }
#pragma unroll
    for (int t = 0; t < NCW; ++t) {
      const int tile = wid * NCW + t, rt = tile / NC, sc = tile % NC;
      if (NC * NC % NW == 0 || tile < NC * NC) {
        aa[t] = mma_split<LB, DO_EXACT>(aa[t], smem, S::doH, S::doL, 16 * rt, S::vnH, S::vnL, 16 * sc);  // do v_new^T
        at2[t] = mma_split<LB, false>(at2[t], smem, S::dvH, S::dvL, 16 * rt, S::bvH, S::bvL, 16 * sc);   // dv_new (beta v)^T
      }
    }
    if (j0 + SJ >= p.Vr) {  // the item's last slab: its outputs (rows past L fall outside the ranges)
      const int64_t t0 = lc.t0;
      const uint32_t bytes = (uint32_t)((lc.L - 1) * ld + D) * 4u, bytc = (uint32_t)((lc.L - 1) * ldc + C) * 4u;
      const rsrc_t rq = store_rsrc(bw.dqt + t0 * ld + h * D, bytes), rk = store_rsrc(bw.dkt + t0 * ld + h * D, bytes);
      const rsrc_t rw = store_rsrc(bw.dw + t0 * ld + h * D, bytes);
      const rsrc_t ra = store_rsrc(bw.dAqk + t0 * ldc + h * C, bytc), rt_ = store_rsrc(bw.dT + t0 * ldc + h * C, bytc);
#pragma unroll
      for (int t = 0; t < NTW; ++t) {
        const int tile = wid * NTW + t, rt = tile / DT, ct = tile % DT;
        if (NC * DT % NW == 0 || tile < NC * DT) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t o = (uint32_t)((16 * rt + tile_row(e)) * ld + 16 * ct + tile_col()) * 4u;
            bstore_f32(rq, o, aq[t][e]);
            bstore_f32(rk, o, ak[t][e]);
            bstore_f32(rw, o, -aw[t][e]);
          }
        }
        aq[t] = ak[t] = aw[t] = zero4();
      }
#pragma unroll
      for (int t = 0; t < NCW; ++t) {
        const int tile = wid * NCW + t, rt = tile / NC, sc = tile % NC;
        if (NC * NC % NW == 0 || tile < NC * NC) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 16 * rt + tile_row(e), s2 = 16 * sc + tile_col();
            const uint32_t o = (uint32_t)(r * ldc + s2) * 4u;
            bstore_f32(ra, o, (s2 <= r) ? aa[t][e] : 0.f);
            bstore_f32(rt_, o, at2[t][e]);
          }
        }
        aa[t] = at2[t] = zero4();
      }
      if (threadIdx.x % (SJ / 4) == 0) {
#pragma unroll
        for (int q = 0; q < R::IH; ++q) {
          const int i = (q * NT + threadIdx.x) / (SJ / 4);
          if (i < D) bw.dlam[((int64_t)lc.gci * p.H + h) * D + i] = dlam[q];
          dlam[q] = 0.f;
        }
      }
    }
    __syncthreads();  // the slab is consumed before the next one is stored
  };
  for (int64_t st = 0; st < steps; st += 2) {
    step(st, regs0);
    if (st + 1 < steps) step(st + 1, regs1);
  }
}

// ---- the WY factors and the triangular inverse ----
// Persistent workgroups of eight waves walk (chunk, head) items; the next
// item's loads are in flight while the current one computes. The products run
// on the bf16 matrix cores with fp32 operands split into high and low parts
// (as in the contractions and the scan): dT = dT_u + beta_s (dw X_w^T) and
// X = dT T^T contract along rows (16x16x32 products from row-major tiles);
// dA_kk = -T^T X, dX_w = T^T dw and dX_u = T^T dv_new contract over tokens
// (16x16x16 products, operands through the transposing LDS load).
template <int C, int D>
struct WySmem {
  static constexpr int LA = C + 8, LT = D + 8, LU = C + 4;  // bf16 strides; fp32 stride of dT_u
  static constexpr size_t tH = 0, tL = tH + 2 * C * LA;     // T [C][LA]
  static constexpr size_t dtH = tL + 2 * C * LA, dtL = dtH + 2 * C * LA;  // dT
  static constexpr size_t dwH = dtL + 2 * C * LA, dwL = dwH + 2 * C * LT;  // dw [C][LT]
  static constexpr size_t xwH = dwL + 2 * C * LT, xwL = xwH + 2 * C * LT;  // X_w = k 2^b, later X = dT T^T [C][LA]
  static constexpr size_t dvH = xwL + 2 * C * LT, dvL = dvH + 2 * C * LT;  // dv_new
  static constexpr size_t dtu = dvL + 2 * C * LT;  // fp32 [C][LU] dT_u
  static constexpr size_t beta = dtu + 4 * C * LU;  // fp32 [C]
  static constexpr size_t dbp = beta + 4 * C;      // fp32 [4][C] partial beta gradients
  static constexpr size_t total = dbp + 16 * C;
  static_assert(total <= 160 * 1024, "LDS");
};

template <typename Tin, int C, int D, int NT>
struct WyRegs {
  static constexpr int EPV = 16 / (int)sizeof(Tin), NB = EPV / 4;
  static constexpr int NA = C * C / 4, IA = (NA + NT - 1) / NT;               // T, dT_u
  static constexpr int NF = C * D / 4, IF = (NF + NT - 1) / NT;               // dw, dv_new
  static constexpr int VPR = D / EPV, NI = C * VPR, II = (NI + NT - 1) / NT;  // k
  u32x4_t tm[IA], dtu[IA], dw[IF], dvn[IF], k[II];
  f32x4_t b[II][NB];
  float beta;

  __device__ __forceinline__ void load(const ChunkParams &p, const BwdParams &bw, int64_t t0, int L, int h) {
    const int t = threadIdx.x;
    const int64_t ld = (int64_t)p.H * D, ldc = (int64_t)p.H * C, ldk = (int64_t)p.H * p.Kr;
    const u32x4_t z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int it = 0; it < IA; ++it) {
      const int idx = it * NT + t, r = idx / (C / 4), c = (idx % (C / 4)) * 4;
      const bool ok = (NA % NT == 0 || idx < NA) && r < L;
      const int64_t o = (t0 + r) * ldc + h * C + c;
      tm[it] = ok ? *reinterpret_cast<const u32x4_t *>(p.Tm + o) : z;
      dtu[it] = ok ? *reinterpret_cast<const u32x4_t *>(bw.dT + o) : z;
    }
#pragma unroll
    for (int it = 0; it < IF; ++it) {
      const int idx = it * NT + t, r = idx / (D / 4), c = (idx % (D / 4)) * 4;
      const bool ok = (NF % NT == 0 || idx < NF) && r < L;
      const int64_t o = (t0 + r) * ld + h * D + c;
      dw[it] = ok ? *reinterpret_cast<const u32x4_t *>(bw.dw + o) : z;
      dvn[it] = ok ? *reinterpret_cast<const u32x4_t *>(bw.dvn + o) : z;
    }
    const Tin *gk = reinterpret_cast<const Tin *>(p.k) + t0 * ldk + h * p.Kr;
    const float *gb = p.b + t0 * ld + h * D;
#pragma unroll
    for (int it = 0; it < II; ++it) {
      const int idx = it * NT + t, r = idx / VPR, c = (idx % VPR) * EPV;
      const bool ok = (NI % NT == 0 || idx < NI) && r < L;
      k[it] = ok && c < p.Kr ? *reinterpret_cast<const u32x4_t *>(gk + r * ldk + c) : z;
#pragma unroll
      for (int j = 0; j < NB; ++j) b[it][j] = ok ? ld4(gb + r * ld + c + 4 * j) : zero4();
    }
    if (t < C) beta = t < L ? beta_at(p, t0 + t, h) : 0.f;
  }

  static __device__ __forceinline__ void put(char *smem, size_t hiOff, size_t loOff, int o, const f32x4_t &x) {
    u32x2_t hi, lo;
    split_bf16x4(x, hi, lo);
    *reinterpret_cast<u32x2_t *>(smem + hiOff + o) = hi;
    *reinterpret_cast<u32x2_t *>(smem + loOff + o) = lo;
  }

  // L masks the columns of T and dT_u
  __device__ __forceinline__ void store(char *smem, int L) const {
    using S = WySmem<C, D>;
    const int t = threadIdx.x;
#pragma unroll
    for (int it = 0; it < IA; ++it) {
      const int idx = it * NT + t, r = idx / (C / 4), c = (idx % (C / 4)) * 4;
      if (NA % NT == 0 || idx < NA) {
        f32x4_t a = __builtin_bit_cast(f32x4_t, tm[it]), d = __builtin_bit_cast(f32x4_t, dtu[it]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          a[e] = (c + e <= r && c + e < L) ? a[e] : 0.f;
          d[e] = (c + e < L) ? d[e] : 0.f;
        }
        put(smem, S::tH, S::tL, 2 * (r * S::LA + c), a);
        *reinterpret_cast<f32x4_t *>(smem + S::dtu + 4 * (r * S::LU + c)) = d;
      }
    }
#pragma unroll
    for (int it = 0; it < IF; ++it) {
      const int idx = it * NT + t, r = idx / (D / 4), c = (idx % (D / 4)) * 4;
      if (NF % NT == 0 || idx < NF) {
        put(smem, S::dwH, S::dwL, 2 * (r * S::LT + c), __builtin_bit_cast(f32x4_t, dw[it]));
        put(smem, S::dvH, S::dvL, 2 * (r * S::LT + c), __builtin_bit_cast(f32x4_t, dvn[it]));
      }
    }
#pragma unroll
    for (int it = 0; it < II; ++it) {
      const int idx = it * NT + t, r = idx / VPR, c = (idx % VPR) * EPV;
      if (NI % NT == 0 || idx < NI) {
        float f[EPV];
        if constexpr (sizeof(Tin) == 4) {
          const f32x4_t x = __builtin_bit_cast(f32x4_t, k[it]);
#pragma unroll
          for (int e = 0; e < EPV; ++e) f[e] = x[e];
        } else {
          const bf16x8_t x = __builtin_bit_cast(bf16x8_t, k[it]);
#pragma unroll
          for (int e = 0; e < EPV; ++e) f[e] = static_cast<float>(x[e]);
        }
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          f32x4_t x;
#pragma unroll
          for (int e = 0; e < 4; ++e) x[e] = f[4 * j + e] * fast_exp2(b[it][j][e]);
          put(smem, S::xwH, S::xwL, 2 * (r * S::LT + c + 4 * j), x);
        }
      }
    }
    if (t < C) reinterpret_cast<float *>(smem + S::beta)[t] = beta;
  }
};

// acc += A B^T over K columns k0 .. k0 + 31 of two [rows][ld] bf16 hi / lo tile pairs
template <int LDR>
__device__ __forceinline__ f32x4_t mma_split_rows(f32x4_t acc, const char *smem, size_t aH, size_t aL, int a0,
                                                  size_t bH, size_t bL, int b0, int k0) {
  using M = Mma<bf16_t>;
  const int lane = tid_opaque() & 63, r = lane & 15, g = lane >> 4;
  const int ao = 2 * ((a0 + r) * LDR + k0 + 8 * g), bo = 2 * ((b0 + r) * LDR + k0 + 8 * g);
  const bf16x8_t ah = *reinterpret_cast<const bf16x8_t *>(smem + aH + ao);
  const bf16x8_t al = *reinterpret_cast<const bf16x8_t *>(smem + aL + ao);
  const bf16x8_t bh = *reinterpret_cast<const bf16x8_t *>(smem + bH + bo);
  const bf16x8_t bl = *reinterpret_cast<const bf16x8_t *>(smem + bL + bo);
  acc = M::mma(ah, bh, acc);
  acc = M::mma(ah, bl, acc);
  return M::mma(al, bh, acc);
}

// acc += A^T B over 16-token blocks: A [C][lda] and B [C][ldb] bf16 hi / lo pairs
// (row = token), output rows a0 .., columns b0 ..
template <int C, int LDA_, int LDB_>
__device__ __forceinline__ f32x4_t mma_split_tokens(f32x4_t acc, const char *smem, size_t aH, size_t aL, int a0,
                                                    size_t bH, size_t bL, int b0, int loA, int loB) {
  const bf16_t *pAh = reinterpret_cast<const bf16_t *>(smem + aH), *pAl = reinterpret_cast<const bf16_t *>(smem + aL);
  const bf16_t *pBh = reinterpret_cast<const bf16_t *>(smem + bH), *pBl = reinterpret_cast<const bf16_t *>(smem + bL);
#pragma unroll
  for (int kb = 0; kb < C / 16; ++kb) {
    const bf16x4_t ah = load_cfrag_at(pAh + 16 * kb * LDA_ + a0, loA), al = load_cfrag_at(pAl + 16 * kb * LDA_ + a0, loA);
    const bf16x4_t bh = load_cfrag_at(pBh + 16 * kb * LDB_ + b0, loB), bl = load_cfrag_at(pBl + 16 * kb * LDB_ + b0, loB);
    acc = mma16(ah, bh, acc);
    acc = mma16(ah, bl, acc);
    acc = mma16(al, bh, acc);
  }
  return acc;
}

constexpr int kWyThreads = 512;

template <typename Tin, int C, int D>
__global__ __launch_bounds__(kWyThreads) void bwd_wy_kernel(ChunkParams p, BwdParams bw) {
  constexpr int NT = kWyThreads, NW = NT / 64, NC = C / 16, DT = D / 16;
  using S = WySmem<C, D>;
  constexpr int LA = S::LA, LT = S::LT, LU = S::LU;
  constexpr int NCW = (NC * NC + NW - 1) / NW, NDW = (NC * DT + NW - 1) / NW;  // tiles per wave
  static_assert(NC * DT % NW == 0, "whole tiles per wave");
  const int wid = threadIdx.x >> 6, lane = threadIdx.x & 63, n16 = lane & 15, grp = lane >> 4;
  const int total = p.cu ? p.chunk_off[p.N] : p.B * ((p.T + C - 1) / C);
  const int64_t items = (int64_t)total * p.H;
  const int64_t ld = (int64_t)p.H * D, ldc = (int64_t)p.H * C, ldv = (int64_t)p.H * p.Vr;
  extern __shared__ __align__(16) char smem[];
  const float *sBeta = reinterpret_cast<const float *>(smem + S::beta);
  const float *sDtu = reinterpret_cast<const float *>(smem + S::dtu);
  float *sDbp = reinterpret_cast<float *>(smem + S::dbp);
  bf16_t *dtH = reinterpret_cast<bf16_t *>(smem + S::dtH), *dtL = reinterpret_cast<bf16_t *>(smem + S::dtL);
  bf16_t *xH = reinterpret_cast<bf16_t *>(smem + S::xwH), *xL = reinterpret_cast<bf16_t *>(smem + S::xwL);

  WyRegs<Tin, C, D, NT> R;
  auto locate = [&](int64_t it, ChunkLoc &lc, int &h) {
    h = (int)(it % p.H);
    locate_chunk(p, (int)(it / p.H), lc);
  };
  int64_t it = blockIdx.x;
  if (it < items) {
    ChunkLoc lc;
    int h;
    locate(it, lc, h);
    R.load(p, bw, lc.t0, lc.L, h);
  }
  for (; it < items; it += gridDim.x) {
    ChunkLoc lc;
    int h;
    locate(it, lc, h);
    const int L = lc.L;
    const int64_t t0 = lc.t0;
    R.store(smem, L);
    // v of this wave's dX_u elements (rows 16 rt + 4 g + e, column 16 ct + n16), for the beta
    // gradient: range-checked buffer loads (rows past L read zeros), issued together, used last
    float vv[NDW][4];
    {
      const rsrc_t rv = store_rsrc(const_cast<Tin *>(reinterpret_cast<const Tin *>(p.v)) + t0 * ldv + h * p.Vr,
                                   (uint32_t)((L - 1) * ldv + p.Vr) * (uint32_t)sizeof(Tin));
#pragma unroll
      for (int t = 0; t < NDW; ++t) {
        const int tile = wid * NDW + t, rt = tile / DT, ct = tile % DT;
        const int j = 16 * ct + n16;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t off = (uint32_t)((16 * rt + tile_row(e)) * ldv + j) * (uint32_t)sizeof(Tin);
          float x;
          if constexpr (sizeof(Tin) == 4) {
            x = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rv, (int)off, 0, 0));
          } else {
            x = __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rv, (int)off, 0, 0) << 16);
          }
          vv[t][e] = j < p.Vr ? x : 0.f;
        }
      }
    }
    __syncthreads();
    if (it + gridDim.x < items) {
      ChunkLoc ln;
      int hn;
      locate(it + gridDim.x, ln, hn);
      R.load(p, bw, ln.t0, ln.L, hn);
    }
    // dT = dT_u + beta_s (dw X_w^T)_rs, to LDS as hi / lo
#pragma unroll
    for (int t = 0; t < NCW; ++t) {
      const int tile = wid * NCW + t, rt = tile / NC, st = tile % NC;
      if (NC * NC % NW == 0 || tile < NC * NC) {
        f32x4_t acc = zero4();
#pragma unroll
        for (int k0 = 0; k0 < D; k0 += 32)
          acc = mma_split_rows<LT>(acc, smem, S::dwH, S::dwL, 16 * rt, S::xwH, S::xwL, 16 * st, k0);
        const int sc = 16 * st + n16;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * rt + tile_row(e);
          const float x = sDtu[r * LU + sc] + sBeta[sc] * acc[e];
          const bf16_t hh = static_cast<bf16_t>(x);
          dtH[r * LA + sc] = hh;
          dtL[r * LA + sc] = static_cast<bf16_t>(x - static_cast<float>(hh));
        }
      }
    }
    __syncthreads();  // dT complete; X_w consumed
    // X = dT T^T, over X_w's place
#pragma unroll
    for (int t = 0; t < NCW; ++t) {
      const int tile = wid * NCW + t, rt = tile / NC, st = tile % NC;
      if (NC * NC % NW == 0 || tile < NC * NC) {
        f32x4_t acc = zero4();
#pragma unroll
        for (int k0 = 0; k0 < C; k0 += 32)
          acc = mma_split_rows<LA>(acc, smem, S::dtH, S::dtL, 16 * rt, S::tH, S::tL, 16 * st, k0);
        const int sc = 16 * st + n16;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * rt + tile_row(e);
          const bf16_t hh = static_cast<bf16_t>(acc[e]);
          xH[r * LA + sc] = hh;
          xL[r * LA + sc] = static_cast<bf16_t>(acc[e] - static_cast<float>(hh));
        }
      }
    }
    __syncthreads();
    const int loA = cfrag_lane_off(LA), loT = cfrag_lane_off(LT);
    // dA_kk = -strict_lower(T^T X) (rows past L fall outside the range)
    const rsrc_t rak = store_rsrc(bw.dAkk + t0 * ldc + h * C, (uint32_t)((L - 1) * ldc + C) * 4u);
#pragma unroll
    for (int t = 0; t < NCW; ++t) {
      const int tile = wid * NCW + t, rt = tile / NC, st = tile % NC;
      if (NC * NC % NW == 0 || tile < NC * NC) {
        const f32x4_t a = mma_split_tokens<C, LA, LA>(zero4(), smem, S::tH, S::tL, 16 * rt, S::xwH, S::xwL, 16 * st,
                                                      loA, loA);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * rt + tile_row(e), sc = 16 * st + n16;
          bstore_f32(rak, (uint32_t)(r * ldc + sc) * 4u, (sc < r) ? -a[e] : 0.f);
        }
      }
    }
    // dX_w = T^T dw; dX_u = T^T dv_new, dv = beta dX_u, and the beta gradient through u
    const rsrc_t rxw = store_rsrc(bw.dXw + t0 * ld + h * D, (uint32_t)((L - 1) * ld + D) * 4u);
    float dbp[NDW][4];
#pragma unroll
    for (int t = 0; t < NDW; ++t) {
      const int tile = wid * NDW + t, rt = tile / DT, ct = tile % DT;
      const f32x4_t a = mma_split_tokens<C, LA, LT>(zero4(), smem, S::tH, S::tL, 16 * rt, S::dwH, S::dwL, 16 * ct,
                                                    loA, loT);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        bstore_f32(rxw, (uint32_t)((16 * rt + tile_row(e)) * ld + 16 * ct + n16) * 4u, a[e]);
      const f32x4_t u = mma_split_tokens<C, LA, LT>(zero4(), smem, S::tH, S::tL, 16 * rt, S::dvH, S::dvL, 16 * ct,
                                                    loA, loT);
      const int j = 16 * ct + n16;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * rt + tile_row(e);
        if (r < L && j < p.Vr)
          reinterpret_cast<Tin *>(bw.dv)[(t0 + r) * ldv + h * p.Vr + j] = from_f32<Tin>(sBeta[r] * u[e]);
        dbp[t][e] = u[e] * vv[t][e];
      }
    }
    // beta gradient: per row, over the lane's columns, then the 16 lanes of a row
    // group, then the waves sharing the row block (in a fixed order)
    {
      constexpr int WPR = DT / NDW;  // waves per 16-row block
      static_assert(WPR >= 1 && WPR <= 4 && DT % NDW == 0, "waves per row block");
      float rs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < NDW; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) rs[e] += dbp[t][e];
#pragma unroll
      for (int e = 0; e < 4; ++e) rs[e] = lanes16_sum(rs[e]);
      const int rt = (wid * NDW) / DT, part = ((wid * NDW) % DT) / NDW;
      if (n16 == 0)
#pragma unroll
        for (int e = 0; e < 4; ++e) sDbp[part * C + 16 * rt + tile_row(e)] = rs[e];
      __syncthreads();
      if (threadIdx.x < C && threadIdx.x < L) {
        float d = sDbp[threadIdx.x];
#pragma unroll
        for (int q = 1; q < WPR; ++q) d += sDbp[q * C + threadIdx.x];
        bw.dbp[(t0 + threadIdx.x) * p.H + h] = d;
      }
    }
    __syncthreads();  // the buffers are rewritten by the next item
  }
}

// ---- pairwise decays: dq, dk, the cumsum gradient, dg and the gate activation ----
// For row r, channel i (E_rs = 2^(b_r - b_s)):
//   Q[r] = sum_{s<r} dA_kk[r,s] k_s E_rs      R[r] = sum_{s<=r} dA_qk[r,s] k_s E_rs
//   U[s] = sum_{r>=s} (dA_kk[r,s] beta_r k_r + dA_qk[r,s] scale q_r) E_rs
// Off-diagonal 16x16 blocks (row block I > column block J) factor the decay
// through the first row a_I of block I, E_rs = 2^(b_r - a_I) 2^(a_I - b_s),
// both exponents non-positive for any decaying gate ("FLA KDA Skill", "Safe
// gate numerical note"), and run as fp32 MFMA products; diagonal blocks take
// E_rs per pair. Each wave owns 16 channels of a 64-channel slab.
// The grams step's operands in registers between their loads and the LDS stores:
// the two gram gradients of a chunk (loaded with the first slab), and one
// 64-channel slab of k, q and b (the next slab's loads are issued while the
// current slab computes).
template <typename Tin, int C, int SI>
struct GramSlabRegs {
  static constexpr int EPV = 16 / (int)sizeof(Tin), VK = SI / EPV, NK = C * VK, IK = (NK + kBT - 1) / kBT;
  static constexpr int VB = SI / 4, NB = C * VB, IB = (NB + kBT - 1) / kBT;
  u32x4_t k[IK], q[IK];
  f32x4_t b[IB];
  float bl;

  // rows >= L of b repeat row L - 1, so every exponent formed from them stays <= 0
  __device__ __forceinline__ void load(const ChunkParams &p, int64_t t0, int L, int h, int i0) {
    const int t = threadIdx.x, Kr = p.Kr;
    const int64_t ld = (int64_t)p.H * (int64_t)p.D, ldk = (int64_t)p.H * Kr;
    const Tin *gk = reinterpret_cast<const Tin *>(p.k) + t0 * ldk + h * Kr + i0;
    const Tin *gq = reinterpret_cast<const Tin *>(p.q) + t0 * ldk + h * Kr + i0;
    const float *gb = p.b + t0 * ld + h * p.D + i0;
    const u32x4_t z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int it = 0; it < IK; ++it) {
      const int idx = it * kBT + t, r = idx / VK, c = (idx % VK) * EPV;
      const bool ok = (NK % kBT == 0 || idx < NK) && r < L && c < Kr - i0;
      k[it] = ok ? *reinterpret_cast<const u32x4_t *>(gk + r * ldk + c) : z;
      q[it] = ok ? *reinterpret_cast<const u32x4_t *>(gq + r * ldk + c) : z;
    }
#pragma unroll
    for (int it = 0; it < IB; ++it) {
      const int idx = it * kBT + t, r = idx / VB, c = (idx % VB) * 4;
      b[it] = (NB % kBT == 0 || idx < NB) ? ld4(gb + (int64_t)min(r, L - 1) * ld + c) : zero4();
    }
    if (t < SI) bl = gb[(int64_t)(L - 1) * ld + t];
  }

  static __device__ __forceinline__ void put(float *s, int lds, int r, int c, u32x4_t raw) {
    if constexpr (sizeof(Tin) == 4) {
      *reinterpret_cast<u32x4_t *>(s + r * lds + c) = raw;
    } else {
      const bf16x8_t f = __builtin_bit_cast(bf16x8_t, raw);
      *reinterpret_cast<f32x4_t *>(s + r * lds + c) = f32x4_t{(float)f[0], (float)f[1], (float)f[2], (float)f[3]};
      *reinterpret_cast<f32x4_t *>(s + r * lds + c + 4) = f32x4_t{(float)f[4], (float)f[5], (float)f[6], (float)f[7]};
    }
  }

  __device__ __forceinline__ void store(float *sK, float *sQ, float *sB, float *sBL, int lds) const {
    const int t = threadIdx.x;
#pragma unroll
    for (int it = 0; it < IK; ++it) {
      const int idx = it * kBT + t, r = idx / VK, c = (idx % VK) * EPV;
      if (NK % kBT == 0 || idx < NK) {
        put(sK, lds, r, c, k[it]);
        put(sQ, lds, r, c, q[it]);
      }
    }
#pragma unroll
    for (int it = 0; it < IB; ++it) {
      const int idx = it * kBT + t, r = idx / VB, c = (idx % VB) * 4;
      if (NB % kBT == 0 || idx < NB) *reinterpret_cast<f32x4_t *>(sB + r * lds + c) = b[it];
    }
    if (t < SI) sBL[t] = bl;
  }
};

template <typename Tin, int C, int D, int GK>
__global__ __launch_bounds__(kBT) void bwd_grams_kernel(ChunkParams p, BwdParams bw) {
  ChunkLoc lc;
  if (!locate_chunk(p, blockIdx.x, lc)) return;
  const int h = blockIdx.y;
  constexpr int SI = 64, LS = SI + 4, LA = C + 4, NC = C / 16, NW = kBT / 64;
  static_assert(SI == 16 * NW, "one 16-channel tile per wave");
  const int Kr = p.Kr, L = lc.L;
  const int64_t t0 = lc.t0;
  const int64_t ld = (int64_t)p.H * D, ldc = (int64_t)p.H * C, ldk = (int64_t)p.H * Kr;
  const int wid = threadIdx.x >> 6, lane = threadIdx.x & 63, n16 = lane & 15, grp = lane >> 4;
  extern __shared__ __align__(16) char smem[];
  // [C][LA], both gradients of the grams in one tile: dA_kk (strictly lower) in
  // place, dA_qk (lower) transposed, so dA_kk[r][s] = sDAg[r][s] for s < r and
  // dA_qk[r][s] = sDAg[s][r] for s <= r
  float *sDAg = reinterpret_cast<float *>(smem);
  float *sK = sDAg + C * LA;                        // [C][LS] slab of SI channels
  float *sQ = sK + C * LS;
  float *sB = sQ + C * LS;   // b; rows >= L repeat row L - 1, so every exponent below stays <= 0
  float *sCT = sB + C * LS;  // [SI] per channel: sum over rows of k 2^(b_L - b) dk~ (b_L's share)
  float *sBeta = sCT + SI;   // [C]
  float *sDbw = sBeta + C;      // [NW][C] per-wave partial beta gradients
  float *sBL = sDbw + NW * C;   // [SI]
  float *sDA = sBL + SI;        // [SI]
  const Tin *gq = reinterpret_cast<const Tin *>(p.q), *gk = reinterpret_cast<const Tin *>(p.k);
  Tin *gdq = reinterpret_cast<Tin *>(bw.dq), *gdk = reinterpret_cast<Tin *>(bw.dk);
  const float scale = p.scale;
  const float expA = (GK == kGateSafe || GK == kGateSoftplus) ? fast_exp2(p.A_log[h] * kLog2e) : 0.f;

  // the gram gradients and the first slab's operands, loaded together
  constexpr int NA = C * C / 4, IA = (NA + kBT - 1) / kBT;
  f32x4_t akk[IA], aqk[IA];
#pragma unroll
  for (int it = 0; it < IA; ++it) {
    const int idx = it * kBT + threadIdx.x, r = idx / (C / 4), c = (idx % (C / 4)) * 4;
    const bool ok = (NA % kBT == 0 || idx < NA) && r < L;
    akk[it] = ok ? ld4(bw.dAkk + (t0 + r) * ldc + h * C + c) : zero4();
    aqk[it] = ok ? ld4(bw.dAqk + (t0 + r) * ldc + h * C + c) : zero4();
  }
  GramSlabRegs<Tin, C, SI> slab;
  slab.load(p, t0, L, h, 0);
#pragma unroll
  for (int it = 0; it < IA; ++it) {
    const int idx = it * kBT + threadIdx.x, r = idx / (C / 4), c = (idx % (C / 4)) * 4;
    if (NA % kBT == 0 || idx < NA) {
      f32x4_t v = akk[it];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = (c + e < r) ? v[e] : 0.f;
      *reinterpret_cast<f32x4_t *>(sDAg + r * LA + c) = v;
    }
  }
  __syncthreads();  // the upper triangle and the diagonal are zero before dA_qk goes in
#pragma unroll
  for (int it = 0; it < IA; ++it) {
    const int idx = it * kBT + threadIdx.x, r = idx / (C / 4), c = (idx % (C / 4)) * 4;
    if (NA % kBT == 0 || idx < NA) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (c + e <= r) sDAg[(c + e) * LA + r] = aqk[it][e];  // dA_qk written transposed
    }
  }
  for (int r = threadIdx.x; r < C; r += kBT) sBeta[r] = r < L ? beta_at(p, t0 + r, h) : 0.f;
  for (int idx = threadIdx.x; idx < NW * C; idx += kBT) sDbw[idx] = 0.f;
  float dA_total = 0.f;
  const float *gb = p.b + t0 * ld + h * D;
  const int cl = 16 * wid + n16;  // this lane's channel within a slab
  // this lane's elements of dq~, dX_w, dk~ of row block I (rows 16I + 4grp + e)
  auto load_p = [&](int i0, int I, float (&pq)[4], float (&px)[4], float (&pk)[4]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 16 * I + 4 * grp + e, i = i0 + cl;
      const bool ok = r < L && i < Kr;
      const int64_t eo = (t0 + (ok ? r : 0)) * ld + h * D + (ok ? i : 0);
      pq[e] = ok ? bw.dqt[eo] : 0.f;
      px[e] = ok ? bw.dXw[eo] : 0.f;
      pk[e] = ok ? bw.dkt[eo] : 0.f;
    }
  };
  // the gate activation's pass: thread = (row group, 4 channels)
  constexpr int CG = SI / 4, RG = kBT / CG, NXR = (C + RG - 1) / RG;
  const int c4 = 4 * (threadIdx.x % CG), rg = threadIdx.x / CG;
  for (int i0 = 0; i0 < Kr; i0 += SI) {
    __syncthreads();
    // issued first, consumed later: block 0's elements and the gate input of the activation pass
    float pq[4], px[4], pk[4];
    load_p(i0, 0, pq, px, pk);
    f32x4_t xs[NXR];
#pragma unroll
    for (int m = 0; m < NXR; ++m) {
      const int rr = rg + RG * m, i = i0 + c4;
      xs[m] = ((GK == kGateSafe || GK == kGateSoftplus) && rr < L && i < Kr)
                  ? ld4(p.g + (t0 + rr) * ldk + h * Kr + i) : zero4();
    }
    slab.store(sK, sQ, sB, sBL, LS);
    if (i0 + SI < Kr) slab.load(p, t0, L, h, i0 + SI);  // the next slab, during this one's products
    __syncthreads();

    float ctl = 0.f;                // sum over this lane's rows of k 2^(b_L - b) dk~
#pragma unroll 1
    for (int I = 0; I < NC; ++I) {
      const float aI = sB[16 * I * LS + cl];
      // the next block's elements, loaded while this block's products run
      float nq[4], nx[4], nk[4];
      if (I + 1 < NC) load_p(i0, I + 1, nq, nx, nk);
      // Q and R of rows 16I + 4grp + e: blocks J < I, then the diagonal block
      f32x4_t aq = zero4(), ar = zero4();
#pragma unroll 1
      for (int J = 0; J < I; ++J) {
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          const int s = 16 * J + 4 * st + grp;
          const float kh = sK[s * LS + cl] * fast_exp2(aI - sB[s * LS + cl]);
          aq = __builtin_amdgcn_mfma_f32_16x16x4f32(sDAg[(16 * I + n16) * LA + s], kh, aq, 0, 0, 0);
          ar = __builtin_amdgcn_mfma_f32_16x16x4f32(sDAg[s * LA + 16 * I + n16], kh, ar, 0, 0, 0);
        }
      }
      // U of rows (as columns) 16I + 4grp + e: row blocks I2 > I
      f32x4_t u = zero4();
#pragma unroll 1
      for (int I2 = I + 1; I2 < NC; ++I2) {
        const float a2 = sB[16 * I2 * LS + cl];
        f32x4_t au = zero4();
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          const int rr = 16 * I2 + 4 * st + grp;
          const float f = fast_exp2(sB[rr * LS + cl] - a2);
          const float xh = sBeta[rr] * sK[rr * LS + cl] * f, qh = scale * sQ[rr * LS + cl] * f;
          au = __builtin_amdgcn_mfma_f32_16x16x4f32(sDAg[rr * LA + 16 * I + n16], xh, au, 0, 0, 0);
          au = __builtin_amdgcn_mfma_f32_16x16x4f32(sDAg[(16 * I + n16) * LA + rr], qh, au, 0, 0, 0);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) u[e] += au[e] * fast_exp2(a2 - sB[(16 * I + 4 * grp + e) * LS + cl]);
      }
      // the diagonal block
      float qd[4], rd[4], ud[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float fo = fast_exp2(sB[(16 * I + 4 * grp + e) * LS + cl] - aI);
        qd[e] = aq[e] * fo;
        rd[e] = ar[e] * fo;
        ud[e] = u[e];
      }
      if constexpr (GK == kGateSafe) {
        // bounded decay: the block's midpoint m (row 16I + 8) anchors both sides,
        // E_rs = 2^(b_r - m) 2^(m - b_s), with |exponents| at most 8 rows of decay
        const float mI = sB[(16 * I + 8) * LS + cl];
        f32x4_t dq4 = zero4(), dr4 = zero4(), du4 = zero4();
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          const int s = 16 * I + 4 * st + grp;  // contraction index
          const float bs = sB[s * LS + cl];
          const float km = sK[s * LS + cl] * fast_exp2(mI - bs);
          const int rl = 16 * I + n16;  // this lane's row (the operand's m index)
          const float akk_rs = s < rl ? sDAg[rl * LA + s] : 0.f, aqk_rs = s <= rl ? sDAg[s * LA + rl] : 0.f;
          const float akk_sr = rl < s ? sDAg[s * LA + rl] : 0.f, aqk_sr = rl <= s ? sDAg[rl * LA + s] : 0.f;
          dq4 = __builtin_amdgcn_mfma_f32_16x16x4f32(akk_rs, km, dq4, 0, 0, 0);
          dr4 = __builtin_amdgcn_mfma_f32_16x16x4f32(aqk_rs, km, dr4, 0, 0, 0);
          const float fm = fast_exp2(bs - mI);
          du4 = __builtin_amdgcn_mfma_f32_16x16x4f32(akk_sr, sBeta[s] * sK[s * LS + cl] * fm, du4, 0, 0, 0);
          du4 = __builtin_amdgcn_mfma_f32_16x16x4f32(aqk_sr, scale * sQ[s * LS + cl] * fm, du4, 0, 0, 0);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float br = sB[(16 * I + 4 * grp + e) * LS + cl];
          const float fr = fast_exp2(br - mI), fc = fast_exp2(mI - br);
          qd[e] += dq4[e] * fr;
          rd[e] += dr4[e] * fr;
          ud[e] += du4[e] * fc;
        }
      } else {
        // unbounded decay: one exponential per pair, every exponent <= 0
        float br[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) br[e] = sB[(16 * I + 4 * grp + e) * LS + cl];
#pragma unroll 4
        for (int sl = 0; sl < 16; ++sl) {
          const int s = 16 * I + sl;
          const float ks = sK[s * LS + cl], bs = sB[s * LS + cl];
          const float xs = sBeta[s] * ks, qs = scale * sQ[s * LS + cl];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 16 * I + 4 * grp + e;
            if (s <= r) {
              const float f = fast_exp2(br[e] - bs) * ks;
              qd[e] += (s < r ? sDAg[r * LA + s] : 0.f) * f;
              rd[e] += sDAg[s * LA + r] * f;
            }
            if (s >= r)
              ud[e] += ((r < s ? sDAg[s * LA + r] : 0.f) * xs + sDAg[r * LA + s] * qs) * fast_exp2(bs - br[e]);
          }
        }
      }
      float dBv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * I + 4 * grp + e, i = i0 + cl;
        const float br = sB[r * LS + cl];
        // dq, dk, the cumsum gradient and the beta gradient of (r, i)
        float dbp = 0.f, dB = 0.f, ct = 0.f;
        if (r < L && i < Kr) {
          const float kr = sK[r * LS + cl], qr = sQ[r * LS + cl], be = sBeta[r];
          const float gam = fast_exp2(br), ktf = fast_exp2(sBL[cl] - br);
          const float t1 = gam * pq[e] + rd[e];
          const float t2 = gam * px[e] + qd[e];
          const float kd = ktf * pk[e];
          const float t3 = kd + ud[e];
          gdq[(t0 + r) * ldk + h * Kr + i] = from_f32<Tin>(scale * t1);
          gdk[(t0 + r) * ldk + h * Kr + i] = from_f32<Tin>(be * t2 + t3);
          dB = scale * qr * t1 + be * kr * t2 - kr * t3;
          ct = kr * kd;
          dbp = kr * t2;
        }
        dBv[e] = dB;
        ctl += ct;
        dbp = lanes16_sum(dbp);
        if (n16 == 0) sDbw[wid * C + r] += dbp;
      }
      // this wave alone reads these rows of its channels again: dB goes over q
#pragma unroll
      for (int e = 0; e < 4; ++e) sQ[(16 * I + 4 * grp + e) * LS + cl] = dBv[e];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pq[e] = nq[e];
        px[e] = nx[e];
        pk[e] = nk[e];
      }
    }
    // b_L's share summed over the rows: the lanes of one channel hold 4 rows each
    ctl += __shfl_xor(ctl, 16);
    ctl += __shfl_xor(ctl, 32);
    if (grp == 0) sCT[cl] = ctl;
    __syncthreads();
    // per channel: b_L's terms and the reverse cumsum, in place in sQ (which holds
    // dB): each channel's rows in NQ quarters, the quarter sums (in sB, free now)
    // added in row order to the later quarters
    {
      constexpr int NQ = kBT / SI, RQ = C / NQ;
      const int ii = threadIdx.x % SI, q = threadIdx.x / SI, i = i0 + ii;
      const int r0 = q * RQ;
      // the quarter's rows in registers (rows past L hold zeros: dB is zero there)
      float vq[RQ];
#pragma unroll
      for (int e = 0; e < RQ; ++e) vq[e] = sQ[(r0 + e) * LS + ii];
      float part = 0.f;
#pragma unroll
      for (int e = 0; e < RQ; ++e) part += vq[e];
      sB[q * SI + ii] = part;
      __syncthreads();
      if (i < Kr) {
        float acc = sCT[ii] + fast_exp2(sBL[ii]) * bw.dlam[((int64_t)lc.gci * p.H + h) * D + i];
#pragma unroll
        for (int q2 = NQ - 1; q2 > 0; --q2)
          if (q2 > q) acc += sB[q2 * SI + ii];
#pragma unroll
        for (int e = RQ - 1; e >= 0; --e) {
          acc += vq[e];
          if (r0 + e < L) sQ[(r0 + e) * LS + ii] = acc;  // gradient of the natural-log decay of token r0 + e
        }
      }
    }
    __syncthreads();
    // per element: the gate activation's derivative; thread = (row group, 4 channels)
    {
      const int i = i0 + c4;
      float ddt4[4] = {0.f, 0.f, 0.f, 0.f}, dA4 = 0.f;
      f32x4_t dt4 = zero4();
      if (p.dt_bias && i < Kr) dt4 = ld4(p.dt_bias + h * Kr + i);
#pragma unroll
      for (int m = 0; m < NXR; ++m) {
        const int rr = rg + RG * m;
        if (rr >= L || i >= Kr) break;
        const f32x4_t g4 = ld4(sQ + rr * LS + c4);
        f32x4_t out = g4;
        if constexpr (GK == kGateSafe || GK == kGateSoftplus) {
          const f32x4_t x4 = xs[m];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float z = x4[e] + dt4[e];
            if constexpr (GK == kGateSafe) {
              const float sg = sigmoid_f32(expA * z);
              out[e] = g4[e] * (p.lower_bound * sg * (1.f - sg) * expA);
              dA4 += out[e] * z;
            } else {
              const float sp = fmaxf(z, 0.f) + log1p_pos(fast_exp2(-fabsf(z) * kLog2e));
              out[e] = g4[e] * (-expA * sigmoid_f32(z));
              dA4 += g4[e] * (-expA * sp);
            }
            ddt4[e] += out[e];
          }
        }
        *reinterpret_cast<f32x4_t *>(bw.dg + (t0 + rr) * ldk + h * Kr + i) = out;
      }
      // per-channel sums over the row groups (sK and sB are free now)
      *reinterpret_cast<f32x4_t *>(sB + rg * LS + c4) = f32x4_t{ddt4[0], ddt4[1], ddt4[2], ddt4[3]};
      sK[rg * LS + c4] = dA4;
    }
    __syncthreads();
    if (threadIdx.x < SI) {
      const int ii = threadIdx.x, i = i0 + ii;
      float dsum = 0.f, dAcc = 0.f;
      for (int g2 = 0; g2 < RG; ++g2) {
        dsum += sB[g2 * LS + ii];
        if ((ii & 3) == 0) dAcc += sK[g2 * LS + ii];
      }
      if (bw.ddt_part && i < Kr) bw.ddt_part[((int64_t)lc.gci * p.H + h) * D + i] = dsum;
      sDA[ii] = dAcc;
    }
    __syncthreads();
    if (threadIdx.x == 0)
      for (int ii = 0; ii < SI; ++ii) dA_total += sDA[ii];
  }
  for (int rr = threadIdx.x; rr < L; rr += kBT) {
    float d = bw.dbp[(t0 + rr) * p.H + h];
#pragma unroll
    for (int w = 0; w < NW; ++w) d += sDbw[w * C + rr];
    if (p.beta_logits) {
      const float b = sBeta[rr];
      d *= b * (1.f - b);
    }
    bw.dbeta[(t0 + rr) * p.H + h] = d;
  }
  if (threadIdx.x == 0 && bw.dA_part) bw.dA_part[(int64_t)lc.gci * p.H + h] = dA_total;
}

// ---- dA_log and ddt_bias: sums of the per-chunk parts ----
// Per head: the chunks split into contiguous ranges, each summed in chunk order
// by one thread, and the range sums added in range order (a fixed order: the
// result does not vary from run to run).
template <int D>
__global__ __launch_bounds__(kBT) void bwd_params_kernel(ChunkParams p, BwdParams bw) {
  constexpr int G = kBT / 64;  // chunk ranges per channel
  __shared__ float sPart[kBT];
  const int h = blockIdx.x, t = threadIdx.x;
  const int total = p.cu ? p.chunk_off[p.N] : p.B * ((p.T + p.C - 1) / p.C);
  if (bw.ddt) {
    const int lane = t % 64, g = t / 64;
    const int g0 = (int)((int64_t)total * g / G), g1 = (int)((int64_t)total * (g + 1) / G);
    for (int i0 = 0; i0 < p.Kr; i0 += 64) {
      const int i = i0 + lane;
      float acc = 0.f;
      if (i < p.Kr) {
#pragma unroll 8
        for (int gc = g0; gc < g1; ++gc) acc += bw.ddt_part[((int64_t)gc * p.H + h) * D + i];
      }
      sPart[t] = acc;
      __syncthreads();
      if (g == 0 && i < p.Kr) {
        float sum = 0.f;
#pragma unroll
        for (int q = 0; q < G; ++q) sum += sPart[64 * q + lane];
        bw.ddt[h * p.Kr + i] = sum;
      }
      __syncthreads();
    }
  }
  if (bw.dA_log) {
    const int g0 = (int)((int64_t)total * t / kBT), g1 = (int)((int64_t)total * (t + 1) / kBT);
    float acc = 0.f;
    for (int gc = g0; gc < g1; ++gc) acc += bw.dA_part[(int64_t)gc * p.H + h];
    sPart[t] = acc;
    __syncthreads();
    if (t == 0) {
      float sum = 0.f;
      for (int q = 0; q < kBT; ++q) sum += sPart[q];
      bw.dA_log[h] = sum;
    }
  }
}

template <typename Kern>
hipError_t launch_k(Kern kernel, dim3 grid, size_t smem, hipStream_t st, const ChunkParams &p, const BwdParams &b,
                    int threads = kBT) {
  if (grid.x == 0 || grid.y == 0 || grid.z == 0) return hipSuccess;
  if (smem > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      return e;
    }
  }
  hipLaunchKernelGGL(kernel, grid, dim3(threads), smem, st, p, b);
  return hipGetLastError();
}

template <typename Tin, int C, int D>
hipError_t launch_bwd_t(const ChunkParams &p, const BwdParams &b, hipStream_t st) {
  constexpr int LA = C + 4, LX = D + 4;
  hipError_t e;
  if constexpr (sizeof(Tin) == 2) {
    if ((e = launch_k(bwd_scan_split_kernel<C, D>, dim3(p.N * p.H), ScanSplitSmem<C, D>::total, st, p, b, 4 * D)) !=
        hipSuccess)
      return e;
  } else {
    if ((e = launch_k(bwd_scan_kernel<Tin, C, D>, dim3(p.N * p.H), ScanSmem<C, D>::total, st, p, b, 4 * D)) !=
        hipSuccess)
      return e;
  }
  const dim3 grid(p.max_chunks, p.H);
  {
    const int64_t items = (int64_t)p.max_chunks * p.H;
    const int wgs = (int)std::min<int64_t>(items, device_cus());
    if ((e = launch_k(bwd_contract_kernel<Tin, C, D>, dim3(wgs), ContractSmem<C, D>::total, st, p, b,
                      kContractThreads)) != hipSuccess)
      return e;
  }
  {
    const int64_t items = (int64_t)p.max_chunks * p.H;
    const int wgs = (int)std::min<int64_t>(items, device_cus());
    if ((e = launch_k(bwd_wy_kernel<Tin, C, D>, dim3(wgs), WySmem<C, D>::total, st, p, b, kWyThreads)) != hipSuccess)
      return e;
  }
  {
    constexpr int LS = 64 + 4, NW = kBT / 64;
    const size_t smem = sizeof(float) * ((size_t)C * LA + 3 * C * LS + 64 + C + NW * C + 2 * 64);
    switch (p.gate_kind) {
      case kGateSafe: e = launch_k(bwd_grams_kernel<Tin, C, D, kGateSafe>, grid, smem, st, p, b); break;
      case kGateSoftplus: e = launch_k(bwd_grams_kernel<Tin, C, D, kGateSoftplus>, grid, smem, st, p, b); break;
      case kGateLogE: e = launch_k(bwd_grams_kernel<Tin, C, D, kGateLogE>, grid, smem, st, p, b); break;
      default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;
  }
  if ((p.gate_kind == kGateSafe || p.gate_kind == kGateSoftplus) && (b.dA_log || b.ddt))
    return launch_k(bwd_params_kernel<D>, dim3(p.H), 0, st, p, b);
  return hipSuccess;
}

}  // namespace

hipError_t launch_bwd(const ChunkParams &p, const BwdParams &b, hipStream_t st) {
#define KDA_BWD_CASE(TIN, CC, DD) \
  if (p.C == CC && p.D == DD) return launch_bwd_t<TIN, CC, DD>(p, b, st);
  if (p.is_bf16) {
    KDA_BWD_CASE(bf16_t, 64, 128) KDA_BWD_CASE(bf16_t, 64, 64) KDA_BWD_CASE(bf16_t, 32, 128)
    KDA_BWD_CASE(bf16_t, 32, 64)
  } else {
    KDA_BWD_CASE(float, 64, 128) KDA_BWD_CASE(float, 64, 64) KDA_BWD_CASE(float, 32, 128)
    KDA_BWD_CASE(float, 32, 64)
  }
#undef KDA_BWD_CASE
  return hipErrorInvalidValue;
}

}  // namespace kda
