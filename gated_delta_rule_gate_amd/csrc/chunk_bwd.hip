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
  const int lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
  const float *pa = A + (m0 + r) * am + g * ak;
  const float *pb = B + g * bk + (n0 + r) * bn;
#pragma unroll 8
  for (int k0 = 0; k0 < KN; k0 += 4) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(pa[k0 * ak], pb[k0 * bk], acc, 0, 0, 0);
  return acc;
}

__device__ __forceinline__ int tile_row(int e) { return 4 * ((threadIdx.x & 63) >> 4) + e; }
__device__ __forceinline__ int tile_col() { return threadIdx.x & 15; }

__device__ __forceinline__ float beta_at(const ChunkParams &p, int64_t row, int h) {
  const float b = p.beta[row * p.H + h];
  return p.beta_logits ? sigmoid_f32(b) : b;
}

// ---- scan: dv_new and the state gradients, reverse over the chunks ----
template <typename Tin, int C, int D>
__global__ __launch_bounds__(kBT) void bwd_scan_kernel(ChunkParams p, BwdParams bw) {
  constexpr int BV = 64, LH = BV + 4, LA = C + 4, LX = D + 4, NC = C / 16, DT = D / 16;
  const int nvb = (p.Vr + BV - 1) / BV;
  const int vb = blockIdx.x % nvb, nh = blockIdx.x / nvb;
  const int n = nh / p.H, h = nh % p.H;
  const int wid = threadIdx.x >> 6;
  const int col0 = vb * BV;
  const int Kr = p.Kr, Vr = p.Vr;
  const SlotRange sr = slot_range(p.cu, n, p.T);
  const int nch = (sr.len + C - 1) / C;
  const int cbase = p.cu ? p.chunk_off[n] : n * ((p.T + C - 1) / C);
  const int64_t sbase = (int64_t)nh * Kr * Vr;
  const int64_t ld = (int64_t)p.H * D, ldc = (int64_t)p.H * C, ldk = (int64_t)p.H * Kr, ldv = (int64_t)p.H * Vr;
  extern __shared__ __align__(16) char smem[];
  float *sDh = reinterpret_cast<float *>(smem);  // [D][LH] gradient of the state (this value block)
  float *sA = sDh + D * LH;                      // [C][LA] A_qk
  float *sDo = sA + C * LA;                      // [C][LH] do
  float *sX = sDo + C * LH;                      // [C][LX] k~, then q~
  float *sW = sX + C * LX;                       // [C][LX] w
  float *sDv = sW + C * LX;                      // [C][LH] dv_new
  float *sBL = sDv + C * LH;                     // [D] b_L
  const Tin *gq = reinterpret_cast<const Tin *>(p.q), *gk = reinterpret_cast<const Tin *>(p.k);
  const Tin *gdo = reinterpret_cast<const Tin *>(bw.dout);

  for (int idx = threadIdx.x; idx < D * BV; idx += kBT) {
    const int i = idx / BV, j = idx % BV;
    sDh[i * LH + j] = (bw.dht && i < Kr && col0 + j < Vr) ? bw.dht[sbase + (int64_t)i * Vr + col0 + j] : 0.f;
  }
  __syncthreads();
  for (int c = nch - 1; c >= 0; --c) {
    const int64_t t0 = sr.t0 + (int64_t)c * C;
    const int L = min(C, sr.len - c * C);
    const int64_t gc = cbase + c;
    const float *gb = p.b + t0 * ld + h * D;  // this chunk's rows of b (log2)
    float *dhn = bw.dhn + (gc * p.H + h) * Kr * Vr;
    for (int idx = threadIdx.x; idx < D * BV; idx += kBT) {
      const int i = idx / BV, j = idx % BV;
      if (i < Kr && col0 + j < Vr) dhn[(int64_t)i * Vr + col0 + j] = sDh[i * LH + j];
    }
    for (int i = threadIdx.x; i < D; i += kBT) sBL[i] = gb[(int64_t)(L - 1) * ld + i];
    for (int idx = threadIdx.x; idx < C * C; idx += kBT) {
      const int r = idx / C, s = idx % C;
      sA[r * LA + s] = (r < L && s <= r) ? p.Aqk[(t0 + r) * ldc + h * C + s] : 0.f;
    }
    for (int idx = threadIdx.x; idx < C * BV; idx += kBT) {
      const int r = idx / BV, j = idx % BV;
      sDo[r * LH + j] = (r < L && col0 + j < Vr) ? to_f32(gdo[(t0 + r) * ldv + h * Vr + col0 + j]) : 0.f;
    }
    for (int idx = threadIdx.x; idx < C * D; idx += kBT) {
      const int r = idx / D, i = idx % D;
      float x = 0.f;
      if (r < L && i < Kr)
        x = to_f32(gk[(t0 + r) * ldk + h * Kr + i]) * fast_exp2(gb[(int64_t)(L - 1) * ld + i] - gb[(int64_t)r * ld + i]);
      sX[r * LX + i] = x;
    }
    __syncthreads();
    // dv_new = A_qk^T do + k~ dh (this wave: value columns 16 wid..)
    for (int rt = 0; rt < NC; ++rt) {
      f32x4_t acc = zero4();
      acc = mm16<C>(acc, sA, 1, LA, sDo, LH, 1, 16 * rt, 16 * wid);
      acc = mm16<D>(acc, sX, LX, 1, sDh, LH, 1, 16 * rt, 16 * wid);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * rt + tile_row(e), j = 16 * wid + tile_col();
        sDv[r * LH + j] = acc[e];
        if (r < L) bw.dvn[(t0 + r) * ld + h * D + col0 + j] = acc[e];
      }
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < C * D; idx += kBT) {
      const int r = idx / D, i = idx % D;
      float x = 0.f, wv = 0.f;
      if (r < L) {
        if (i < Kr) x = p.scale * to_f32(gq[(t0 + r) * ldk + h * Kr + i]) * fast_exp2(gb[(int64_t)r * ld + i]);
        wv = p.w[(t0 + r) * ld + h * D + i];
      }
      sX[r * LX + i] = x;
      sW[r * LX + i] = wv;
    }
    __syncthreads();
    // dh <- 2^b_L dh + q~^T do - w^T dv_new (this wave's columns only)
    for (int it = 0; it < DT; ++it) {
      f32x4_t a1 = zero4(), a2 = zero4();
      a1 = mm16<C>(a1, sX, 1, LX, sDo, LH, 1, 16 * it, 16 * wid);
      a2 = mm16<C>(a2, sW, 1, LX, sDv, LH, 1, 16 * it, 16 * wid);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 16 * it + tile_row(e), j = 16 * wid + tile_col();
        sDh[i * LH + j] = fast_exp2(sBL[i]) * sDh[i * LH + j] + a1[e] - a2[e];
      }
    }
    __syncthreads();
  }
  if (bw.dh0) {
    for (int idx = threadIdx.x; idx < D * BV; idx += kBT) {
      const int i = idx / BV, j = idx % BV;
      if (i < Kr && col0 + j < Vr) bw.dh0[sbase + (int64_t)i * Vr + col0 + j] = sDh[i * LH + j];
    }
  }
}

// ---- contractions over the value columns ----
template <typename Tin, int C, int D>
__global__ __launch_bounds__(kBT) void bwd_contract_kernel(ChunkParams p, BwdParams bw) {
  ChunkLoc lc;
  if (!locate_chunk(p, blockIdx.x, lc)) return;
  const int h = blockIdx.y;
  constexpr int SJ = 32, LS = SJ + 4, NC = C / 16, DT = D / 16;
  constexpr int NTW = NC * DT / 4, NCW = NC * NC / 4;  // tiles per wave of a [C][D] and a [C][C] product
  static_assert(NTW >= 1 && NCW >= 1, "tiles per wave");
  const int wid = threadIdx.x >> 6;
  const int Kr = p.Kr, Vr = p.Vr, L = lc.L;
  const int64_t t0 = lc.t0;
  const int64_t ld = (int64_t)p.H * D, ldc = (int64_t)p.H * C, ldv = (int64_t)p.H * Vr;
  const int64_t hbase = ((int64_t)lc.gci * p.H + h) * Kr * Vr;
  extern __shared__ __align__(16) char smem[];
  float *sDo = reinterpret_cast<float *>(smem);  // [C][LS] slabs of SJ value columns
  float *sVn = sDo + C * LS;
  float *sDvn = sVn + C * LS;
  float *sBv = sDvn + C * LS;
  float *sH = sBv + C * LS;  // [D][LS]
  float *sDhn = sH + D * LS;
  const Tin *gdo = reinterpret_cast<const Tin *>(bw.dout), *gv = reinterpret_cast<const Tin *>(p.v);

  f32x4_t aq[NTW], ak[NTW], aw[NTW], aa[NCW], at[NCW];
#pragma unroll
  for (int t = 0; t < NTW; ++t) aq[t] = ak[t] = aw[t] = zero4();
#pragma unroll
  for (int t = 0; t < NCW; ++t) aa[t] = at[t] = zero4();

  for (int j0 = 0; j0 < Vr; j0 += SJ) {
    __syncthreads();  // the previous slab is consumed
    for (int idx = threadIdx.x; idx < C * SJ; idx += kBT) {
      const int r = idx / SJ, j = idx % SJ, jj = j0 + j;
      const bool ok = r < L && jj < Vr;
      const int64_t row = t0 + r;
      sDo[r * LS + j] = ok ? to_f32(gdo[row * ldv + h * Vr + jj]) : 0.f;
      sVn[r * LS + j] = ok ? p.vnew[row * ld + h * D + jj] : 0.f;
      sDvn[r * LS + j] = ok ? bw.dvn[row * ld + h * D + jj] : 0.f;
      sBv[r * LS + j] = ok ? beta_at(p, row, h) * to_f32(gv[row * ldv + h * Vr + jj]) : 0.f;
    }
    for (int idx = threadIdx.x; idx < D * SJ; idx += kBT) {
      const int i = idx / SJ, j = idx % SJ, jj = j0 + j;
      const bool ok = i < Kr && jj < Vr;
      sH[i * LS + j] = ok ? p.hc[hbase + (int64_t)i * Vr + jj] : 0.f;
      sDhn[i * LS + j] = ok ? bw.dhn[hbase + (int64_t)i * Vr + jj] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < NTW; ++t) {
      const int tile = wid * NTW + t, rt = tile / DT, ct = tile % DT;
      aq[t] = mm16<SJ>(aq[t], sDo, LS, 1, sH, 1, LS, 16 * rt, 16 * ct);    // do h^T
      ak[t] = mm16<SJ>(ak[t], sVn, LS, 1, sDhn, 1, LS, 16 * rt, 16 * ct);  // v_new dh'^T
      aw[t] = mm16<SJ>(aw[t], sDvn, LS, 1, sH, 1, LS, 16 * rt, 16 * ct);   // dv_new h^T
    }
#pragma unroll
    for (int t = 0; t < NCW; ++t) {
      const int tile = wid * NCW + t, rt = tile / NC, st = tile % NC;
      aa[t] = mm16<SJ>(aa[t], sDo, LS, 1, sVn, 1, LS, 16 * rt, 16 * st);   // do v_new^T
      at[t] = mm16<SJ>(at[t], sDvn, LS, 1, sBv, 1, LS, 16 * rt, 16 * st);  // dv_new (beta v)^T
    }
  }
#pragma unroll
  for (int t = 0; t < NTW; ++t) {
    const int tile = wid * NTW + t, rt = tile / DT, ct = tile % DT;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 16 * rt + tile_row(e), i = 16 * ct + tile_col();
      if (r < L) {
        const int64_t o = (t0 + r) * ld + h * D + i;
        bw.dqt[o] = aq[t][e];
        bw.dkt[o] = ak[t][e];
        bw.dw[o] = -aw[t][e];
      }
    }
  }
#pragma unroll
  for (int t = 0; t < NCW; ++t) {
    const int tile = wid * NCW + t, rt = tile / NC, st = tile % NC;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 16 * rt + tile_row(e), s = 16 * st + tile_col();
      if (r < L) {
        const int64_t o = (t0 + r) * ldc + h * C + s;
        bw.dAqk[o] = (s <= r) ? aa[t][e] : 0.f;
        bw.dT[o] = at[t][e];
      }
    }
  }
  for (int i = threadIdx.x; i < D; i += kBT) {
    float acc = 0.f;
    if (i < Kr)
      for (int j = 0; j < Vr; ++j) acc += p.hc[hbase + (int64_t)i * Vr + j] * bw.dhn[hbase + (int64_t)i * Vr + j];
    bw.dlam[((int64_t)lc.gci * p.H + h) * D + i] = acc;
  }
}

// ---- the WY factors and the triangular inverse ----
template <typename Tin, int C, int D>
__global__ __launch_bounds__(kBT) void bwd_wy_kernel(ChunkParams p, BwdParams bw) {
  ChunkLoc lc;
  if (!locate_chunk(p, blockIdx.x, lc)) return;
  const int h = blockIdx.y;
  constexpr int LA = C + 4, LX = D + 4, NC = C / 16, DT = D / 16;
  constexpr int NTW = NC * DT / 4, NCW = NC * NC / 4, TPR = kBT / C;
  const int wid = threadIdx.x >> 6;
  const int Kr = p.Kr, Vr = p.Vr, L = lc.L;
  const int64_t t0 = lc.t0;
  const int64_t ld = (int64_t)p.H * D, ldc = (int64_t)p.H * C, ldk = (int64_t)p.H * Kr, ldv = (int64_t)p.H * Vr;
  extern __shared__ __align__(16) char smem[];
  float *sT = reinterpret_cast<float *>(smem);  // [C][LA] T
  float *sDT = sT + C * LA;                     // [C][LA] dT
  float *sX = sDT + C * LA;                     // [C][LA] dT T^T
  float *sDw = sX + C * LA;                     // [C][LX] dw, later dX_u
  float *sKG = sDw + C * LX;                    // [C][LX] k 2^b
  float *sDvn = sKG + C * LX;                   // [C][LX] dv_new
  float *sBeta = sDvn + C * LX;                 // [C]
  const Tin *gk = reinterpret_cast<const Tin *>(p.k), *gv = reinterpret_cast<const Tin *>(p.v);

  for (int idx = threadIdx.x; idx < C * C; idx += kBT) {
    const int r = idx / C, s = idx % C;
    const bool ok = r < L && s < L;
    const int64_t o = (t0 + r) * ldc + h * C + s;
    sT[r * LA + s] = (ok && s <= r) ? p.Tm[o] : 0.f;
    sDT[r * LA + s] = ok ? bw.dT[o] : 0.f;
  }
  for (int idx = threadIdx.x; idx < C * D; idx += kBT) {
    const int r = idx / D, i = idx % D;
    const int64_t o = (t0 + r) * ld + h * D + i;
    sDw[r * LX + i] = r < L ? bw.dw[o] : 0.f;
    sDvn[r * LX + i] = r < L ? bw.dvn[o] : 0.f;
    sKG[r * LX + i] = (r < L && i < Kr) ? to_f32(gk[(t0 + r) * ldk + h * Kr + i]) * fast_exp2(p.b[o]) : 0.f;
  }
  for (int r = threadIdx.x; r < C; r += kBT) sBeta[r] = r < L ? beta_at(p, t0 + r, h) : 0.f;
  __syncthreads();
  // dT = dT_u + beta_s (dw (k 2^b)^T)_rs
#pragma unroll
  for (int t = 0; t < NCW; ++t) {
    const int tile = wid * NCW + t, rt = tile / NC, st = tile % NC;
    const f32x4_t acc = mm16<D>(zero4(), sDw, LX, 1, sKG, 1, LX, 16 * rt, 16 * st);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 16 * rt + tile_row(e), s = 16 * st + tile_col();
      sDT[r * LA + s] += sBeta[s] * acc[e];
    }
  }
  __syncthreads();
  // X = dT T^T
#pragma unroll
  for (int t = 0; t < NCW; ++t) {
    const int tile = wid * NCW + t, rt = tile / NC, st = tile % NC;
    const f32x4_t acc = mm16<C>(zero4(), sDT, LA, 1, sT, 1, LA, 16 * rt, 16 * st);
#pragma unroll
    for (int e = 0; e < 4; ++e) sX[(16 * rt + tile_row(e)) * LA + 16 * st + tile_col()] = acc[e];
  }
  __syncthreads();
  // dA_kk = -strict_lower(T^T X); dX_w = T^T dw
#pragma unroll
  for (int t = 0; t < NCW; ++t) {
    const int tile = wid * NCW + t, rt = tile / NC, st = tile % NC;
    const f32x4_t acc = mm16<C>(zero4(), sT, 1, LA, sX, LA, 1, 16 * rt, 16 * st);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 16 * rt + tile_row(e), s = 16 * st + tile_col();
      if (r < L) bw.dAkk[(t0 + r) * ldc + h * C + s] = (s < r) ? -acc[e] : 0.f;
    }
  }
#pragma unroll
  for (int t = 0; t < NTW; ++t) {
    const int tile = wid * NTW + t, rt = tile / DT, ct = tile % DT;
    const f32x4_t acc = mm16<C>(zero4(), sT, 1, LA, sDw, LX, 1, 16 * rt, 16 * ct);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 16 * rt + tile_row(e), i = 16 * ct + tile_col();
      if (r < L) bw.dXw[(t0 + r) * ld + h * D + i] = acc[e];
    }
  }
  __syncthreads();
  // dX_u = T^T dv_new, into sDw
#pragma unroll
  for (int t = 0; t < NTW; ++t) {
    const int tile = wid * NTW + t, rt = tile / DT, ct = tile % DT;
    const f32x4_t acc = mm16<C>(zero4(), sT, 1, LA, sDvn, LX, 1, 16 * rt, 16 * ct);
#pragma unroll
    for (int e = 0; e < 4; ++e) sDw[(16 * rt + tile_row(e)) * LX + 16 * ct + tile_col()] = acc[e];
  }
  __syncthreads();
  // dv = beta dX_u; the beta gradient through u: sum over j of dX_u v
  {
    const int r = threadIdx.x / TPR, q = threadIdx.x % TPR;
    float acc = 0.f;
    if (r < L) {
      Tin *gdv = reinterpret_cast<Tin *>(bw.dv) + (t0 + r) * ldv + h * Vr;
      for (int j = q; j < Vr; j += TPR) {
        const float x = sDw[r * LX + j];
        acc += x * to_f32(gv[(t0 + r) * ldv + h * Vr + j]);
        gdv[j] = from_f32<Tin>(sBeta[r] * x);
      }
    }
#pragma unroll
    for (int m = 1; m < TPR; m <<= 1) acc += __shfl_xor(acc, m);
    if (q == 0 && r < L) bw.dbp[(t0 + r) * p.H + h] = acc;
  }
}

// ---- pairwise decays: dq, dk, the cumsum gradient, dg and the gate activation ----
template <typename Tin, int C, int D, int GK>
__global__ __launch_bounds__(kBT) void bwd_grams_kernel(ChunkParams p, BwdParams bw) {
  ChunkLoc lc;
  if (!locate_chunk(p, blockIdx.x, lc)) return;
  const int h = blockIdx.y;
  constexpr int SI = 32, LS = SI + 1, LA = C + 1, TPR = kBT / C, CPT = SI / TPR;
  const int Kr = p.Kr, L = lc.L;
  const int64_t t0 = lc.t0;
  const int64_t ld = (int64_t)p.H * D, ldc = (int64_t)p.H * C, ldk = (int64_t)p.H * Kr;
  extern __shared__ __align__(16) char smem[];
  float *sDAkk = reinterpret_cast<float *>(smem);  // [C][LA]
  float *sDAqk = sDAkk + C * LA;                   // [C][LA]
  float *sK = sDAqk + C * LA;                      // [C][LS] slabs of SI channels
  float *sQ = sK + C * LS;
  float *sB = sQ + C * LS;
  float *sDB = sB + C * LS;
  float *sCT = sDB + C * LS;
  float *sBeta = sCT + C * LS;  // [C]
  float *sDbeta = sBeta + C;    // [C]
  float *sBL = sDbeta + C;      // [SI]
  float *sDA = sBL + SI;        // [SI]
  const Tin *gq = reinterpret_cast<const Tin *>(p.q), *gk = reinterpret_cast<const Tin *>(p.k);
  Tin *gdq = reinterpret_cast<Tin *>(bw.dq), *gdk = reinterpret_cast<Tin *>(bw.dk);
  const float scale = p.scale;
  const float expA = (GK == kGateSafe || GK == kGateSoftplus) ? fast_exp2(p.A_log[h] * kLog2e) : 0.f;

  for (int idx = threadIdx.x; idx < C * C; idx += kBT) {
    const int r = idx / C, s = idx % C;
    const int64_t o = (t0 + r) * ldc + h * C + s;
    sDAkk[r * LA + s] = (r < L && s < r) ? bw.dAkk[o] : 0.f;
    sDAqk[r * LA + s] = (r < L && s <= r) ? bw.dAqk[o] : 0.f;
  }
  for (int r = threadIdx.x; r < C; r += kBT) {
    sBeta[r] = r < L ? beta_at(p, t0 + r, h) : 0.f;
    sDbeta[r] = 0.f;
  }
  float dA_total = 0.f;
  const int r = threadIdx.x / TPR, q4 = threadIdx.x % TPR;
  for (int i0 = 0; i0 < Kr; i0 += SI) {
    __syncthreads();
    for (int idx = threadIdx.x; idx < C * SI; idx += kBT) {
      const int rr = idx / SI, ii = idx % SI, i = i0 + ii;
      const bool ok = rr < L && i < Kr;
      sK[rr * LS + ii] = ok ? to_f32(gk[(t0 + rr) * ldk + h * Kr + i]) : 0.f;
      sQ[rr * LS + ii] = ok ? to_f32(gq[(t0 + rr) * ldk + h * Kr + i]) : 0.f;
      sB[rr * LS + ii] = rr < L ? p.b[(t0 + rr) * ld + h * D + i] : 0.f;
    }
    for (int ii = threadIdx.x; ii < SI; ii += kBT) sBL[ii] = p.b[(t0 + L - 1) * ld + h * D + i0 + ii];
    __syncthreads();
    float dbr = 0.f;
    for (int cc = 0; cc < CPT; ++cc) {
      const int ii = cc * TPR + q4, i = i0 + ii;
      if (r >= L || i >= Kr) {
        sDB[r * LS + ii] = 0.f;
        sCT[r * LS + ii] = 0.f;
        continue;
      }
      const float br = sB[r * LS + ii], kr = sK[r * LS + ii], qr = sQ[r * LS + ii], be = sBeta[r];
      const float gam = fast_exp2(br), ktf = fast_exp2(sBL[ii] - br);
      const int64_t eo = (t0 + r) * ld + h * D + i;
      const float dqt = bw.dqt[eo], dkt = bw.dkt[eo], dxw = bw.dXw[eo];
      float Q = 0.f, R = 0.f, U = 0.f;
      for (int s = 0; s <= r; ++s) {
        const float ks = sK[s * LS + ii] * fast_exp2(br - sB[s * LS + ii]);
        Q += sDAkk[r * LA + s] * ks;
        R += sDAqk[r * LA + s] * ks;
      }
      for (int t = r; t < L; ++t) {
        const float e = fast_exp2(sB[t * LS + ii] - br);
        U += (sDAkk[t * LA + r] * sBeta[t] * sK[t * LS + ii] + sDAqk[t * LA + r] * scale * sQ[t * LS + ii]) * e;
      }
      const float dq = scale * (gam * dqt + R);
      const float dk = be * (gam * dxw + Q) + ktf * dkt + U;
      const float dB = scale * qr * (gam * dqt + R) + be * kr * (gam * dxw + Q) - kr * (ktf * dkt + U);
      dbr += kr * (gam * dxw + Q);
      sDB[r * LS + ii] = dB;
      sCT[r * LS + ii] = kr * ktf * dkt;
      gdq[(t0 + r) * ldk + h * Kr + i] = from_f32<Tin>(dq);
      gdk[(t0 + r) * ldk + h * Kr + i] = from_f32<Tin>(dk);
    }
#pragma unroll
    for (int m = 1; m < TPR; m <<= 1) dbr += __shfl_xor(dbr, m);
    if (q4 == 0 && r < L) sDbeta[r] += dbr;
    __syncthreads();
    // per channel: b_L's terms, the reverse cumsum and the gate activation
    if (threadIdx.x < SI) {
      const int ii = threadIdx.x, i = i0 + ii;
      float dsum = 0.f, dAcc = 0.f;
      if (i < Kr) {
        float ct = 0.f;
        for (int rr = 0; rr < L; ++rr) ct += sCT[rr * LS + ii];
        const float extra = ct + fast_exp2(sBL[ii]) * bw.dlam[((int64_t)lc.gci * p.H + h) * D + i];
        const float dt = p.dt_bias ? p.dt_bias[h * Kr + i] : 0.f;
        float acc = extra;
        for (int rr = L - 1; rr >= 0; --rr) {
          acc += sDB[rr * LS + ii];
          float out = acc;  // gradient of the natural-log decay of token rr
          if constexpr (GK == kGateSafe || GK == kGateSoftplus) {
            const float x = p.g[(t0 + rr) * ldk + h * Kr + i];
            if constexpr (GK == kGateSafe) {
              const float s = sigmoid_f32(expA * (x + dt));
              out = acc * (p.lower_bound * s * (1.f - s) * expA);
              dAcc += out * (x + dt);
            } else {
              const float z = x + dt;
              const float sp = fmaxf(z, 0.f) + log1p_pos(fast_exp2(-fabsf(z) * kLog2e));
              out = acc * (-expA * sigmoid_f32(z));
              dAcc += acc * (-expA * sp);
            }
            dsum += out;
          }
          bw.dg[(t0 + rr) * ldk + h * Kr + i] = out;
        }
        if (bw.ddt_part) bw.ddt_part[((int64_t)lc.gci * p.H + h) * D + i] = dsum;
      }
      sDA[ii] = dAcc;
    }
    __syncthreads();
    if (threadIdx.x == 0)
      for (int ii = 0; ii < SI; ++ii) dA_total += sDA[ii];
  }
  for (int rr = threadIdx.x; rr < L; rr += kBT) {
    float d = sDbeta[rr] + bw.dbp[(t0 + rr) * p.H + h];
    if (p.beta_logits) {
      const float b = sBeta[rr];
      d *= b * (1.f - b);
    }
    bw.dbeta[(t0 + rr) * p.H + h] = d;
  }
  if (threadIdx.x == 0 && bw.dA_part) bw.dA_part[(int64_t)lc.gci * p.H + h] = dA_total;
}

// ---- dA_log and ddt_bias: sums of the per-chunk parts, in chunk order ----
template <int D>
__global__ __launch_bounds__(kBT) void bwd_params_kernel(ChunkParams p, BwdParams bw) {
  const int h = blockIdx.x;
  const int total = p.cu ? p.chunk_off[p.N] : p.B * ((p.T + p.C - 1) / p.C);
  if (bw.ddt) {
    for (int i = threadIdx.x; i < p.Kr; i += kBT) {
      float acc = 0.f;
      for (int gc = 0; gc < total; ++gc) acc += bw.ddt_part[((int64_t)gc * p.H + h) * D + i];
      bw.ddt[h * p.Kr + i] = acc;
    }
  }
  if (bw.dA_log && threadIdx.x == 0) {
    float acc = 0.f;
    for (int gc = 0; gc < total; ++gc) acc += bw.dA_part[(int64_t)gc * p.H + h];
    bw.dA_log[h] = acc;
  }
}

template <typename Kern>
hipError_t launch_k(Kern kernel, dim3 grid, size_t smem, hipStream_t st, const ChunkParams &p, const BwdParams &b) {
  if (grid.x == 0 || grid.y == 0 || grid.z == 0) return hipSuccess;
  if (smem > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      return e;
    }
  }
  hipLaunchKernelGGL(kernel, grid, dim3(kBT), smem, st, p, b);
  return hipGetLastError();
}

template <typename Tin, int C, int D>
hipError_t launch_bwd_t(const ChunkParams &p, const BwdParams &b, hipStream_t st) {
  constexpr int LA = C + 4, LX = D + 4;
  hipError_t e;
  {
    constexpr int LH = 64 + 4;
    const size_t smem = sizeof(float) * ((size_t)D * LH + C * LA + 2 * C * LH + 2 * C * LX + D);
    const int nvb = (p.Vr + 63) / 64;
    if ((e = launch_k(bwd_scan_kernel<Tin, C, D>, dim3(p.N * p.H * nvb), smem, st, p, b)) != hipSuccess) return e;
  }
  const dim3 grid(p.max_chunks, p.H);
  {
    constexpr int LS = 32 + 4;
    const size_t smem = sizeof(float) * ((size_t)4 * C * LS + 2 * D * LS);
    if ((e = launch_k(bwd_contract_kernel<Tin, C, D>, grid, smem, st, p, b)) != hipSuccess) return e;
  }
  {
    const size_t smem = sizeof(float) * ((size_t)3 * C * LA + 3 * C * LX + C);
    if ((e = launch_k(bwd_wy_kernel<Tin, C, D>, grid, smem, st, p, b)) != hipSuccess) return e;
  }
  {
    constexpr int LS = 32 + 1, LA1 = C + 1;
    const size_t smem = sizeof(float) * ((size_t)2 * C * LA1 + 5 * C * LS + 2 * C + 2 * 32);
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
