// The split schedule of the chunked KDA forward (bf16, D <= 128): a persistent
// key-side kernel runs steps (1)-(4) for every (chunk, head) and leaves each
// chunk's operands in a workspace record; a state-side kernel per (sequence,
// head, four value tiles) then walks the chunks with steps (5)-(6) and the state
// update only.
#include "chunk_fused_layout.h"
#include "chunk_loc.h"
#include "kda_launch.h"

// Threads per workgroup of the key side: as the fused kernel (512 when the state
// has at least 8 column tiles, else 256).
#ifndef KDA_FUSED_THREADS
#define KDA_FUSED_THREADS 0
#endif

namespace kda {

// Why: with fewer (sequence, head) pairs than compute units, the fused kernel's
// workgroups each walk a long chain of chunks at the full per-chunk latency
// while most of the chip idles. Steps (1)-(4) depend on no state, so here they
// run for all chunks in parallel, and only steps (5)-(6) and the state update
// stay in the chain.

// The workspace of one (chunk, head), written by the key side and read by the
// state side: bf16 [q~ (operand order) C*D | k~ C*D | w^T D*C | A_qk C*C], and
// fp32 [u in accumulator-fragment order C*D | 2^b_L D | q row scales C]. u's
// fragment order: for value tile t, lane l, row block i, the lane's four rows
// 16i + 4(l/16) + e of column 16t + l%16 as one 16-byte vector.
template <int C, int D>
struct SplitLayout {
  static constexpr int64_t nq = (int64_t)C * D, na = (int64_t)C * C;
  static constexpr int64_t bf = 3 * nq + na;       // bf16 elements per (chunk, head)
  static constexpr int64_t dec = nq, qn = nq + D;  // fp32 offsets
  static constexpr int64_t f32 = nq + D + C;       // fp32 elements per (chunk, head)
  static_assert((bf * 2) % 16 == 0 && (f32 * 4) % 16 == 0, "16-byte aligned records");
};

size_t split_workspace_bytes(int C, int D, int64_t chunk_heads) {
  const int64_t bf = 3LL * C * D + (int64_t)C * C, f = (int64_t)C * D + D + C;
  return (size_t)chunk_heads * (size_t)(2 * bf + 4 * f);
}


// Steps (1)-(4) for a contiguous range of (chunk, head) items per workgroup (one
// workgroup per compute unit), the next item's inputs loaded while the current
// one computes, as in the fused kernel.
template <int C, int D, int NT, int GK>
__global__ __launch_bounds__(NT) void split_key_kernel(ChunkParams p) {
  using Tin = bf16_t;
  using TL = Tile<Tin, C, D>;
  using S = FusedSmem<C, D, NT>;
  using SL = SplitLayout<C, D>;
  constexpr bool SAFE = (GK == kGateSafe);
  constexpr int NW = NT / 64, NC = TL::NC, DT = TL::DT, LDT = TL::LDT, LDB = TL::LDB, LDA = TL::LDA;
  static_assert(DT == NW, "one w column tile and one value tile per wave");
  // chunks in total (the prefix's last entry when packed) and this workgroup's items
  const int total = p.cu ? p.chunk_off[p.N] : p.B * ((p.T + C - 1) / C);
  const int64_t M = (int64_t)total * p.H;
  const int64_t i0 = M * blockIdx.x / gridDim.x, i1 = M * (blockIdx.x + 1) / gridDim.x;
  if (i0 >= i1) return;

  extern __shared__ __align__(16) char smem[];
  char *baseB = lds_base(smem, S::b), *baseA = lds_base(smem, S::akk), *baseT = lds_base(smem, S::t1);
  Tin *sQ = reinterpret_cast<Tin *>(smem + S::q);
  Tin *sK = reinterpret_cast<Tin *>(smem + S::k);
  Tin *sV = reinterpret_cast<Tin *>(smem + S::v);
  float *sB = reinterpret_cast<float *>(smem + S::b);
  Tin *sXw = reinterpret_cast<Tin *>(smem + S::b + S::xw_off);
  Tin *sWT = reinterpret_cast<Tin *>(baseB + S::wt_off);
  float *sAkk = reinterpret_cast<float *>(baseA);
  Tin *sKt = reinterpret_cast<Tin *>(baseA + (S::kt - S::akk));
  float *sAqk = reinterpret_cast<float *>(baseA + (S::aqk - S::akk));
  Tin *sAqh = reinterpret_cast<Tin *>(baseA + (S::aqh - S::akk));
  Tin *sTd = reinterpret_cast<Tin *>(baseA + (S::td - S::akk));
  float *sT1 = reinterpret_cast<float *>(baseT);
  float *sT2 = reinterpret_cast<float *>(baseT + (S::t2 - S::t1));
  float *sT0 = reinterpret_cast<float *>(baseT + (S::t0 - S::t1));
  float *sBeta = reinterpret_cast<float *>(baseT + (S::beta - S::t1));
  float *sBL = reinterpret_cast<float *>(baseT + (S::bl - S::t1));
  float *sDecay = reinterpret_cast<float *>(baseT + (S::decay - S::t1));
  float *sDt = reinterpret_cast<float *>(baseT + (S::dt - S::t1));
  float *sSeg = reinterpret_cast<float *>(baseT + (S::seg - S::t1));
  float *sQn = reinterpret_cast<float *>(baseT + (S::qn - S::t1));
  float *sPart = reinterpret_cast<float *>(baseT + (S::part - S::t1));
  bf16x8_t *sXc = reinterpret_cast<bf16x8_t *>(baseT + (S::xc - S::t1));

  const int wid = wave_id();
  const bool owner = wid * 16 < p.Vr;
  // the grams issue the next chunk's q, k, v loads, from half the waves
  constexpr bool GRAM_LOADS = (NW / NC >= 2);
  constexpr int NL = GRAM_LOADS ? NT / 2 : NT;
  const bool loader = !GRAM_LOADS || gram_loader<NW, NC>(wid);
  ChunkRegs<Tin, C, D, NT, NL, gram_shares<NW, NC>() == 4> regs;
  // item i is (chunk i % total, head i / total): the items of a head are consecutive
  int h = (int)(i0 / total), gc = (int)(i0 % total);
  ChunkLoc lc;
  locate_chunk(p, gc, lc);
  regs.load_gate(p, lc.t0, lc.L, h);
  if (loader) regs.load_qkv(p, lc.t0, lc.L, h);
  int hdt = -1;  // head whose dt_bias sDt and exp(A_log) expA hold
  float expA = 0.f;

  for (int64_t it = i0; it < i1; ++it) {
    const int L = lc.L;
    const int64_t t0 = lc.t0, gh = (int64_t)lc.gci * p.H + h;
    if (h != hdt) {  // uniform: a new head (the first item, or a range that crosses heads)
      expA = (GK == kGateSafe || GK == kGateSoftplus) ? fast_exp2(p.A_log[h] * kLog2e) : 0.f;
      for (int i = tid_opaque(); i < D; i += NT) {
        const float dt = (p.dt_bias && i < p.Kr) ? p.dt_bias[h * p.Kr + i] : 0.f;
        sDt[i] = (GK == kGateSafe) ? dt * (-expA * kLog2e) : dt;
      }
      hdt = h;
      __syncthreads();
    }
    regs.template store<GK>(loader, sQ, sK, sV, sB, sBeta, sDt, L, expA, p.lower_bound, p.q_l2norm != 0, sQn,
                            p.beta_logits != 0);
    __syncthreads();
    // the next item, loaded while this one computes
    ChunkLoc ln = lc;
    const bool more = it + 1 < i1;
    const bool wrap = gc + 1 == total;
    const int hn = wrap ? h + 1 : h, gn = wrap ? 0 : gc + 1;
    if (more) locate_chunk(p, gn, ln);
    // (1)
    if constexpr (GK == kGateLog2Cumsum) {
      gate_pad<NT, C, D>(sB, LDB, sBL, L);
      for (int i = tid_opaque(); i < D; i += NT) sDecay[i] = fast_exp2(sBL[i]);
    } else {
      gate_cumsum_tables<NT, C, D, SAFE>(sB, LDB, sBL, sSeg, sDecay, sT0, sT1, sT2, p.scale);
    }
    // (2), (3)
    auto load_next = [&]() {
      if (more) regs.load_qkv(p, ln.t0, ln.L, hn);
    };
    auto none = []() {};
    auto gate_next = [&]() {
      if (more) regs.load_gate(p, ln.t0, ln.L, hn);
    };
    if constexpr (GRAM_LOADS)
      grams_fused<NT, C, D, SAFE>(sQ, sK, LDT, sB, LDB, sBeta, p.scale, sAkk, sAqk, LDA, sAqh, S::LDAH, L, sT0, sT1,
                                  sT2, sBL, sKt, sXw, sTd, S::LDTD, sPart, sXc, load_next, gate_next);
    else
      grams_fused<NT, C, D, SAFE>(sQ, sK, LDT, sB, LDB, sBeta, p.scale, sAkk, sAqk, LDA, sAqh, S::LDAH, L, sT0, sT1,
                                  sT2, sBL, sKt, sXw, sTd, S::LDTD, sPart, sXc, none, gate_next);
    __syncthreads();
    if (!GRAM_LOADS && more) regs.load_qkv(p, ln.t0, ln.L, hn);
    // (4): w^T to LDS, u of this wave's value tile straight to the workspace
    {
      f32x4_t W[NC], U[NC];
      if (owner) wy_subst2<C, true>(sXw, wid, sV, wid, LDT, sBeta, sAkk, LDA, sTd, S::LDTD, W, U);
      else wy_subst2<C, false>(sXw, wid, sV, 0, LDT, sBeta, sAkk, LDA, sTd, S::LDTD, W, U);
      store_wT<C>(sWT, S::LDW, wid, W);
      if (owner) {
        f32x4_t *gu = reinterpret_cast<f32x4_t *>(p.swf + gh * SL::f32) + (wid * 64 + (tid_opaque() & 63)) * NC;
#pragma unroll
        for (int i = 0; i < NC; ++i) gu[i] = U[i];
      }
    }
    __syncthreads();
    u32x4_t *gb = reinterpret_cast<u32x4_t *>(static_cast<bf16_t *>(p.sws) + gh * SL::bf);
    constexpr int VQ = D / 8, VC = C / 8, NQ = C * VQ, NA = C * VC;
    for (int idx = tid_opaque(); idx < NQ; idx += NT) {
      const int r = idx / VQ, c = (idx % VQ) * 8;
      gb[idx] = *reinterpret_cast<const u32x4_t *>(sQ + r * LDT + c);
      gb[NQ + idx] = *reinterpret_cast<const u32x4_t *>(sKt + r * LDT + c);
      const int rw = idx / VC, cw = (idx % VC) * 8;
      gb[2 * NQ + idx] = *reinterpret_cast<const u32x4_t *>(sWT + rw * S::LDW + cw);
    }
    for (int idx = tid_opaque(); idx < NA; idx += NT) {
      const int r = idx / VC, c = (idx % VC) * 8;
      gb[3 * NQ + idx] = *reinterpret_cast<const u32x4_t *>(sAqh + r * S::LDAH + c);
    }
    float *gf = p.swf + gh * SL::f32;
    for (int i = tid_opaque(); i < D; i += NT) gf[SL::dec + i] = sDecay[i];
    if (p.q_l2norm)
      for (int i = tid_opaque(); i < C; i += NT) gf[SL::qn + i] = sQn[i];
    __syncthreads();  // the tiles are read out before the next item's store
    lc = ln;
    h = hn;
    gc = gn;
  }
}

// Threads of the state side: four waves, one value tile each, one per SIMD.
constexpr int kSplitThreads = 256;

template <int C, int D>
struct SplitSmem {
  static constexpr int LDT = Tile<bf16_t, C, D>::LDT, LDW = C + 8, LDAH = C + 8;
  static constexpr size_t q = 0, kt = q + 2 * C * LDT, wt = kt + 2 * C * LDT, aqh = wt + 2 * D * LDW;
  static constexpr size_t decay = aqh + 2 * C * LDAH;  // [2][D], by chunk parity
  static constexpr size_t qn = decay + 2 * 4 * D;
  static constexpr size_t total = qn + 4 * C;
};

// One chunk's state-side operands, from the workspace to registers (issued a
// chunk ahead) and from there to LDS.
template <int C, int D, int NT>
struct SplitRegs {
  using SL = SplitLayout<C, D>;
  static constexpr int VQ = D / 8, VC = C / 8, NQ = C * VQ, NA = C * VC;  // 16-byte vectors
  static constexpr int IQ = (NQ + NT - 1) / NT, IA = (NA + NT - 1) / NT, NC = C / 16;
  u32x4_t q[IQ], kt[IQ], wt[IQ], aq[IA];
  f32x4_t u[NC];
  float dec, qn;

  __device__ __forceinline__ void load(const ChunkParams &p, int64_t gh, int ctu, bool owner) {
    const u32x4_t *gb = reinterpret_cast<const u32x4_t *>(static_cast<const bf16_t *>(p.sws) + gh * SL::bf);
#pragma unroll
    for (int it = 0; it < IQ; ++it) {
      const int idx = it * NT + tid_opaque();
      if (NQ % NT == 0 || idx < NQ) {
        q[it] = gb[idx];
        kt[it] = gb[NQ + idx];
        wt[it] = gb[2 * NQ + idx];
      }
    }
#pragma unroll
    for (int it = 0; it < IA; ++it) {
      const int idx = it * NT + tid_opaque();
      if (NA % NT == 0 || idx < NA) aq[it] = gb[3 * NQ + idx];
    }
    const float *gf = p.swf + gh * SL::f32;
    if (owner) {
      const f32x4_t *gu = reinterpret_cast<const f32x4_t *>(gf) + (ctu * 64 + (tid_opaque() & 63)) * NC;
#pragma unroll
      for (int i = 0; i < NC; ++i) u[i] = gu[i];
    }
    const int t = tid_opaque();
    if (t < D) dec = gf[SL::dec + t];
    if (p.q_l2norm && t < C) qn = gf[SL::qn + t];
  }

  __device__ __forceinline__ void store(bf16_t *sQ, bf16_t *sKt, bf16_t *sWT, bf16_t *sAqh, int ldt, int ldw,
                                        int ldh, float *sDecay, float *sQn, bool qnorm) const {
#pragma unroll
    for (int it = 0; it < IQ; ++it) {
      const int idx = it * NT + tid_opaque();
      if (NQ % NT == 0 || idx < NQ) {
        const int r = idx / VQ, c = (idx % VQ) * 8, rw = idx / VC, cw = (idx % VC) * 8;
        *reinterpret_cast<u32x4_t *>(sQ + r * ldt + c) = q[it];
        *reinterpret_cast<u32x4_t *>(sKt + r * ldt + c) = kt[it];
        *reinterpret_cast<u32x4_t *>(sWT + rw * ldw + cw) = wt[it];
      }
    }
#pragma unroll
    for (int it = 0; it < IA; ++it) {
      const int idx = it * NT + tid_opaque();
      if (NA % NT == 0 || idx < NA) *reinterpret_cast<u32x4_t *>(sAqh + (idx / VC) * ldh + (idx % VC) * 8) = aq[it];
    }
    const int t = tid_opaque();
    if (t < D) sDecay[t] = dec;
    if (qnorm && t < C) sQn[t] = qn;
  }
};

// Workgroup index -> (unit, block) for `units` units of nb workgroups each:
// workgroups are dealt to the eight XCDs in turn, so with a multiple of eight
// units, unit u goes to XCD u % 8 and all nb workgroups of a unit to the same
// XCD (they read the same records, through its L2). Units of unequal length
// (packed slots) then spread over all XCDs instead of one XCD holding a run of
// long ones while another idles.
__device__ __forceinline__ void xcd_unit(int bid, int units, int nb, int &unit, int &blk) {
  if (units % 8 == 0) {
    const int x = bid % 8, k = bid / 8;
    blk = k % nb;
    unit = 8 * (k / nb) + x;
  } else {
    unit = bid / nb;
    blk = bid % nb;
  }
}

// (5), (6) and the state update of one (sequence, head, block of value tiles),
// walking the sequence's chunks with the key side's operands from the
// workspace.
template <int C, int D>
__global__ __launch_bounds__(kSplitThreads) void split_state_kernel(ChunkParams p) {
  using Tin = bf16_t;
  using TL = Tile<Tin, C, D>;
  using S = SplitSmem<C, D>;
  constexpr int NT = kSplitThreads, NC = TL::NC, DT = TL::DT, LDT = TL::LDT;
  constexpr int NVW = 1;
  static_assert(DT * 64 == NT * (D / 64), "four value tiles per workgroup");
  static_assert(S::total <= 65536, "DS immediate offsets");
  extern __shared__ __align__(16) char smem[];
  Tin *sQ = reinterpret_cast<Tin *>(smem + S::q);
  Tin *sKt = reinterpret_cast<Tin *>(smem + S::kt);
  Tin *sWT = reinterpret_cast<Tin *>(smem + S::wt);
  Tin *sAqh = reinterpret_cast<Tin *>(smem + S::aqh);
  float *sDecay2 = reinterpret_cast<float *>(smem + S::decay);
  float *sQn = reinterpret_cast<float *>(smem + S::qn);

  const int vs = D / 64;  // value-tile blocks per (sequence, head)
  int nh, vb;
  xcd_unit(blockIdx.x, p.N * p.H, vs, nh, vb);
  const int n = nh / p.H, h = nh % p.H;
  const int wid = wave_id();
  const int ctu = vb * 4 + wid;
  const bool owner = ctu * 16 < p.Vr;
  const int col0 = ctu * 16;
  const int Kr = p.Kr, Vr = p.Vr;
  const SlotRange sr = slot_range(p.cu, n, p.T);
  const int nch = (sr.len + C - 1) / C;
  const int cbase = p.cu ? p.chunk_off[n] : n * ((p.T + C - 1) / C);
  const int64_t sbase = (int64_t)nh * Kr * Vr;
  const int64_t ld = (int64_t)p.H * Vr;
  float *hcs = p.hc ? p.hc + ((int64_t)cbase * p.H + h) * Kr * Vr : nullptr;

  // two chunks' operands in flight: chunk c's are stored to LDS as chunk c + 2's are requested
  SplitRegs<C, D, NT> R0, R1;
  if (nch > 0) R0.load(p, (int64_t)cbase * p.H + h, ctu, owner);
  if (nch > 1) R1.load(p, (int64_t)(cbase + 1) * p.H + h, ctu, owner);
  f32x4_t hs[DT][NVW];
  if (p.h0 && owner) {
    load_strip<DT, NVW>(hs, p.h0 + sbase, Vr, col0, Kr, Vr);
  } else {
#pragma unroll
    for (int t = 0; t < DT; ++t) hs[t][0] = zero4();
  }
  bf16x8_t vprev[NC / 2][NVW];
#pragma unroll
  for (int s2 = 0; s2 < NC / 2; ++s2) vprev[s2][0] = bf16x8_t{};
  for (int i = tid_opaque(); i < D; i += NT) sDecay2[D + i] = 1.f;
  for (int i = tid_opaque(); i < C * LDT / 8; i += NT) reinterpret_cast<u32x4_t *>(sKt)[i] = u32x4_t{0u, 0u, 0u, 0u};
  __syncthreads();

  auto step = [&](int c, SplitRegs<C, D, NT> &R) {
    const int64_t t0 = sr.t0 + (int64_t)c * C;
    const int L = min(C, sr.len - c * C);
    // chunk c - 1's state update (the identity before the first chunk)
    if (owner) state_update_kt<C, D, NVW>(hs, sKt, LDT, vprev, sDecay2 + ((c + 1) & 1) * D);
    if (hcs && owner) store_strip<float, DT, NVW>(hcs + (int64_t)c * p.H * Kr * Vr, Vr, col0, Kr, hs, Vr);
    __syncthreads();  // every wave is done with chunk c - 1's operands
    R.store(sQ, sKt, sWT, sAqh, LDT, S::LDW, S::LDAH, sDecay2 + (c & 1) * D, sQn, p.q_l2norm != 0);
    f32x4_t uv[NC][NVW];
#pragma unroll
    for (int i = 0; i < NC; ++i) uv[i][0] = R.u[i];
    __syncthreads();
    if (c + 2 < nch) R.load(p, (int64_t)(cbase + c + 2) * p.H + h, ctu, owner);
    if (owner) {
      f32x4_t p1[NC][NVW], o[NC][NVW];
#pragma unroll
      for (int i = 0; i < NC; ++i) {
        p1[i][0] = zero4();
        o[i][0] = zero4();
      }
      q_times_state<C, D, NVW>(o, sQ, LDT, hs);
      w_times_state<C, D, NVW>(p1, sWT, S::LDW, hs);
#pragma unroll
      for (int i = 0; i < NC; ++i) uv[i][0] = uv[i][0] - p1[i][0];
      causal_times_h<C, NVW>(o, sAqh, S::LDAH, uv);
      vnew_frags<C, NVW>(vprev, uv);
      if (p.q_l2norm) {
        const int n16 = tid_opaque() & 15;
#pragma unroll
        for (int i = 0; i < NC; ++i) o[i][0] = o[i][0] * sQn[16 * i + n16];
      }
      store_oT<C, NVW>(reinterpret_cast<Tin *>(p.o) + t0 * ld + h * Vr, ld, col0, L, o, Vr);
    }
  };
  for (int c = 0; c < nch; c += 2) {
    step(c, R0);
    if (c + 1 < nch) step(c + 1, R1);
  }
  if (nch > 0 && owner) state_update_kt<C, D, NVW>(hs, sKt, LDT, vprev, sDecay2 + ((nch - 1) & 1) * D);
  if (owner && p.ht && !(sr.len == 0 && p.ht == p.h0)) store_strip<float, DT, NVW>(p.ht + sbase, Vr, col0, Kr, hs, Vr);
}

// ---------------------------------------------------------------------------------------------
// Chain-parallel state side. One chunk's state map is affine in the incoming
// state, h' = (Diag(2^b_L) - k~^T w) h + k~^T u, so a run of chunks maps
// h_out = M h_in + B; the run's outputs are affine in h_in as well,
// o = o_local + E h_in, where E is what the output step makes of the columns of
// M (q~ M - A_qk w M per chunk, with the row scales). A sequence's chunks are
// cut into segments of seg_len chunks. Its first segment runs from h0 and
// writes o itself; every later one runs the state side over 2D columns: D from
// the identity with u = 0 (M, and E per chunk) and the value columns from zero
// (B, and o_local per chunk). The segments run side by side; a combine pass
// then chains their maps, h_in(s + 1) = M_s h_in(s) + B_s, in fp32, and a
// correction pass adds E h_in to o_local for every chunk after the first
// segment, all chunks at once. Channels >= Kr stay exact: their columns of M
// only decay (k~, q~ and w vanish there) and the states' rows there are zero.
// ---------------------------------------------------------------------------------------------

struct SegLoc {
  int n, s, nseg;  // slot, segment within the slot, segments of the slot
  int c0, c1;      // chunks [c0, c1) of the slot
  int gs0;         // global index of the slot's first segment
};

__device__ __forceinline__ int dense_segments(const ChunkParams &p) {
  const int nt = (p.T + p.C - 1) / p.C;
  return max(1, (nt + p.seg_len - 1) / p.seg_len);
}

// Maps a global segment index to its slot and chunk range (false past the last).
__device__ __forceinline__ bool locate_segment(const ChunkParams &p, int gs, SegLoc &sl) {
  int nch;
  if (!p.cu) {
    const int ns = dense_segments(p);
    if (gs >= p.B * ns) return false;
    sl.n = gs / ns;
    sl.nseg = ns;
    sl.gs0 = sl.n * ns;
    nch = (p.T + p.C - 1) / p.C;
  } else {
    if (gs >= p.seg_off[p.N]) return false;
    int lo = 0, hi = p.N;  // largest n with seg_off[n] <= gs (every slot has a segment)
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (p.seg_off[mid] <= gs) lo = mid;
      else hi = mid;
    }
    sl.n = lo;
    sl.gs0 = p.seg_off[lo];
    sl.nseg = p.seg_off[lo + 1] - sl.gs0;
    nch = p.chunk_off[lo + 1] - p.chunk_off[lo];
  }
  sl.s = gs - sl.gs0;
  sl.c0 = sl.s * p.seg_len;
  sl.c1 = min(sl.c0 + p.seg_len, nch);
  return true;
}

// One (segment, head, block of four 16-column tiles) of the 2D columns [M | B]:
// the walk of split_state_kernel over the segment's chunks, from the identity
// (M tiles, u = 0), from zero (B tiles) or from h0 (the first segment, which
// has B tiles only and writes o). Two workgroups fit a compute unit.
template <int C, int D>
__global__ __launch_bounds__(kSplitThreads, 2) void split_seg_kernel(ChunkParams p) {
  using Tin = bf16_t;
  using TL = Tile<Tin, C, D>;
  using S = SplitSmem<C, D>;
  constexpr int NT = kSplitThreads, NC = TL::NC, DT = TL::DT, LDT = TL::LDT;
  constexpr int NVW = 1, NB = 2 * (D / 64);
  static_assert(S::total <= 65536, "DS immediate offsets");
  extern __shared__ __align__(16) char smem[];
  Tin *sQ = reinterpret_cast<Tin *>(smem + S::q);
  Tin *sKt = reinterpret_cast<Tin *>(smem + S::kt);
  Tin *sWT = reinterpret_cast<Tin *>(smem + S::wt);
  Tin *sAqh = reinterpret_cast<Tin *>(smem + S::aqh);
  float *sDecay2 = reinterpret_cast<float *>(smem + S::decay);
  float *sQn = reinterpret_cast<float *>(smem + S::qn);

  // the NB workgroups of one (segment, head) share an XCD and its L2; each XCD
  // takes a contiguous range of (segment, head) units (segments of dense
  // batches are of equal length, and the heads of one segment read adjacent records)
  const int G = p.seg_max * p.H * NB;
  const int bid = blockIdx.x;
  const int li = (G % 8 == 0) ? (bid % 8) * (G / 8) + bid / 8 : bid;
  const int cb = li % NB, gh = li / NB;
  const int h = gh % p.H, gs = gh / p.H;
  SegLoc sg;
  if (!locate_segment(p, gs, sg)) return;
  const bool isM = cb < D / 64;
  if (isM && sg.s == 0) return;
  const int wid = wave_id();
  const int ctu = (isM ? cb : cb - D / 64) * 4 + wid;
  const int col0 = ctu * 16;
  const bool owner = isM || col0 < p.Vr;
  const int Kr = p.Kr, Vr = p.Vr, n = sg.n;
  const SlotRange sr = slot_range(p.cu, n, p.T);
  const int cbase = p.cu ? p.chunk_off[n] : n * ((p.T + C - 1) / C);
  const int64_t ld = (int64_t)p.H * Vr;
  const int64_t sbase = ((int64_t)n * p.H + h) * Kr * Vr;
  const int lane = tid_opaque() & 63;
  const int n16 = lane & 15, grp = lane >> 4;

  SplitRegs<C, D, NT> R;
  if (sg.c0 < sg.c1) R.load(p, (int64_t)(cbase + sg.c0) * p.H + h, ctu, owner && !isM);
  f32x4_t hs[DT][NVW];
  if (isM) {
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) hs[t][0][e] = (16 * t + 4 * grp + e == col0 + n16) ? 1.f : 0.f;
  } else if (sg.s == 0 && p.h0 && owner) {
    load_strip<DT, NVW>(hs, p.h0 + sbase, Vr, col0, Kr, Vr);
  } else {
#pragma unroll
    for (int t = 0; t < DT; ++t) hs[t][0] = zero4();
  }
  bf16x8_t vprev[NC / 2][NVW];
#pragma unroll
  for (int s2 = 0; s2 < NC / 2; ++s2) vprev[s2][0] = bf16x8_t{};
  // the first chunk's "previous" update is the identity: decay 1, k~ = 0
  for (int i = tid_opaque(); i < D; i += NT) sDecay2[((sg.c0 + 1) & 1) * D + i] = 1.f;
  for (int i = tid_opaque(); i < C * LDT / 8; i += NT) reinterpret_cast<u32x4_t *>(sKt)[i] = u32x4_t{0u, 0u, 0u, 0u};
  __syncthreads();

  for (int c = sg.c0; c < sg.c1; ++c) {
    const int64_t t0 = sr.t0 + (int64_t)c * C;
    const int L = min(C, sr.len - c * C);
    const int64_t gch = (int64_t)(cbase + c) * p.H + h;
    // chunk c - 1's state update
    if (owner) state_update_kt<C, D, NVW>(hs, sKt, LDT, vprev, sDecay2 + ((c + 1) & 1) * D);
    __syncthreads();  // every wave is done with chunk c - 1's operands
    R.store(sQ, sKt, sWT, sAqh, LDT, S::LDW, S::LDAH, sDecay2 + (c & 1) * D, sQn, p.q_l2norm != 0);
    f32x4_t uv[NC][NVW];
#pragma unroll
    for (int i = 0; i < NC; ++i) uv[i][0] = isM ? zero4() : R.u[i];
    __syncthreads();
    if (c + 1 < sg.c1) R.load(p, gch + p.H, ctu, owner && !isM);
    if (owner) {
      f32x4_t p1[NC][NVW], o[NC][NVW];
#pragma unroll
      for (int i = 0; i < NC; ++i) {
        p1[i][0] = zero4();
        o[i][0] = zero4();
      }
      q_times_state<C, D, NVW>(o, sQ, LDT, hs);
      w_times_state<C, D, NVW>(p1, sWT, S::LDW, hs);
#pragma unroll
      for (int i = 0; i < NC; ++i) uv[i][0] = uv[i][0] - p1[i][0];
      causal_times_h<C, NVW>(o, sAqh, S::LDAH, uv);
      vnew_frags<C, NVW>(vprev, uv);
      if (p.q_l2norm) {
#pragma unroll
        for (int i = 0; i < NC; ++i) o[i][0] = o[i][0] * sQn[16 * i + n16];
      }
      if (sg.s == 0) {
        store_oT<C, NVW>(reinterpret_cast<Tin *>(p.o) + t0 * ld + h * Vr, ld, col0, L, o, Vr);
      } else if (isM) {
        // E rows with the channels of each 32-block in the operand order of q~
        // (the lane's channels 4g.., 16 + 4g.. of the block side by side at 8g)
        Tin *E = static_cast<Tin *>(p.seg_e) + gch * C * D + 32 * (ctu >> 1) + 8 * grp + 4 * (ctu & 1);
#pragma unroll
        for (int i = 0; i < NC; ++i) *reinterpret_cast<bf16x4_t *>(E + (16 * i + n16) * D) = to_bf16x4(o[i][0]);
      } else {
        float *OL = p.seg_ol + gch * C * D + col0 + 4 * grp;
#pragma unroll
        for (int i = 0; i < NC; ++i) *reinterpret_cast<f32x4_t *>(OL + (16 * i + n16) * D) = o[i][0];
      }
    }
  }
  if (sg.c1 > sg.c0 && owner) state_update_kt<C, D, NVW>(hs, sKt, LDT, vprev, sDecay2 + ((sg.c1 - 1) & 1) * D);
  if (sg.nseg == 1) {
    if (owner && p.ht && !(sr.len == 0 && p.ht == p.h0)) store_strip<float, DT, NVW>(p.ht + sbase, Vr, col0, Kr, hs, Vr);
  } else if (owner) {
    float *mb = p.seg_mb + ((int64_t)gs * p.H + h) * (int64_t)D * (2 * D);
    store_strip<float, DT, NVW>(mb, 2 * D, (isM ? 0 : D) + col0, D, hs);
  }
}

// The segments' incoming states, h_in(s + 1) = M_s h_in(s) + B_s with h_in(1) =
// B_0, in fp32, and the final state. One workgroup per (slot, head, 16-column
// tile): wave w forms row tiles w*DT/4.. of the next state with 16x16x4 fp32
// products (a C-layout state tile is the B operand as it stands, contraction
// index of step (t, e) at rows 16t + 4g + e), and the whole strip goes through
// LDS to every wave for the next step. Each h_in(s) also goes out as the bf16
// operand fragments of the correction's product.
template <int D>
__global__ __launch_bounds__(256) void seg_combine_kernel(ChunkParams p) {
  constexpr int DT = D / 16, SD = D / 32, IW = DT / 4, LDS_ = 20;
  constexpr int64_t MBS = (int64_t)D * 2 * D;
  __shared__ __align__(16) float sS[2][D * LDS_];
  const int bid = blockIdx.x;
  const int ctu = bid % DT, nh = bid / DT;
  const int n = nh / p.H, h = nh % p.H;
  int gs0, nseg;
  if (p.cu) {
    gs0 = p.seg_off[n];
    nseg = p.seg_off[n + 1] - gs0;
  } else {
    nseg = dense_segments(p);
    gs0 = n * nseg;
  }
  const int col0 = 16 * ctu;
  if (nseg <= 1 || col0 >= p.Vr) return;  // uniform over the workgroup
  const int w = wave_id(), lane = tid_opaque() & 63;
  const int n16 = lane & 15, grp = lane >> 4;
  const float *mb0 = p.seg_mb + ((int64_t)gs0 * p.H + h) * MBS;
  f32x4_t acc[IW];
  // B_0 rows of this wave's tiles
#pragma unroll
  for (int i = 0; i < IW; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[i][e] = mb0[(int64_t)(16 * (w * IW + i) + 4 * grp + e) * (2 * D) + D + col0 + n16];
  int cur = 0;
#pragma unroll
  for (int i = 0; i < IW; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) sS[0][(16 * (w * IW + i) + 4 * grp + e) * LDS_ + n16] = acc[i][e];
  __syncthreads();
  for (int s = 1; s < nseg; ++s) {
    const int64_t gsh = (int64_t)(gs0 + s) * p.H + h;
    const float *S = sS[cur];
    // h_in(s) as bf16 fragments: k-step j holds rows 32j + 4g + e and 32j + 16 + 4g + e
    for (int j = w; j < SD; j += 4) {
      u32x4_t f;
      f[0] = pack_bf16x2(S[(32 * j + 4 * grp) * LDS_ + n16], S[(32 * j + 4 * grp + 1) * LDS_ + n16]);
      f[1] = pack_bf16x2(S[(32 * j + 4 * grp + 2) * LDS_ + n16], S[(32 * j + 4 * grp + 3) * LDS_ + n16]);
      f[2] = pack_bf16x2(S[(32 * j + 16 + 4 * grp) * LDS_ + n16], S[(32 * j + 16 + 4 * grp + 1) * LDS_ + n16]);
      f[3] = pack_bf16x2(S[(32 * j + 16 + 4 * grp + 2) * LDS_ + n16], S[(32 * j + 16 + 4 * grp + 3) * LDS_ + n16]);
      static_cast<u32x4_t *>(p.seg_sin)[((gsh * DT + ctu) * SD + j) * 64 + lane] = f;
    }
    const float *mb = p.seg_mb + gsh * MBS;
    // two accumulators per row tile (even and odd contraction tiles) keep the
    // dependent products apart
    f32x4_t a2[IW][2];
#pragma unroll
    for (int i = 0; i < IW; ++i) {
#pragma unroll
      for (int e = 0; e < 4; ++e) a2[i][0][e] = mb[(int64_t)(16 * (w * IW + i) + 4 * grp + e) * (2 * D) + D + col0 + n16];
      a2[i][1] = zero4();
    }
#pragma unroll
    for (int t = 0; t < DT; ++t) {
      f32x4_t a[IW];
#pragma unroll
      for (int i = 0; i < IW; ++i)
        a[i] = *reinterpret_cast<const f32x4_t *>(mb + (int64_t)(16 * (w * IW + i) + n16) * (2 * D) + 16 * t + 4 * grp);
      f32x4_t b;
#pragma unroll
      for (int e = 0; e < 4; ++e) b[e] = S[(16 * t + 4 * grp + e) * LDS_ + n16];
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int i = 0; i < IW; ++i) a2[i][t & 1] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i][e], b[e], a2[i][t & 1], 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < IW; ++i) acc[i] = a2[i][0] + a2[i][1];
#pragma unroll
    for (int i = 0; i < IW; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) sS[cur ^ 1][(16 * (w * IW + i) + 4 * grp + e) * LDS_ + n16] = acc[i][e];
    __syncthreads();
    cur ^= 1;
  }
  if (p.ht) {
    float *ht = p.ht + (int64_t)nh * p.Kr * p.Vr;
#pragma unroll
    for (int i = 0; i < IW; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * (w * IW + i) + 4 * grp + e, c = col0 + n16;
        if (r < p.Kr && c < p.Vr) ht[(int64_t)r * p.Vr + c] = acc[i][e];
      }
  }
}

// Chunks per workgroup of the correction: they share one load of h_in.
constexpr int kCorrChunks = 8;

// o = o_local + E h_in for every chunk after its sequence's first segment: one
// workgroup of D/16 waves (one 16-column tile each) per (segment, head,
// kCorrChunks chunks). h_in's fragments are loaded once; each chunk's E is
// staged in LDS for all waves, and the next chunk's E and o_local are in flight
// while a chunk computes.
template <int C, int D>
__global__ __launch_bounds__(4 * D) void seg_correct_kernel(ChunkParams p) {
  using M = Mma<bf16_t>;
  constexpr int NT = 4 * D, NC = C / 16, DT = D / 16, SD = D / 32, LDE = D + 8;
  constexpr int EV = C * D / 8, EI = EV / NT;  // 16-byte vectors of E per chunk, per thread
  static_assert(EV % NT == 0, "whole vectors per thread");
  __shared__ __align__(16) bf16_t sE[C * LDE];
  const int NGR = (p.seg_len + kCorrChunks - 1) / kCorrChunks;
  const int64_t G = (int64_t)p.seg_max * p.H * NGR;
  const int64_t bid = blockIdx.x;
  const int64_t li = (G % 8 == 0) ? (bid % 8) * (G / 8) + bid / 8 : bid;
  const int gr = (int)(li % NGR);
  const int64_t gh = li / NGR;
  const int h = (int)(gh % p.H), gs = (int)(gh / p.H);
  SegLoc sg;
  if (!locate_segment(p, gs, sg) || sg.s == 0) return;
  const int ca = sg.c0 + gr * kCorrChunks, cz = min(ca + kCorrChunks, sg.c1);
  if (ca >= cz) return;  // uniform over the workgroup
  const int ctu = wave_id(), col0 = 16 * ctu, t = tid_opaque();
  const bool owner = col0 < p.Vr;
  const int lane = t & 63;
  const int n16 = lane & 15, grp = lane >> 4;
  const int64_t gsh = (int64_t)gs * p.H + h;
  bf16x8_t fh[SD];
#pragma unroll
  for (int j = 0; j < SD; ++j)
    fh[j] = owner ? __builtin_bit_cast(bf16x8_t, static_cast<const u32x4_t *>(p.seg_sin)[((gsh * DT + ctu) * SD + j) * 64 + lane])
                  : bf16x8_t{};
  const SlotRange sr = slot_range(p.cu, sg.n, p.T);
  const int cbase = p.cu ? p.chunk_off[sg.n] : sg.n * ((p.T + C - 1) / C);
  const int64_t ld = (int64_t)p.H * p.Vr;
  u32x4_t ev[EI];
  f32x4_t ol[NC];
  auto fetch = [&](int c) {
    const int64_t gch = (int64_t)(cbase + c) * p.H + h;
    const u32x4_t *E = reinterpret_cast<const u32x4_t *>(static_cast<const bf16_t *>(p.seg_e) + gch * C * D);
#pragma unroll
    for (int i = 0; i < EI; ++i) ev[i] = E[i * NT + t];
    if (owner) {
      const float *OL = p.seg_ol + gch * C * D + col0 + 4 * grp;
#pragma unroll
      for (int i = 0; i < NC; ++i) ol[i] = *reinterpret_cast<const f32x4_t *>(OL + (16 * i + n16) * D);
    }
  };
  fetch(ca);
  for (int c = ca; c < cz; ++c) {
    __syncthreads();  // the previous chunk's reads of sE are done
#pragma unroll
    for (int i = 0; i < EI; ++i) {
      const int v = i * NT + t;
      *reinterpret_cast<u32x4_t *>(sE + (v / (D / 8)) * LDE + (v % (D / 8)) * 8) = ev[i];
    }
    f32x4_t o[NC][1];
#pragma unroll
    for (int i = 0; i < NC; ++i) o[i][0] = ol[i];
    __syncthreads();
    if (c + 1 < cz) fetch(c + 1);
    if (owner) {
      const bf16_t *eRow = sE + n16 * LDE + 8 * grp;
#pragma unroll
      for (int j = 0; j < SD; ++j)
#pragma unroll
        for (int i = 0; i < NC; ++i) {
          const bf16x8_t fq = *reinterpret_cast<const bf16x8_t *>(eRow + 16 * i * LDE + 32 * j);
          o[i][0] = M::mma(fh[j], fq, o[i][0]);
        }
      const int64_t t0 = sr.t0 + (int64_t)c * C;
      store_oT<C, 1>(reinterpret_cast<bf16_t *>(p.o) + t0 * ld + h * p.Vr, ld, col0, min(C, sr.len - c * C), o, p.Vr);
    }
  }
}

// Whether the split schedule is expected to beat the fused one, from a cost
// model of the two measured on MI355X (C = 64, D = 128, safe gate): the fused
// kernel walks each (sequence, head)'s chunks at ~8.7 us a chunk, one pair per
// compute unit; the split key side costs ~11 us per (chunk, head) item per
// compute unit, and its state side ~3.3 us a chunk with one workgroup per
// D / 64 value tiles a unit. The chain is the longest sequence in chunks (for
// packed calls, bounded by the capacity T); items are the (chunk, head) pairs.
bool split_supported(const ChunkParams &p) { return p.is_bf16 && (p.D == 64 || p.D == 128); }

bool split_preferred(int64_t chain, int64_t pairs, int64_t items, int D) {
  const int64_t cus = device_cus();
  const double fused = 8.7 * chain * ((pairs + cus - 1) / cus);
  const int64_t wgs = pairs * (D / 64);
  const double split = 11.0 * ((items + cus - 1) / cus) + 3.3 * chain * ((wgs + cus - 1) / cus);
  return split < 0.9 * fused;
}

// The segment length from a cost model of the state side measured on MI355X
// (C = 64, D = 128): the serial chain takes ~3.4 us a chunk with one workgroup
// per compute unit; the segment walk ~5.9 us a chunk per round of two
// workgroups per compute unit; the combine ~8 us plus ~4 us a step; the
// correction ~18 ns per (chunk, head) after the first segment. Segments double
// the state side's work past the first, so they pay only where the serial chain
// leaves most compute units idle (few pairs, long sequences).
int split_segment_len(int64_t chain, int64_t pairs, int D, int C) {
  (void)C;
  if (chain < 8 || pairs <= 0) return 0;
  const int64_t cus = device_cus(), nb = D / 64;
  const double serial = 3.4 * chain * ((pairs * nb + cus - 1) / cus);
  double best = 0.9 * serial;
  int best_len = 0;
  for (int64_t P = 2; P <= 64; P *= 2) {
    const int64_t len = (chain + P - 1) / P;
    if (len < 4) break;
    const int64_t ns = (chain + len - 1) / len;
    const int64_t wgs = pairs * nb * (2 * ns - 1);
    const double t = 5.9 * len * ((wgs + 2 * cus - 1) / (2 * cus)) + 8.0 + 4.0 * (ns - 1) + 5.0 +
                     0.018 * pairs * (chain - len);
    if (t < best) {
      best = t;
      best_len = (int)len;
    }
  }
  return best_len;
}

int64_t split_segment_bound(int B, int N, int64_t nt, bool packed, int seg_len) {
  if (seg_len <= 0) return 0;
  if (packed) return (int64_t)N + (nt + N + seg_len - 1) / seg_len;
  return (int64_t)B * std::max<int64_t>(1, (nt + seg_len - 1) / seg_len);
}

size_t split_segment_bytes(int C, int D, int64_t chunk_heads, int64_t seg_heads) {
  return (size_t)chunk_heads * C * D * (2 + 4) + (size_t)seg_heads * D * D * (2 * 4 + 2);
}

namespace {

template <int C, int D, int NT, int GK>
hipError_t launch_split_g(const ChunkParams &p, hipStream_t st) {
  if (p.max_chunks > 0 && p.H > 0) {
    const size_t smem = FusedSmem<C, D, NT>::total;
    auto kern = split_key_kernel<C, D, NT, GK>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      return e;
    }
    // one workgroup per compute unit, each over a contiguous range of items
    const int64_t items = (int64_t)p.max_chunks * p.H;
    const int grid = (int)std::min<int64_t>(items, device_cus());
    hipLaunchKernelGGL(kern, dim3(grid), dim3(NT), smem, st, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (p.N * p.H == 0) return hipSuccess;
  constexpr size_t smem2 = SplitSmem<C, D>::total;
  if (p.seg_len > 0) {
    // segments side by side, then the combine chain, then the correction
    const int64_t G = (int64_t)p.seg_max * p.H * (2 * D / 64);
    if (G > 0) {
      hipLaunchKernelGGL((split_seg_kernel<C, D>), dim3(G), dim3(kSplitThreads), smem2, st, p);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((seg_combine_kernel<D>), dim3(p.N * p.H * (D / 16)), dim3(256), 0, st, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || G == 0) return e;
    const int64_t G2 = (int64_t)p.seg_max * p.H * ((p.seg_len + kCorrChunks - 1) / kCorrChunks);
    hipLaunchKernelGGL((seg_correct_kernel<C, D>), dim3(G2), dim3(4 * D), 0, st, p);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((split_state_kernel<C, D>), dim3(p.N * p.H * (D / 64)), dim3(kSplitThreads), smem2, st, p);
  return hipGetLastError();
}

template <int C, int D>
hipError_t launch_split_t(const ChunkParams &p, hipStream_t st) {
  constexpr int NT = (KDA_FUSED_THREADS > 0) ? KDA_FUSED_THREADS : ((D / 16 >= 8) ? 512 : 256);
  switch (p.gate_kind) {
    case kGateSafe: return launch_split_g<C, D, NT, kGateSafe>(p, st);
    case kGateSoftplus: return launch_split_g<C, D, NT, kGateSoftplus>(p, st);
    case kGateLogE: return launch_split_g<C, D, NT, kGateLogE>(p, st);
    case kGateLog2Cumsum: return launch_split_g<C, D, NT, kGateLog2Cumsum>(p, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_split(const ChunkParams &p, hipStream_t st) {
  if (!p.is_bf16) return hipErrorInvalidValue;
  if (p.C == 64 && p.D == 128) return launch_split_t<64, 128>(p, st);
  if (p.C == 64 && p.D == 64) return launch_split_t<64, 64>(p, st);
  if (p.C == 32 && p.D == 128) return launch_split_t<32, 128>(p, st);
  if (p.C == 32 && p.D == 64) return launch_split_t<32, 64>(p, st);
  return hipErrorInvalidValue;
}

}  // namespace kda
