// The fused schedule of the chunked KDA forward: one persistent workgroup per
// (sequence, head) walks the sequence's chunks in order and runs steps (1)-(6)
// for each chunk entirely on chip. Inputs are read from HBM exactly once and
// only o and the final state are written (plus, when asked for, the state at
// the start of every chunk); the [D, D] FP32 state lives in MFMA
// accumulator registers for the whole sequence (each of the NT/64 waves owns
// a 16*NVW-column strip of it). bf16 inputs only (fp32 inputs run the staged
// schedule).
//
// The next chunk's raw inputs are loaded into registers while the current
// chunk computes, so HBM latency overlaps the on-chip work.
//
// Per chunk:
//   store   raw q, k, v and the activated gate to LDS
//   (1)     chunk-local cumsum of the gate (b), 2^b_L
//   (2)     grams A_kk (fp32), A_qk (bf16), and from the same exponentials
//           q~ = scale q 2^b, X_w = beta k 2^b and k~ = k 2^(b_L-b)
//   (3)     one wave inverts the four 16x16 diagonal blocks of I + A_kk
//   (4)     each wave solves its 16-column tiles of w and u by blocked
//           forward substitution; w goes to LDS transposed, u stays in registers
//   (5)+(6) v_new = u - w h, o = q~ h + A_qk v_new, h <- 2^b_L h + k~^T v_new
//   o       formed transposed, so each lane stores four adjacent columns
//
// LDS (C = 64, D = 128: about 156 KB): q (-> q~), k, v, gate (-> b -> X_w and
// w^T), A_kk, k~, A_qk (fp32 partial sums and the bf16 result), the diagonal
// inverses, the midpoint tables, beta, b_L, 2^b_L, dt_bias.
#include "chunk_fused_layout.h"
#include "kda_launch.h"

// Threads per workgroup of the fused kernel (0: 512 when the state has at
// least 8 column tiles, else 256). A build-time knob for tuning.
#ifndef KDA_FUSED_THREADS
#define KDA_FUSED_THREADS 0
#endif

namespace kda {

template <int C, int D, int NT, int GK>
__global__ __launch_bounds__(NT) void fused_chunk_kernel(ChunkParams p) {
  using Tin = bf16_t;
  using TL = Tile<Tin, C, D>;
  using S = FusedSmem<C, D, NT>;
  constexpr bool SAFE = (GK == kGateSafe);
  constexpr int NW = NT / 64, NC = TL::NC, DT = TL::DT, LDT = TL::LDT, LDB = TL::LDB, LDA = TL::LDA;
  // one value tile per wave; at D = 256 the eight waves also solve two w tiles
  // each (with the whole state in eight waves, half of every wave's 256 VGPRs
  // would hold state and the rest spill: 1.39 against 1.12 ms at B8 T2048 H32)
  constexpr int NVW = 1;
  constexpr int WT = DT / NW;
  static_assert(WT * NW == DT && (WT == 1 || WT == 2), "w column tiles per wave");

  extern __shared__ __align__(16) char smem[];
  // buffers below 64 KB at constant offsets; the others from three opaque bases
  char *baseB = lds_base(smem, S::b), *baseA = lds_base(smem, S::akk), *baseT = lds_base(smem, S::t1);
  static_assert(S::b % 16 == 0 && S::wt_off % 16 == 0 && S::akk % 16 == 0 && S::kt % 16 == 0 && S::aqk % 16 == 0 &&
                    S::aqh % 16 == 0 && S::td % 16 == 0 && S::t1 % 16 == 0 && S::t2 % 16 == 0 && S::t0 % 16 == 0 && S::beta % 16 == 0 &&
                    S::bl % 16 == 0 && S::decay % 16 == 0 && S::dt % 16 == 0 && S::seg % 16 == 0 && S::qn % 16 == 0 && S::part % 16 == 0 && S::xc % 16 == 0,
                "16-byte aligned buffers");
  static_assert( S::td + 2 * C * S::LDTD - S::akk <= 65536 &&
                    S::total - S::t1 <= 65536 && S::v + S::tile <= 65536,
                "DS immediate offsets below 64 KB");
  Tin *sQ = reinterpret_cast<Tin *>(smem + S::q);    // q, then q~
  Tin *sK = reinterpret_cast<Tin *>(smem + S::k);    // k, then beta k 2^b
  Tin *sV = reinterpret_cast<Tin *>(smem + S::v);
  float *sB = reinterpret_cast<float *>(smem + S::b);             // gate, then b
  Tin *sXw = reinterpret_cast<Tin *>(smem + S::b + S::xw_off);  // beta k 2^b once b is consumed
  Tin *sWT = reinterpret_cast<Tin *>(baseB + S::wt_off);        // w^T
  float *sAkk = reinterpret_cast<float *>(baseA);
  Tin *sKt = reinterpret_cast<Tin *>(baseA + (S::kt - S::akk));
  float *sAqk = reinterpret_cast<float *>(baseA + (S::aqk - S::akk));  // partial sums of A_qk
  Tin *sAqh = reinterpret_cast<Tin *>(baseA + (S::aqh - S::akk));      // A_qk
  Tin *sTd = reinterpret_cast<Tin *>(baseA + (S::td - S::akk));
  float *sT1 = reinterpret_cast<float *>(baseT);
  float *sT2 = reinterpret_cast<float *>(baseT + (S::t2 - S::t1));
  float *sT0 = reinterpret_cast<float *>(baseT + (S::t0 - S::t1));
  float *sBeta = reinterpret_cast<float *>(baseT + (S::beta - S::t1));
  float *sBL = reinterpret_cast<float *>(baseT + (S::bl - S::t1));
  float *sDecay2 = reinterpret_cast<float *>(baseT + (S::decay - S::t1));  // [2][D], by chunk parity
  float *sDt = reinterpret_cast<float *>(baseT + (S::dt - S::t1));
  float *sSeg = reinterpret_cast<float *>(baseT + (S::seg - S::t1));
  float *sQn = reinterpret_cast<float *>(baseT + (S::qn - S::t1));
  float *sPart = reinterpret_cast<float *>(baseT + (S::part - S::t1));
  bf16x8_t *sXc = reinterpret_cast<bf16x8_t *>(baseT + (S::xc - S::t1));

  // workgroup = (sequence, head, block vb of D / vsplit value columns); waves
  // below tpb own one 16-column tile of the state, all waves share the key side
  const int vs = p.vsplit, tpb = DT / vs;
  const int nh = blockIdx.x / vs, vb = blockIdx.x % vs;
  const int n = nh / p.H, h = nh % p.H;
  const int wid = wave_id();
  const int ctu = vb * tpb + wid;  // this wave's value tile (owners)
  const bool owner = wid < tpb && ctu * 16 < p.Vr;  // tiles wholly past Vr are zero
  const int col0 = ctu * 16;
  const int Kr = p.Kr, Vr = p.Vr;
  const SlotRange sr = slot_range(p.cu, n, p.T);
  const int nch = (sr.len + C - 1) / C;
  const int64_t sbase = (int64_t)nh * Kr * Vr;  // states [Kr, Vr]
  const int64_t ld = (int64_t)p.H * Vr;
  // chunk-start states, if asked for: chunks numbered slot by slot
  float *hcs = p.hc ? p.hc + ((int64_t)(p.cu ? p.chunk_off[n] : n * ((p.T + C - 1) / C)) * p.H + h) * Kr * Vr : nullptr;
  const float expA = (GK == kGateSafe || GK == kGateSoftplus) ? fast_exp2(p.A_log[h] * kLog2e) : 0.f;
  for (int i = tid_opaque(); i < D; i += NT) {
    const float dt = (p.dt_bias && i < Kr) ? p.dt_bias[h * Kr + i] : 0.f;
    sDt[i] = (GK == kGateSafe) ? dt * (-expA * kLog2e) : dt;
  }

  f32x4_t hs[DT][NVW];
  if (p.h0 && owner) {
    load_strip<DT, NVW>(hs, p.h0 + sbase, Vr, col0, Kr, Vr);
  } else {
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int v = 0; v < NVW; ++v) hs[t][v] = zero4();
  }

  // with two waves per row block of the grams, the even waves load the next
  // chunk's q, k, v while the odd ones invert the diagonal blocks
  // the grams issue the next chunk's q, k, v loads, from half the waves
  constexpr bool GRAM_LOADS = (NW / NC >= 2);
  constexpr int NL = GRAM_LOADS ? NT / 2 : NT;
  const bool loader = !GRAM_LOADS || gram_loader<NW, NC>(wid);
  // the next chunk's raw inputs wait in registers while a chunk computes
  constexpr bool PREFETCH = true;
  ChunkRegs<Tin, C, D, NT, NL, gram_shares<NW, NC>() == 4> regs;
  if (PREFETCH && nch > 0) {
    regs.load_gate(p, sr.t0, min(C, sr.len), h);
    if (loader) regs.load_qkv(p, sr.t0, min(C, sr.len), h);
  }
  // v_new of the chunk as bf16 operand fragments of its state update
  // h <- Diag(2^b_L) h + k~^T v_new
  bf16x8_t vprev[NC / 2][NVW];
  __syncthreads();  // sDt visible

  for (int c = 0; c < nch; ++c) {
    const int64_t t0 = sr.t0 + (int64_t)c * C;
    const int L = min(C, sr.len - c * C);
    const int64_t off = t0 * ld + h * Vr;
    float *sDecay = sDecay2 + (c & 1) * D;
    if constexpr (!PREFETCH) {
      regs.load_gate(p, t0, L, h);
      if (loader) regs.load_qkv(p, t0, L, h);
    }
    regs.template store<GK>(loader, sQ, sK, sV, sB, sBeta, sDt, L, expA, p.lower_bound, p.q_l2norm != 0, sQn,
                            p.beta_logits != 0);
    if (hcs && owner) store_strip<float, DT, NVW>(hcs + (int64_t)c * p.H * Kr * Vr, Vr, col0, Kr, hs, Vr);
    __syncthreads();
    // the next chunk's inputs are loaded in two parts while this chunk computes:
    // the gate by every wave as it finishes the grams' first phase (the waves get
    // there at different times, so their loads do not queue at once), then q, k, v
    const bool more = PREFETCH && c + 1 < nch;
    const int Ln = more ? min(C, sr.len - (c + 1) * C) : 0;

    // (1)
    if constexpr (GK == kGateLog2Cumsum) {
      gate_pad<NT, C, D>(sB, LDB, sBL, L);
      for (int i = tid_opaque(); i < D; i += NT) sDecay[i] = fast_exp2(sBL[i]);  // read after later barriers
    } else {
      gate_cumsum_tables<NT, C, D, SAFE>(sB, LDB, sBL, sSeg, sDecay, sT0, sT1, sT2, p.scale);
    }
    // (2) the grams, and q~, k~, beta k 2^b; (3) the diagonal inverses
    auto load_next = [&]() {
      if (more) regs.load_qkv(p, t0 + C, Ln, h);
    };
    auto none = []() {};
    auto gate_next = [&]() {
      if (more) regs.load_gate(p, t0 + C, Ln, h);
    };
    if constexpr (GRAM_LOADS)
      grams_fused<NT, C, D, SAFE>(sQ, sK, LDT, sB, LDB, sBeta, p.scale, sAkk, sAqk, LDA, sAqh, S::LDAH, L, sT0, sT1,
                                  sT2, sBL, sKt, sXw, sTd, S::LDTD, sPart, sXc, load_next, gate_next);
    else
      grams_fused<NT, C, D, SAFE>(sQ, sK, LDT, sB, LDB, sBeta, p.scale, sAkk, sAqk, LDA, sAqh, S::LDAH, L, sT0, sT1,
                                  sT2, sBL, sKt, sXw, sTd, S::LDTD, sPart, sXc, none, gate_next);
    __syncthreads();
    if (!GRAM_LOADS && more) regs.load_qkv(p, t0 + C, Ln, h);
    // (4) this wave's column tiles of w (channels) and u (values)
    f32x4_t uv[NC][NVW];
    {
      f32x4_t W[NC], U[NC];
      if (owner) {
        wy_subst2<C, true>(sXw, wid, sV, ctu, LDT, sBeta, sAkk, LDA, sTd, S::LDTD, W, U);
      } else {
        wy_subst2<C, false>(sXw, wid, sV, 0, LDT, sBeta, sAkk, LDA, sTd, S::LDTD, W, U);
      }
      store_wT<C>(sWT, S::LDW, wid, W);
#pragma unroll
      for (int i = 0; i < NC; ++i) uv[i][0] = U[i];
      if constexpr (WT == 2) {  // the wave's second w tile
        wy_subst2<C, false>(sXw, wid + NW, sXw, 0, LDT, sBeta, sAkk, LDA, sTd, S::LDTD, W, W);
        store_wT<C>(sWT, S::LDW, wid + NW, W);
      }
    }
    __syncthreads();
    // (5) + (6) on the waves that own a value tile
    if (owner) {
      f32x4_t p1[NC][NVW], o[NC][NVW];
#pragma unroll
      for (int i = 0; i < NC; ++i)
#pragma unroll
        for (int v = 0; v < NVW; ++v) {
          p1[i][v] = zero4();
          o[i][v] = zero4();
        }
      q_times_state<C, D, NVW>(o, sQ, LDT, hs);
      w_times_state<C, D, NVW>(p1, sWT, S::LDW, hs);
#pragma unroll
      for (int i = 0; i < NC; ++i)
#pragma unroll
        for (int v = 0; v < NVW; ++v) uv[i][v] = uv[i][v] - p1[i][v];
      causal_times_h<C, NVW>(o, sAqh, S::LDAH, uv);
      vnew_frags<C, NVW>(vprev, uv);
      if (p.q_l2norm) {  // raw q: o is linear in each q row
        const int n16 = tid_opaque() & 15;
#pragma unroll
        for (int i = 0; i < NC; ++i)
#pragma unroll
          for (int v = 0; v < NVW; ++v) o[i][v] = o[i][v] * sQn[16 * i + n16];
      }
      // o from registers: four adjacent value columns per lane and row
      store_oT<C, NVW>(reinterpret_cast<Tin *>(p.o) + off, ld, col0, L, o, Vr);
      // this chunk's state update, before the barrier: it reads only k~ and 2^b_L,
      // which the next chunk's store leaves alone, so each wave runs it while the
      // slower waves finish their products
      state_update_kt<C, D, NVW>(hs, sKt, LDT, vprev, sDecay);
    }
    __syncthreads();
  }
  if (owner && p.ht && !(sr.len == 0 && p.ht == p.h0)) store_strip<float, DT, NVW>(p.ht + sbase, Vr, col0, Kr, hs, Vr);
}

// D = 256 runs 32-row chunks with eight waves (two w tiles each) and the value
// columns split over two workgroups, each holding half the state; 131 KB of LDS
bool fused_supported(const ChunkParams &p) {
  return p.is_bf16 && (p.D == 64 || p.D == 128 || (p.D == 256 && p.C == 32));
}

// Compute units of the current device (cached per device).
int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
    cus[dev] = v;
  }
  return cus[dev];
}

namespace {

template <int C, int D, int NT, int GK>
hipError_t launch_fused_g(const ChunkParams &p, hipStream_t st) {
  const size_t smem = FusedSmem<C, D, NT>::total;
  auto kern = fused_chunk_kernel<C, D, NT, GK>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)smem);
  if (e != hipSuccess) {
    (void)hipGetLastError();  // do not leave the error for the next launch to report
    return e;
  }
  hipLaunchKernelGGL(kern, dim3(p.N * p.H * p.vsplit), dim3(NT), smem, st, p);
  return hipGetLastError();
}


template <int C, int D>
hipError_t launch_fused_t(const ChunkParams &p0, hipStream_t st) {
  // one wave per 16-column tile of w (and of the state); at D = 256 eight waves
  // with two w tiles each, and at least two value blocks
  constexpr int NT = (KDA_FUSED_THREADS > 0 && D <= 128) ? KDA_FUSED_THREADS : (D == 256 ? 512 : 4 * D);
  constexpr int VS0 = (D / 16) / (NT / 64);
  if (p0.N * p0.H == 0) return hipSuccess;
  // with fewer (sequence, head) pairs than compute units, split the value
  // columns so that the workgroups still cover the chip
  ChunkParams p = p0;
  const int cus = device_cus();
  p.vsplit = VS0;
  while (2 * p.vsplit <= D / 16 && (int64_t)p.N * p.H * 2 * p.vsplit <= cus) p.vsplit *= 2;
  switch (p.gate_kind) {
    case kGateSafe: return launch_fused_g<C, D, NT, kGateSafe>(p, st);
    case kGateSoftplus: return launch_fused_g<C, D, NT, kGateSoftplus>(p, st);
    case kGateLogE: return launch_fused_g<C, D, NT, kGateLogE>(p, st);
    case kGateLog2Cumsum: return launch_fused_g<C, D, NT, kGateLog2Cumsum>(p, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_fused(const ChunkParams &p, hipStream_t st) {
  if (!p.is_bf16) return hipErrorInvalidValue;
  if (p.C == 64 && p.D == 128) return launch_fused_t<64, 128>(p, st);
  if (p.C == 64 && p.D == 64) return launch_fused_t<64, 64>(p, st);
  if (p.C == 32 && p.D == 128) return launch_fused_t<32, 128>(p, st);
  if (p.C == 32 && p.D == 64) return launch_fused_t<32, 64>(p, st);
  if (p.C == 32 && p.D == 256) return launch_fused_t<32, 256>(p, st);
  return hipErrorInvalidValue;
}

}  // namespace kda
