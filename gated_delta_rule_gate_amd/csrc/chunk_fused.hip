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
#include "chunk_fused_tiles.h"
#include "chunk_loc.h"
#include "kda_launch.h"

// Threads per workgroup of the fused kernel (0: 512 when the state has at
// least 8 column tiles, else 256). A build-time knob for tuning.
#ifndef KDA_FUSED_THREADS
#define KDA_FUSED_THREADS 0
#endif

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
  static constexpr size_t total = qn + 4 * C;
};

// One chunk's raw inputs held in registers between the HBM load and the LDS store.
// q, k and v are loaded and stored by NL threads (loader index in [0, NL)):
// all of them, or one wave of each pair 2m, 2m + 1 (the pair's first half of
// the grams), which issues those loads while the other inverts a diagonal
// block. The gate input and beta use every thread.
template <typename Tin, int C, int D, int NT, int NL>
struct ChunkRegs {
  static constexpr int EPV = 16 / (int)sizeof(Tin);
  static constexpr int VPR = D / EPV, NVT = C * VPR, IT = (NVT + NL - 1) / NL;  // q, k, v tiles
  static constexpr int XPR = D / 4, NVX = C * XPR, IX = (NVX + NT - 1) / NT;    // gate tile (fp32)
  // the q/k/v loader index of this thread (valid on loader waves)
  static __device__ __forceinline__ unsigned loader_index() {
    const unsigned t = (unsigned)tid_opaque();
    return (NL == NT) ? t : (((t >> 7) << 6) | (t & 63));
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

template <int C, int D, int NT, int GK>
__global__ __launch_bounds__(NT) void fused_chunk_kernel(ChunkParams p) {
  using Tin = bf16_t;
  using TL = Tile<Tin, C, D>;
  using S = FusedSmem<C, D, NT>;
  constexpr bool SAFE = (GK == kGateSafe);
  constexpr int NW = NT / 64, NC = TL::NC, DT = TL::DT, LDT = TL::LDT, LDB = TL::LDB, LDA = TL::LDA;
  constexpr int NVW = 1;  // value tiles (and w column tiles) per wave
  static_assert(DT == NW, "one w column tile and at most one value tile per wave");

  extern __shared__ __align__(16) char smem[];
  // buffers below 64 KB at constant offsets; the others from three opaque bases
  char *baseB = lds_base(smem, S::b), *baseA = lds_base(smem, S::akk), *baseT = lds_base(smem, S::t1);
  static_assert(S::b % 16 == 0 && S::wt_off % 16 == 0 && S::akk % 16 == 0 && S::kt % 16 == 0 && S::aqk % 16 == 0 &&
                    S::aqh % 16 == 0 && S::td % 16 == 0 && S::t1 % 16 == 0 && S::t2 % 16 == 0 && S::t0 % 16 == 0 && S::beta % 16 == 0 &&
                    S::bl % 16 == 0 && S::decay % 16 == 0 && S::dt % 16 == 0 && S::seg % 16 == 0 && S::qn % 16 == 0,
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
  constexpr bool HALF_LOAD = (NW / NC >= 2);
  constexpr int NL = HALF_LOAD ? NT / 2 : NT;
  const bool loader = !HALF_LOAD || gram_half<NW, NC>(wid) == 0;
  ChunkRegs<Tin, C, D, NT, NL> regs;
  if (nch > 0) {
    regs.load_gate(p, sr.t0, min(C, sr.len), h);
    if (loader) regs.load_qkv(p, sr.t0, min(C, sr.len), h);
  }
  // v_new of the previous chunk: its state update h <- Diag(2^b_L) h + k~^T v_new
  // runs right after the next chunk's inputs are stored, beside their gate
  // activation; before the first chunk it is the identity (v_new = 0, k~ = 0,
  // decay 1)
  bf16x8_t vprev[NC / 2][NVW];
#pragma unroll
  for (int s2 = 0; s2 < NC / 2; ++s2)
#pragma unroll
    for (int v = 0; v < NVW; ++v) vprev[s2][v] = bf16x8_t{};
  for (int i = tid_opaque(); i < D; i += NT) sDecay2[D + i] = 1.f;
  for (int i = tid_opaque(); i < C * LDT / 8; i += NT) reinterpret_cast<u32x4_t *>(sKt)[i] = u32x4_t{0u, 0u, 0u, 0u};
  __syncthreads();  // sDt, the identity update's operands visible

  for (int c = 0; c < nch; ++c) {
    const int64_t t0 = sr.t0 + (int64_t)c * C;
    const int L = min(C, sr.len - c * C);
    const int64_t off = t0 * ld + h * Vr;
    float *sDecay = sDecay2 + (c & 1) * D;
    // chunk c - 1's state update first: it needs no new input, so the loads of
    // this chunk's inputs land meanwhile
    state_update_kt<C, D, NVW>(hs, sKt, LDT, vprev, sDecay2 + ((c + 1) & 1) * D);
    regs.template store<GK>(loader, sQ, sK, sV, sB, sBeta, sDt, L, expA, p.lower_bound, p.q_l2norm != 0, sQn,
                            p.beta_logits != 0);
    if (hcs && owner) store_strip<float, DT, NVW>(hcs + (int64_t)c * p.H * Kr * Vr, Vr, col0, Kr, hs, Vr);
    __syncthreads();
    // the next chunk's inputs are loaded in two parts while this chunk computes:
    // the gate by every wave as it finishes the grams' first phase (the waves get
    // there at different times, so their loads do not queue at once), then q, k, v
    const bool more = c + 1 < nch;
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
    if constexpr (HALF_LOAD)
      grams_fused<NT, C, D, SAFE>(sQ, sK, LDT, sB, LDB, sBeta, p.scale, sAkk, sAqk, LDA, sAqh, S::LDAH, L, sT0, sT1,
                                  sT2, sBL, sKt, sXw, sTd, S::LDTD, load_next, gate_next);
    else
      grams_fused<NT, C, D, SAFE>(sQ, sK, LDT, sB, LDB, sBeta, p.scale, sAkk, sAqk, LDA, sAqh, S::LDAH, L, sT0, sT1,
                                  sT2, sBL, sKt, sXw, sTd, S::LDTD, none, gate_next);
    __syncthreads();
    if (!HALF_LOAD && more) regs.load_qkv(p, t0 + C, Ln, h);
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
    }
    __syncthreads();
  }
  if (nch > 0) state_update_kt<C, D, NVW>(hs, sKt, LDT, vprev, sDecay2 + ((nch - 1) & 1) * D);
  if (owner && p.ht && !(sr.len == 0 && p.ht == p.h0)) store_strip<float, DT, NVW>(p.ht + sbase, Vr, col0, Kr, hs, Vr);
}

bool fused_supported(const ChunkParams &p) { return p.is_bf16 && (p.D == 64 || p.D == 128); }

// ---------------------------------------------------------------------------------------------
// Split schedule. With fewer (sequence, head) pairs than compute units, the
// fused kernel's workgroups each walk a long chain of chunks at the full
// per-chunk latency. Here the key side -- steps (1)-(4), which depend on no
// state -- runs for every chunk at once, one workgroup per (chunk, head), and
// leaves its operands in the workspace; the state side then walks the chunks
// with only steps (5)-(6) and the state update in its chain.
// ---------------------------------------------------------------------------------------------

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

  const int wid = wave_id();
  const bool owner = wid * 16 < p.Vr;
  constexpr bool HALF_LOAD = (NW / NC >= 2);
  constexpr int NL = HALF_LOAD ? NT / 2 : NT;
  const bool loader = !HALF_LOAD || gram_half<NW, NC>(wid) == 0;
  ChunkRegs<Tin, C, D, NT, NL> regs;
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
    if constexpr (HALF_LOAD)
      grams_fused<NT, C, D, SAFE>(sQ, sK, LDT, sB, LDB, sBeta, p.scale, sAkk, sAqk, LDA, sAqh, S::LDAH, L, sT0, sT1,
                                  sT2, sBL, sKt, sXw, sTd, S::LDTD, load_next, gate_next);
    else
      grams_fused<NT, C, D, SAFE>(sQ, sK, LDT, sB, LDB, sBeta, p.scale, sAkk, sAqk, LDA, sAqh, S::LDAH, L, sT0, sT1,
                                  sT2, sBL, sKt, sXw, sTd, S::LDTD, none, gate_next);
    __syncthreads();
    if (!HALF_LOAD && more) regs.load_qkv(p, ln.t0, ln.L, hn);
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

// (5), (6) and the state update of one (sequence, head, block of value tiles),
// walking the sequence's chunks with the key side's operands from the
// workspace. Workgroups of one (sequence, head) sit on one XCD (workgroups are
// dealt to the XCDs round-robin), so they share its L2.
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
  const int G = p.N * p.H * vs;
  const int bid = blockIdx.x;
  const int li = (G % 8 == 0) ? (bid % 8) * (G / 8) + bid / 8 : bid;
  const int nh = li / vs, vb = li % vs;
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

// Whether the split schedule is expected to beat the fused one, from a cost
// model of the two measured on MI355X (C = 64, D = 128, safe gate): the fused
// kernel walks each (sequence, head)'s chunks at ~8.7 us a chunk, one pair per
// compute unit; the split key side costs ~11 us per (chunk, head) item per
// compute unit, and its state side ~3.3 us a chunk with one workgroup per
// D / 64 value tiles a unit. The chain is the longest sequence in chunks (for
// packed calls, bounded by the capacity T); items are the (chunk, head) pairs.
bool split_preferred(int64_t chain, int64_t pairs, int64_t items, int D) {
  const int64_t cus = device_cus();
  const double fused = 8.7 * chain * ((pairs + cus - 1) / cus);
  const int64_t wgs = pairs * (D / 64);
  const double split = 11.0 * ((items + cus - 1) / cus) + 3.3 * chain * ((wgs + cus - 1) / cus);
  return split < 0.9 * fused;
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
  constexpr int NT = (KDA_FUSED_THREADS > 0) ? KDA_FUSED_THREADS : ((D / 16 >= 8) ? 512 : 256);
  if (p0.N * p0.H == 0) return hipSuccess;
  // with fewer (sequence, head) pairs than compute units, split the value
  // columns so that the workgroups still cover the chip
  ChunkParams p = p0;
  const int cus = device_cus();
  p.vsplit = 1;
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

hipError_t launch_fused(const ChunkParams &p, hipStream_t st) {
  if (!p.is_bf16) return hipErrorInvalidValue;
  if (p.C == 64 && p.D == 128) return launch_fused_t<64, 128>(p, st);
  if (p.C == 64 && p.D == 64) return launch_fused_t<64, 64>(p, st);
  if (p.C == 32 && p.D == 128) return launch_fused_t<32, 128>(p, st);
  if (p.C == 32 && p.D == 64) return launch_fused_t<32, 64>(p, st);
  return hipErrorInvalidValue;
}

}  // namespace kda
