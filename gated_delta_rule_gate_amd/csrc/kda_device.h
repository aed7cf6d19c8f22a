// Device-side helpers shared by the gfx950 kernels of the KDA library:
// storage-type loads/stores, the gate activations in log2 units, and the
// 16x16 MFMA tile conventions used by every contraction.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __bf16 bf16_t;
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));  // raw 16-byte chunk

constexpr float kLog2e = 1.4426950408889634f;  // 1 / ln 2 (the RCP_LN2 conversion)
constexpr float kLn2 = 0.6931471805599453f;

// Gate kinds (values match kda_gate_kind in include/kda.h).
enum GateKind : int { kGateLogE = 0, kGateSafe = 1, kGateSoftplus = 2, kGateLog2Cumsum = 3, kGateLog2 = 4 };

// ---------------------------------------------------------------------------------------------
// Storage types: bf16 (round-to-nearest-even on store) or fp32.
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) { return static_cast<float>(x); }

template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) { return static_cast<bf16_t>(x); }

// Two floats rounded to nearest-even bf16 in one dword (lo in bits 0..15):
// one v_cvt_pk_bf16_f32. Vectors that feed a matrix instruction are built
// from these dwords; assembled element by element, the compiler converts each
// element on its own and merges the halves with extra permutes.
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ unsigned pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}
__device__ __forceinline__ bf16x8_t pack_bf16x8(const float (&x)[8]) {
  return __builtin_bit_cast(bf16x8_t, u32x4_t{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]),
                                              pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7])});
}

// threadIdx.x behind an empty volatile asm: values derived from it cannot be
// hoisted out of loops, so per-thread LDS/global addresses are recomputed
// where they are used instead of being held in registers across a whole loop
// (which otherwise spills the chunk loop's live state).
__device__ __forceinline__ int tid_opaque() {
  int t = threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}

// Row K (lanes 16K .. 16K + 15) of x, in every row at the same position within
// the row: a v_permlane16_swap of x with itself leaves rows (0, 0, 2, 2) in its
// first result and (1, 1, 3, 3) in its second, and a v_permlane32_swap of one
// of those with itself leaves its first half-wave's row in the first result and
// its second's in the second. Two VALU permutes instead of an LDS permute.
template <int K>
__device__ __forceinline__ float row_bcast(float x) {
  static_assert(K >= 0 && K < 4, "four rows of 16 lanes");
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const unsigned h = (K & 1) ? r[1] : r[0];
  const auto t = __builtin_amdgcn_permlane32_swap(h, h, false, false);
  return __uint_as_float((K & 2) ? t[1] : t[0]);
}

// The wave's index within the workgroup as a wave-uniform (scalar) value.
// Branches on it are scalar branches; a branch on a per-lane value would
// instead run both sides under an EXEC mask, and MFMA instructions do not
// honour an empty EXEC mask.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(tid_opaque() >> 6); }

// Hardware base-2 exponential / logarithm / reciprocal (v_exp_f32, v_log_f32, v_rcp_f32).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// log(1 + x) for x >= 0 by Goldberg's correction ("What Every Computer Scientist Should
// Know About Floating-Point Arithmetic", 1991, Theorem 4): with u = fl(1 + x),
// log1p(x) = log(u) * x / (u - 1), exact to a few ulps even when x is tiny.
__device__ __forceinline__ float log1p_pos(float x) {
  float u = 1.0f + x;
  if (u == 1.0f) return x;
  return fast_log2(u) * kLn2 * (x / (u - 1.0f));
}

// Per-token decay in log2 units from the gate input of one channel.
//   kGateLog2:     g is already log2 (kGateLog2Cumsum: already the chunk-local
//                  cumsum in log2; callers skip their own cumsum)
//   kGateLogE:     g * log2(e)
//   kGateSafe:     lower_bound * sigmoid(expA * (x + dt)) * log2(e)
//   kGateSoftplus: -expA * softplus(x + dt) * log2(e)
// The activations follow "FLA KDA Skill", section "Gate modes".
__device__ __forceinline__ float gate_log2(int kind, float x, float dt, float expA, float lower_bound) {
  if (kind == kGateLog2 || kind == kGateLog2Cumsum) return x;
  if (kind == kGateLogE) return x * kLog2e;
  // the coefficients depend on per-head values only, so loops hoist them
  const float z = x + dt;
  if (kind == kGateSafe) {
    const float c1 = -expA * kLog2e, c2 = lower_bound * kLog2e;
    return c2 * fast_rcp(1.0f + fast_exp2(z * c1));
  }
  const float c3 = -expA * kLog2e;
  const float sp = fmaxf(z, 0.0f) + log1p_pos(fast_exp2(-fabsf(z) * kLog2e));
  return c3 * sp;
}

// beta from its logit: 1 / (1 + e^-x), hardware exp2 and reciprocal.
__device__ __forceinline__ float sigmoid_f32(float x) { return fast_rcp(1.0f + fast_exp2(-x * kLog2e)); }

// s_waitcnt vmcnt(0): every vector memory load this wave issued has returned.
// Used where registers filled by a prefetch issued in an earlier loop
// iteration are consumed, so the wait never depends on the compiler's
// tracking of loop-carried loads.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// An LDS address the compiler cannot see as a constant. The DS offset field
// holds 16 bits: with a buffer at a known offset beyond 64 KB, every access
// would pay its own address add; from an opaque base (one SGPR) the lane part
// is added once and the tile offsets stay immediates.
__device__ __forceinline__ char *lds_base(char *smem, unsigned off) {
  asm volatile("" : "+s"(off));
  return static_cast<char *>(__builtin_assume_aligned(smem + off, 16));  // every buffer offset is a multiple of 16
}

// Lets one wave read back, from other lanes, what it has just written to LDS:
// the LDS unit completes one wave's instructions in issue order, so it only
// keeps the compiler from moving LDS accesses across this point.
__device__ __forceinline__ void lds_wave_order() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_wave_barrier();
  asm volatile("" ::: "memory");
}

// ---------------------------------------------------------------------------------------------
// Slot / chunk location for packed (cu_seqlens) and dense batches.
// ---------------------------------------------------------------------------------------------
struct SlotRange {
  int64_t t0;  // first token (flattened B*T axis)
  int len;     // tokens in the slot
};

__device__ __forceinline__ SlotRange slot_range(const int32_t *cu, int n, int T) {
  SlotRange r;
  if (cu) {
    int a = cu[n], b = cu[n + 1];
    r.t0 = a;
    r.len = b - a;
  } else {
    r.t0 = (int64_t)n * T;
    r.len = T;
  }
  return r;
}

}  // namespace kda
