// Step (1) of the chunked KDA forward as a kernel of its own: the gate
// activation followed by the chunk-local inclusive cumsum in log2 units
// ("FLA KDA Skill", sections "Gate modes" and "Safe gate numerical note"),
//
//   out[t, h, i] = sum over s from the start of t's chunk to t of act(g[s, h, i]),
//
// where chunks of C rows start at every sequence start (dense: every T rows;
// packed: every cu_seqlens[n]). C = 1 yields the per-token log2 decay that
// the recurrent entry point takes.
//
// One workgroup of K threads owns 64 consecutive rows of one head; thread i
// owns channel i and scans the rows in order, so each row is one coalesced
// K-float read and write. A chunk that began before the workgroup's first
// row contributes its earlier rows as a carry-in (re-read, never written),
// which is why the output must not overlap the input.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

namespace {

constexpr int kRows = 64;  // rows per workgroup

// Last slot n with cu[n] <= r (r < cu[N]); empty slots are skipped over.
__device__ __forceinline__ int slot_of(const int32_t *cu, int N, int64_t r) {
  int lo = 0, hi = N;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu[mid] <= r) lo = mid;
    else hi = mid;
  }
  return lo;
}

// One thread per channel: KP >= K threads, the ones past K idle.
template <int KP>
__global__ __launch_bounds__(KP) void gate_cumsum_kernel(GateCumsumParams p) {
  const int h = blockIdx.y;
  const int i = threadIdx.x;
  const int K = p.K;
  if (i >= K) return;  // no barriers below
  // rows outside [cu_seqlens[0], cu_seqlens[N]) are neither read nor written
  const int64_t beg = p.cu ? (int64_t)p.cu[0] : 0;
  const int64_t end = p.cu ? (int64_t)p.cu[p.N] : (int64_t)p.B * p.T;
  const int64_t r0 = (int64_t)blockIdx.x * kRows;
  if (r0 >= end || r0 + kRows <= beg) return;
  const int n_rows = (int)min((int64_t)kRows, end - r0);
  const int64_t ld = (int64_t)p.H * K;
  const float *g = p.g + h * K + i;
  float *out = p.out + h * K + i;

  const float expA = (p.gate_kind == kGateSafe || p.gate_kind == kGateSoftplus) ? fast_exp2(p.A_log[h] * kLog2e) : 0.f;
  const float dt = p.dt_bias ? p.dt_bias[h * K + i] : 0.f;
  auto act = [&](float x) { return gate_log2(p.gate_kind, x, dt, expA, p.lower_bound); };

  // all rows of the block in flight at once
  float x[kRows];
#pragma unroll
  for (int r = 0; r < kRows; ++r) x[r] = (r < n_rows && r0 + r >= beg) ? g[(r0 + r) * ld] : 0.f;

  // the slot holding r0 (or the first slot, for rows before cu_seqlens[0]) and
  // the start of r0's chunk
  int n = 0;
  int64_t s_begin, s_end;
  if (p.cu) {
    n = slot_of(p.cu, p.N, r0);
    s_begin = p.cu[n];
    s_end = p.cu[n + 1];
  } else {
    n = (int)(r0 / p.T);
    s_begin = (int64_t)n * p.T;
    s_end = s_begin + p.T;
  }
  float acc = 0.f;
  if (r0 > s_begin) {
    const int64_t c_begin = s_begin + (r0 - s_begin) / p.C * p.C;
    for (int64_t r = c_begin; r < r0; ++r) acc += act(g[r * ld]);
  }

#pragma unroll
  for (int r = 0; r < kRows; ++r) {
    if (r < n_rows) {
      const int64_t t = r0 + r;
      while (t >= s_end) {  // next non-empty slot (uniform across the workgroup)
        ++n;
        if (p.cu) {
          s_begin = p.cu[n];
          s_end = p.cu[n + 1];
        } else {
          s_begin = s_end;
          s_end = s_begin + p.T;
        }
      }
      if (t < s_begin) continue;  // before cu_seqlens[0]: outside the contract
      if ((t - s_begin) % p.C == 0) acc = 0.f;
      acc += act(x[r]);
      out[t * ld] = acc;
    }
  }
}

}  // namespace

hipError_t launch_gate_cumsum(const GateCumsumParams &p, hipStream_t st) {
  const int64_t rows = (int64_t)p.B * p.T;
  const int64_t nblk = (rows + kRows - 1) / kRows;
  if (nblk == 0 || p.H == 0) return hipSuccess;
  if (nblk > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid((unsigned)nblk, p.H);
  if (p.K < 1 || p.K > 256) return hipErrorInvalidValue;
  if (p.K <= 64) hipLaunchKernelGGL(gate_cumsum_kernel<64>, grid, dim3(64), 0, st, p);
  else if (p.K <= 128) hipLaunchKernelGGL(gate_cumsum_kernel<128>, grid, dim3(128), 0, st, p);
  else hipLaunchKernelGGL(gate_cumsum_kernel<256>, grid, dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace kda
