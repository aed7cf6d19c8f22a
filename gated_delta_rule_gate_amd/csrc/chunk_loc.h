// Where a chunk lives: the map from a global chunk index (chunks numbered slot
// by slot) to its slot, first token and rows, shared by the kernels that run
// one workgroup per (chunk, head).
#pragma once

#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

struct ChunkLoc {
  int n, c, gci, L;
  int64_t t0;
};

// Maps a global chunk index to (slot, chunk in slot, first token, rows).
__device__ __forceinline__ bool locate_chunk(const ChunkParams &p, int gc, ChunkLoc &lc) {
  if (!p.cu) {
    const int nt = (p.T + p.C - 1) / p.C;
    if (gc >= p.B * nt) return false;
    lc.n = gc / nt;
    lc.c = gc % nt;
    lc.t0 = (int64_t)lc.n * p.T + (int64_t)lc.c * p.C;
    lc.L = min(p.C, p.T - lc.c * p.C);
    lc.gci = gc;
    return true;
  }
  if (gc >= p.chunk_off[p.N]) return false;
  int lo = 0, hi = p.N;  // largest n with chunk_off[n] <= gc
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (p.chunk_off[mid] <= gc) lo = mid;
    else hi = mid;
  }
  lc.n = lo;
  lc.c = gc - p.chunk_off[lo];
  lc.t0 = (int64_t)p.cu[lo] + (int64_t)lc.c * p.C;
  lc.L = min((int64_t)p.C, (int64_t)p.cu[lo + 1] - lc.t0);
  lc.gci = gc;
  return true;
}

}  // namespace kda
