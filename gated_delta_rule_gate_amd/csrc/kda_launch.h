// Kernel parameter blocks and launcher declarations shared by the host API
// (kda_api.hip) and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

struct RecurrentParams {
  const void *q, *k, *v;
  const float *g, *beta, *h0;
  const int32_t *cu;
  void *o;
  float *ht;
  const float *A_log, *dt_bias;
  float lower_bound, scale;
  int gate_kind;
  int B, T, H, K, V, N;
  bool is_bf16;
};

hipError_t launch_recurrent(const RecurrentParams &p, hipStream_t st);

}  // namespace kda
