/*
 * kda_stages.h -- per-step entry points of the staged chunk schedule.
 *
 * For testing and profiling each step of the chunked prefill on its own. The
 * staged schedule of kda_chunk_fwd (KDA_SCHED_STAGED) is exactly the sequence
 * INDEX, GATE, GRAMS, SOLVE, WY, SCAN, OUTPUT of kda_chunk_stage calls on one
 * workspace. Intermediates live in that workspace at the byte offsets that
 * kda_staged_workspace_offset reports, all fp32, token-major like the inputs:
 *
 *   CHUNK_OFF int32 [N + 1]   chunks before each slot (packed batches only)
 *   (D = the tile width: 64, 128 or 256, the smallest >= max(K, V); columns
 *   past K or V hold zeros)
 *   B         [B*T, H, D]     chunk-local gate cumsum, log2 units (step 1)
 *   AKK, AQK  [B*T, H, C]     intra-chunk grams; column = row within the chunk;
 *                             beta folded into A_kk rows, the query scale into
 *                             A_qk (step 2)
 *   T         [B*T, H, C]     (I + A_kk)^-1 (step 3)
 *   W, U      [B*T, H, D]     WY factors (step 4)
 *   VNEW      [B*T, H, D]     u - w h (step 5)
 *   HC        [n_chunks, H, K, V]  state at the start of each chunk, chunks
 *                             numbered slot by slot (step 5)
 *
 * The steps follow the same passages as kda_chunk_fwd in kda.h. Arguments,
 * layouts, ownership and errors are those of kda_chunk_fwd; `ws` must hold at
 * least kda_chunk_workspace_bytes() for args with schedule KDA_SCHED_STAGED.
 * Each step reads only what earlier steps (or the caller) left in the
 * workspace, so a test may write an intermediate and run one step alone.
 */
#ifndef KDA_STAGES_H_
#define KDA_STAGES_H_

#include "kda.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KDA_STAGE_INDEX = 0,  /* chunk prefix per slot (no-op for dense batches)          */
  KDA_STAGE_GATE = 1,   /* (1) gate activation + chunk-local cumsum, base 2         */
  KDA_STAGE_GRAMS = 2,  /* (2) A_kk, A_qk over causal 16x16 blocks                  */
  KDA_STAGE_SOLVE = 3,  /* (3) T = (I + A_kk)^-1, blocked forward substitution      */
  KDA_STAGE_WY = 4,     /* (4) w = T (beta k 2^b), u = T (beta v)                   */
  KDA_STAGE_SCAN = 5,   /* (5) inter-chunk state scan: v_new, chunk states, ht      */
  KDA_STAGE_OUTPUT = 6  /* (6) o = scale (q 2^b) h + A_qk v_new                      */
} kda_stage;

typedef enum {
  KDA_WS_CHUNK_OFF = 0,
  KDA_WS_B = 1,
  KDA_WS_AKK = 2,
  KDA_WS_AQK = 3,
  KDA_WS_T = 4,
  KDA_WS_W = 5,
  KDA_WS_U = 6,
  KDA_WS_VNEW = 7,
  KDA_WS_HC = 8
} kda_ws_field;

/* Byte offset of an intermediate inside the staged workspace ((size_t)-1 on
 * invalid arguments). Offsets are 256-byte aligned. */
size_t kda_staged_workspace_offset(const kda_args *args, kda_ws_field field);

/* Runs one step of the staged schedule on `stream`. */
kda_status kda_chunk_stage(const kda_args *args, kda_stage stage, const void *q, const void *k, const void *v,
                           const float *g, const float *beta, const float *h0, const int32_t *cu_seqlens, void *o,
                           float *ht, void *workspace, size_t ws_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* KDA_STAGES_H_ */
