// Kernel parameter blocks and launcher declarations shared by the host API
// (kda_api.hip) and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

constexpr float kQNormEps = 1e-6f;  // eps floor of the deferred q l2-normalisation

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
  int q_l2norm;  // scale each output row by 1/sqrt(|q|^2 + 1e-6)
  int Hk;        // q/k heads; value head h reads q/k head h / (H / Hk)
  int beta_logits;  // beta holds logits: the kernel applies the sigmoid
};

hipError_t launch_recurrent(const RecurrentParams &p, hipStream_t st);
// the blocked recurrence (bf16, K = V = 128, sequences longer than one token)
bool recurrent_block_supported(const RecurrentParams &p);
hipError_t launch_recurrent_block(const RecurrentParams &p, hipStream_t st);

// Step (1) on its own: gate activation and chunk-local cumsum in log2 units
// over [B*T, H, K] rows; C in {1, 32, 64}.
struct GateCumsumParams {
  const float *g;
  float *out;
  const int32_t *cu;
  const float *A_log, *dt_bias;
  float lower_bound;
  int gate_kind;
  int B, T, H, K, N, C;
};

hipError_t launch_gate_cumsum(const GateCumsumParams &p, hipStream_t st);

// Chunked prefill. The kernels run at a tile width D in {64, 128, 256} that
// covers both real widths Kr (q, k, g channels) and Vr (v, o columns); channels
// >= Kr and columns >= Vr are loaded as zeros, which leaves every product
// exact, and are never stored. Intermediates of the staged schedule are fp32,
// token-major like the inputs: b, w, u, vnew [B*T, H, D]; Akk, Aqk, Tm
// [B*T, H, C] (column = row within the chunk); hc [n_chunks, H, Kr, Vr], the
// state at the start of every chunk, chunks numbered slot by slot (the layout
// of h0 and ht).
struct ChunkParams {
  const void *q, *k, *v;
  const float *g, *beta, *h0;
  const int32_t *cu;
  void *o;
  float *ht;
  const float *A_log, *dt_bias;
  float lower_bound, scale;
  int gate_kind;
  int B, T, H, D, N, C;
  int Kr, Vr;          // real widths of q/k/g and of v/o (<= D, multiples of 8)
  bool is_bf16;
  int q_l2norm;        // scale each output row by 1/sqrt(|q|^2 + 1e-6)
  int Hk;              // q/k heads; value head h reads q/k head h / (H / Hk)
  int beta_logits;     // beta holds logits: the kernels apply the sigmoid
  int32_t *chunk_off;  // [N + 1] chunk prefix per slot (packed batches only)
  int max_chunks;      // upper bound of the number of chunks (grid size)
  int vsplit;          // fused schedule: value-column blocks per (sequence, head), set by its launcher
  float *b, *Akk, *Aqk, *Tm, *w, *u, *vnew, *hc;
  // split schedule: the key side's operands per (chunk, head), bf16 and fp32
  // records (sizes from split_workspace_bytes)
  void *sws;
  float *swf;
  // split schedule, chain-parallel state side: each sequence's chunks are cut
  // into segments of seg_len chunks (0: one segment, the serial chain). A
  // segment after the first runs from the identity (the columns of M) and from
  // zero (those of B), giving its affine map h_out = M h_in + B, per-chunk
  // output parts E (o = o_local + E h_in) and o_local; a combine pass chains
  // the maps for every segment's incoming state and a correction pass adds
  // E h_in to o_local.
  int seg_len;
  int seg_max;          // upper bound of the number of segments (grid size)
  int32_t *seg_off;     // [N + 1] segment prefix per slot (packed batches only)
  float *seg_mb;        // [seg_max, H, D, 2D] fp32: [M | B] of each segment
  void *seg_sin;        // [seg_max, H, D/16, D/32, 64] 16-byte bf16 operand fragments of each
                        // segment's incoming state (column tile, contraction step, lane)
  void *seg_e;          // [n_chunks, H, C, D] bf16: E, channels in operand order
  float *seg_ol;        // [n_chunks, H, C, D] fp32: o_local
};

// Backward of the chunked forward (staged). The forward intermediates come from
// the staged steps (1)-(5) in the same workspace (ChunkParams b, Akk, Aqk, Tm,
// w, vnew, hc); the backward's own fp32 intermediates follow them:
//   dvn, dqt, dkt, dw, dXw [B*T, H, D]   gradients of v_new, q~, k~, w, beta k 2^b
//   dAqk, dT, dAkk         [B*T, H, C]   gradients of A_qk, T (first its u part), A_kk
//   dbp                    [B*T, H]      the beta gradient through u
//   dhn                    [n_chunks, H, Kr, Vr]  gradient of the state after each chunk
//   dlam, ddt_part         [n_chunks, H, D]; dA_part [n_chunks, H]
struct BwdParams {
  const void *dout;  // [B*T, H, Vr] dtype of q
  const float *dht;  // [N, H, Kr, Vr] or null
  void *dq, *dk, *dv;
  float *dg, *dbeta, *dh0, *dA_log, *ddt;
  float *dvn, *dqt, *dkt, *dw, *dXw, *dAqk, *dT, *dAkk, *dbp, *dhn, *dlam, *ddt_part, *dA_part;
};

hipError_t launch_bwd(const ChunkParams &p, const BwdParams &b, hipStream_t st);

hipError_t launch_chunk_index(const ChunkParams &p, hipStream_t st);
// flag bits (kda.h) of the contract of cu_seqlens [N + 1] for capacity T, into flags[0]
hipError_t launch_check_offsets(const int32_t *cu, int N, int T, int32_t *flags, hipStream_t st);
hipError_t launch_stage_gate(const ChunkParams &p, hipStream_t st);
hipError_t launch_stage_grams(const ChunkParams &p, hipStream_t st);
hipError_t launch_stage_solve(const ChunkParams &p, hipStream_t st);
hipError_t launch_stage_wy(const ChunkParams &p, hipStream_t st);
hipError_t launch_stage_scan(const ChunkParams &p, hipStream_t st);
hipError_t launch_stage_output(const ChunkParams &p, hipStream_t st);
hipError_t launch_fused(const ChunkParams &p, hipStream_t st);
bool fused_supported(const ChunkParams &p);
// the pipelined fused kernel (bf16, C = 64, D = 128, safe gate; one workgroup per
// (sequence, head))
bool pipe_supported(const ChunkParams &p);
hipError_t launch_pipe(const ChunkParams &p, hipStream_t st);
// split schedule: the key side of every chunk in parallel, then the state side
// (bf16, D in {64, 128})
bool split_supported(const ChunkParams &p);
hipError_t launch_split(const ChunkParams &p, hipStream_t st);
// workspace of the split schedule for chunk_heads (chunk, head) pairs: the bf16
// records, then the fp32 ones
size_t split_workspace_bytes(int C, int D, int64_t chunk_heads);
// whether the split schedule is expected to beat the fused one for a longest
// chain of `chain` chunks, `pairs` (sequence, head) pairs and `items` (chunk,
// head) pairs at tile width D
bool split_preferred(int64_t chain, int64_t pairs, int64_t items, int D);
// chunks per segment of the split schedule's chain-parallel state side for a
// chain of `chain` chunks over `pairs` (sequence, head) pairs at tile width D,
// or 0 where the serial chain is expected to be faster
int split_segment_len(int64_t chain, int64_t pairs, int D, int C);
// upper bound of the number of segments of seg_len chunks: dense B * ceil(nt /
// seg_len) with nt = ceil(T / C); packed N + ceil((nt + N) / seg_len)
int64_t split_segment_bound(int B, int N, int64_t nt, bool packed, int seg_len);
// workspace of the chain-parallel state side beyond the records: E and o_local
// for chunk_heads (chunk, head) pairs, [M | B] and the incoming state for
// seg_heads (segment, head) pairs
size_t split_segment_bytes(int C, int D, int64_t chunk_heads, int64_t seg_heads);
// compute units of the current device (cached per device)
int device_cus();

}  // namespace kda
