/*
 * kda.h -- C ABI of the MI355X (gfx950) Kimi Delta Attention forward library.
 *
 * KDA is a gated delta rule with a per-channel decay. Per (sequence, head) it
 * keeps an FP32 state S in R^{K x V} and, token by token,
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(exp g_t) S_{t-1} + beta_t k_t v_t^T
 *     o_t = S_t^T (q_t * scale),        scale = 1/sqrt(K) unless given.
 *
 * Conventions shared by every entry point
 *   - Every tensor pointer is a DEVICE pointer. Every call is asynchronous on
 *     `stream` (a hipStream_t; NULL is the default stream), never synchronises
 *     the host, never allocates, and never reads `cu_seqlens` on the host, so
 *     calls can be captured in a HIP graph and replayed with new offsets.
 *     This contract (device-resident int32 offsets, graph replay with mutated
 *     boundaries) follows "Add fused recurrent_kda for decode and inference
 *     prefill" (attention-gym PR #317), sections "Agent note" and "Test Plan".
 *   - The caller owns every buffer, including the workspace.
 *   - Layouts are contiguous, row-major:
 *       q, k [B, T, H, K]   v, o [B, T, H, V]   (dtype: bf16 or fp32)
 *       g    [B, T, H, K]   fp32 (meaning set by gate_kind)
 *       beta [B, T, H]      fp32, post-sigmoid
 *       h0, ht [N, H, K, V] fp32, one entry per logical sequence
 *       cu_seqlens [N + 1]  int32, device-resident
 *   - Packed (variable-length) batches pass B == 1, T == physical capacity and
 *     N + 1 offsets. A repeated offset is an empty slot: its final state is h0
 *     bit for bit (zeros when h0 is NULL). Rows at or beyond cu_seqlens[N] are
 *     outside the contract: they are neither read nor written. Dense batches
 *     pass cu_seqlens == NULL and N == B.
 *   - q and k arrive l2-normalised per row; the library does not normalise
 *     them ("Add fused recurrent_kda ...", PR #345 text: k keeps an explicit
 *     l2norm; inference callers normalise q before the op).
 *   - ht may alias h0 (in-place state update). ht == NULL skips the final state.
 *   - With T == 0 there are no tokens: the per-token tensors (q, k, v, g, beta,
 *     o; in the backward d_o and the per-token gradients) are never touched and
 *     may be NULL, and every final state is its h0 (the backward: dh0 = dht).
 *   - Errors: arguments that the host can check return a status code and
 *     launch nothing. Device-side contract violations (offsets that decrease,
 *     cu_seqlens[N] > T) are undefined behaviour. A failed launch returns
 *     KDA_ERR_HIP; kda_last_error() then names the HIP error.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KDA_OK = 0,
  KDA_ERR_NULL = 1,        /* a required pointer is NULL                          */
  KDA_ERR_SHAPE = 2,       /* B, T, H, N, K or V out of range or inconsistent      */
  KDA_ERR_DTYPE = 3,       /* unknown dtype                                        */
  KDA_ERR_CHUNK = 4,       /* chunk size not in {32, 64} (cumsum: {1, 32, 64})     */
  KDA_ERR_GATE = 5,        /* gate kind unknown, A_log missing, lower bound range  */
  KDA_ERR_ALIGN = 6,       /* a tensor pointer is not 16-byte aligned              */
  KDA_ERR_WORKSPACE = 7,   /* workspace NULL or smaller than the query says        */
  KDA_ERR_UNSUPPORTED = 8, /* valid but not implemented (e.g. K or V not a multiple of 8 in [8, 256]) */
  KDA_ERR_HIP = 9          /* a HIP launch failed                                  */
} kda_status;

typedef enum { KDA_BF16 = 0, KDA_F32 = 1 } kda_dtype;

/*
 * Gate input contracts ("FLA KDA Skill", section "Gate modes"; the log2 forms
 * follow "Add fused recurrent_kda ...", section "Agent note").
 */
typedef enum {
  KDA_GATE_LOGE = 0,     /* g is the per-token natural-log decay (pre-gated), g <= 0        */
  KDA_GATE_SAFE = 1,     /* g is raw x: lower_bound * sigmoid(exp(A_log) * (x + dt_bias)),
                            requires A_log and -5 <= lower_bound < 0                       */
  KDA_GATE_SOFTPLUS = 2, /* g is raw x: -exp(A_log) * softplus(x + dt_bias), requires A_log */
  KDA_GATE_LOG2_CUMSUM = 3, /* g is the chunk-local log2 cumsum that kda_gate_cumsum writes
                               with the same chunk size (kda_chunk_fwd only)               */
  KDA_GATE_LOG2 = 4      /* g is the per-token log2 decay (kda_recurrent_fwd, kda_gate_cumsum) */
} kda_gate_kind;

/* Execution schedule of kda_chunk_fwd. All schedules compute the same function. */
typedef enum {
  KDA_SCHED_AUTO = 0,   /* pick per shape                                                   */
  KDA_SCHED_STAGED = 1, /* six kernels, one per step, intermediates in the workspace        */
  KDA_SCHED_FUSED = 2,  /* one persistent kernel per (sequence, head); state kept on chip.
                           bf16, max(K, V) <= 128, or up to 256 with 32-row chunks; AUTO
                           runs it at width 256 with 32-row chunks also when 64 are asked
                           for (same o and ht up to rounding) unless the call returns the
                           chunk-start states                                              */
  KDA_SCHED_SPLIT = 3,  /* steps (1)-(4) for every chunk at once, their operands through the
                           workspace, then steps (5)-(6) and the state per (sequence, head),
                           the chain cut into segments that run side by side where that pays
                           (see kda_args.segment); for few (sequence, head) pairs with long
                           sequences                                                         */
  KDA_SCHED_PIPE = 4    /* the fused schedule's pipelined kernel (bf16, chunk 64, max(K, V) in
                           (64, 128], safe gate): per (sequence, head), four waves run steps
                           (1)-(4) of one chunk while four run steps (5)-(6) of the previous
                           one. AUTO runs it where it applies and the (sequence, head) pairs
                           fill the device; KDA_SCHED_FUSED always runs the fused kernel      */
} kda_schedule;

typedef struct {
  int B, T, H, K, V;       /* dense: tensors [B, T, H, *] (q, k: [B, T, Hk, K]); packed: B == 1,
                              T = capacity. 1 <= H <= 4096 (else KDA_ERR_SHAPE): the kernels
                              address one chunk's rows of a head with 32-bit byte offsets   */
  int N;                   /* sequences (slots); cu_seqlens has N + 1 entries (dense: N == B)   */
  int chunk_size;          /* chunk path: 32 or 64 (sub-chunk fixed at 16 rows)                 */
  kda_dtype dtype;         /* dtype of q, k, v and o                                            */
  float scale;             /* query scale; <= 0 selects 1/sqrt(K)                               */
  kda_gate_kind gate_kind; /* meaning of g                                                      */
  const float *A_log;      /* [H] device pointer (SAFE, SOFTPLUS)                               */
  const float *dt_bias;    /* [H, K] device pointer or NULL (SAFE, SOFTPLUS)                    */
  float lower_bound;       /* SAFE only                                                         */
  kda_schedule schedule;   /* kda_chunk_fwd only                                                */
  int Hk;                  /* heads of q and k; 0 means H. H must be a multiple of Hk: value head h
                              (of v, g, beta, o and the states) reads q/k head h / (H / Hk)
                              (grouped value heads, GVA)                                      */
  int q_l2norm;            /* 0: q arrives l2-normalised (the contract). 1: q arrives raw and each
                              output row is scaled by 1 / sqrt(sum over K of q^2 + 1e-6), which
                              equals running on l2-normalised q (see below). Other values:
                              KDA_ERR_SHAPE                                                   */
  int beta_logits;         /* 0: beta arrives post-sigmoid (the contract). 1: beta holds raw
                              logits and every kernel uses 1 / (1 + exp(-beta)) ("FLA KDA
                              Skill", section "Correctness checklist": raw beta logits and
                              post-sigmoid beta). Other values: KDA_ERR_SHAPE                 */
  int segment;             /* KDA_SCHED_SPLIT's state scan: chunks per segment. 0 chooses from
                              the sizes (kda_chunk_segment reports it), < 0 keeps one chain per
                              (sequence, head). Segments after a sequence's first run side by
                              side from the identity and from zero, and their affine maps are
                              chained afterwards (see below); o and ht agree with the serial
                              chain up to rounding. kda_chunk_fwd_states always runs the serial
                              chain. The workspace size depends on it                          */
} kda_args;

/*
 * Segments of the state scan (the context-parallel path that "FLA KDA Skill",
 * section "Correctness checklist", lists beside initial and final states and
 * long-sequence cumulative decay): one chunk maps the incoming state affinely,
 * h' = (Diag(2^b_L) - k~^T w) h + k~^T u, so a segment of chunks maps
 * h_out = M h_in + B and its outputs are o = o_local + E h_in. Each later
 * segment computes M, B, E and o_local from the identity and from zero, in
 * parallel with the others; an fp32 pass chains h_in(s + 1) = M_s h_in(s) + B_s
 * and a last pass adds E h_in to o_local. It trades about twice the state-side
 * work after the first segment for a chain of seg_len chunks instead of the
 * whole sequence.
 */

/*
 * q_l2norm ("Add fused recurrent_kda ...", the stacked description of the
 * fused q-l2norm option): every q-dependent term of the forward is linear in
 * q's row and lands in the same output row, so the normalisation of q can be
 * deferred to one 1/||q|| scale of that row of o. The eps floor is 1e-6, the
 * default of the l2norm it replaces. The grams then run in the raw-q basis,
 * about sqrt(K) larger, which the bounded safe gate tolerates. Forward only;
 * kda_chunk_fwd (every schedule) and kda_recurrent_fwd honour it.
 */

/* Human-readable name of a status code. */
const char *kda_status_string(kda_status s);

/* Text of the last KDA_ERR_HIP (thread-local); "" if none. */
const char *kda_last_error(void);

/*
 * Checks the device-side contract of packed offsets, which the other calls
 * cannot check without a host read ("Add fused recurrent_kda for decode and
 * inference prefill", section "Agent note": the varlen contract, offsets that
 * never decrease and end within the capacity). One
 * asynchronous launch on `stream` reads cu_seqlens [N + 1] (device) and writes
 * into flags[0] (device int32, caller-owned) the OR of
 *   KDA_OFFSETS_DECREASE   some cu_seqlens[n + 1] < cu_seqlens[n]
 *   KDA_OFFSETS_NEGATIVE   cu_seqlens[0] < 0
 *   KDA_OFFSETS_PAST_END   cu_seqlens[N] > T
 * or 0 when the offsets are valid for a call with capacity T. A debugging aid:
 * run it before kda_chunk_fwd or kda_recurrent_fwd and read the flag at the
 * next synchronisation. Errors: KDA_ERR_NULL (cu_seqlens or flags NULL),
 * KDA_ERR_SHAPE (N < 0 or T < 0), KDA_ERR_HIP (launch failure).
 */
#define KDA_OFFSETS_DECREASE 1
#define KDA_OFFSETS_NEGATIVE 2
#define KDA_OFFSETS_PAST_END 4
kda_status kda_check_offsets(const int32_t *cu_seqlens, int N, int T, int32_t *flags, void *stream);

/*
 * Bytes of device workspace that kda_chunk_fwd needs for these arguments
 * (0 when the arguments are invalid). Depends on B, T, H, K, V, N, chunk_size,
 * dtype and schedule only -- and, under KDA_SCHED_AUTO, on the compute units of
 * the current device, which the choice between the fused and split schedules
 * weighs (call it with the device current that kda_chunk_fwd will run on).
 */
size_t kda_chunk_workspace_bytes(const kda_args *args);

/*
 * The schedule kda_chunk_fwd runs for these arguments: KDA_SCHED_STAGED,
 * KDA_SCHED_FUSED, KDA_SCHED_SPLIT or KDA_SCHED_PIPE (what KDA_SCHED_AUTO
 * resolves to on the current device), or -1 when the arguments' sizes are
 * invalid or the named schedule does not take them (fused and split: bf16 with
 * K, V <= 128; pipe: as listed at KDA_SCHED_PIPE).
 */
int kda_chunk_schedule(const kda_args *args);

/*
 * Chunks per segment of the split schedule's state scan for these arguments
 * (args->segment if positive, else the choice of a cost model of the state side
 * from the sizes and the device's compute units; a packed batch keeps one chain
 * per slot unless args->segment asks otherwise), or 0 when kda_chunk_fwd runs
 * one serial chain per (sequence, head) or another schedule. Host-only.
 */
int kda_chunk_segment(const kda_args *args);

/*
 * Step (1) of the chunked forward on its own: the gate activation and the
 * chunk-local inclusive cumsum in base 2 ("FLA KDA Skill", sections "Gate
 * modes" and "Safe gate numerical note": RCP_LN2 conversion),
 *     g_out[t, h, i] = sum over s in [start of t's chunk, t] of act(g_in[s, h, i]),
 * with chunks of chunk_size rows restarting at every sequence start.
 * act() is the gate of args->gate_kind in log2 units: LOGE (times log2 e),
 * SAFE, SOFTPLUS (activation of the raw input) or LOG2 (as is).
 *   chunk_size 1      g_out is the per-token log2 decay kda_recurrent_fwd takes
 *                     (KDA_GATE_LOG2);
 *   chunk_size 32/64  g_out is the input of kda_chunk_fwd under
 *                     KDA_GATE_LOG2_CUMSUM with the same chunk size (the
 *                     pre-cumsummed gate contract of "Add fused recurrent_kda ...",
 *                     section "Agent note").
 * Arguments:
 *   args        B, T, H, K, N, gate_kind, A_log, dt_bias, lower_bound are used;
 *               V, dtype, scale, chunk_size and schedule are ignored
 *   g_in        fp32 [B, T, H, K] device pointer
 *   cu_seqlens  int32 [N + 1] or NULL (dense: sequences of T rows)
 *   g_out       fp32 [B, T, H, K] device pointer; must not overlap g_in
 *               (KDA_ERR_SHAPE). Rows at or beyond cu_seqlens[N] are not written.
 * Supported: K a multiple of 8 in [8, 256]; chunk_size in {1, 32, 64} (else KDA_ERR_CHUNK).
 */
kda_status kda_gate_cumsum(const kda_args *args, const float *g_in, const int32_t *cu_seqlens, int chunk_size,
                           float *g_out, void *stream);

/*
 * Chunked prefill (chunk_kda forward). Steps, per (sequence, head, chunk):
 *  (1) gate activation and chunk-local cumsum in base 2 ("FLA KDA Skill",
 *      section "Safe gate numerical note": RCP_LN2 conversion);
 *  (2) the intra-chunk grams A_kk and A_qk over causal 16-row blocks only
 *      ("[examples] Read only the causal columns in chunk_fwd_A_diag_anchored",
 *      description), midpoint offsets on diagonal blocks and paired
 *      non-positive offsets off-diagonal for the safe gate, per-pair
 *      exponents on diagonal blocks otherwise ("FLA KDA Skill", sections
 *      "Safe gate numerical note" and "Safe vs non-safe intra path");
 *  (3) T = (I + A_kk)^-1 by blocked forward substitution;
 *  (4) w = T (beta k 2^b), u = T (beta v);
 *  (5) the inter-chunk state scan; (6) o = scale (q 2^b) h + A_qk (u - w h).
 * Arguments:
 *   q, k, v, o   see the layout conventions; dtype args->dtype
 *   g            fp32 [B, T, H, K]; gate_kind LOGE, SAFE, SOFTPLUS or
 *                LOG2_CUMSUM (step (1) already done by kda_gate_cumsum)
 *   beta         fp32 [B, T, H] (logits when args->beta_logits)
 *   h0           fp32 [N, H, K, V] or NULL (zero initial state)
 *   cu_seqlens   int32 [N + 1] or NULL (dense)
 *   ht           fp32 [N, H, K, V] or NULL; may alias h0
 *   workspace    device buffer of ws_bytes >= kda_chunk_workspace_bytes(args),
 *                256-byte aligned; contents on entry are ignored
 * Supported: K and V multiples of 8 in [8, 256], equal or not ("FLA KDA Skill",
 * section "Correctness checklist": D != Dv); chunk_size in {32, 64}; dtype bf16
 * or fp32. The kernels run at the tile width 64, 128 or 256 that covers
 * max(K, V), with channels past K and value columns past V masked to zero, so
 * other widths cost what the next tile width costs. The fused and split
 * schedules run bf16 with max(K, V) <= 128 (KDA_ERR_UNSUPPORTED when named for
 * other cases); other cases run the staged one. KDA_SCHED_AUTO picks
 * (kda_chunk_schedule reports which).
 */
kda_status kda_chunk_fwd(const kda_args *args, const void *q, const void *k, const void *v, const float *g,
                         const float *beta, const float *h0, const int32_t *cu_seqlens, void *o, float *ht,
                         void *workspace, size_t ws_bytes, void *stream);

/*
 * kda_chunk_fwd for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc. Same
 * arguments and results as kda_chunk_fwd without the workspace: the
 * intermediates live in a library-owned static device array of
 * kda_chunk_noalloc_max_bytes() bytes (64 MiB), one copy per GPU the library
 * runs on, held until the process ends. The call allocates nothing (no
 * hipMalloc, hipFree or allocating library routine); the caller still passes
 * every input and output.
 *   - Schedules: the one kda_chunk_fwd would run, when its workspace fits the
 *     array; under KDA_SCHED_AUTO a split schedule whose records would not fit
 *     runs the fused schedule instead (the same function). Otherwise
 *     KDA_ERR_WORKSPACE, with the sizes in kda_last_error(), and nothing runs.
 *   - Every call on one GPU shares that GPU's array, which keeps the last call's
 *     contents (no kernel here needs it cleared). Calls that overlap on one GPU
 *     (concurrent streams or host threads) race on it: serialise them.
 *   - The first call on each device looks up that device's address of the
 *     array (KDA_ERR_HIP if the lookup fails).
 */
kda_status kda_chunk_fwd_noalloc(const kda_args *args, const void *q, const void *k, const void *v, const float *g,
                                 const float *beta, const float *h0, const int32_t *cu_seqlens, void *o,
                                 float *ht, void *stream);

/* Bytes of the static device array behind kda_chunk_fwd_noalloc. */
size_t kda_chunk_noalloc_max_bytes(void);

/*
 * Entries of [H, K, V] floats that h_states of kda_chunk_fwd_states must hold
 * (0 when the arguments are invalid or packed does not match B and N):
 *   dense  (packed == 0, N == B)  B * ceil(T / C), exactly the chunks;
 *   packed (packed != 0, B == 1)  ceil(T / C) + N, an upper bound of the sum
 *                                 over slots of ceil(len_n / C), since the
 *                                 offsets stay on the device.
 */
size_t kda_chunk_states_count(const kda_args *args, int packed);

/*
 * kda_chunk_fwd that also writes the state entering every chunk (the
 * return_intermediate_states option that "FLA KDA Skill", section
 * "Correctness checklist", lists as an axis of the forward):
 *   h_states[j] = the fp32 [H, K, V] state before the first token of chunk j,
 * chunks numbered slot by slot and in order within a slot: dense j = n *
 * ceil(T / C) + c; packed j = (sum over m < n of ceil(len_m / C)) + c. A
 * slot's first chunk holds h0 (zeros when h0 is NULL). Empty slots own no
 * chunk. Entries past the last chunk of a packed batch are not written.
 * Arguments: those of kda_chunk_fwd, plus
 *   h_states   fp32 device pointer, kda_chunk_states_count(args, cu_seqlens
 *              != NULL) * H * K * V floats, 16-byte aligned (KDA_ERR_ALIGN),
 *              not NULL unless that count is 0 (KDA_ERR_NULL); must not overlap
 *              any other buffer.
 * Every schedule honours it; the workspace is the one kda_chunk_fwd takes.
 * The extra traffic is K * V * 4 bytes per chunk and head, written once.
 */
kda_status kda_chunk_fwd_states(const kda_args *args, const void *q, const void *k, const void *v, const float *g,
                                const float *beta, const float *h0, const int32_t *cu_seqlens, void *o, float *ht,
                                float *h_states, void *workspace, size_t ws_bytes, void *stream);

/*
 * Bytes of device workspace that kda_chunk_bwd needs (0 when the arguments are
 * invalid or not supported by the backward).
 */
size_t kda_chunk_bwd_workspace_bytes(const kda_args *args);

/*
 * Backward of kda_chunk_fwd (the chunk_kda_bwd family that "FLA KDA Skill",
 * section "Public code map", names without printing it). Returns the gradients
 * of L = sum(d_o * o) + sum(dht * ht) for the forward of the same arguments.
 * The forward's steps (1)-(5) are recomputed inside (staged), then the chunks
 * are walked in reverse for the state gradient and each chunk's gradients are
 * formed on its own; every product is fp32.
 * Arguments (all device pointers; the caller owns every buffer):
 *   q, k, v, g, beta, h0, cu_seqlens   as kda_chunk_fwd
 *   d_o      [B, T, H, V], dtype args->dtype: gradient of o
 *   dht      fp32 [N, H, K, V] or NULL (zero): gradient of ht
 *   dq, dk   [B, T, H, K], dtype args->dtype     dv  [B, T, H, V], dtype args->dtype
 *   dg       fp32 [B, T, H, K]: gradient of g as passed (the raw gate input
 *            for SAFE and SOFTPLUS, the natural-log decay for LOGE)
 *   dbeta    fp32 [B, T, H] (of the logits when args->beta_logits)
 *   dh0      fp32 [N, H, K, V] or NULL; an empty slot gets dht (zeros without dht)
 *   dA_log   fp32 [H] or NULL, ddt_bias fp32 [H, K] or NULL: parameter
 *            gradients of the SAFE and SOFTPLUS gates (not written for LOGE)
 *   workspace  ws_bytes >= kda_chunk_bwd_workspace_bytes(args), 256-byte aligned
 * Rows at or beyond cu_seqlens[N] are not written. dq..dbeta are required
 * (KDA_ERR_NULL); they must not overlap the inputs.
 * Supported: K and V multiples of 8 with max(K, V) <= 128, chunk_size 32 or 64,
 * bf16 or fp32, gate kinds LOGE, SAFE and SOFTPLUS, Hk == H and q_l2norm == 0;
 * other valid arguments return KDA_ERR_UNSUPPORTED.
 */
kda_status kda_chunk_bwd(const kda_args *args, const void *q, const void *k, const void *v, const float *g,
                         const float *beta, const float *h0, const int32_t *cu_seqlens, const void *d_o,
                         const float *dht, void *dq, void *dk, void *dv, float *dg, float *dbeta, float *dh0,
                         float *dA_log, float *ddt_bias, void *workspace, size_t ws_bytes, void *stream);

/*
 * Fused token-sequential recurrence (recurrent_kda forward), for decode and
 * inference prefill ("Add fused recurrent_kda ...", section "Agent note"):
 * one kernel; each workgroup owns a (sequence, head, value-block) and scans its
 * tokens with the [K, BV] FP32 state held in registers, computing in FP32
 * whatever the input dtype.
 * Same arguments and layouts as kda_chunk_fwd, with no workspace; g is the
 * per-token decay of gate_kind LOG2 (log2 units, as the recurrent contract
 * has it), LOGE, SAFE or SOFTPLUS. args->chunk_size and args->schedule are ignored.
 * Supported: K and V multiples of 8 in [8, 256] (non-power-of-two widths run
 * in the next power-of-two tile with the rest masked, "Add fused recurrent_kda
 * ...", section "Test Plan").
 */
kda_status kda_recurrent_fwd(const kda_args *args, const void *q, const void *k, const void *v, const float *g,
                             const float *beta, const float *h0, const int32_t *cu_seqlens, void *o, float *ht,
                             void *stream);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
