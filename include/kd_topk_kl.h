/*
 * kd_topk_kl.h -- C ABI of the fused chunked top-K KL distillation loss on
 * AMD Instinct MI355X (gfx950).
 *
 * The operation.  A student's hidden states are projected through its output
 * head one sequence chunk at a time; a chunk's full-vocabulary logits are
 * reduced into the loss and then dropped, and the gradient pass forms them
 * again rather than keeping a sequence x vocabulary grid
 * (Glonce, "Multiverse Computing cuts LLM distillation VRAM by 15x with
 * chunked KL loss", paragraph on Multiverse's two-part fix).  The teacher is
 * represented by an offline cache of its K largest logits per position
 * (same paragraph: top-100; epoka.news, "Two systems changes that cut the
 * cost of knowledge distillation", section "The two proposed changes").
 *
 * The pages give no formula; the loss computed here is, with S = z / tau and
 * z = h W^T over the whole vocabulary V:
 *   p[t,k]  = softmax over the K cached ids of teacher_logit[t,:] / tau
 *   log q   = S[t,:] - logsumexp_v S[t,:]
 *   KL_t    = sum_k p[t,k] (log p[t,k] - log q[t, teacher_idx[t,k]])
 *   loss    = tau^2 * sum_t m_t KL_t / N,   N = #positions with mask != 0
 * and the outputs are its exact gradients: with
 *   G[t,v] = (tau/N) m_t (q[t,v] - P[t,v]),  P[t,v] = sum_k p[t,k][idx=v]
 * (duplicate ids add), grad_hidden = G W and grad_W = G^T H.  N = 0 gives
 * loss 0 and zero gradients.
 *
 * Conventions for every entry point below.
 *  - Pointers named as device pointers are device memory owned by the
 *    caller.  The library allocates no device memory, keeps no pointer after
 *    a call returns and holds no global state.  Calls on different streams
 *    need distinct workspaces (and distinct outputs).
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *    the call returns without synchronising.  `loss` is a device scalar.
 *  - Argument errors are returned synchronously before anything is enqueued.
 *  - Ids outside [0, V) are reported on the device: *status_dev is set to
 *    KD_ERR_BAD_INDEX (if status_dev is not NULL) and the entry contributes
 *    nothing to the loss or the gradients; p is still normalised over all K
 *    logits of the row.  NaN or Inf inputs propagate.
 *  - Results are deterministic: two calls on the same inputs give the same
 *    bits (fixed-order reductions, no floating-point atomics).
 */
#ifndef KD_TOPK_KL_H
#define KD_TOPK_KL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define KD_OK 0
#define KD_ERR_NULL_ARG 1    /* a required pointer is NULL                      */
#define KD_ERR_BAD_SHAPE 2   /* T, d, V or K < 1, K > V, K > KD_MAX_K, V*d,     */
                             /* chunk*V or T*d beyond what the kernels address, */
                             /* or (loss) V > 2096896                           */
#define KD_ERR_BAD_TAU 3     /* tau <= 0 or not finite                          */
#define KD_ERR_BAD_CHUNK 4   /* chunk < 1                                       */
#define KD_ERR_DTYPE 5       /* in_dtype is not KD_BF16 or KD_F32               */
#define KD_ERR_WORKSPACE 6   /* workspace NULL or smaller than required         */
#define KD_ERR_BAD_INDEX 7   /* (device) a teacher id is outside [0, V)         */
#define KD_ERR_HIP 8         /* a HIP launch failed                             */
#define KD_ERR_NOALLOC_SIZE 9 /* kd_topk_kl_fwd_bwd_noalloc: the sizes need more */
                             /* than KD_NOALLOC_SCRATCH_BYTES of workspace      */

/* Input element types of `hidden` and `W`. */
#define KD_BF16 0            /* bfloat16, row-major                             */
#define KD_F32 1             /* float32, row-major ("fp32 everywhere": the      */
                             /* gradient chunk is also kept in fp32)            */

/* Largest cache width K accepted (duplicate ids are merged per row in LDS). */
#define KD_MAX_K 4096

/*
 * Bytes of device workspace kd_topk_kl_fwd_bwd needs for these sizes; 0 if
 * the arguments are invalid.  A chunk larger than T is treated as T.  The
 * size grows as O(chunk*V + V*d) and does not depend on T beyond the chunk:
 * it holds one chunk's gradient row-major, the transposed gradient of the
 * chunks one head-gradient GEMM contracts (kd_topk_kl_dw_chunks), the
 * transposed head and per-chunk row statistics.
 */
size_t kd_topk_kl_workspace_bytes(int64_t T, int64_t d, int64_t V, int64_t K,
                                  int64_t chunk, int32_t in_dtype);

/*
 * Number of consecutive chunks whose gradient one launch of the
 * head-gradient GEMM (grad_W += G^T H) contracts, for these sizes; 0 if the
 * arguments are invalid.  Each launch reads and writes the whole fp32
 * grad_W once, so a launch takes as many consecutive chunks as fit in 8192
 * rows (the chunk counted rounded up to a multiple of 256), at least one and
 * never more than there are: max(1, min(nchunks, 8192 / chunk_256)).  The
 * workspace holds the transposed gradient of that many chunks.  The same
 * grouping applies to kd_topk_kl_bwd.  It changes neither the results'
 * meaning nor the summation's determinism (fp32 sums in a fixed order).
 */
int32_t kd_topk_kl_dw_chunks(int64_t T, int64_t d, int64_t V, int64_t K,
                             int64_t chunk, int32_t in_dtype);

/*
 * Forward and backward of the loss above in one call.
 *
 *  hidden        device [T, d] in_dtype, row-major: the student's final hidden
 *                states (one row per sequence position).
 *  W             device [V, d] in_dtype, row-major: the output head (lm_head).
 *  teacher_idx   device [T, K] int32, row-major: cached teacher token ids.
 *  teacher_logit device [T, K] float32, row-major: their cached logits (any
 *                per-row offset; only differences matter).
 *  mask          device [T] uint8, nonzero = the position counts; NULL = all
 *                positions count.
 *  tau           temperature > 0 (divides student and teacher logits; the
 *                loss is multiplied by tau^2).
 *  chunk         number of sequence rows whose V logits are live at once
 *                (>= 1; values above T mean T).  The last chunk may be ragged.
 *  loss          device float32 scalar (written).
 *  grad_hidden   device [T, d] float32 (overwritten).
 *  grad_W        device [V, d] float32 (overwritten, accumulated in fp32
 *                across chunks).
 *  row_lse       device [T] float32 or NULL: logsumexp_v S[t,:] per row.
 *  row_kl        device [T] float32 or NULL: KL_t per row (masked rows too).
 *  workspace     device buffer of at least kd_topk_kl_workspace_bytes(...)
 *                bytes, 256-byte aligned; its contents on entry do not matter.
 *  status_dev    device int32 or NULL: set to KD_OK at the start of the
 *                enqueued work, and to KD_ERR_BAD_INDEX if any id is invalid.
 *  stream        hipStream_t to enqueue on.
 *
 * Returns KD_OK or a host-side error code (nothing is enqueued on error,
 * except KD_ERR_HIP, after which the outputs are unspecified).
 */
int32_t kd_topk_kl_fwd_bwd(const void* hidden, const void* W, int32_t in_dtype,
                           const int32_t* teacher_idx,
                           const float* teacher_logit, const uint8_t* mask,
                           int64_t T, int64_t d, int64_t V, int64_t K,
                           float tau, int64_t chunk,
                           float* loss, float* grad_hidden, float* grad_W,
                           float* row_lse, float* row_kl,
                           void* workspace, size_t workspace_bytes,
                           int32_t* status_dev, void* stream);

/*
 * kd_topk_kl_fwd_bwd for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  It takes no workspace and allocates nothing (no hipMalloc,
 * hipFree or allocating library call): its workspace is a fixed device
 * array of KD_NOALLOC_SCRATCH_BYTES inside the library, which every GPU the
 * library runs on holds from the library's first use on that GPU until the
 * process ends.  The caller still passes inputs and outputs, as for
 * kd_topk_kl_fwd_bwd (same arguments and meaning, minus the workspace).
 *
 * The head gradient is contracted one chunk per launch (the smallest
 * workspace), so with several chunks grad_W's fp32 sums run in another
 * fixed order than kd_topk_kl_fwd_bwd's (results agree to rounding; with a
 * single chunk they are the same bits).  Sizes whose workspace would exceed
 * KD_NOALLOC_SCRATCH_BYTES return KD_ERR_NOALLOC_SIZE before anything is
 * enqueued; other errors as for kd_topk_kl_fwd_bwd, and KD_ERR_HIP if the
 * scratch's device address cannot be obtained.
 *
 * All calls on one GPU share that GPU's scratch, which keeps the last call's
 * contents (none of which a later call relies on): calls that can overlap
 * on one GPU -- concurrent streams, or threads -- race and must be
 * serialised by the caller.
 */
#define KD_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)
int32_t kd_topk_kl_fwd_bwd_noalloc(const void* hidden, const void* W, int32_t in_dtype,
                                   const int32_t* teacher_idx,
                                   const float* teacher_logit, const uint8_t* mask,
                                   int64_t T, int64_t d, int64_t V, int64_t K,
                                   float tau, int64_t chunk,
                                   float* loss, float* grad_hidden, float* grad_W,
                                   float* row_lse, float* row_kl,
                                   int32_t* status_dev, void* stream);

/* Number of timed phases per chunk (see kd_topk_kl_fwd_bwd_timed). */
#define KD_NUM_PHASES 8

/*
 * kd_topk_kl_fwd_bwd with timing markers, for measurement.  `events` points
 * to 2 * (KD_NUM_PHASES * nchunks + 2) hipEvent_t created by the caller,
 * nchunks = ceil(T / min(chunk, T)).  The call records events[2*i] before and
 * events[2*i + 1] after the launches of
 *   i = c * KD_NUM_PHASES + p   phase p of chunk c:
 *       0 zero-padded H_c and H_c^T and the teacher-id hit lists,
 *       1 forward GEMM with the logsumexp partials and the logits at the
 *       teacher ids, 2 logsumexp merge, KL rows and the chunk's loss sum,
 *       3 recompute GEMM with the gradient epilogue, 4 the teacher
 *       probabilities of the backward-only call (recorded ahead of phase 3;
 *       empty in the fused call), 5 hidden-gradient GEMM, 6 its split-K
 *       reduction,
 *       7 head-gradient GEMM (launched in the last chunk of each group of
 *       kd_topk_kl_dw_chunks(...) chunks; empty in the group's others);
 *   i = KD_NUM_PHASES * nchunks      the prologue (count N, W^T);
 *   i = KD_NUM_PHASES * nchunks + 1  the final loss.
 * Everything else is as for kd_topk_kl_fwd_bwd; KD_ERR_NULL_ARG if events is
 * NULL.
 */
int32_t kd_topk_kl_fwd_bwd_timed(const void* hidden, const void* W, int32_t in_dtype,
                                 const int32_t* teacher_idx,
                                 const float* teacher_logit, const uint8_t* mask,
                                 int64_t T, int64_t d, int64_t V, int64_t K,
                                 float tau, int64_t chunk,
                                 float* loss, float* grad_hidden, float* grad_W,
                                 float* row_lse, float* row_kl,
                                 void* workspace, size_t workspace_bytes,
                                 int32_t* status_dev, void* stream,
                                 void* const* events);

/*
 * Split entry points, for a training step whose forward and backward are
 * separate calls (the loss sits inside a model and the backward runs when
 * the framework back-propagates).  The method is the same: the forward
 * projects one chunk at a time, folds it into the loss and discards it, and
 * the backward rebuilds each chunk's logits when it needs them (the second
 * half of the fix described on the same Glonce page, paragraph on
 * Multiverse's two-part fix).  The only state carried from the forward to
 * the backward is the per-row logsumexp, O(T) floats.
 *
 * Workspace sizes for the two calls (0 if the arguments are invalid); each
 * is at most that of the fused call, and neither depends on T beyond the
 * chunk.
 */
size_t kd_topk_kl_fwd_workspace_bytes(int64_t T, int64_t d, int64_t V, int64_t K,
                                      int64_t chunk, int32_t in_dtype);
size_t kd_topk_kl_bwd_workspace_bytes(int64_t T, int64_t d, int64_t V, int64_t K,
                                      int64_t chunk, int32_t in_dtype);

/*
 * Forward only: `loss` (device fp32 scalar) and `row_lse` (device [T] fp32,
 * required: logsumexp_v S[t,:], to be passed to kd_topk_kl_bwd), `row_kl`
 * optional as in kd_topk_kl_fwd_bwd.  Inputs, workspace, status and stream
 * as for kd_topk_kl_fwd_bwd (workspace of kd_topk_kl_fwd_workspace_bytes).
 * The loss and row statistics are bitwise those of the fused call.
 */
int32_t kd_topk_kl_fwd(const void* hidden, const void* W, int32_t in_dtype,
                       const int32_t* teacher_idx, const float* teacher_logit,
                       const uint8_t* mask, int64_t T, int64_t d, int64_t V, int64_t K,
                       float tau, int64_t chunk,
                       float* loss, float* row_lse, float* row_kl,
                       void* workspace, size_t workspace_bytes,
                       int32_t* status_dev, void* stream);

/*
 * kd_topk_kl_fwd with timing markers, for measurement: `events` as for
 * kd_topk_kl_fwd_bwd_timed (phases 0-2 of every chunk carry the forward's
 * launches; phases 3-7 are recorded as empty intervals).  KD_ERR_NULL_ARG
 * if events is NULL.
 */
int32_t kd_topk_kl_fwd_timed(const void* hidden, const void* W, int32_t in_dtype,
                             const int32_t* teacher_idx, const float* teacher_logit,
                             const uint8_t* mask, int64_t T, int64_t d, int64_t V, int64_t K,
                             float tau, int64_t chunk,
                             float* loss, float* row_lse, float* row_kl,
                             void* workspace, size_t workspace_bytes,
                             int32_t* status_dev, void* stream, void* const* events);

/*
 * Backward only: the gradients of g * loss, with g = *grad_loss (device fp32
 * scalar; NULL means 1), recomputing every chunk's logits.
 *  row_lse            device [T] fp32 from kd_topk_kl_fwd on the same inputs.
 *  grad_hidden        device [T, d] of grad_hidden_dtype (KD_F32, or KD_BF16
 *                     rounded to nearest even), overwritten; NULL: not
 *                     computed (its GEMM is skipped).
 *  grad_W             device [V, d] fp32; overwritten, or, with
 *                     accumulate_grad_W != 0, added to (fp32 accumulation,
 *                     e.g. across micro-batches); NULL: not computed.
 *  grad_W_bf16        device [V, d] bf16 or NULL: a copy of the final grad_W
 *                     rounded to nearest even (requires grad_W).
 * At least one of grad_hidden and grad_W must be given (else
 * KD_ERR_NULL_ARG); KD_ERR_DTYPE for another grad_hidden_dtype.  Inputs,
 * workspace (kd_topk_kl_bwd_workspace_bytes), status and stream as for
 * kd_topk_kl_fwd_bwd; invalid ids are reported here too.
 */
int32_t kd_topk_kl_bwd(const void* hidden, const void* W, int32_t in_dtype,
                       const int32_t* teacher_idx, const float* teacher_logit,
                       const uint8_t* mask, int64_t T, int64_t d, int64_t V, int64_t K,
                       float tau, int64_t chunk,
                       const float* row_lse, const float* grad_loss,
                       void* grad_hidden, int32_t grad_hidden_dtype,
                       float* grad_W, int32_t accumulate_grad_W, uint16_t* grad_W_bf16,
                       void* workspace, size_t workspace_bytes,
                       int32_t* status_dev, void* stream);

/*
 * kd_topk_kl_bwd with timing markers, for measurement: `events` as for
 * kd_topk_kl_fwd_bwd_timed (phase 0 carries the chunk's H^T copy, phases
 * 3-7 the backward's launches; phases 1-2, and those of a gradient not
 * asked for, are recorded as empty intervals).  KD_ERR_NULL_ARG if events
 * is NULL.
 */
int32_t kd_topk_kl_bwd_timed(const void* hidden, const void* W, int32_t in_dtype,
                             const int32_t* teacher_idx, const float* teacher_logit,
                             const uint8_t* mask, int64_t T, int64_t d, int64_t V, int64_t K,
                             float tau, int64_t chunk,
                             const float* row_lse, const float* grad_loss,
                             void* grad_hidden, int32_t grad_hidden_dtype,
                             float* grad_W, int32_t accumulate_grad_W, uint16_t* grad_W_bf16,
                             void* workspace, size_t workspace_bytes,
                             int32_t* status_dev, void* stream, void* const* events);

/*
 * Offline top-K teacher-logit cache: the record the loss reads as
 * teacher_idx / teacher_logit.  The teacher runs once ahead of training and
 * its K largest output logits per position are stored with their token ids
 * (Glonce, "Multiverse Computing cuts LLM distillation VRAM by 15x with
 * chunked KL loss", paragraph on Multiverse's two-part fix: K = 100;
 * ainewsbank.com, "Multiverse Computing Tests Lower-Memory Long-Context
 * Distillation", section "Two changes remove different bottlenecks").
 *
 *  hidden     device [T, d] in_dtype: the teacher's final hidden states.
 *  W          device [V, d] in_dtype: the teacher's output head.
 *  out_idx    device [T, K] int32 (written): per row the ids of the K largest
 *             logits z[t, v] = h_t . W_v, in descending order of z; equal
 *             logits are ordered by the lower id.
 *  out_logit  device [T, K] float32 (written): those logits.
 *  chunk      rows processed at a time (the chunk's logits are computed once,
 *             kept in the workspace as fp32 and scanned once more for the
 *             candidates of each row).
 * Workspace: kd_topk_cache_workspace_bytes(...) bytes, 256-byte aligned;
 * O(chunk * V), independent of T beyond the chunk.  Host errors
 * as for kd_topk_kl_fwd_bwd.  Logits are fp32 sums of exact bf16 (or fp32)
 * products; rows where more than about 2K logits tie at or above the
 * selection threshold are recomputed by a slower exact path with plain dot
 * products.
 */
size_t kd_topk_cache_workspace_bytes(int64_t T, int64_t d, int64_t V, int64_t K,
                                     int64_t chunk, int32_t in_dtype);
int32_t kd_topk_cache_build(const void* hidden, const void* W, int32_t in_dtype,
                            int64_t T, int64_t d, int64_t V, int64_t K, int64_t chunk,
                            int32_t* out_idx, float* out_logit,
                            void* workspace, size_t workspace_bytes, void* stream);

/* Number of timed phases per chunk of the cache builder. */
#define KD_CACHE_PHASES 4

/*
 * kd_topk_cache_build with timing markers, for measurement.  `events` points
 * to 2 * (KD_CACHE_PHASES * nchunks + 1) hipEvent_t created by the caller
 * (nchunks = ceil(T / min(chunk, T))); events[2*i] is recorded before and
 * events[2*i + 1] after
 *   i = c * KD_CACHE_PHASES + p   phase p of chunk c: 0 the head GEMM
 *       (per-row block maxima and the stored logits, after the chunk's
 *       padded copy if any), 1 the threshold selection, 2 the scan of the
 *       stored logits for candidates, 3 the sort of the candidates and the
 *       exact fallback;
 *   i = KD_CACHE_PHASES * nchunks  the prologue (padded copy of W, if any).
 * Everything else is as for kd_topk_cache_build; KD_ERR_NULL_ARG if events
 * is NULL.
 */
int32_t kd_topk_cache_build_timed(const void* hidden, const void* W, int32_t in_dtype,
                                  int64_t T, int64_t d, int64_t V, int64_t K, int64_t chunk,
                                  int32_t* out_idx, float* out_logit,
                                  void* workspace, size_t workspace_bytes, void* stream,
                                  void* const* events);

/*
 * Measurement only (not part of the loss): the sustained bf16 MFMA ceiling.
 * Enqueues `blocks` blocks of 512 threads; every wave issues
 * 64 * iters v_mfma_f32_32x32x16_bf16 (32768 FLOPs each) back to back on
 * register operands, in the GEMMs' wave shape, with random bf16 operands
 * (or zeros when zero_operands != 0).  Timing it with events gives the
 * MFMA throughput at the clock the chip sustains under that load, the
 * ceiling the GEMMs are compared against beside the datasheet peak.
 *  out   device float32 [blocks * 512] (written: per-thread accumulator
 *        sums, 0 exactly with zero operands).
 * Returns KD_ERR_NULL_ARG, KD_ERR_BAD_SHAPE (blocks or iters < 1) or
 * KD_ERR_HIP on a launch failure, else KD_OK.
 */
int32_t kd_mfma_probe(int32_t blocks, int32_t iters, int32_t zero_operands, float* out, void* stream);

/* Static, NUL-terminated description of a status code. */
const char* kd_status_str(int32_t status);

#ifdef __cplusplus
}
#endif

#endif /* KD_TOPK_KL_H */
