/*
 * ra.h -- C ABI of one rank's ring step of softmax attention on gfx950.
 *
 * The operation (pages cited by title and section):
 *   "Ring Attention Paper Breakdown: Blockwise Distributed Transformers for
 *   Near-Infinite Context", section 2 (ring schedule): at ring step s rank i
 *   holds key/value block j = (i - s) mod P and folds it into the running
 *   softmax state of its resident query block Q_i; section 3 gives the update
 *   of that state (row max m, normaliser l, unnormalised output O) and the
 *   single division O / l after the last step.
 *   "Ring Attention Math Deep", section "The online-softmax identity that makes
 *   streaming legal": the same recurrence per query row.
 *   "Ring Attention：把超长序列沿设备环流动", section "Causal Attention
 *   让环不再完全对称": under a causal mask a block strictly in the future is
 *   skipped, the diagonal block is masked element by element, earlier blocks
 *   are used whole.
 *
 * Conventions common to every call
 *   - Every pointer to tensor data is a device pointer (hipMalloc'd or torch
 *     CUDA memory) owned by the caller.  The library never allocates, frees or
 *     retains memory and never writes q, k or v.
 *   - Tensors are dense row-major: q and o are [batch, heads, rows,
 *     head_dim], k and v [batch, heads, kv_rows, head_dim]; m, l and lse are
 *     [batch, heads, rows].  Every non-empty tensor pointer must be 16-byte
 *     aligned, except the per-row vectors (the state's m and l, and lse),
 *     which need 4 bytes (so that a batch or row slice of a state or of an
 *     output is itself valid).
 *   - Every call is asynchronous and ordered on `stream` (0 = the null
 *     stream); no call synchronises.  Buffers must stay valid and unmodified
 *     until the stream has passed the call.
 *   - All checks run on the host before anything is enqueued.  On a negative
 *     return nothing was enqueued and the state is untouched; ra_last_error()
 *     then names the check that failed.  RA_ERR_HIP means a HIP launch or copy
 *     failed to enqueue.  No exception or abort crosses this boundary.
 *   - Calls that share a state or an output must not overlap on different
 *     streams unless the caller orders them with events.
 *   - Within one call, every buffer the call writes (state m, l, o; outputs;
 *     gradients) must be disjoint from every other buffer the call names, and
 *     a state's m, l and o from each other.  Overlapping byte ranges are
 *     rejected with RA_ERR_INVALID_ARG before anything is enqueued.
 */
#ifndef RA_H_
#define RA_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  RA_OK = 0,
  RA_ERR_INVALID_ARG = -1,  /* bad shape, index, pointer, alignment or scale   */
  RA_ERR_UNSUPPORTED = -2,  /* valid but not implemented (head_dim, kv_rows,
                               bf16 blocks of 2^31 bytes or more per
                               (batch, head)) */
  RA_ERR_HIP = -3           /* HIP refused to enqueue a kernel or copy         */
} ra_status;

typedef enum { RA_F32 = 0, RA_BF16 = 1 } ra_dtype;

/* Result of the causal case test (ra_step_case). */
typedef enum { RA_CASE_SKIP = 0, RA_CASE_DIAG = 1, RA_CASE_FULL = 2 } ra_case;

/* Flags of ra_step_ex. */
typedef enum {
  RA_STEP_FRESH = 1,    /* the state is not read: the step starts from the empty
                           state, as right after ra_state_init */
  RA_STEP_FINALIZE = 2, /* the step writes ra_finalize's outputs instead of the
                           state, which keeps its previous contents */
  RA_STEP_Q_BROADCAST = 4 /* q holds one batch entry, [1, heads, rows, head_dim],
                             read by every batch entry of the state and of k, v */
} ra_step_flags;

/*
 * Running online-softmax state of one rank's query block ("Ring Attention
 * Paper Breakdown ...", section 3: m, l in R^c and O in R^{c x d} per head,
 * kept on the rank for the whole ring).  All buffers are caller-owned fp32
 * device memory.
 *   m  [batch, heads, rows]           running maximum of the scaled scores
 *                                     (natural-log units); empty = -inf
 *   l  [batch, heads, rows]           running sum of exp(score - m); empty = 0
 *   o  [batch, heads, rows, head_dim] unnormalised output; empty = 0
 * batch, heads, rows >= 0 (0 = empty, every call is then a no-op returning
 * RA_OK); head_dim is 64 or 128.
 */
typedef struct {
  int32_t batch, heads, rows, head_dim;
  float *m;
  float *l;
  float *o;
} ra_state;

/*
 * Set the state to the empty state (m = -inf, l = 0, O = 0), the identity of
 * the merge ("Ring Attention Math Deep", section "Accumulation math, step by
 * step"; aicassindra architecture article, section "End-to-end flow").
 * Implemented with a fill kernel, never hipMemset, so it can be captured.
 */
ra_status ra_state_init(ra_state *st, hipStream_t stream);

/*
 * Host-only causal case test for query block i = q_block against key/value
 * block j = kv_block of num_blocks contiguous blocks ("Ring Attention：...",
 * section "Causal Attention 让环不再完全对称"):
 *   causal == 0            -> RA_CASE_FULL
 *   causal, j > i          -> RA_CASE_SKIP   (block strictly in the future)
 *   causal, j == i         -> RA_CASE_DIAG   (key t visible to query r iff t <= r)
 *   causal, j < i          -> RA_CASE_FULL
 * Returns the case (>= 0) or RA_ERR_INVALID_ARG unless 0 <= i, j < num_blocks
 * and causal is 0 or 1.  Enqueues nothing; needs no GPU.
 */
int32_t ra_step_case(int32_t q_block, int32_t kv_block, int32_t num_blocks, int32_t causal);

/*
 * Fold one visiting key/value block into the state ("Ring Attention Paper
 * Breakdown ...", section 3, steps 1-7; the FlashAttention_Update of its
 * section 2):
 *   S = scale * Q_i K_j^T  (masked per ra_step_case), m' = max(m, rowmax S),
 *   l' = exp(m - m') l + rowsum exp(S - m'),  O' = exp(m - m') O + exp(S - m') V_j.
 * On return of the kernel the state is again in the canonical form above
 * (m is the running maximum).
 *   q          [batch, heads, rows, head_dim] in in_dtype (RA_BF16 or RA_F32),
 *              the rank's block i.
 *   k, v       [batch, heads, kv_rows, head_dim] in in_dtype, block j.
 *   kv_rows    rows of k and v, >= 0.  Under the causal mask it must equal
 *              st->rows (the pages' equal blocks), else RA_ERR_UNSUPPORTED.
 *              Without it any length is accepted: a short query block against
 *              a key/value shard, as in decoding.  kv_rows == 0 folds nothing
 *              (k and v may then be NULL).
 *   q_block, kv_block, num_blocks, causal   as in ra_step_case; global
 *              positions are q_block*rows + r and kv_block*rows + t.
 *   scale      score multiplier, finite and > 0 (1/sqrt(head_dim) normally).
 * bf16 inputs use the MFMA path (fp32 accumulation, P rounded to bf16 before
 * the P V product) and must stay below 2^31 bytes per (batch, head) block of
 * q, k or v (else RA_ERR_UNSUPPORTED; the fp32 O state of such a block then
 * stays below 2^32 bytes); f32 inputs use an fp32 path.  A skipped block returns
 * RA_OK and enqueues nothing, leaving the state bit-identical.
 */
ra_status ra_step(ra_state *st, const void *q, const void *k, const void *v, ra_dtype in_dtype,
                  int32_t kv_rows, int32_t q_block, int32_t kv_block, int32_t num_blocks,
                  int32_t causal, float scale, hipStream_t stream);

/*
 * ra_step with the first and the last fold of a ring fused with ra_state_init
 * and ra_finalize (the normalisation of the pages' last step, RAMD section
 * "Accumulation math, step by step": out = O / l; the saved LSE of the
 * backward section of "Ring Attention：把超长序列沿设备环流动"), so a ring needs
 * no separate init and finalize launches.  Arguments as in ra_step, plus:
 *   flags      any combination of RA_STEP_FRESH, RA_STEP_FINALIZE and
 *              RA_STEP_Q_BROADCAST (else RA_ERR_INVALID_ARG).  RA_STEP_FRESH:
 *              m, l and o are not read;
 *              the result is that of ra_state_init followed by ra_step.
 *              RA_STEP_FINALIZE: instead of storing the new state the step
 *              writes o_out and lse_out exactly as ra_finalize would from it
 *              (bit-identical); m, l and o keep their previous contents.
 *              RA_STEP_Q_BROADCAST: q is [1, heads, rows, head_dim] and batch
 *              entry b of the state folds it against batch entry b of k, v
 *              (decoding one query block against a cache laid out as chunks
 *              along the batch axis, without copying the query block per
 *              chunk); the result is that of a q repeated along the batch.
 *   o_out, out_dtype, lse_out   as in ra_finalize (used with
 *              RA_STEP_FINALIZE only; either may be NULL; o_out 16-byte,
 *              lse_out 4-byte aligned).
 * A step that folds nothing (a skipped causal block, kv_rows == 0) still
 * applies its flags, by enqueueing ra_state_init and ra_finalize.
 */
ra_status ra_step_ex(ra_state *st, const void *q, const void *k, const void *v, ra_dtype in_dtype,
                     int32_t kv_rows, int32_t q_block, int32_t kv_block, int32_t num_blocks,
                     int32_t causal, float scale, uint32_t flags, void *o_out, ra_dtype out_dtype,
                     float *lse_out, hipStream_t stream);

/*
 * ra_step_ex for a caller that times every step while the ring runs (the
 * per-kernel durations of a profiler's kernel trace, taken live).  Arguments
 * as in ra_step_ex, plus two HIP events, created by the caller with timing
 * enabled on the device of `stream` (either may be NULL; the caller keeps
 * ownership and may reuse them once the stream has passed this call):
 *   start, stop   when the call folds a block, they take the begin and end
 *                 timestamps of the step kernel's own dispatch packet
 *                 (hipExtLaunchKernel), so timing adds no marker between two
 *                 steps on the stream; when it folds nothing (a skipped
 *                 block, kv_rows == 0, an empty state), start is recorded on
 *                 the stream before whatever the flags enqueue and stop after.
 * Results are those of ra_step_ex.  On an error return nothing is enqueued
 * and neither event is recorded.
 */
ra_status ra_step_timed(ra_state *st, const void *q, const void *k, const void *v,
                        ra_dtype in_dtype, int32_t kv_rows, int32_t q_block, int32_t kv_block,
                        int32_t num_blocks, int32_t causal, float scale, uint32_t flags,
                        void *o_out, ra_dtype out_dtype, float *lse_out, hipEvent_t start,
                        hipEvent_t stop, hipStream_t stream);

/*
 * dst <- dst (+) src: merge two partial states over disjoint key sets
 * (aicassindra architecture article, section "The architecture: every piece
 * explained": take the larger maximum, rescale each side by exp(its max - new
 * max), add).  Shapes must match.  A row empty on one side takes the other
 * side's values bit-exactly.  dst and src must not overlap.
 */
ra_status ra_lse_merge(ra_state *dst, const ra_state *src, hipStream_t stream);

/*
 * Final division and log-sum-exp ("Ring Attention Math Deep", section
 * "Accumulation math, step by step": out = o / l; "Ring Attention：...",
 * section "Backward 需要让梯度也沿环传播": the per-row log-sum-exp kept for the
 * backward).
 *   o_out   [batch, heads, rows, head_dim] in out_dtype (RA_F32 or RA_BF16,
 *           round to nearest even); may be NULL to skip.
 *   lse_out [batch, heads, rows] fp32, = m + ln l; may be NULL to skip.
 * A row with l == 0 gives o_out = 0 and lse_out = -inf.  The state is not
 * modified, so more blocks may be folded in afterwards.
 */
ra_status ra_finalize(const ra_state *st, void *o_out, ra_dtype out_dtype, float *lse_out,
                      hipStream_t stream);

/*
 * Reduce partial states and finalize in one pass: the global online-softmax
 * reduction of decoding against a sharded key/value cache ("Ring Attention：
 * 把超长序列沿设备环流动", section "训练与推理的适用方式不同": each shard
 * holder folds the broadcast query block into a partial state, then the
 * partial states are combined), followed by ra_finalize.  The state holds
 * batch = out_batch * parts partial states: state batch b * parts + p is part
 * p of output batch b, each over a disjoint key set.  Per row, with
 * m = max_p m_p and w_p = exp(m_p - m) (w_p = 0 for a part whose m_p is -inf,
 * i.e. that saw no key), l = sum_p w_p l_p and
 *   o_out   [out_batch, heads, rows, head_dim] in out_dtype (RA_F32 or
 *           RA_BF16, round to nearest even) = (sum_p w_p o_p) / l; may be
 *           NULL to skip.
 *   lse_out [out_batch, heads, rows] fp32 = m + ln l; may be NULL to skip.
 * The same result as merging the parts pairwise with ra_lse_merge (any
 * order) and finalizing, up to rounding.  A row no part saw gives o_out = 0
 * and lse_out = -inf.  parts must divide batch (RA_ERR_INVALID_ARG
 * otherwise); o_out 16-byte, lse_out 4-byte aligned.  The state is not
 * modified.
 */
ra_status ra_merge_finalize(const ra_state *st, int32_t parts, void *o_out, ra_dtype out_dtype,
                            float *lse_out, hipStream_t stream);

/*
 * Stage a block: asynchronous device-to-device copy of `bytes` bytes from src
 * to dst on `stream`.  On one GPU this stands in for the receive of the next
 * key/value block from the previous rank into the free buffer ("Ring Attention
 * Paper Breakdown ...", section 2: receive into buffer B while buffer A is
 * computed on, then swap).  Runs as a kernel of this library built to run
 * beside a step: non-temporal loads and stores, a small grid that leaves the
 * compute units to the step, and few registers per wavefront, so that its
 * wavefronts fit on compute units that also run step workgroups; a copy alone
 * is slower than a full-chip copy but overlaps well.  bytes == 0 is a no-op;
 * otherwise both pointers must be non-NULL and 16-byte aligned, bytes a
 * multiple of 16, and the ranges must not overlap.
 */
ra_status ra_stage_block(void *dst, const void *src, size_t bytes, hipStream_t stream);

/*
 * ra_stage_block with flags.  RA_STAGE_ALONE: no step runs beside this copy
 * (in a ring, the step it overlaps is a skipped causal block, "Ring
 * Attention：把超长序列沿设备环流动", section "Causal Attention
 * 让环不再完全对称": such a rank only forwards the block), so the copy takes a
 * full-chip grid instead of the small one built to run beside a step; it
 * still runs correctly beside a step, only slows it.  flags == 0 is
 * ra_stage_block.  Other flag bits: RA_ERR_INVALID_ARG.  Same argument rules
 * as ra_stage_block.
 */
typedef enum {
  RA_STAGE_ALONE = 1 /* no step runs beside the copy: full-chip grid */
} ra_stage_flags;
ra_status ra_stage_block_ex(void *dst, const void *src, size_t bytes, uint32_t flags, hipStream_t stream);

/*
 * One device-to-device copy carried by ra_step_staged.
 */
typedef struct {
  void *dst;        /* written; 16-byte aligned */
  const void *src;  /* read; 16-byte aligned */
  size_t bytes;     /* a multiple of 16, below 2^31; 0: nothing */
} ra_copy;

#define RA_MAX_STEP_COPIES 2

/*
 * ra_step_timed that also carries out the staging of the next block (the
 * receive of the next key/value block into the free buffer while the current
 * one is folded, "Ring Attention Paper Breakdown ...", section 2) inside the
 * step's own launch: the step kernel's workgroups copy slices of the
 * n_copies copies between their key tiles, one 16-byte chunk per thread per
 * tile, each workgroup a share proportional to its key tiles.  A ring then
 * needs one stream and no events: the next step is ordered after this one's
 * copies by the stream, and this step's copies after the previous step's
 * reads of the buffer they refill.  Arguments as in ra_step_timed, plus:
 *   copies     n_copies ra_copy entries (0 <= n_copies <= RA_MAX_STEP_COPIES,
 *              copies may be NULL when n_copies == 0).  Every dst range must be
 *              disjoint from every other dst and src range, from q, k, v, the
 *              state and the outputs; a src range must be disjoint from what
 *              the step writes (the state, or o_out and lse_out).
 * The copies complete when the call completes on the stream.  They run inside
 * the step kernel for bf16 inputs; for fp32 inputs, and when the call folds
 * nothing (a skipped block, kv_rows == 0, an empty state), as full-chip copy
 * kernels (ra_stage_block_ex with RA_STAGE_ALONE) enqueued after whatever the
 * step enqueues, outside start and stop.  The fold's results are those of
 * ra_step_timed.  On an error return nothing is enqueued.
 */
ra_status ra_step_staged(ra_state *st, const void *q, const void *k, const void *v,
                         ra_dtype in_dtype, int32_t kv_rows, int32_t q_block, int32_t kv_block,
                         int32_t num_blocks, int32_t causal, float scale, uint32_t flags,
                         void *o_out, ra_dtype out_dtype, float *lse_out, const ra_copy *copies,
                         int32_t n_copies, hipEvent_t start, hipEvent_t stop, hipStream_t stream);

/*
 * ra_step_staged on tensors whose (batch, head) entries are not packed: the
 * entry e = b * heads + h of q, of the state's m, l and o and of o_out and
 * lse_out starts at row e * row_stride (element e * row_stride * head_dim of
 * q, o and o_out, element e * row_stride of m, l and lse_out), that of k and v
 * at row e * kv_row_stride; within an entry rows stay packed.  One launch can
 * so fold a row range of a longer block (query rows [r0, r0 + rows) of every
 * head: pointers advanced by r0 rows, row_stride the longer block's rows)
 * against a row range of another.  The zigzag partition of "Ring
 * Attention：...", section "Causal Attention 让环不再完全对称", uses it: a
 * rank keeps its two sub-blocks in position order, one block per head, and
 * every visit of another rank's two sub-blocks is one such launch (the later
 * sub-block against both, or both against the earlier one), the visit of its
 * own one causal diagonal launch.
 *   row_stride     >= st->rows (st->rows: packed), else RA_ERR_INVALID_ARG
 *   kv_row_stride  >= kv_rows (kv_rows: packed), else RA_ERR_INVALID_ARG
 * The overlap checks compare each buffer's whole extent, from the first row of
 * entry 0 to the end of the last entry.  RA_STEP_FRESH and RA_STEP_FINALIZE
 * on a call that folds nothing (skipped block, kv_rows == 0) with row_stride
 * != st->rows return RA_ERR_UNSUPPORTED (the state kernels take packed
 * states).  Everything else, and the error behaviour, as ra_step_staged.
 */
ra_status ra_step_strided(ra_state *st, int32_t row_stride, const void *q, const void *k,
                          const void *v, ra_dtype in_dtype, int32_t kv_rows, int32_t kv_row_stride,
                          int32_t q_block, int32_t kv_block, int32_t num_blocks, int32_t causal,
                          float scale, uint32_t flags, void *o_out, ra_dtype out_dtype,
                          float *lse_out, const ra_copy *copies, int32_t n_copies, hipEvent_t start,
                          hipEvent_t stop, hipStream_t stream);

/*
 * Backward, per-row term ("Ring Attention：...", section "Backward 需要让梯度也
 * 沿环传播": gradients of every block interaction, probabilities recomputed
 * from the saved log-sum-exp):  delta[row] = sum_x dout[row][x] * o[row][x],
 * the D of dS = P (dP - D), computed once per rank before its backward ring.
 *   o       [batch, heads, rows, head_dim] the forward output (ra_finalize's
 *           o_out, normalised) in o_dtype (RA_F32 or RA_BF16)
 *   dout    [batch, heads, rows, head_dim] gradient of the loss with respect
 *           to that output, in do_dtype
 *   delta   [batch, heads, rows] fp32, written
 *   dq      [batch, heads, rows, head_dim] fp32, set to zero (the rank's dQ
 *           accumulator before its backward ring); may be NULL to skip;
 *           16-byte aligned
 * head_dim 64 or 128 (else RA_ERR_UNSUPPORTED); checks and errors as for
 * ra_step.
 */
ra_status ra_bwd_prepare(int32_t batch, int32_t heads, int32_t rows, int32_t head_dim,
                         const void *o, ra_dtype o_dtype, const void *dout, ra_dtype do_dtype,
                         float *delta, float *dq, hipStream_t stream);

/*
 * Backward of one ring step: the contribution of visiting block j to the
 * gradients of query block i (same section; the query owner accumulates dq,
 * the dk and dv of block j accumulate while it travels the ring and return to
 * its owner):
 *   P = exp(scale * q k^T - lse)   (masked per ra_step_case; a row with
 *                                   lse = -inf contributes nothing)
 *   dP = dout v^T,  dS = P * (dP - delta)
 *   dq += scale * dS k,   dk += scale * dS^T q,   dv += P^T dout
 *   q, dout   [batch, heads, rows, head_dim] in in_dtype, block i
 *   lse       [batch, heads, rows] fp32, natural log (ra_finalize's lse_out)
 *   delta     [batch, heads, rows] fp32 (ra_bwd_prepare)
 *   k, v      [batch, heads, rows, head_dim] in in_dtype, block j (equal blocks)
 *   dq        [batch, heads, rows, head_dim] fp32, accumulated (block i)
 *   dk, dv    [batch, heads, rows, head_dim] fp32, accumulated (block j)
 *   q_block, kv_block, num_blocks, causal, scale   as in ra_step.
 * The caller zeroes the accumulators before a ring.  A skipped block returns
 * RA_OK and enqueues nothing.  bf16 inputs use the MFMA path: two kernels (query-stationary for dq, key-stationary for dk and dv),
 * fp32 accumulation, P and dS rounded to bf16 before their products; each
 * output row is updated by one workgroup, so results are run-to-run
 * identical.  fp32 inputs use an fp32-arithmetic kernel that adds dk and dv
 * with fp32 atomics (low bits may differ between runs).  bf16 blocks are
 * limited as in ra_step.
 */
ra_status ra_bwd_step(int32_t batch, int32_t heads, int32_t rows, int32_t head_dim, const void *q,
                      const void *dout, const float *lse, const float *delta, const void *k,
                      const void *v, ra_dtype in_dtype, float *dq, float *dk, float *dv,
                      int32_t q_block, int32_t kv_block, int32_t num_blocks, int32_t causal,
                      float scale, hipStream_t stream);

/*
 * ra_bwd_step with timing events as in ra_step_timed: start takes the begin
 * of the step's first kernel, stop the end of its last (bf16: the dq kernel,
 * then the dk/dv kernel; fp32: one kernel); a skipped block records both on
 * the stream back to back.  Results are those of ra_bwd_step.
 */
ra_status ra_bwd_step_timed(int32_t batch, int32_t heads, int32_t rows, int32_t head_dim,
                            const void *q, const void *dout, const float *lse, const float *delta,
                            const void *k, const void *v, ra_dtype in_dtype, float *dq, float *dk,
                            float *dv, int32_t q_block, int32_t kv_block, int32_t num_blocks,
                            int32_t causal, float scale, hipEvent_t start, hipEvent_t stop,
                            hipStream_t stream);

/* Static string naming a status code. */
const char *ra_status_string(ra_status s);

/* Thread-local detail of the last non-OK return on the calling thread ("" if
 * none).  Valid until the next library call on this thread. */
const char *ra_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* RA_H_ */
