/*
 * fwpkm.h -- C ABI of the FwPKM chunked read-then-write step on MI355X (gfx950).
 *
 * Fast-weight Product Key Memory keeps, per memory unit (one sequence x one
 * head), fast weights theta = (K1, K2, V): two sub-key tables of n rows and a
 * value table of N = n*n rows.  One call processes one chunk of tokens:
 *
 *   read   each query is split into two halves scored against K1 and K2,
 *          the per-half best k sub-keys are combined into k*k candidate slots
 *          (slot = a*n + b), the best k slots are kept, and the retrieved
 *          vector is the softmax-weighted sum of their value rows.
 *          [gist.science "Fast-weight Product Key Memory", section 2,
 *          Core Architecture (two codebooks, top-k slots with O(sqrt N)
 *          scoring) and Key Technical Choices (IDW score
 *          -log(eps + ||q - K||^2)); agifrontier tutorial "Fast-weight
 *          Product Key Memory", Product Key addressing]
 *   write  one local gradient step theta' = theta - lr * grad L on the
 *          summed MSE loss L = sum_t 1/2 ||retrieved_t - target_t||^2, held
 *          at the chunk's starting weights, applied to every touched V, K1
 *          and K2 row; a row touched by several tokens gets the mean of their
 *          gradients; no clipping.
 *          [agifrontier tutorial, update equation; sciencestack.ai
 *          "Fast-weight Product Key Memory", contents: MSE loss, reducing MSE
 *          losses to a scalar by summation, weighting gradient by row
 *          contribution, no gradient clipping; gist.science section 2,
 *          gradient aggregation by averaging]
 *   chain  predictions inside the chunk use only the weights from before the
 *          chunk; the next call reads the updated weights.
 *          [gist.science section 2, Causality Preservation; PyPI
 *          "fast-weight-product-key-memory 0.2.2", Usage: chained
 *          past_memories -> next_memories]
 *
 * All tensors are fp32, row-major and contiguous, in device memory owned by
 * the caller.  All work is enqueued on the caller's stream; no call
 * synchronises the host with the device except where stated.
 *
 * Errors: every entry point returns FWPKM_OK (0) or a negative code, never
 * throws, and leaves a message for fwpkm_last_error() in thread-local storage.
 * Argument validation runs before anything is enqueued: on a validation error
 * no device memory is written.  Device faults are asynchronous and surface at
 * a later HIP call or stream synchronisation.
 */
#ifndef FWPKM_H
#define FWPKM_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
#define FWPKM_OK               0
#define FWPKM_ERR_INVALID_ARG (-1) /* null pointer, bad size, k out of range, non-finite lr */
#define FWPKM_ERR_ALIAS       (-2) /* partial overlap of past/next state, or an output aliasing an input */
#define FWPKM_ERR_OOM         (-3) /* device workspace allocation failed */
#define FWPKM_ERR_HIP         (-4) /* HIP runtime error; fwpkm_last_error() holds its text */
#define FWPKM_ERR_UNSUPPORTED (-5) /* valid shape outside the kernels' limits (listed below) */
#define FWPKM_ERR_DEVICE_CHECK (-6) /* checked builds only: a kernel found one of its invariants
                                       broken (fwpkm_last_error() names which); the call's
                                       outputs and state are then not meaningful */

/* Scoring modes.
 * IDW: score = -log(eps + ||q - K||^2) over the full key [K1[a]; K2[b]]
 *      [gist.science section 2, Key Technical Choices].
 * DOT: score = q . K, the standard product-key memory score that the same
 *      passage contrasts IDW with. */
#define FWPKM_SCORE_IDW 0
#define FWPKM_SCORE_DOT 1

/* Kernel limits (FWPKM_ERR_UNSUPPORTED beyond them). */
#define FWPKM_MAX_TOPK      32      /* k */
#define FWPKM_MAX_SQRT_SLOTS 4096   /* n, so N <= 2^24 */
#define FWPKM_MAX_HALF      1024    /* d_qk / 2 */
#define FWPKM_MAX_DIM_V     2048    /* d_v */
#define FWPKM_MAX_CHUNK     1024    /* chunk_size */

/* Opaque handle: owns the device workspace of one configuration, nothing else. */
typedef struct fwpkm_handle fwpkm_handle;

/* Configuration, mirroring the constructor arguments on the PyPI page's Usage
 * section (num_memories = sqrt_slots^2, dim_queries_keys, dim_values, topk,
 * learning_rate per call, chunk_size) plus the multi-head count. */
typedef struct {
    int32_t sqrt_slots;  /* n >= 1; N = n*n slots; n <= FWPKM_MAX_SQRT_SLOTS           */
    int32_t dim_qk;      /* d_qk, even; each half d_h = d_qk/2, d_h % 4 == 0            */
    int32_t dim_v;       /* d_v, d_v % 4 == 0                                          */
    int32_t topk;        /* 1 <= k <= min(n*n, FWPKM_MAX_TOPK), and k <= n              */
    int32_t chunk_size;  /* C, the most tokens one call may carry                      */
    int32_t num_heads;   /* H >= 1, an independent memory per head                     */
    int32_t max_batch;   /* most sequences one call may carry; sizes the workspace     */
    float   eps;         /* IDW epsilon, finite and > 0 (the pages give no value)      */
    int32_t score_mode;  /* FWPKM_SCORE_IDW or FWPKM_SCORE_DOT                          */
    float   addr_weight; /* lambda of the marginal-entropy addressing loss; finite; 0 = off.
                          * [gist.science "Fast-weight Product Key Memory", section 2:
                          * a negative-entropy loss on the key matrices keeps slot usage
                          * balanced across a chunk.]  Per half h, p_h = chunk mean of the
                          * per-token softmax of the scores over all n sub-keys; the loss
                          * lambda * sum_i p_h[i] log p_h[i] adds its gradient to every
                          * K1 / K2 row in the chunk's SGD step (at the chunk's starting
                          * weights).  Non-zero costs three extra kernels per chunk and a
                          * [units, 2, tokens, n] score buffer in the workspace.           */
} fwpkm_config;

/* Fast-weight state in caller-owned device memory (fp32, contiguous):
 *   k1, k2 : per sequence [H, n, d_h]
 *   v      : per sequence [H, N, d_v]
 * Sequence b's tables start at k1 + b*batch_stride_k (likewise k2) and
 * v + b*batch_stride_v.  A stride of 0 means one set of tables shared by the
 * whole batch (allowed for a past state only). */
typedef struct {
    float*  k1;
    float*  k2;
    float*  v;
    int64_t batch_stride_k;  /* elements; 0 or >= H*n*d_h */
    int64_t batch_stride_v;  /* elements; 0 or >= H*N*d_v */
} fwpkm_state;

/* Validate *cfg and create a handle.  The device workspace is allocated on
 * the current device at the first fwpkm_forward_chunk call, so creation
 * itself makes no HIP call.  Returns FWPKM_ERR_INVALID_ARG or
 * FWPKM_ERR_UNSUPPORTED for a bad configuration, FWPKM_ERR_OOM if the handle
 * cannot be allocated.  *out is set only on success. */
int fwpkm_create(const fwpkm_config* cfg, fwpkm_handle** out);

/* Device workspace bytes a handle of this configuration allocates
 * (0 for an invalid configuration). */
size_t fwpkm_workspace_bytes(const fwpkm_config* cfg);

/* One chunk: read with past_state, write the updated state into next_state.
 *
 *   queries   [batch, tokens, H, d_qk]   read
 *   targets   [batch, tokens, H, d_v]    read; already paired with the
 *                                        queries (a lookahead shift, if any,
 *                                        is the caller's)
 *   batch     1..max_batch;  tokens 1..chunk_size
 *   lr        learning rate eta, finite; 0 skips the write entirely and
 *             next_state then equals past_state bit for bit
 *   past_state  weights before the chunk (read)
 *   next_state  weights after the chunk (written).  Either the very same
 *             pointers and strides as past_state (in-place update, the fast
 *             path), or tables disjoint from past_state: then past_state is
 *             first copied into next_state on the stream (this is also how a
 *             shared, stride-0 past state is expanded into per-sequence
 *             tables; next_state strides must then be non-zero when
 *             batch > 1).  Any partial overlap is FWPKM_ERR_ALIAS.
 *   retrieved [batch, tokens, H, d_v]    written; must not overlap any input
 *   out_slots   nullable [batch, tokens, H, k] int32: selected slots, best
 *               first (ties by lower slot)
 *   out_weights nullable [batch, tokens, H, k] fp32: their softmax weights
 *   stream    HIP stream to enqueue on (0 = null stream)
 *
 * The handle's workspace is reused by every call: calls on one handle must
 * be ordered (one stream at a time); the handle is not thread-safe. */
int fwpkm_forward_chunk(fwpkm_handle* h,
                        const float* queries, const float* targets,
                        int32_t batch, int32_t tokens, float lr,
                        const fwpkm_state* past_state, const fwpkm_state* next_state,
                        float* retrieved, int32_t* out_slots, float* out_weights,
                        hipStream_t stream);

/* fwpkm_forward_chunk with per-token importance weights on the memorisation
 * loss [sciencestack.ai "Fast-weight Product Key Memory", contents entry
 * "Weighting MSE loss by token importance"]:
 *
 *   token_weights  nullable [batch, tokens, H] fp32, finite.  Token t's loss
 *                  becomes lambda_t/2 ||retrieved_t - target_t||^2, so its
 *                  gradients are scaled by lambda_t; a token with
 *                  lambda_t == 0 is read (retrieved, out_slots, out_weights
 *                  as usual) but writes nothing and is not counted in the
 *                  per-row mean (e.g. the last token of a sequence, which
 *                  has no lookahead target).  NULL means every weight is 1:
 *                  the call is then exactly fwpkm_forward_chunk.
 *
 * Every other argument, the aliasing rules (token_weights is an input: it
 * must not overlap retrieved or next_state) and the return codes are those
 * of fwpkm_forward_chunk. */
int fwpkm_forward_chunk_weighted(fwpkm_handle* h,
                                 const float* queries, const float* targets,
                                 const float* token_weights,
                                 int32_t batch, int32_t tokens, float lr,
                                 const fwpkm_state* past_state, const fwpkm_state* next_state,
                                 float* retrieved, int32_t* out_slots, float* out_weights,
                                 hipStream_t stream);

/* ---- without device allocation --------------------------------------------
 * For callers that cannot allocate device memory: code being captured into a
 * HIP graph, tight serving loops, harnesses that forbid hipMalloc.
 *
 * fwpkm_forward_chunk with the same arguments, rules and results (the same
 * kernels run), except where the workspace lives: a fixed array of
 * FWPKM_NOALLOC_SCRATCH_BYTES bytes in the library's device data instead of
 * the handle's allocation.  The call never calls hipMalloc, hipFree or any
 * other allocating routine, and neither allocates nor touches the handle's
 * own workspace (the handle supplies the configuration only).
 *
 *   - Limit: the call's workspace, fwpkm_workspace_bytes of the
 *     configuration with max_batch = batch and chunk_size = tokens, must not
 *     exceed FWPKM_NOALLOC_SCRATCH_BYTES, else FWPKM_ERR_UNSUPPORTED (checked
 *     with the other arguments, before anything is enqueued).
 *   - Each GPU holds its own copy of the array from library load until the
 *     process ends.  The first call on a device looks its address up (a
 *     symbol query, not an allocation) with that device current.
 *   - Every call on one GPU shares that GPU's array, which keeps the last
 *     call's contents: calls that overlap in time on one GPU (other streams,
 *     threads or handles) race and give undefined results; order them on one
 *     stream.  Nothing in the array needs to start at zero: every call
 *     writes each part before reading it.
 *   - Per-kernel timing (fwpkm_profile_enable) does not record these calls. */
#define FWPKM_NOALLOC_SCRATCH_BYTES (64u << 20)
int fwpkm_forward_chunk_noalloc(fwpkm_handle* h,
                                const float* queries, const float* targets,
                                int32_t batch, int32_t tokens, float lr,
                                const fwpkm_state* past_state, const fwpkm_state* next_state,
                                float* retrieved, int32_t* out_slots, float* out_weights,
                                hipStream_t stream);

/* ---- sequence-level layer ------------------------------------------------
 * Whole token sequences through the memory [PyPI page
 * "fast-weight-product-key-memory", Usage: model-width tokens in, memories
 * chained from call to call; gist.science "Fast-weight Product Key Memory",
 * section 2: Core Architecture (gated residual output) and Key Technical
 * Choices (lookahead targets)].  With D = num_heads * dim_v the model width
 * and, per token t of a sequence of S tokens:
 *
 *   [q_t | v_t] = w_in x_t               fp32 projection (queries of head
 *                                         0..H-1, then values of head 0..H-1)
 *   target of q_t = v_{t+1}              the last token has none: it reads
 *                                         but does not write (weight 0)
 *   chunks of chunk_size tokens (the last may be shorter), each read with
 *   the tables left by the chunks before it, then written
 *   (fwpkm_forward_chunk_weighted's step, addr_weight included)
 *   g = sigmoid(w_gate[h] . x_t + b_gate[h])
 *   out_t[h*dim_v .. (h+1)*dim_v) = g * r_t[h] + (1 - g) * x_t[same slice]
 *
 * The gate's and the projections' forms are readings: the pages name the
 * gate and the lookahead pairing but give no formula for either. */

/* Bytes of workspace fwpkm_forward_sequence needs for (batch, seq); 0 on
 * an invalid configuration or size (see fwpkm_last_error). */
size_t fwpkm_sequence_workspace_bytes(const fwpkm_config* cfg, int32_t batch, int32_t seq);

/* Arguments (device pointers unless noted; all row-major fp32):
 *   x          [batch, seq, D] tokens
 *   w_in       [H*dim_qk + H*dim_v, D] projection rows
 *   w_gate     [H, D] gate weights;  b_gate  nullable [H] gate biases (0)
 *   batch      1 .. max_batch;  seq  >= 1 (batch * seq <= 2^30)
 *   lr         learning rate of every chunk's step (0: read only)
 *   past_state, next_state  as for fwpkm_forward_chunk: the first chunk
 *              reads past_state (copied into next_state when they differ),
 *              later chunks update next_state in place
 *   out        [batch, seq, D] written: the gated output
 *   out_slots, out_weights  nullable [batch, seq, H, k]: every token's
 *              selection, as fwpkm_forward_chunk reports it
 *   workspace  caller-owned device memory of at least
 *              fwpkm_sequence_workspace_bytes(cfg, batch, seq) bytes (its
 *              contents need no initialisation and are scratch afterwards)
 *   stream     HIP stream to enqueue on
 * Aliasing: out, out_slots, out_weights, the workspace and next_state must
 * not overlap x, w_in, w_gate or b_gate; outputs must not overlap the
 * workspace or the state; the workspace must not overlap the state
 * (FWPKM_ERR_ALIAS).  Every size and pointer is checked before anything is
 * enqueued; a HIP error during enqueueing leaves out and next_state
 * unspecified.  The handle's own workspace is used by each chunk, as for
 * fwpkm_forward_chunk: calls on one handle must be ordered. */
int fwpkm_forward_sequence(fwpkm_handle* h,
                           const float* x, const float* w_in,
                           const float* w_gate, const float* b_gate,
                           int32_t batch, int32_t seq, float lr,
                           const fwpkm_state* past_state, const fwpkm_state* next_state,
                           float* out, int32_t* out_slots, float* out_weights,
                           void* workspace, size_t workspace_bytes,
                           hipStream_t stream);

/* Release the handle and its workspace (synchronises the device before the
 * workspace is freed).  NULL-safe. */
void fwpkm_destroy(fwpkm_handle* h);

/* Message of the last failing call on this thread ("" if none). */
const char* fwpkm_last_error(void);

/* ---- per-kernel timing (measurement support, off by default) ------------
 * With profiling enabled, every fwpkm_forward_chunk call on the handle also
 * records a pair of HIP events around each kernel (and the state copy) on the
 * call's stream.  The events are timing-only markers: they add no
 * synchronisation.  Kernel ids are stable:
 *   0 score  (sub-key scoring + per-half top-k)
 *   1 read   (Cartesian top-k, weights, gather, backward)
 *   2 sort   (pair-list radix sort)
 *   3 update (segmented mean gradient + SGD)
 *   4 copy   (past -> next state copy, copy mode only)
 *   5 addr_stats   (addressing loss: softmax statistics and marginal usage)
 *   6 addr_grad    (addressing loss: key gradient contraction)
 *   7 addr_apply   (addressing loss: key step)
 *   8 project  (sequence layer: query/value projection and last-token prep)
 *   9 gate     (sequence layer: gated output)                             */
#define FWPKM_NUM_TIMED 10

/* enable != 0: clear the totals and start recording; 0: stop recording. */
int fwpkm_profile_enable(fwpkm_handle* h, int32_t enable);

/* Wait for the recorded events, add their elapsed times to the totals and
 * report them: ms[i] = total milliseconds of kernel i, launches[i] = how many
 * launches were timed.  Arrays hold FWPKM_NUM_TIMED entries; either may be
 * NULL.  Synchronises with the recorded events (not with the whole device). */
int fwpkm_profile_read(fwpkm_handle* h, double* ms, int64_t* launches);

/* Short name of timed kernel i ("" outside 0..FWPKM_NUM_TIMED-1). */
const char* fwpkm_kernel_name(int32_t i);

/* 1 in a checked build of this library, else 0.
 *
 * A checked build (compiled with FWPKM_DEVICE_CHECKS=1; the package's build
 * script makes it with --checked, as libfwpkm_checked.so) runs the same
 * kernels with device-side tests of the invariants the indexing rests on:
 * every per-half candidate index below n, k Cartesian candidates per token,
 * every selected slot in [0, N) and distinct, every selection weight finite
 * and in [0, 1], every grouped entry's row and token in range, equal to its
 * pair's row and in row order, and every update batch within its LDS lists.
 * Every chunk call first fills its whole workspace with 0xFF bytes (NaN as a
 * float, -1 as an index), so that a kernel reading workspace the call never
 * wrote gets values the tests or the results expose.  A failed test sets a
 * bit in a word of the workspace; each chunk call then waits for its stream
 * and returns FWPKM_ERR_DEVICE_CHECK naming the tests that failed.  The wait
 * makes a checked build unsuitable for stream capture and for timing; the
 * tests never trap, so a failure cannot fault the device.  For debugging
 * and test runs, not for production. */
int32_t fwpkm_checked_build(void);

#ifdef __cplusplus
}
#endif

#endif /* FWPKM_H */
