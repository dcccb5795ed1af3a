/*
 * ttt.h — C ABI of the chunk-wise test-time-training (TTT) inner loop on MI355X (gfx950).
 *
 * What the library computes (pages: "End-to-End Test-Time Training for Long Context",
 * review on kimjy99.github.io = [E2E]; "In-Place Test-Time Training", review on
 * blog.secrett2633.cloud = [IPT]; "Self-Generated Feedback Destabilizes Test-Time
 * Training", summary on onedev.kr = [SGF]):
 *
 *   f(x; W) = LMhead( block_L( ... block_1( E_in[x] ) ) )       (no final norm, untied head)
 *   block_l(h) = h + MLP_l(norm(h)),  norm = none | RMSNorm without gain (eps from the config)
 *   MLP = GELU(n W1) W2 with W1, W2 fast                         ([E2E] section 3.1)
 *       | (SiLU(n Wg) * (n Wu)) W2 with Wg, Wu frozen, W2 fast   ([IPT] section 1)
 *   l_t(W) = CE(f(x_{t-1}; W), x_t)                              ([E2E] eq. 1)
 *   for chunk i = 1..T/b, in sequence, tokens of a chunk in parallel ([E2E] eq. 5):
 *       G_i = (1/b) sum_{t in chunk i} grad l_t(W_{i-1})
 *       g_i = ||G_i||_2 over all fast tensors; s_i = min(1, clip/g_i) (clip <= 0: s_i = 1)
 *                                                                ([SGF] one clipped step per chunk)
 *       W_i = W_{i-1} - lr * s_i * G_i
 *   the loss recorded for token t is l_t(W_{i-1}), its chunk's weights before the step
 *                                                                ([E2E] eq. 6)
 *
 * Conventions for every call:
 *   - All tensor pointers are HIP device pointers unless stated otherwise; row-major.
 *   - Tokens are int32 ids in [0, vocab).
 *   - Every function returns a ttt_status and never throws or aborts.
 *   - A context is bound to one HIP stream (given at creation) and is not thread-safe.
 *     Separate contexts are independent.
 *   - Conditions the device detects (an id out of range, a non-finite gradient norm)
 *     are recorded in a sticky device flag and returned by the next synchronising call
 *     (ttt_sync, ttt_token_losses, ttt_token_argmax, ttt_chunk_stats, ttt_fast_weights).
 *     After that, ttt_prefill_chunks returns TTT_ESTATE until ttt_reset or ttt_destroy.
 */
#ifndef TTT_H_
#define TTT_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TTT_ABI_VERSION 1

typedef struct ttt_ctx ttt_ctx;

typedef enum {
  TTT_OK = 0,
  TTT_EINVAL = -1,     /* bad argument or configuration; nothing was enqueued            */
  TTT_ENOMEM = -2,     /* device allocation failed                                         */
  TTT_EDEVICE = -3,    /* no usable HIP device, or a HIP runtime call failed               */
  TTT_ERANGE = -4,     /* a token id outside [0, vocab) was seen (it was read as id 0)     */
  TTT_ENONFINITE = -5, /* a chunk's gradient norm was not finite; that chunk took no step  */
  TTT_ESTATE = -6      /* the context holds a sticky error; reset or destroy it            */
} ttt_status;

enum { TTT_MLP_GELU = 0, TTT_MLP_SWIGLU_W2 = 1 };
enum { TTT_NORM_NONE = 0, TTT_NORM_RMS = 1 };
/* TTT_FP32: fp32 GEMM operands and fp32 fast weights (kept as W0 + D, D the fp32
 *           accumulated update).
 * TTT_BF16: bf16 GEMM operands (weights and activations rounded to nearest even),
 *           fp32 accumulation, fp32 residual stream and losses. The fast state is kept as
 *           W0 + D with D the fp32 accumulated update. The forward products read it as two
 *           bf16 K-segments, W0 and rn(D) (a single rn(W0 + D) would drop updates smaller
 *           than half a bf16 ulp of W0); the backward products read rn(W0 + D). Chunk
 *           gradients are stored in bf16; their squared norm is summed from the fp32
 *           accumulators. */
enum { TTT_FP32 = 0, TTT_BF16 = 1 };

typedef struct {
  int32_t abi_version;  /* must be TTT_ABI_VERSION                                        */
  int32_t vocab;        /* V >= 2, multiple of 8                                          */
  int32_t d_model;      /* d >= 8, multiple of 8                                          */
  int32_t d_hidden;     /* m >= 8, multiple of 8                                          */
  int32_t n_blocks;     /* L >= 0; 0 = LM head on the embeddings (no fast weights).
                           TTT_MLP_SWIGLU_W2 supports L = 1 only.                         */
  int32_t mlp;          /* TTT_MLP_*                                                       */
  int32_t norm;         /* TTT_NORM_*                                                      */
  int32_t precision;    /* TTT_FP32 | TTT_BF16                                             */
  int32_t chunk;        /* b >= 1 tokens per TTT step                                      */
  int32_t reserved;     /* must be 0                                                       */
  int64_t max_tokens;   /* capacity of the per-token loss / argmax record (multiple of b) */
  float lr;             /* eta >= 0                                                        */
  float clip;           /* c; <= 0 disables clipping                                       */
  float rms_eps;        /* epsilon of RMSNorm (ignored for TTT_NORM_NONE)                  */
  float reserved_f;     /* must be 0                                                       */
} ttt_config;

/* Initial weights. Element type is bf16 (raw 16-bit patterns) for TTT_BF16, fp32 for
 * TTT_FP32. Shapes, row-major:
 *   embed    [V x d]  input embedding E_in (frozen)
 *   lm_head  [V x d]  output head E_out (frozen; logits z = h E_out^T)
 *   w1[l]    [d x m]  GELU: fast W1 of block l.  SWIGLU: frozen gate Wg.
 *   w_up[l]  [d x m]  SWIGLU only: frozen up projection Wu; NULL array for GELU.
 *   w2[l]    [m x d]  fast down projection W2 of block l.
 * The arrays w1, w_up, w2 are HOST arrays of n_blocks device pointers. */
typedef struct {
  const void* embed;
  const void* lm_head;
  const void* const* w1;
  const void* const* w_up;
  const void* const* w2;
} ttt_weights;

/* Create a context for one token stream ([E2E] Method: the model reads a prefix x_0..x_T
 * with x_0 = BOS and keeps learning from it; [IPT] section 1: the fast weights are private
 * state of the stream, updated while it is read, the rest of the model frozen). Validates
 * the configuration, allocates all device memory the chunk loop needs, and copies every
 * weight into library-owned memory (the caller may free its tensors when this returns). Synchronous. `stream` is a hipStream_t (NULL =
 * the default stream) on which every later call of this context is enqueued.
 * Errors: TTT_EINVAL (config), TTT_ENOMEM, TTT_EDEVICE. On error *out is NULL. */
ttt_status ttt_create(const ttt_config* cfg, const ttt_weights* w, void* stream, ttt_ctx** out);

/* Largest number of streams of one batched context. */
#define TTT_MAX_STREAMS 4096

/* Create a context that advances `streams` independent token streams together ([SGF], How
 * it works: several sequences are adapted side by side, each stream from the same initial
 * weights with its own fast weights and its own clipped step per chunk). The frozen weights
 * and W0 are stored once; each stream has its own fast state D, records (losses, argmax,
 * chunk statistics) and clip. Every result of a stream equals that of a single-stream
 * context fed the same tokens, up to the summation order of products that now cover all
 * streams' rows. One chunk step covers all streams: the products with a stream's own fast
 * weights run as grouped launches, those with frozen weights (LM head, CE backward) once
 * over the streams' stacked rows. Each stream beyond the first costs 10 bytes (bf16) or 16
 * bytes (fp32) per fast parameter (D, Wop, WtT, G) and its share of the per-token buffers
 * (the largest, the CE numerators, chunk x vocab elements).
 * streams in [1, TTT_MAX_STREAMS]; with streams > 1 the chunk size must be a multiple of
 * 64 and streams * chunk at most 2^21. ttt_create(...) is ttt_create_batch(..., 1, ...).
 * A batched context (streams > 1) supports ttt_prefill_batch, the ttt_stream_* readers, the
 * stream-0 readers, ttt_reset, ttt_sync, the profiling calls and ttt_destroy; ttt_prefill_chunks,
 * ttt_decode, ttt_evaluate, ttt_snapshot, ttt_restore and ttt_settle_chunk return TTT_EINVAL.
 * Errors: as ttt_create. */
ttt_status ttt_create_batch(const ttt_config* cfg, const ttt_weights* w, int32_t streams, void* stream,
                            ttt_ctx** out);

/* Number of streams of the context (-1 for NULL). */
int32_t ttt_streams(const ttt_ctx* ctx);

/* Frozen layers added to every TTT'd block, before its fast MLP, each with its own pre-norm
 * and residual:
 *   h <- h + Attn(norm(h))                (swa_window = k > 0: sliding-window attention,
 *                                          [E2E] section 3, window k >= chunk recommended)
 *   h <- h + GELU(norm(h) Ws1) Ws2        (static_hidden = m_s > 0: the static MLP of
 *                                          [E2E] section 3.1, "two MLP layers per block")
 *   h <- h + MLP(norm(h))                 (the fast MLP of ttt_config)
 * The inner loop backpropagates through the frozen layers of the blocks above each fast
 * one; nothing of them is updated. TTT_MLP_GELU only.
 * Attention: swa_heads heads of 128 (d_model = 128 swa_heads), TTT_BF16 only;
 * q = n Wq, k = n Wk, v = n Wv, softmax(q.k / sqrt(128)) over the keys of the last k
 * positions up to the query's own (no positional encoding), output o Wo. Each position's key
 * and value are computed once, at the weights of the chunk (or the decoded token) that first
 * processes it, and kept in a ring of k + chunk positions per block and stream, in half
 * precision (read by the forward and decode) and in bf16 (read by the backward): 8 (k +
 * chunk) d bytes; later chunks read them as constants. A single-stream
 * context keeps a second set of rings for passages: ttt_evaluate scores a passage as a
 * sequence of its own (its positions attend only within it) and leaves the stream's rings as
 * they are ([SGF], Settlement: the two scores leave the attention unchanged). Snapshots hold
 * the fast state only; a Settlement candidate's keys and values join the stream's rings
 * whatever the decision, as its tokens join the stream. A batched context with attention
 * supports prefill and the readers.
 *   ws1[l] [d x m_s], ws2[l] [m_s x d], wq/wk/wv/wo[l] [d x d]: HOST arrays of n_blocks
 *   device pointers, element type as the other weights; copied at creation like them.
 *   Arrays of an absent layer are ignored. */
typedef struct {
  int32_t static_hidden;   /* m_s, a multiple of 8 (0: no static MLP)            */
  int32_t swa_window;      /* k (0: no attention)                               */
  int32_t swa_heads;       /* heads of 128                                      */
  int32_t reserved;        /* must be 0                                         */
  const void* const* ws1;
  const void* const* ws2;
  const void* const* wq;
  const void* const* wk;
  const void* const* wv;
  const void* const* wo;
} ttt_block_ext;

/* ttt_create_batch with the block extension (NULL ext: none). Errors: as ttt_create_batch,
 * TTT_EINVAL for a bad extension (m_s not a multiple of 8, a missing pointer, the SwiGLU
 * block, attention outside bf16 or with d_model != 128 heads, a nonzero reserved field). */
ttt_status ttt_create_ext(const ttt_config* cfg, const ttt_weights* w, const ttt_block_ext* ext, int32_t streams,
                          void* stream, ttt_ctx** out);

/* Run the inner loop over n_tokens new tokens ([E2E] Method: prefill; section 3 eq. 5).
 * tokens: device int32 [n_tokens + 1]; tokens[0] conditions the first prediction (BOS on
 *         the first call, else the previous call's last token); tokens[1..n_tokens] are
 *         scored and trained on. Borrowed until the stream passes this call.
 * n_tokens must be a positive multiple of the chunk size and fit in the remaining
 * capacity (max_tokens - tokens already consumed). Enqueued; returns immediately.
 * Errors (nothing enqueued): TTT_EINVAL, TTT_ESTATE. */
ttt_status ttt_prefill_chunks(ttt_ctx* ctx, const int32_t* tokens, int64_t n_tokens);

/* ttt_prefill_chunks for every stream of the context at once: tokens is device int32
 * [streams x ld_tokens], row z holding stream z's n_tokens + 1 ids (as for
 * ttt_prefill_chunks); ld_tokens >= n_tokens + 1 when streams > 1 (ignored for one stream).
 * Chunk i of every stream is computed in one step, the streams' chunks in lockstep; the
 * streams never exchange data. Enqueued. Errors (nothing enqueued): TTT_EINVAL, TTT_ESTATE. */
ttt_status ttt_prefill_batch(ttt_ctx* ctx, const int32_t* tokens, int64_t ld_tokens, int64_t n_tokens);

/* Decode n tokens one at a time ([E2E] Method: decoding predicts the next token's
 * distribution from the current weights; section 3.2: a gradient step is taken only when
 * the decoded tokens fill a mini-batch, and decoding continues with the updated weights).
 * tokens: device int32 [n + 1]; tokens[0] is the stream's last token so far (the last id of
 *         the previous prefill or decode call, BOS if nothing came before); for i in [0, n),
 *         prediction i is f(tokens[i]; W) at the current fast weights and scores tokens[i + 1].
 *         Borrowed until the stream passes this call.
 * For every prediction, the loss and argmax are recorded at the next token position (read
 * back with ttt_token_losses / ttt_token_argmax, like prefilled tokens); argmax (device int32
 * [n]) and logits (device fp32 [n x vocab], row i = prediction i) receive them too when
 * non-NULL. Each time b decoded pairs complete a chunk, that chunk takes the same step as in
 * ttt_prefill_chunks (which also re-records its losses, then with the bf16 loss compensation)
 * before the next prediction. Decoded pairs that do not yet fill a chunk stay pending across
 * calls (ttt_decode_pending); ttt_prefill_chunks is refused (TTT_EINVAL) while any are.
 * Predictions use fp32 activations against the stored fast weights (bf16: W0 and rn(D) as two
 * segments, as in the forward GEMMs), so their losses carry no operand rounding. Ids out of
 * range raise the sticky TTT_ERANGE and read id 0. n = 0 is a no-op. With attention, each
 * prediction's key and value join the stream's rings at its position before it attends over
 * the window (fp32 arithmetic over the rings' half-precision keys and values); a filled
 * chunk's step re-files the
 * chunk's keys and values from its own forward pass, as prefill would.
 * Errors (nothing enqueued): TTT_EINVAL (n < 0, NULL tokens, capacity, a batched context),
 * TTT_ESTATE. */
ttt_status ttt_decode(ttt_ctx* ctx, const int32_t* tokens, int64_t n, int32_t* argmax, float* logits);

/* Decoded pairs waiting for their chunk to fill (0 .. chunk - 1; -1 for NULL). */
int64_t ttt_decode_pending(const ttt_ctx* ctx);

/* Loss of a passage at the current fast weights, without any step ([SGF]: a held-out
 * real-text passage is scored against the state; scoring changes nothing).
 * q: device int32 [nq + 1]; q[0] conditions q[1]; nq a positive multiple of the chunk size.
 * losses: device fp32 [nq], per-token losses (bf16: with the same loss compensation as the
 * recorded prefill losses); mean: device fp32 scalar, their mean. Either may be NULL. The
 * stream (token count, records, pending decode pairs, fast weights) is unchanged.
 * Errors (nothing enqueued): TTT_EINVAL, TTT_ESTATE. */
ttt_status ttt_evaluate(ttt_ctx* ctx, const int32_t* q, int64_t nq, float* losses, float* mean);

/* Snapshot of the fast state (one slot per context; the first call allocates it, about
 * 8 bytes per fast parameter in bf16 mode), and restore of that snapshot. Enqueued.
 * ttt_restore returns TTT_ESTATE when no snapshot was taken. ttt_settle_chunk uses the same
 * slot. Errors: TTT_EINVAL, TTT_ESTATE. */
ttt_status ttt_snapshot(ttt_ctx* ctx);
ttt_status ttt_restore(ttt_ctx* ctx);

/* The Settlement rule ([SGF], Settlement): the candidate chunk (tokens: device int32
 * [chunk + 1], as for one prefill chunk) is scored at W and stepped to W + delta as in
 * ttt_prefill_chunks; the held-out passage q (as for ttt_evaluate) gives
 *   A = L(q, W) - L(q, W + delta)   (mean per-token losses),
 * and delta is kept only if A >= 0; otherwise the fast weights return to W. The candidate's
 * losses, argmax and chunk statistics are recorded either way and the token count advances
 * by one chunk. A (device fp32) and committed (device int32, 1 = kept) receive the outcome
 * when non-NULL. The decision and the restore happen on the device: nothing synchronises.
 * Refused (TTT_EINVAL) while decoded pairs are pending. Errors: TTT_EINVAL, TTT_ESTATE. */
ttt_status ttt_settle_chunk(ttt_ctx* ctx, const int32_t* tokens, const int32_t* q, int64_t nq, float* A,
                            int32_t* committed);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): ttt_settle_chunk with the pre-candidate
 * snapshot kept in the library's static scratch, a device array of
 * TTT_STATIC_SCRATCH_BYTES bytes per GPU, instead of the context's snapshot slot that
 * ttt_settle_chunk allocates on first use. The array's device address is looked up when the
 * first context is created on a GPU (the runtime may back it with memory then), and the GPU
 * holds it until the process ends. This call itself allocates nothing: no hipMalloc, no
 * hipFree, no allocating library routine. Results (A, the decision, the recorded losses and the
 * state it leaves) are those of ttt_settle_chunk; the context's own snapshot slot is
 * neither used nor changed (ttt_restore still returns to the last ttt_snapshot).
 * The snapshot needs, per fast tensor of n parameters, 4 n + 2 n e bytes, each part rounded
 * up to 256 (e = 2 in bf16, 4 in fp32): about 8 bytes per fast parameter in bf16, so
 * contexts up to about 8.3M fast parameters in bf16 (5.5M in fp32).
 * Every call on one GPU uses that GPU's one array: calls whose work may overlap on the GPU
 * (other streams, other contexts) race on it and must be ordered by the caller; calls on one
 * context are ordered by its stream. The array keeps the last call's contents; nothing in it
 * needs to start at zero (the snapshot is written before it is read).
 * Errors (nothing enqueued): TTT_EINVAL (as ttt_settle_chunk, and a snapshot larger than
 * TTT_STATIC_SCRATCH_BYTES), TTT_ESTATE, TTT_EDEVICE (the array's address is unavailable). */
#define TTT_STATIC_SCRATCH_BYTES (64ll << 20)
ttt_status ttt_settle_chunk_noalloc(ttt_ctx* ctx, const int32_t* tokens, const int32_t* q, int64_t nq, float* A,
                                    int32_t* committed);

/* Copy the recorded losses l_t(W_{i-1}) of tokens [offset, offset + n) (counted from the
 * first token of the first prefill since creation or reset) into dst (device fp32 [n]).
 * These are the summands of [E2E] eq. (6), L = (1/T) sum_i sum_{t in chunk i} l_t(W_{i-1}):
 * each token is scored at its chunk's weights before that chunk's step.
 * Synchronises the context's stream; returns a pending sticky error if there is one
 * (the copy is still made). Errors: TTT_EINVAL (range), TTT_ERANGE, TTT_ENONFINITE. */
ttt_status ttt_token_losses(ttt_ctx* ctx, float* dst, int64_t offset, int64_t n);

/* Same for the argmax of each scored token's logits (lowest index on ties); dst int32 [n]. */
ttt_status ttt_token_argmax(ttt_ctx* ctx, int32_t* dst, int64_t offset, int64_t n);

/* Per-chunk clip statistics: dst device fp32 [n x 2] = (g_i, s_i) for chunks
 * [offset, offset + n); s_i = 0 marks a chunk that took no step. Synchronises. */
ttt_status ttt_chunk_stats(ttt_ctx* ctx, float* dst, int64_t offset, int64_t n);

/* Export a fast tensor as fp32 into dst (device, same shape/layout as its initial
 * weight: W1 [d x m], W2 [m x d]): the fast weights W_i after the last step of [E2E]
 * eq. (5) ([E2E] section 3.1: the MLP weights; [IPT] section 1: the final projection only).
 * which: 1 = W1 (GELU only), 2 = W2.
 * kind: 0 = current W = W0 + D;  1 = accumulated update D = W - W0. Synchronises.
 * Errors: TTT_EINVAL (block/which/kind). */
ttt_status ttt_fast_weights(ttt_ctx* ctx, int32_t block, int32_t which, int32_t kind, float* dst);

/* The readers above for stream s of the context (the ones above read stream 0). Errors as
 * there, and TTT_EINVAL for s outside [0, streams). */
ttt_status ttt_stream_token_losses(ttt_ctx* ctx, int32_t s, float* dst, int64_t offset, int64_t n);
ttt_status ttt_stream_token_argmax(ttt_ctx* ctx, int32_t s, int32_t* dst, int64_t offset, int64_t n);
ttt_status ttt_stream_chunk_stats(ttt_ctx* ctx, int32_t s, float* dst, int64_t offset, int64_t n);
ttt_status ttt_stream_fast_weights(ttt_ctx* ctx, int32_t s, int32_t block, int32_t which, int32_t kind, float* dst);

/* Restore W = W0 (every stream), forget recorded losses, and clear a sticky error. Enqueued. */
ttt_status ttt_reset(ttt_ctx* ctx);

/* Wait for the context's stream; return a pending sticky error if there is one. */
ttt_status ttt_sync(ttt_ctx* ctx);

/* Number of tokens consumed since creation or reset (host-side counter). */
int64_t ttt_tokens_consumed(const ttt_ctx* ctx);

/* Free all device memory of the context (synchronises first). NULL is allowed. */
ttt_status ttt_destroy(ttt_ctx* ctx);

/* Kernel kinds of the chunk loop, for event-based timing. */
typedef enum {
  TTT_K_GATHER = 0,    /* embedding gather                                   */
  TTT_K_NORM = 1,      /* block pre-norm                                     */
  TTT_K_TRANSPOSE = 2, /* transposed copies of activations / gradients       */
  TTT_K_UP = 3,        /* up-projection GEMM + activation epilogue           */
  TTT_K_DOWN = 4,      /* down-projection GEMM (split-K partials)            */
  TTT_K_RESIDUAL = 5,  /* residual add of the down-projection partials       */
  TTT_K_CE_FWD = 6,    /* LM-head GEMM + online-softmax partials             */
  TTT_K_CE_MERGE = 7,  /* per-token merge of the vocab-tile partials         */
  TTT_K_CE_PROB = 8,   /* dlogits from the stored softmax numerators         */
  TTT_K_CE_DY = 9,     /* dlogits x E_out GEMM (split over the vocab)        */
  TTT_K_DY_SUM = 10,   /* sum of the dY partials                             */
  TTT_K_DU = 11,       /* dY W2^T GEMM + GELU' epilogue                      */
  TTT_K_DW = 12,       /* weight-gradient GEMMs (+ sum of squares per tile)  */
  TTT_K_DHN = 13,      /* dU W1^T GEMM (split-K partials)                    */
  TTT_K_NORM_BWD = 14, /* norm backward into the residual gradient           */
  TTT_K_GRADNORM = 15, /* global gradient norm and clip scale                */
  TTT_K_UPDATE = 16,   /* clipped SGD step of one fast tensor (bracketed on
                          the library's second stream, beside the main one)  */
  TTT_K_DEC_GEMV = 17, /* decode: one-row products with the weights         */
  TTT_K_ATTN = 18,     /* sliding-window attention forward (online softmax)  */
  TTT_K_ATTN_BWD = 19, /* sliding-window attention backward (dQ, dK, dV)     */
  TTT_K_COUNT = 20
} ttt_kernel_kind;

/* Tracing: when bit k of `mask` is set, every later launch of kind k by this context is
 * bracketed by a pair of HIP events recorded on the context stream. mask = 0 turns it off.
 * Events cost a few microseconds of stream time each; leave the mask at 0 for timing runs
 * that do not need per-kernel figures. */
ttt_status ttt_profile_enable(ttt_ctx* ctx, uint32_t mask);

/* Trace only every period-th chunk (period >= 1, default 1), counting from the next chunk;
 * the other chunks run without events. Returns TTT_EINVAL for period < 1. */
ttt_status ttt_profile_period(ttt_ctx* ctx, int32_t period);

/* Synchronise, then add the bracketed durations recorded since the last read into
 * total_ms[TTT_K_COUNT] and launches[TTT_K_COUNT] (host arrays, overwritten), and forget them. */
ttt_status ttt_profile_read(ttt_ctx* ctx, double* total_ms, int64_t* launches);

/* Static English description of a status code. */
const char* ttt_status_string(ttt_status s);

/* Test hook: the library's own tiled MFMA GEMM, C = X Y^T in fp32, with X [M x K] (row
 * stride ldx elements) and Y [N x K] (row stride ldy), both bf16 (precision = TTT_BF16)
 * or fp32 (TTT_FP32), C [M x N] fp32 (row stride ldc). K must be a multiple of 8 (bf16)
 * or 4 (fp32); rows and K-offsets must keep 16-byte alignment. Enqueued on `stream`.
 * It exposes the kernel the inner loop uses so that its tiling can be tested on ragged
 * shapes; it is not a second code path. Errors: TTT_EINVAL. */
ttt_status ttt_test_gemm(int32_t precision, const void* X, int64_t ldx, const void* Y, int64_t ldy,
                         float* C, int64_t ldc, int32_t M, int32_t N, int32_t K, void* stream);

/* Test hook: the forward product of a fast weight in bf16 mode, C = X (Y + Y2)^T in fp32, with
 * X [M x K], Y and Y2 [N x K] bf16 (row strides ldx, ldy, ldy2 elements): the bf16 path
 * multiplies the block input by the frozen W0 and by the rounded accumulated update as two
 * K-segments over the same rows of X ([E2E] section 3, eq. (5): the weights a chunk is scored
 * with are W0 plus the sum of the earlier steps). The K range is cut into `splits` slabs
 * (1 .. 8), each written to its own M x ldc fp32 block of C (C holds splits * M * ldc
 * floats; the caller sums the slabs). `form` picks how the tile engine walks the two
 * segments: 0 as the inner loop does (its tile plan decides), 1 one segment after the other,
 * 2 both weights' slices against one staged slice of X wherever the tile plan allows it, so
 * that tests can hold both forms to the product. K a multiple of 8; 16-byte aligned rows;
 * enqueued on `stream`. It exposes the kernels the inner loop uses on ragged shapes; it is
 * not a second code path. Errors: TTT_EINVAL. */
ttt_status ttt_test_gemm_pair(const void* X, int64_t ldx, const void* Y, int64_t ldy, const void* Y2,
                              int64_t ldy2, float* C, int64_t ldc, int32_t M, int32_t N, int32_t K,
                              int32_t splits, int32_t form, void* stream);

/* Test hook: the library's weight-gradient GEMM (bf16), G = sum over k < K of X_k^T Y_k
 * ([E2E] eq. 5: a fast tensor's chunk gradient, summed over the chunk's tokens), stored in
 * bf16 into G [M x N] (row stride ldg), and each output tile's sum of squared fp32 values
 * into slots[tile] (the partials of the global gradient norm, [SGF] "how it works").
 *   token_major = 1: X [K x M], Y [K x N] row-major (row strides ldx, ldy): the activations
 *     as the chunk's products write them; K a multiple of 64, M and N multiples of 8.
 *   token_major = 0: X [M x K], Y [N x K] row-major: their transposed copies; K a multiple of
 *     64.
 * Both forms run the same output tiles (192 x 192 or 128 x 128, by shape); slots must hold
 * at least ceil(M / 128) ceil(N / 128) floats. Device pointers, 16-byte aligned rows;
 * enqueued on `stream`. It exposes the kernels the inner loop uses so that the two operand
 * layouts can be compared; it is not a second code path. Errors: TTT_EINVAL. */
ttt_status ttt_test_grad(const void* X, int64_t ldx, const void* Y, int64_t ldy, void* G, int64_t ldg,
                         float* slots, int32_t M, int32_t N, int32_t K, int32_t token_major, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TTT_H_ */
