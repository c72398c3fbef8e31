/*
 * dualar.h -- C ABI of the Dual-AR per-frame decode step on AMD Instinct
 * MI355X (gfx950).
 *
 * The method (Fish Audio S2 pages):
 *   [P1] "How the Dual-Autoregressive Architecture Works in Fish Speech S2:
 *        A Deep Dive" -- sections "Slow Transformer: BaseTransformer",
 *        "Fast Transformer: The Codebook Decoder", "DualARModelArgs
 *        Configuration", "Inference Pipeline".
 *   [P2] "Fish Audio S2: a Qwen3-4B on the time axis, four layers on the
 *        codebook axis, and tags that are only text" -- sections "Two
 *        autoregressions, because ten codebooks is ten times the sequence"
 *        (decode loop, logit bias, Eq. 1 fusion and its sqrt(N+1) scale),
 *        "The slow AR is Qwen3-4B. The fast AR is not small" (shapes),
 *        "Streaming: whose numbers" (bf16 RoPE table).
 *
 * One decode frame = multi-codebook fusion of the previous frame, one slow-AR
 * pass at the next time position, the semantic-logit-biased sample of the
 * semantic token, then N fast-AR passes along codebook depth against an
 * N-slot cache rewritten every frame ([P2] "Two autoregressions").
 *
 * Conventions for every call:
 *   - Pointers marked "device" are HIP device memory; "host" is host memory.
 *   - Weights, workspace, prompts, uniforms, outputs and taps belong to the
 *     caller and must outlive the context (weights, workspace) or the call.
 *   - Matrices are [out, in] row-major (nn.Linear layout); element type is
 *     bf16 (raw uint16 bit patterns) or fp32 per dualar_config.weight_dtype.
 *   - Activations, norms, softmax and accumulation are fp32; the K/V caches
 *     hold kv_dtype (default: the weight type); the RoPE tables hold bf16
 *     values.
 *   - Every call validates its arguments on the host first.  On failure it
 *     enqueues nothing, leaves the context unchanged and returns an error;
 *     dualar_last_error() then gives a message.
 *   - Work is enqueued asynchronously on the context's stream.  Faults found
 *     on the device (an out-of-range id in a prompt, a non-finite logit) are
 *     latched in a status word and reported by dualar_sync().
 *   - The checked build of the library (libdualar_checked.so, compiled with
 *     DUALAR_DEVICE_CHECKS) also checks, in the kernels, every cache
 *     position it appends at or reads up to against max_seq_len and every
 *     partial-sum slot against its buffer; a failing check keeps the access
 *     inside the buffer, latches a status bit and makes dualar_sync() return
 *     DUALAR_ERR_DEVICE_INDEX.  The normal build compiles the checks out.
 *   - A context is bound to one stream and one device and is not thread-safe.
 */
#ifndef DUALAR_H
#define DUALAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DUALAR_OK = 0,
  DUALAR_ERR_INVALID_ARG = -1,   /* bad config / pointer / size            */
  DUALAR_ERR_NO_DEVICE = -2,     /* no HIP device visible                  */
  DUALAR_ERR_WORKSPACE = -3,     /* workspace smaller than required        */
  DUALAR_ERR_CONTEXT_FULL = -4,  /* positions would pass max_seq_len       */
  DUALAR_ERR_BAD_TOKEN = -5,     /* device saw an id outside its range     */
  DUALAR_ERR_STATE = -6,         /* call out of order (decode before prefill) */
  DUALAR_ERR_HIP = -7,           /* a HIP runtime call failed              */
  DUALAR_ERR_DEVICE_FAULT = -8,  /* device saw a non-finite logit          */
  DUALAR_ERR_DEVICE_INDEX = -9   /* checked build only: a device index check failed */
} dualar_status;

typedef enum { DUALAR_F32 = 0, DUALAR_BF16 = 1 } dualar_dtype;

typedef struct dualar_ctx dualar_ctx_t;   /* opaque */

/* Model hyper-parameters.  [P1] "DualARModelArgs Configuration": a fast_*
 * field left unset falls back to the slow value -- here 0 means "inherit"
 * for every fast_* size, and -1 means "inherit" for fast_qk_norm. */
typedef struct {
  int32_t n_layer, dim, n_head, n_kv_head, head_dim, ffn_dim, vocab_size;
  int32_t n_fast_layer, fast_dim, fast_n_head, fast_n_kv_head, fast_head_dim, fast_ffn_dim;
  int32_t slow_qk_norm;          /* 1: per-head RMSNorm of q and k before RoPE */
  int32_t fast_qk_norm;          /* 1 / 0 / -1 (inherit)                        */
  int32_t num_codebooks;         /* N: codebooks per frame (10 at S2)           */
  int32_t codebook_size;         /* C: rows per codebook (4096 at S2)           */
  int32_t semantic_begin_id;     /* first <|semantic:i|> id (inclusive)         */
  int32_t semantic_end_id;       /* last  <|semantic:i|> id (inclusive)         */
  int32_t end_id;                /* <|im_end|>                                  */
  int32_t scale_codebook_embeddings; /* 1: divide the fused sum by sqrt(N+1)   */
  float rope_base;               /* 1e6 at S2; the fast AR uses the same base   */
  float norm_eps;                /* RMSNorm epsilon                             */
  int32_t weight_dtype;          /* dualar_dtype                                */
  int32_t max_batch;             /* sequences held by the workspace             */
  int32_t max_seq_len;           /* slow-AR positions per sequence              */
  int32_t kv_dtype;              /* K/V cache type: dualar_dtype, -1 = weight_dtype */
  int32_t prefill_chunk;         /* prompt positions per sequence per prefill
                                    step (0 = min(4096, max(1, 8192 /
                                    max_batch))); the
                                    workspace holds max_batch * prefill_chunk
                                    activation rows                             */
  int32_t semantic_head;         /* 0: the tied head computes the whole
                                    vocabulary, as [P2] "The slow AR is Qwen3-4B"
                                    describes (then the bias masks it); 1: only
                                    the C semantic rows and the end row, the
                                    ids the biased sample can pick (same draws;
                                    the full head still runs when the
                                    slow_logits tap is requested)              */
} dualar_config;

/* One transformer layer.  q_norm / k_norm are [head_dim] gains shared by all
 * heads, used only when QK-norm is on (else may be NULL). */
typedef struct {
  const void *attention_norm;    /* [dim]                      */
  const void *wq, *wk, *wv;      /* [H*hd, dim], [KV*hd, dim]  */
  const void *q_norm, *k_norm;   /* [hd] or NULL               */
  const void *wo;                /* [dim, H*hd]                */
  const void *ffn_norm;          /* [dim]                      */
  const void *w1, *w3;           /* [ffn, dim]  (gate, up)     */
  const void *w2;                /* [dim, ffn]  (down)         */
} dualar_layer_weights;

/* W4A16 form of a layer's linear matrices ([P3], the model card of a W4A16
 * S2 variant that keeps the attention of its last 12 layers in bf16; it
 * prints no format, so the format is this library's reading).  For each of
 * wq, wk, wv, wo, w1, w3, w2 (index 0..6): q4 = NULL uses the bf16 matrix of
 * dualar_layer_weights; otherwise q4 holds the matrix [rows, in] as 4-bit
 * two's-complement values, two per byte ([rows, in/2] bytes; input 2j in the
 * low nibble of byte j, 2j+1 in the high one) and s4 its bf16 scales
 * [rows, in/128], one per row and group of 128 consecutive inputs; the
 * weight is q * scale.  Device pointers, 16-byte aligned.  wq/wk/wv must be
 * all 4-bit or all bf16, and so must w1/w3.  A 4-bit matrix's rows must be
 * a multiple of 512 inputs, at most 10,240.  Only for bf16 models with
 * max_batch <= 8 and prefill_chunk = 1 or >= 256 (decode products run as
 * 4-bit GEMVs over the batch's rows; prefill steps of 256+ positions run on
 * the matrix cores with each group's sum scaled in fp32); dualar_create
 * rejects other uses with DUALAR_ERR_INVALID_ARG.  With 4-bit fast layers,
 * dualar_fast_teacher_forced needs n * num_codebooks <= 8 or >= 256. */
typedef struct {
  const void *q4[7];             /* wq, wk, wv, wo, w1, w3, w2, or NULL */
  const void *s4[7];
} dualar_layer_w4;

/* All device pointers, each 16-byte aligned (tensors are read with 16-byte
 * vector loads; dualar_create rejects others with DUALAR_ERR_INVALID_ARG);
 * the layer arrays are HOST arrays of n_layer and n_fast_layer entries
 * (copied at create); layers_w4 / fast_layers_w4 may be NULL (all bf16). */
typedef struct {
  const void *tok_embedding;        /* [vocab, dim]; also the tied slow head   */
  const void *codebook_embedding;   /* [N*C, dim]; codebook k = rows k*C..     */
  const void *norm;                 /* [dim] final slow norm                   */
  const dualar_layer_weights *layers;
  const dualar_layer_weights *fast_layers;
  const void *fast_embeddings;      /* [C, fast_dim]                           */
  const void *fast_norm;            /* [fast_dim]                              */
  const void *fast_output;          /* [C, fast_dim]                           */
  const dualar_layer_w4 *layers_w4;       /* NULL or n_layer entries           */
  const dualar_layer_w4 *fast_layers_w4;  /* NULL or n_fast_layer entries      */
} dualar_weights;

/* Sampling ([P2] `decode_one_token_ar` excerpt): greedy, or temperature +
 * top-p driven by caller-supplied uniforms.  Top-p keeps the shortest
 * prefix, in (probability desc, id asc) order, whose mass reaches top_p and
 * draws the first kept id whose renormalised cumulative mass exceeds u.
 * <|im_end|> stays masked until a sequence has emitted min_frames frames.
 *
 * Loop breaker (RAS, [P2] "Two autoregressions, because ten codebooks is
 * ten times the sequence", the paragraph after Eq. 1): with ras_window > 0
 * every slow draw that repeats a semantic id the sequence emitted in its
 * previous ras_window frames is replaced by a second top-p draw at
 * (ras_temperature, ras_top_p) from the same biased logits.  The uniforms
 * then hold N + 1 draws per (frame, sequence), slot N being the second
 * draw's, and may not be NULL.  <|im_end|> is never replaced; the id
 * emitted enters the window.  dualar_fast_frames ignores it (no slow draw). */
#define DUALAR_RAS_MAX_WINDOW 16
typedef struct {
  float temperature;             /* > 0 */
  float top_p;                   /* (0, 1] */
  int32_t greedy;                /* 1: argmax (lowest id on ties) */
  int32_t min_frames;
  int32_t ras_window;            /* 0 = off, 1..DUALAR_RAS_MAX_WINDOW ([P2]: 10) */
  float ras_temperature;         /* > 0 when ras_window > 0 ([P2]: 1.0) */
  float ras_top_p;               /* (0, 1] when ras_window > 0 ([P2]: 0.9) */
} dualar_sampling;

/* Optional fp32 device buffers filled with the LAST frame of a call. */
typedef struct {
  float *fused_x;                /* [batch][dim]   slow-AR input of the frame     */
  float *slow_hidden;            /* [batch][dim]   residual before the final norm */
  float *slow_logits;            /* [batch][vocab] unbiased slow logits           */
  float *fast_logits;            /* [batch][N-1][C] logits of q^(1..N-1)          */
} dualar_taps;

/* Bytes of device workspace a context needs for this config: slow and fast
 * K/V caches, RoPE tables, activations, logits, per-sequence state.  Returns
 * 0 for an invalid config. */
size_t dualar_workspace_bytes(const dualar_config *cfg);

/* Create a context.  Validates cfg and weights, binds the stream (a
 * hipStream_t, NULL = default stream) and the current device, and enqueues
 * the workspace initialisation (zeroed state, RoPE tables).  *out is set
 * only on success. */
dualar_status dualar_create(const dualar_config *cfg, const dualar_weights *w,
                            void *workspace, size_t workspace_bytes,
                            void *hip_stream, dualar_ctx_t **out);

/* Largest workspace dualar_create_static can provide (32 MiB). */
#define DUALAR_STATIC_WORKSPACE_BYTES (32u << 20)

/* dualar_create without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The workspace is a static device array
 * of DUALAR_STATIC_WORKSPACE_BYTES that the library holds on every GPU it
 * runs on until the process ends; this call allocates no device memory (no
 * hipMalloc / hipFree, no framework allocator).  Everything else is as in
 * dualar_create: the same validation, the same initialisation (zeroed state,
 * RoPE tables) enqueued on hip_stream, and the same kernels and results for
 * every later call on the context.
 * Fails with DUALAR_ERR_WORKSPACE (nothing created) when
 * dualar_workspace_bytes(cfg) exceeds DUALAR_STATIC_WORKSPACE_BYTES (small
 * models, batches and prefill chunks fit), and DUALAR_ERR_HIP if the
 * array's device address cannot be obtained.
 * Every context made by this call on one GPU uses the same array, which
 * keeps what the last context wrote: at most one of them may be in use per
 * GPU at a time; creating another (or using two at once) races on that
 * memory.  Destroy as usual with dualar_destroy. */
dualar_status dualar_create_static(const dualar_config *cfg, const dualar_weights *w,
                                   void *hip_stream, dualar_ctx_t **out);

/* Prefill a batch of prompts and emit frame 0 of every sequence.
 *   tokens     device int32 [batch][N+1][t_max]: row 0 = LM ids, rows 1..N =
 *              codebook ids q^(0..N-1) (read at semantic positions only);
 *              a semantic position is fused as in decode, a text position
 *              takes its LM embedding alone.
 *   prompt_len host int32 [batch], 1 <= prompt_len[b] <= t_max.
 *   uniforms   device fp32 [batch][N] for top-p, or NULL when greedy;
 *              [batch][N + 1] with the loop breaker on (slot N).
 *   frame0     device int32 [batch][N+1]: (id, q^(0..N-1)); a sequence whose
 *              first sample is <|im_end|> gets (end_id, -1, ..., -1).
 *   taps       NULL, or buffers for frame 0's slow hidden state, slow logits
 *              and fast logits (fused_x is not written by prefill).
 * Resets every sequence of the context.  Requires batch <= max_batch and
 * prompt_len[b] < max_seq_len. */
dualar_status dualar_prefill(dualar_ctx_t *ctx, int32_t batch, const int32_t *tokens,
                             int32_t t_max, const int32_t *prompt_len,
                             const dualar_sampling *s, const float *uniforms,
                             int32_t *frame0, const dualar_taps *taps);

/* Decode n_frames frames for every sequence of the last prefill.
 *   uniforms  device fp32 [n_frames][batch][N] (slot 0: slow draw, slot k:
 *             draw of q^(k)), or NULL when greedy; [n_frames][batch][N + 1]
 *             with the loop breaker on (slot N: its second draw).
 *   codes     device int32 [batch][n_frames][N+1]; rows after a sequence has
 *             ended are -1; the row that samples <|im_end|> is
 *             (end_id, -1, ..., -1).
 *   n_emitted device int32 [batch] or NULL: frames emitted so far by each
 *             sequence, frame 0 included.
 *   taps      NULL, or buffers filled with the last frame's intermediates.
 * Fails with DUALAR_ERR_CONTEXT_FULL if a sequence would pass max_seq_len. */
dualar_status dualar_decode_frames(dualar_ctx_t *ctx, int32_t n_frames,
                                   const dualar_sampling *s, const float *uniforms,
                                   int32_t *codes, int32_t *n_emitted,
                                   const dualar_taps *taps);

/* The fast AR alone (no slow pass): for each frame f and sequence b, N fast
 * passes seeded by a given slow hidden state and first code.
 *   hidden   device fp32 [n_frames][batch][fast_dim]
 *   q0       device int32 [n_frames][batch], 0 <= q0 < C
 *   uniforms device fp32 [n_frames][batch][N] (slot k draws q^(k)) or NULL
 *   codes    device int32 [batch][n_frames][N]: q^(0..N-1)
 *   taps     only fast_logits is used (last frame). */
dualar_status dualar_fast_frames(dualar_ctx_t *ctx, int32_t batch, int32_t n_frames,
                                 const float *hidden, const int32_t *q0,
                                 const dualar_sampling *s, const float *uniforms,
                                 int32_t *codes, const dualar_taps *taps);

/* Teacher-forced fast AR (the training forward of [P1] "Fast Transformer:
 * The Codebook Decoder", Step 3, in scoring form): for each of n pairs of a
 * slow hidden state and that frame's codes, the fast layers run over
 * [h, E_F(q^(0)), ..., E_F(q^(N-2))] with causal attention along depth, all
 * pairs at once (n*N rows through the products), then fast_norm and the
 * fast head on every row.
 *   hidden  device fp32 [n][fast_dim]
 *   codes   device int32 [n][N], 0 <= code < C (q^(N-1) is not read; an
 *           out-of-range code is latched for dualar_sync and row 0 used)
 *   logits  device fp32 [n][N][C]: slot k >= 1 holds the logits of q^(k)
 *           given q^(0..k-1); slot 0 is the head over the hidden state
 *           itself, which the method does not use.
 * n * N must not exceed max_batch * prefill_chunk (the prefill rows of the
 * workspace).  Needs N <= 11, a fast head_dim <= 128 that is a multiple of
 * 4, and 1, 2, 4 or 8 query heads per KV head (else
 * DUALAR_ERR_INVALID_ARG).  The decode state of the context is not touched. */
dualar_status dualar_fast_teacher_forced(dualar_ctx_t *ctx, int32_t n, const float *hidden,
                                         const int32_t *codes, float *logits);

/* Retire sequences of the current batch: each listed slot ends as a
 * sequence that sampled <|im_end|> does ([P1] "Inference Pipeline",
 * "generate: Full Sequence Generation": a generation emits frames until its
 * end token; [P2] "Two autoregressions ...", the decode_one_token_ar loop),
 * so that one finished or faulted sequence can be dropped without a new
 * prefill of the whole batch.
 *   seq_ids host int32 [n], each in [0, batch) of the last prefill
 *           (duplicates allowed); n = 0 is a no-op.
 * Enqueued on the context's stream.  The slot's frame count, pending frame
 * and loop-breaker window are cleared; later dualar_decode_frames calls
 * write -1 code rows for it and report 0 frames emitted, and the other
 * sequences' codes and taps are bit-identical to a run without the reset.
 * The slot's rows keep being computed (on zero input) with the batch, at
 * positions that keep advancing, so the batch's context limit is unchanged.
 * The next dualar_prefill brings every slot back.  Validation happens on the
 * host before anything is enqueued: DUALAR_ERR_STATE before a successful
 * prefill, DUALAR_ERR_INVALID_ARG for a NULL ctx or seq_ids (n > 0), n
 * outside [0, batch] or an id outside [0, batch); a failing call changes
 * nothing. */
dualar_status dualar_reset(dualar_ctx_t *ctx, const int32_t *seq_ids, int32_t n);

/* Block until the stream's work is done; report latched device faults and
 * clear them.  *device_status (host, may be NULL) receives the raw status
 * word: bit 0 an id outside its range (DUALAR_ERR_BAD_TOKEN), bit 1 a
 * non-finite logit (DUALAR_ERR_DEVICE_FAULT), bit 2 a failed index check of
 * the checked build (DUALAR_ERR_DEVICE_INDEX); with several bits set the
 * first of these is returned. */
dualar_status dualar_sync(dualar_ctx_t *ctx, int32_t *device_status);

/* Measurement: after dualar_profile_begin(ctx, class), every launch of that
 * kernel class on the context's stream is bracketed by a pair of hipEvents;
 * dualar_profile_end() synchronises the stream and returns the number of
 * launches, their summed event-to-event time (ms) and their summed
 * algorithmic HBM bytes (weights + activations read and written, caches
 * read and appended).  Classes: 0 matrix-vector (GEMV), 1 attention,
 * 2 sampler, 3 fusion, 4 the SwiGLU gate|up GEMV alone (W1, W3).  Profiling
 * adds a few microseconds per launch; do not time throughput with it on. */
typedef enum {
  DUALAR_K_GEMV = 0, DUALAR_K_ATTN = 1, DUALAR_K_SAMPLE = 2, DUALAR_K_EMBED = 3, DUALAR_K_GEMV_SWIGLU = 4
} dualar_kernel_class;
dualar_status dualar_profile_begin(dualar_ctx_t *ctx, int32_t kernel_class);
dualar_status dualar_profile_end(dualar_ctx_t *ctx, int64_t *launches, double *total_ms, double *bytes);

void dualar_destroy(dualar_ctx_t *ctx);

const char *dualar_status_string(dualar_status s);

/* Message of the last failing call on ctx (or of the last failing
 * dualar_create in this thread when ctx is NULL). */
const char *dualar_last_error(const dualar_ctx_t *ctx);

#ifdef __cplusplus
}
#endif
#endif /* DUALAR_H */
