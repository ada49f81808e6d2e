/*
 * dllm.h: C ABI of the MI355X (gfx950) library for cached block-wise
 * masked-diffusion LLM decoding.
 *
 * The method (Fast-dLLM v1, training-free): the generated region is split into
 * blocks that are denoised left to right; in each step every still-masked
 * position of the current block gets the softmax of the model's logits, and
 * every position whose top probability clears the threshold is committed at
 * once, never to be revised; K/V of positions outside the recomputed rows are
 * reused from a cache that is refreshed only when a block starts.
 *   - Fast-dLLM README, track table ("KV Cache + Parallel Decoding") and Quick
 *     Start (knobs --gen_length --steps --block_size; Dream command
 *     alg=confidence_threshold, threshold=0.9, use_cache=true).
 *   - "Fast-dLLM: Four Acceleration Tracks ...", sections "The v1 Mechanism"
 *     and "Fast-dLLM v1 Versus a Standard Diffusion Sampler".
 *   - Streaming-dLLM README, throughput tables: "Prefix-Cache" and
 *     "Fast-dLLM" columns against the no-cache backbones.
 *
 * Conventions for every function below
 *   - Return 0 on success or a negative DLLM_E* code; dllm_last_error() gives
 *     a message.  No C++ exception crosses this boundary.
 *   - Device pointers are HIP device addresses on the current device; "host"
 *     arguments are ordinary host memory.
 *   - All device work is enqueued on cfg.stream (a hipStream_t; NULL = the
 *     null stream).  Calls that read or write host arrays synchronise that
 *     stream before returning; dllm_block_begin does not.
 *   - One host thread at a time per handle.  Several handles may share the
 *     same weights read-only.
 *   - Environment: DLLM_DEBUG_SYNC=1 synchronises the stream after every HIP
 *     call of the library, so an asynchronous failure is reported (as DLLM_EHIP)
 *     by the call that caused it.
 *   - The library allocates no device memory: the caller passes the weights
 *     and one workspace of dllm_workspace_bytes() bytes, owns both, and must
 *     keep both alive until dllm_destroy.  The handle owns host state only.
 */
#ifndef DLLM_H
#define DLLM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Error codes. */
#define DLLM_OK 0
#define DLLM_EINVAL -1     /* bad argument or configuration */
#define DLLM_ENOSPACE -2   /* workspace smaller than dllm_workspace_bytes() */
#define DLLM_ESTATE -3     /* call out of order (e.g. a step before prefill) */
#define DLLM_EHIP -4       /* a HIP runtime call failed; the message names it */
#define DLLM_EINTERNAL -5  /* unexpected internal failure */

/* Storage type of weights and KV cache. */
#define DLLM_F32 0
#define DLLM_BF16 1

/* Attention pattern (attention). */
#define DLLM_ATTN_FULL 0         /* bidirectional over the whole context (v1)          */
#define DLLM_ATTN_BLOCK_CAUSAL 1 /* a query sees its own block and the ones before it   */

/* Cache policy (use_cache). */
#define DLLM_NO_CACHE 0     /* every step is a full forward                      */
#define DLLM_PREFIX_CACHE 1 /* steps recompute the block and every later row      */
#define DLLM_DUAL_CACHE 2   /* steps recompute the block rows only                */

/*
 * Model shape and decode knobs.
 *   Shape: an LLaDA/Dream-style bidirectional transformer (Fast-dLLM README
 *   track table, backbones Dream and LLaDA): pre-norm RMSNorm, rotary positions
 *   (rotate-half form), attention with n_heads query heads over n_kv_heads K/V
 *   heads (n_heads % n_kv_heads == 0), SwiGLU feed-forward, untied embedding
 *   and lm_head, no biases.  Constraints: head_dim in {32, 64, 128};
 *   d_model a multiple of 64 and at most 8192; for DLLM_BF16, n_heads*head_dim
 *   and ffn_dim are multiples of 64.
 *   mask_id < vocab is the mask token; it is excluded from every softmax.
 *   logit_scale multiplies the lm_head output before the softmax.
 *   Knobs (Fast-dLLM README, Quick Start): gen_length is a multiple of
 *   block_size; steps (0 = gen_length) is the diffusion step budget, a multiple
 *   of gen_length/block_size, and sets the per-step commit floor (the block's
 *   positions spread evenly over its steps/n_blocks steps; 1 per step by
 *   default); threshold: a masked position commits when its confidence (top
 *   softmax probability) is strictly greater; use_cache: DLLM_*_CACHE.
 *   block_size <= 256.  refresh_every_step != 0 refreshes the whole cache at
 *   every step (a test hook: it must reproduce no-cache decoding).
 *   suffix_window >= 0 turns on approximate suffix pruning (Streaming-dLLM
 *   README, figure caption on approximated suffix pruning): while block [s, e)
 *   is decoded the model sees only positions [0, e + suffix_window) and the
 *   last position, each at its own rotary position, for the block's refresh
 *   and its steps; the other suffix positions are absent.  < 0: whole context.
 *   attention = DLLM_ATTN_BLOCK_CAUSAL (block diffusion: Fast-dLLM README track
 *   table, v2 "Block Diffusion"; Streaming-dLLM README, note on block-causal
 *   models): the prompt is one block, then blocks of block_size; a query sees
 *   its own block and every earlier one.  Finished blocks' K/V are final, so the
 *   refresh at block b recomputes only blocks b-1 (the prompt for b = 0) and b,
 *   and use_cache / suffix_window change nothing.
 *   exit_steps N > 0 turns on early exit for converged tokens (ES-dLLM paper
 *   card, Streaming-dLLM abstract: a dynamic confidence-aware strategy with an
 *   early exit mechanism): a masked position's run counts the consecutive steps
 *   of the block, up to this one, in which its argmax stayed the same with a
 *   confidence strictly above exit_floor; after a step's commit, when every
 *   position of a batch row that is still masked has a run of at least N, all
 *   of them are committed with their argmax and the row's block ends.
 *   first_threshold t1 >= 0 turns on first-step confidence scheduling (ES-dLLM
 *   paper card, CAI-DLLM abstract): a block's first step commits with threshold
 *   t1 (the easy tokens go at once); the positions still masked after it (the
 *   hard ones) are spread over the block's remaining steps/n_blocks - 1 steps of
 *   the budget, which sets the floor of each later step, per batch row.
 *   All batch rows share prompt_len and advance block by block together.
 */
typedef struct dllm_cfg {
  int32_t n_layers, d_model, n_heads, n_kv_heads, head_dim, ffn_dim, vocab, mask_id;
  float rms_eps, rope_base, logit_scale;
  int32_t dtype; /* DLLM_F32 | DLLM_BF16 */
  int32_t batch, prompt_len, gen_length, block_size;
  int32_t steps;
  float threshold;
  int32_t use_cache;
  int32_t refresh_every_step;
  int32_t suffix_window;
  int32_t attention; /* DLLM_ATTN_* */
  int32_t exit_steps;    /* early exit for converged tokens (0: off)                   */
  float exit_floor;      /* ... confidence a converged token stays above               */
  float first_threshold; /* first-step confidence scheduling (< 0: off)                */
  void *stream;      /* hipStream_t */
} dllm_cfg;

/*
 * Device pointers to the weights, in cfg.dtype, torch Linear layout
 * [out_features, in_features], row-major, contiguous:
 *   embed [vocab, d_model], final_norm [d_model], lm_head [vocab, d_model];
 *   layer[9*l + j] for layer l, j in order:
 *     0 attn_norm [d_model]            1 wq [n_heads*head_dim, d_model]
 *     2 wk [n_kv_heads*head_dim, d_model]  3 wv [n_kv_heads*head_dim, d_model]
 *     4 wo [d_model, n_heads*head_dim]  5 ffn_norm [d_model]
 *     6 w_gate [ffn_dim, d_model]       7 w_up [ffn_dim, d_model]
 *     8 w_down [d_model, ffn_dim]
 * Device pointers must be 16-byte aligned.  The array `layer` itself is host
 * memory and is copied by dllm_create.
 */
typedef struct dllm_weights {
  const void *embed, *final_norm, *lm_head;
  const void *const *layer; /* host array of 9*n_layers device pointers */
} dllm_weights;

/*
 * Counters of a handle since the last dllm_prefill (dllm_generate starts with one), or since
 * dllm_create when there has been none.  The two times are GPU time on cfg.stream, measured with
 * HIP events around the work each call enqueues: a refresh (dllm_block_begin is asynchronous) is
 * booked once it has completed, at the next call that synchronises.
 */
typedef struct dllm_stats {
  int64_t steps;            /* denoising steps taken                         */
  int64_t full_forwards;    /* refresh / no-cache forwards                   */
  int64_t cached_forwards;  /* cached-step forwards                          */
  int64_t committed;        /* tokens committed (all batch rows)             */
  int64_t commits_hist[9];  /* steps by tokens committed per row per step:
                               [0]=0, [1]=1, [2]=2, [3]=3-4, [4]=5-8, [5]=9-16,
                               [6]=17-32, [7]=33-64, [8]=65+                 */
  double ms_refresh;        /* GPU time of the block refreshes (ms)          */
  double ms_step;           /* GPU time of the denoise steps' own work (ms):
                               cached forwards, statistics and commits       */
  int64_t nan_count;        /* masked positions whose confidence was NaN
                               (ranked last by the commit; should stay 0)    */
  int64_t early_exits;      /* (batch row, step) pairs that ended a block by
                               the early exit (exit_steps > 0)               */
} dllm_stats;

typedef struct dllm_handle dllm_t;

/* Check a configuration without touching the GPU.  Host only. */
int dllm_validate_cfg(const dllm_cfg *cfg);

/* Workspace bytes that a handle for cfg needs.  Host only.  EINVAL for a bad cfg. */
int dllm_workspace_bytes(const dllm_cfg *cfg, size_t *bytes);

/*
 * Create a handle.  `workspace` is caller-owned device memory of ws_bytes
 * (>= dllm_workspace_bytes, 256-byte aligned); it holds the token state, the
 * KV cache (n_layers x batch x n_kv_heads x (prompt_len+gen_length) x head_dim
 * for K and V, 4 bytes per element: fp32, or a bf16 hi and a bf16 lo plane),
 * all intermediate buffers and, for DLLM_BF16, a packed copy of every linear
 * weight (q/k/v, o, gate/up, down, lm_head): rows grouped into 128-row panels
 * of 32-column blocks, so that a GEMM's weight tile is a few contiguous runs.
 * dllm_create packs them; afterwards the linear weights are read only from the
 * copy (embed and the norm gains are still read from the caller's pointers).
 * Initialises the workspace on cfg.stream and synchronises it.
 */
int dllm_create(const dllm_weights *w, const dllm_cfg *cfg, void *workspace, size_t ws_bytes,
                dllm_t **out);

/*
 * For callers that cannot allocate device memory while they run (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the same handle as dllm_create, except
 * that its scratch (split-K partial tiles, attention key-chunk partials, lm_head tile partials:
 * values that live only within one call's launches) is a static device array of the library,
 * DLLM_STATIC_SCRATCH_BYTES bytes on each GPU it runs on, held until the process ends, and no
 * longer part of the workspace.  The function itself allocates nothing.
 *   - workspace == NULL: host-only size query; *ws_bytes receives the workspace bytes this
 *     variant needs (dllm_workspace_bytes(cfg) less the scratch region).  w and out unused.
 *   - otherwise: as dllm_create with *ws_bytes as the workspace size.  The scratch address is
 *     that of the device current at this call; every call on the handle must run there.
 *   - DLLM_ENOSPACE (query or create) when cfg's scratch exceeds DLLM_STATIC_SCRATCH_BYTES;
 *     DLLM_EINVAL when ws_bytes is NULL or as for dllm_create.
 * All handles of this kind on one GPU share the array, which keeps whatever the last call wrote
 * (nothing in it needs to start at zero): calls on two such handles must not overlap in time
 * (different streams or host threads race).  Handles made by dllm_create are unaffected.
 */
#define DLLM_STATIC_SCRATCH_BYTES ((size_t)256 << 20)
int dllm_create_static_scratch(const dllm_weights *w, const dllm_cfg *cfg, void *workspace,
                               size_t *ws_bytes, dllm_t **out);

/*
 * Start of a decode: x = [prompt | mask_id x gen_length] for every batch row
 * (the whole generated region starts masked: Fast-dLLM README, Quick Start,
 * --gen_length), then the refresh of block 0 (full forward over all positions,
 * every cache slot written; its block-row statistics serve the block's first
 * step, "Fast-dLLM: Four Acceleration Tracks ...", section "The v1 Mechanism").
 * Resets the dllm_stats counters.  prompt: host int32 [batch, prompt_len], ids
 * in [0, vocab).  Synchronises.
 */
int dllm_prefill(dllm_t *h, const int32_t *prompt);

/*
 * Block-boundary refresh (Fast-dLLM v1: the cache is refreshed when a block
 * starts): full forward of all rows of every batch row on the current token
 * state; all K/V cache slots are rewritten; the block's first-step statistics
 * are kept for the next dllm_denoise_step.  0 <= block < gen_length/block_size.
 * Asynchronous.  ESTATE before dllm_prefill or dllm_set_tokens.
 */
int dllm_block_begin(dllm_t *h, int32_t block);

/*
 * One denoising step of the current block ("Fast-dLLM: Four Acceleration
 * Tracks ...", section "The v1 Mechanism": confident positions are committed in
 * parallel and never revised; section "Fast-dLLM v1 Versus a Standard Diffusion
 * Sampler": the conventional schedule stays as the floor).  The statistics come
 * from the refresh on the block's first step, otherwise from a cached forward:
 * block rows for the dual cache, block and later rows for the prefix cache, all
 * rows with no cache (Streaming-dLLM README tables, "Prefix-Cache" and
 * "Fast-dLLM" columns).  Then the commit: in every batch row, each masked block
 * position with confidence > threshold, plus at least the floor's number of
 * most confident ones (ties: lower position), gets its argmax token.
 * n_committed: host int32 [batch] or NULL; block_done: host int32 or NULL,
 * set to 1 when no batch row has a masked position left in the block.
 * Synchronises (one small device-to-host copy).
 */
int dllm_denoise_step(dllm_t *h, int32_t *n_committed, int32_t *block_done);

/*
 * Whole decode (Fast-dLLM README, Quick Start: gen_length tokens in blocks of
 * block_size, decoded left to right; ES-dLLM paper card, Streaming-dLLM
 * abstract: block-wise diffusion): prefill, then every block in order
 * (block_begin for b > 0, steps until the block is done).  out: host int32
 * [batch, prompt_len + gen_length] or NULL; stats: host or NULL (counters of
 * this call).  Fails with EINTERNAL if the steps exceed gen_length + the number
 * of blocks (every step commits at least one position, so this never happens).
 */
int dllm_generate(dllm_t *h, const int32_t *prompt, int32_t *out, dllm_stats *stats);

/* Token state [batch, prompt_len + gen_length] to host.  Synchronises. */
int dllm_get_tokens(dllm_t *h, int32_t *x);

/*
 * Overwrite the token state from host (teacher forcing, resume).  The cache
 * and the current block are left as they are; call dllm_block_begin to
 * refresh the cache from the new state.  Ids must be in [0, vocab).
 */
int dllm_set_tokens(dllm_t *h, const int32_t *x);

/*
 * Statistics of the last step's forward and its commit, host arrays
 * [batch, block_size] each (any may be NULL): argmax token, confidence (top
 * probability), runner-up probability, and 1 where the position was committed
 * by that step.  Synchronises.
 */
int dllm_get_step_info(dllm_t *h, int32_t *tok, float *conf, float *p2, uint8_t *committed);

/*
 * Test aid, never used by the decode: write the scaled logits of the block rows
 * of the last forward (mask id = -inf) to a caller-owned DEVICE buffer of
 * batch*block_size*vocab floats, row-major.  Synchronises.
 */
int dllm_debug_block_logits(dllm_t *h, float *logits_dev);

/* Counters since the last dllm_prefill (see dllm_stats).  Waits for a refresh in flight. */
int dllm_get_stats(dllm_t *h, dllm_stats *stats);

/* Device-side phase of the handle for tests: current block, step index in it. */
int dllm_get_position(dllm_t *h, int32_t *block, int32_t *step);

/*
 * Per-kernel-class timing, a measurement aid.  While enabled, every launch of a selected class
 * is bracketed by HIP events on cfg.stream; durations are collected at the next synchronising
 * call together with each launch's algorithmic work: bytes = every weight, activation and
 * output element the launch must read or write once; flops = 2*M*N*K for a GEMM and
 * 4*queries*keys*head_dim for attention.  Classes:
 */
#define DLLM_KC_GEMM_SKINNY 0 /* weight-streaming GEMM, <= 64 rows (cached steps, lm_head)     */
#define DLLM_KC_GEMM_TILED 1  /* tiled MFMA GEMM, > 64 rows (block refresh, no-cache forward)   */
#define DLLM_KC_ATTENTION 2   /* attention (with its split merge)                               */
#define DLLM_KC_COUNT 3
typedef struct dllm_kernel_prof {
  int64_t launches;
  double ms;     /* summed event-measured duration */
  double bytes;  /* summed algorithmic bytes       */
  double flops;  /* summed algorithmic flops       */
} dllm_kernel_prof;

/* Enable (mask bit 1 << class) or disable (0) timing, and clear the counters. */
int dllm_set_profiling(dllm_t *h, int class_mask);

/* Counters per class since dllm_set_profiling; out: host array of DLLM_KC_COUNT.  Synchronises. */
int dllm_get_profile(dllm_t *h, dllm_kernel_prof *out);

/* Message of the last error on h (or of the last failed dllm_create when h is NULL). */
const char *dllm_last_error(const dllm_t *h);

/* Free the handle's host state.  Does not touch the weights or the workspace. */
void dllm_destroy(dllm_t *h);

#ifdef __cplusplus
}
#endif
#endif /* DLLM_H */
