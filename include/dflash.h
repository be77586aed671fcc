/*
 * dflash.h -- C ABI of the MI355X (gfx950) lossless block speculative-decoding step.
 *
 * Sources cited below by short key:
 *   [P1] "DFlash2 用投机解码给 Qwen 提速" (bml.asia)
 *   [P2] "你的大模型为啥突然快了，下一代投机解码 DFlash 拆给你看" (xiaodao.ai)
 *   [P3] "无损加速是真的吗？Qwen3.8-27B-DFlash2如何保证输出与目标模型完全一致" (rytg.cn)
 *
 * One step of the method ([P1] pseudocode; [P3] section "投机解码如何白嫖速度"):
 *   dflash_draft_block     the drafter fills a block [anchor, MASK x (B-1)] in one forward, after the
 *                          target hidden states of the positions committed by the previous step have
 *                          been projected into every drafter layer's KV cache (KV injection,
 *                          [P2] "DFlash 的第二招" and the SGLang paragraph of "但研究跑通").
 *   dflash_verify_block    the target runs the block once over its paged KV prefix ([P1] pseudocode step 2).
 *   dflash_accept_resample drafts are accepted in order with probability p(x); the first rejected
 *                          position is redrawn from the target distribution with x removed; a fully
 *                          accepted block adds a bonus token ([P1] step 3; [P3] "先说结论").
 *
 * Conventions
 *   - Every pointer named d_* is device memory; everything else is host memory.  The library never
 *     allocates or frees device memory: the caller provides the weights, both KV pools and one
 *     workspace, sized by the *_bytes functions, and keeps them alive until dflash_destroy.
 *   - Step calls only enqueue work on the given HIP stream (asynchronous, stream ordered) and never
 *     synchronise, except dflash_device_status.  A context is used from one thread and one stream
 *     at a time.
 *   - Arguments are checked on the host before anything is enqueued.  On error a call returns a
 *     negative status, enqueues nothing and changes no state; dflash_last_error() then describes it.
 *   - Conditions only the device can see (a token id outside [0, vocab), a position without a
 *     reserved KV page) are caught by bounds checks inside the kernels, which skip the access and
 *     raise a sticky flag; dflash_device_status reports it as DFLASH_E_DEVICE.
 *   - Weight layout: projections are row-major [out, in] (y = x W^T) in the model dtype (bf16, or
 *     fp32 for DFLASH_F32 models); RMSNorm gains are fp32 vectors.  Nothing is copied or repacked.
 *   - KV pool layout, per layer: [page][2 (K, V)][kv_heads][page_tokens * head_dim], K token-major
 *     ([token][dim]) and V dim-major ([dim][token]) inside a page, in IEEE fp16 for DFLASH_BF16 models
 *     (the attention operands keep 11 significant bits; K is RMS-normalised, |V| saturates at 65504)
 *     and fp32 for DFLASH_F32 models.  Page ids are shared by the target pool (layers 0..L_t-1) and the
 *     drafter pool (layers 0..L_d-1): a slot's block table maps its position p to page
 *     table[p / page_tokens] -- except for a windowed drafter's page ring (dflash_drafter_pool_bytes).
 *   - Activations of DFLASH_BF16 models that meet a weight matrix or the attention -- projection
 *     inputs, target features (verify output, draft input), q and the KV cache -- are IEEE fp16 (11
 *     significant bits where bf16 keeps 8; magnitudes saturate at 65504); the bf16 weights enter those
 *     products converted to fp16 (exactly for |w| in [2^-14, 65504]).  DFLASH_F32 models keep fp32.
 */
#ifndef DFLASH_H
#define DFLASH_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DFLASH_MAX_TAPS 16
#define DFLASH_MAX_BATCH 64
#define DFLASH_MAX_BLOCK 16
#define DFLASH_MAX_TOPK 256
/* Calls of DFLASH_BF16 models over at least this many rows run their projections on the tiled MFMA kernel
 * (dflash_op_linear_f16x) and apply every RMSNorm at once; smaller calls stream the weights through the
 * row-chunked kernels (dflash_op_linear) with the norms deferred into the next projection. */
#define DFLASH_F16_MIN_ROWS 32

typedef enum {
  DFLASH_OK = 0,
  DFLASH_E_INVAL = -1,  /* bad argument or unsupported shape */
  DFLASH_E_NOMEM = -2,  /* KV page pool exhausted (other slots unaffected) */
  DFLASH_E_DEVICE = -3, /* HIP error, or a device-side bounds check fired */
  DFLASH_E_STATE = -4   /* call out of order for this slot */
} dflash_status;

typedef enum { DFLASH_BF16 = 0, DFLASH_F32 = 1 } dflash_dtype;

/* A Qwen3-like pre-norm decoder ([P3] "结构一览": the drafter is Qwen3-structured; the target is the
 * Qwen3-family model it serves): RMSNorm (eps), grouped-query attention with per-head q/k RMSNorm and
 * rotate-half RoPE (rope_theta), SwiGLU feed-forward of width ffn, no biases. */
typedef struct {
  int32_t layers, hidden, q_heads, kv_heads, head_dim, ffn, vocab;
  float rope_theta, rms_eps;
  int32_t dtype; /* dflash_dtype */
} dflash_model_cfg;

/* The drafter: `layers` layers of the target's shape; the residual streams after target layers
 * taps[0..n_taps-1] are injected ([P3] "结构一览", target_layer_ids); block_size B positions per
 * draft, the first being the anchor and the rest mask_id ([P3] "DFlash 2 的三个设计"); context keys
 * limited to a sliding window of `window` tokens (0 = unbounded; [P3] "结构一览").  The drafter
 * uses the target's embedding table and LM head.
 * DFlash2 variants ([P3] "DFlash 2 的三个设计", configuration values only; 0 switches each off):
 *   conv_kernel (1..4) taps of a dynamic convolution along the block applied to every drafter layer's
 *     normed attention input before its q/k/v projections: y_i[c] = sum_{t < taps, i - t >= 0}
 *     a_i[c / conv_group][t] x_{i-t}[c] with a_i[g][.] = softmax over t of (W_conv x_i)[g * taps + t]
 *     (W_conv: dflash_layer_weights.w_conv, [conv_kernel * hidden / conv_group, hidden]);
 *   selector_top_k (1..32) candidates per draft position (logit desc, id asc) and the draft path
 *     through them maximising sum_i z_i + (U E[t_{i-1}]) . (V E[t_i]) / sqrt(selector_rank) from the
 *     anchor t_0 (Viterbi in fp32; ties to the lowest candidate index; U, V: dflash_drafter_weights
 *     sel_u, sel_v [selector_rank, hidden], selector_rank a multiple of 32 up to 512; E the embedding
 *     table).  Not with stochastic drafts. */
typedef struct {
  int32_t layers;
  int32_t n_taps;
  int32_t taps[DFLASH_MAX_TAPS];
  int32_t block_size, mask_id, window;
  int32_t conv_kernel, conv_group;
  int32_t selector_top_k, selector_rank;
} dflash_drafter_cfg;

/* One decoder layer: device pointers, borrowed. */
typedef struct {
  const void *attn_norm; /* fp32 [hidden] */
  const void *wq;        /* [q_heads*head_dim, hidden] */
  const void *wk;        /* [kv_heads*head_dim, hidden] */
  const void *wv;        /* [kv_heads*head_dim, hidden] */
  const void *q_norm;    /* fp32 [head_dim] */
  const void *k_norm;    /* fp32 [head_dim] */
  const void *wo;        /* [hidden, q_heads*head_dim] */
  const void *ffn_norm;  /* fp32 [hidden] */
  const void *w_gate;    /* [ffn, hidden] */
  const void *w_up;      /* [ffn, hidden] */
  const void *w_down;    /* [hidden, ffn] */
  const void *w_conv;    /* drafter layers with conv_kernel > 0: [conv_kernel*hidden/conv_group, hidden]; else null */
} dflash_layer_weights;

typedef struct {
  const void *embed;                  /* [vocab, hidden] */
  const void *final_norm;             /* fp32 [hidden] */
  const void *lm_head;                /* [vocab, hidden] */
  const dflash_layer_weights *layers; /* host array [layers] */
} dflash_target_weights;

typedef struct {
  const void *fc;                     /* [hidden, n_taps*hidden] */
  const void *hidden_norm;            /* fp32 [hidden] */
  const void *final_norm;             /* fp32 [hidden] */
  const dflash_layer_weights *layers; /* host array [layers] (wq..w_down as for the target) */
  const void *sel_u, *sel_v;          /* selector_top_k > 0: [selector_rank, hidden] each; else null */
} dflash_drafter_weights;

/* Per-request sampling ([P1] model-card paragraph; [P3] "实测数据": temperature 1.0, top-p 0.95,
 * top-k 20).  temperature 0 = greedy (argmax, lowest id on ties).  1 <= top_k <= DFLASH_MAX_TOPK
 * when temperature > 0.  top_p in (0, 1]; 1 disables the nucleus cut.  Uniforms come from
 * Philox4x64-10 with key (seed, 0) and counter (position, slot, 0, 0). */
typedef struct {
  float temperature;
  int32_t top_k;
  float top_p;
  uint64_t seed;
} dflash_sampling;

/* Capacity fixed at creation. */
typedef struct {
  int32_t max_slots;         /* sequences that may hold KV pages at once, <= DFLASH_MAX_BATCH */
  int32_t max_rows;          /* max batch * q_len of any call (prefill included) */
  int32_t page_tokens;       /* tokens per KV page (16) */
  int32_t num_pages;         /* pages in each pool */
  int32_t max_pages_per_seq; /* block-table width */
} dflash_capacity;

typedef struct dflash_ctx dflash_ctx;

/* Bytes of one KV pool holding `pages` pages for `layers` layers. */
size_t dflash_kv_pool_bytes(const dflash_model_cfg *cfg, int32_t layers, const dflash_capacity *cap);

/* Bytes of the drafter's KV pool (0 if an argument is NULL or dcfg->layers < 1).  With a window W
 * ([P3] "结构一览") the drafter never reads keys more than W positions behind a block, so each slot
 * recycles a ring of R = ceil((W + 2 B) / page_tokens) + 1 pages (page index i of a slot lives in ring
 * page slot * R + i mod R): dcfg->layers * max_slots * R pages.  Without a window, or when that is not
 * smaller than num_pages (or R >= max_pages_per_seq), it is dflash_kv_pool_bytes(cfg, dcfg->layers,
 * cap) and the drafter uses the target's page ids.  With the ring, dflash_draft_block must follow a
 * dflash_accept_resample of at most (page_tokens * R - W) / 2 drafts (at least B + 8), else it returns
 * DFLASH_E_STATE: one draft touches up to W + nd + max(B, nd) consecutive positions after an accept of
 * nd drafts. */
size_t dflash_drafter_pool_bytes(const dflash_model_cfg *cfg, const dflash_drafter_cfg *dcfg,
                                 const dflash_capacity *cap);

/* Bytes of the workspace for this model, drafter and capacity (0 if the arguments are invalid). */
size_t dflash_workspace_bytes(const dflash_model_cfg *cfg, const dflash_drafter_cfg *dcfg,
                              const dflash_capacity *cap);

/* Create a context.  Pointers are borrowed.  d_target_kv must hold dflash_kv_pool_bytes(cfg,
 * cfg->layers, cap) bytes, d_drafter_kv dflash_drafter_pool_bytes(cfg, dcfg, cap) bytes and
 * d_workspace dflash_workspace_bytes(...) bytes, 256-byte aligned.  Zero-fills both KV pools and the
 * workspace's state on `stream` and waits for it (unwritten key slots of a page take part in the
 * attention product with zero weight, which is exact only for finite contents). */
dflash_status dflash_create(const dflash_model_cfg *cfg, const dflash_drafter_cfg *dcfg,
                            const dflash_target_weights *tw, const dflash_drafter_weights *dw,
                            const dflash_capacity *cap, void *d_target_kv, void *d_drafter_kv,
                            void *d_workspace, hipStream_t stream, dflash_ctx **out);
dflash_status dflash_destroy(dflash_ctx *ctx);

/* Reserve pages so that `slot` can hold positions 0 .. n_tokens-1 in both caches (host page table;
 * the device mirror is updated with a synchronous copy of the new entries only, which running
 * kernels never read).  DFLASH_E_NOMEM leaves the slot as it was. */
dflash_status dflash_kv_alloc(dflash_ctx *ctx, int32_t slot, int32_t n_tokens);
/* Return all pages of `slot` to the pool.  The slot must be re-prefilled before it is used again. */
dflash_status dflash_kv_free(dflash_ctx *ctx, int32_t slot);

/* Target forward over a block ([P1] pseudocode step 2: one forward whatever the block length, the
 * prefix coming from the KV cache).  For each request b (slot slots[b]) the tokens
 * d_tokens[b*q_len .. +q_len) sit at positions start .. start+q_len-1 where start is 0 when
 * new_sequence != 0 (prefill) and the slot's committed length otherwise.  Query at position p attends
 * to keys 0 .. p.  The block's K/V are written into the target cache (positions past the committed
 * length are overwritten by later blocks; rollback is a length update).
 * Outputs: d_logits fp32 [batch][n_logit_rows][vocab] for the last n_logit_rows rows of each block;
 * d_feats: the residual stream after each tapped layer, for KV injection by the next
 * dflash_draft_block -- [batch][q_len][n_taps][hidden], fp16 for DFLASH_BF16 models and fp32 for
 * DFLASH_F32 models. */
dflash_status dflash_verify_block(dflash_ctx *ctx, hipStream_t stream, int32_t batch, const int32_t *slots,
                                  const int32_t *d_tokens, int32_t q_len, int32_t new_sequence,
                                  int32_t n_logit_rows, float *d_logits, void *d_feats);

/* Accept / resample one verified block per request ([P1] step 3; [P3] "先说结论" and
 * "投机解码如何白嫖速度").  d_logits as written by dflash_verify_block with n_logit_rows = n_draft+1;
 * d_block[b*(n_draft+1) + i] (i = 1 .. n_draft) is the draft for the i-th position after the anchor,
 * i.e. d_block is the verified block as produced by dflash_draft_block (NULL when n_draft is 0, as
 * after a prefill).  sampling is a host array [batch].
 * Emits tau in 1 .. n_draft+1 tokens per request into d_out[b*(n_draft+1) ..] (the rest set to -1)
 * and tau into d_n_out[b]; commits the anchor and the accepted drafts to both caches' lengths; the
 * last emitted token becomes the new anchor.  Any drafts may be passed (a planted drafter needs no
 * other entry point).  d_cand_ids / d_cand_p (may be NULL): [batch][n_draft+1][DFLASH_MAX_TOPK]
 * candidate ids and fp32 probabilities in sorted order, -1 / 0 past the kept ones (test access to
 * the filter). */
dflash_status dflash_accept_resample(dflash_ctx *ctx, hipStream_t stream, int32_t batch, const int32_t *slots,
                                     const float *d_logits, const int32_t *d_block, int32_t n_draft,
                                     const dflash_sampling *sampling, int32_t *d_out, int32_t *d_n_out,
                                     int32_t *d_cand_ids, float *d_cand_p);

/* Drafter forward ([P2] "DFlash 的第一招"/"第二招"; [P3] "DFlash 2 的三个设计").  First injects, for each
 * request, the target features of the positions committed by the last dflash_accept_resample
 * (read from d_feats as written by the preceding dflash_verify_block for the same slots in the same
 * order): c = RMSNorm(W_fc [h_tap1..h_tapm]), then every drafter layer's K = RoPE(k_norm(W_k c)) and
 * V = W_v c go into the drafter cache.  With a window W, rows that no later draft can see (those more
 * than W + n_draft before the end of a long verified block, i.e. of a prefill) are not injected.  Then
 * runs the block [anchor, MASK x (B-1)] at positions
 * n .. n+B-1 (n = committed length): block queries see all block keys and the injected context keys
 * within the window.  Writes the block to verify, d_block [batch][B] = [anchor, d_1 .. d_{B-1}], where
 * d_i is the argmax (lowest id on ties) of the drafter's fp32 logits at position n+i.  Optionally
 * (d_logits != NULL) also writes those logits, fp32 [batch][B-1][vocab]. */
dflash_status dflash_draft_block(dflash_ctx *ctx, hipStream_t stream, int32_t batch, const int32_t *slots,
                                 const void *d_feats, int32_t *d_block, float *d_logits);

/* Stochastic drafts (the general rejection-sampling rule behind [P1]'s cost-model sentence on
 * rejection sampling; a reading where the pages are silent: drafts drawn from the drafter's own
 * distribution instead of its argmax).  As dflash_draft_block, except that d_i is drawn from q_i, the drafter's fp32 logits at
 * position n+i passed through the same filter as the target's rows with the request's sampling
 * (temperature 0: a point mass at the argmax), by inverse CDF with u = top 24 bits of word 0 of
 * Philox4x64-10 with key (seed, 0) and counter (n+i, slot, 1, 0) (stream 1; dflash_accept_resample uses
 * stream 0).  sampling is a host array [batch].  q_i's candidates go to d_q_ids / d_q_p
 * [batch][B-1][DFLASH_MAX_TOPK] (sorted as the filter sorts them, ids -1 / probabilities 0 past the kept
 * ones), caller-allocated; pass them to dflash_accept_resample_q.  d_logits as in dflash_draft_block. */
dflash_status dflash_draft_block_sampled(dflash_ctx *ctx, hipStream_t stream, int32_t batch, const int32_t *slots,
                                         const void *d_feats, const dflash_sampling *sampling, int32_t *d_block,
                                         int32_t *d_q_ids, float *d_q_p, float *d_logits);

/* Test access to the selector of the last dflash_draft_block call (selector_top_k > 0): the candidate
 * ids [batch][B-1][K] and their logits, and the transitions [batch][B-1][K][K] (entry [b][i][k'][k]:
 * from candidate k' of draft row i-1 -- the anchor, k' = 0, for i = 0 -- to candidate k of row i) in
 * fp32, copied on `stream` into device buffers of the caller. */
dflash_status dflash_selector_state(dflash_ctx *ctx, hipStream_t stream, int32_t batch, int32_t *d_cand_ids,
                                    float *d_cand_logits, float *d_trans);

/* Accept / resample for drafts drawn from known distributions q (d_q_ids / d_q_p as written by
 * dflash_draft_block_sampled, or any caller-built rows in that layout whose q(d_i) > 0): draft d at
 * position t is accepted iff u_acc(t) * q(d) < p(d) in fp32, i.e. with probability min(1, p(d)/q(d));
 * at the first rejection the token is drawn by inverse CDF (u_smp(t)) from max(0, p - q) over p's
 * candidates in their order, renormalised (from p itself should that residual be all zero).  The
 * output law of every position is then p, whatever q is.  Everything else (uniforms, bonus token,
 * commit, outputs, errors) as dflash_accept_resample, which is the case of q a point mass at the draft
 * (the same decisions bit for bit).  d_q_ids / d_q_p may be NULL only when n_draft is 0. */
dflash_status dflash_accept_resample_q(dflash_ctx *ctx, hipStream_t stream, int32_t batch, const int32_t *slots,
                                       const float *d_logits, const int32_t *d_block, int32_t n_draft,
                                       const dflash_sampling *sampling, const int32_t *d_q_ids, const float *d_q_p,
                                       int32_t *d_out, int32_t *d_n_out, int32_t *d_cand_ids, float *d_cand_p);

/* Operator-level access to the projection kernel used by every step (test and measurement access):
 * d_y[m][n] = sum_k d_x[m][k] * d_w[n][k] (fp32 output) for m < M, with d_w [N][K] in `dtype`
 * (dflash_dtype) and d_x [M][K] in the model's activation type (fp16 for DFLASH_BF16, fp32 for
 * DFLASH_F32), on the row-chunked kernels of the model's projections.  N must be a multiple of 16 and K
 * of 32 (bf16) or 16 (fp32).  Asynchronous on `stream`; needs no context. */
dflash_status dflash_op_linear(hipStream_t stream, int32_t dtype, int32_t M, int32_t N, int32_t K, const void *d_x,
                               const void *d_w, float *d_y);

/* The projection kernel of calls over many rows (decode batches of 32 or more rows, prefill) on its
 * own: d_y = d_x d_w^T with d_x [M][K] in fp16, d_w [N][K] in bf16 (converted to fp16 inside the
 * kernel, exactly for |w| in [2^-14, 65504]), fp32 accumulation on the matrix cores.  M >= 1,
 * N a multiple of 32, K a multiple of 64.  The launch may cut K into up to max_ranges ranges (1 <=
 * max_ranges <= 8): range z writes its fp32 sums to d_y + z * M * N (d_y holds max_ranges * M * N
 * floats) and *ranges (host memory; may be null when max_ranges is 1) receives the count; the product
 * is the sum of the ranges in order.  Asynchronous on `stream`; needs no context. */
dflash_status dflash_op_linear_f16x(hipStream_t stream, int32_t M, int32_t N, int32_t K, const void *d_x,
                                    const void *d_w, float *d_y, int32_t max_ranges, int32_t *ranges);

/* The same product on the stream-K projection kernel that the step uses for its residual and SwiGLU
 * projections (operator-level test and measurement access): the (16-or-32-column tile, 256-byte K
 * window) items of the product are cut into equal ranges, one work-group per compute unit, and a tile
 * shared by several work-groups is finished by the last to arrive.  1 <= M <= 16, N a multiple of 32,
 * K a multiple of 128 (bf16) or 64 (fp32); d_x [M][K], d_w [N][K], d_y [M][N] fp32 as for
 * dflash_op_linear.  d_scratch: caller device memory of dflash_op_linear_sk_scratch_bytes(N) bytes,
 * 256-byte aligned (partial tiles and per-tile arrival counters; the call zeroes the counters on
 * `stream` before its launch, so its contents need no preparation); calls that overlap on one
 * scratch block race.  Asynchronous on `stream`; needs no context. */
size_t dflash_op_linear_sk_scratch_bytes(int32_t N); /* 0 if N is not a positive multiple of 32 */
dflash_status dflash_op_linear_sk(hipStream_t stream, int32_t dtype, int32_t M, int32_t N, int32_t K,
                                  const void *d_x, const void *d_w, float *d_y, void *d_scratch,
                                  size_t scratch_bytes);

/* dflash_op_linear_sk for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the same kernel and result bit for bit, with
 * the scratch in a static device array of the library (4.2 MB, held by each GPU the library runs on
 * until the process ends) instead of caller memory.  N must not exceed 131072 (DFLASH_E_INVAL); other
 * arguments and errors as dflash_op_linear_sk.  The call allocates nothing.  Every call on one GPU
 * shares that GPU's array (the call clears its counters before launching): calls that overlap on one
 * GPU race. */
dflash_status dflash_op_linear_sk_noalloc(hipStream_t stream, int32_t dtype, int32_t M, int32_t N, int32_t K,
                                          const void *d_x, const void *d_w, float *d_y);

/* Measurement access.  While profiling is enabled, the library records the projection launches
 * (kernel, shape and pointers) issued by the step calls.  dflash_profile_replay, called with
 * profiling disabled, re-issues exactly those launches `iters` times back to back on `stream`
 * (the optional feature-tap side output is suppressed; every other buffer they write is workspace
 * scratch), bracketed by one pair of HIP events, and returns the elapsed ms, the algorithmic weight
 * bytes of one pass over the recorded launches (every weight once per projection) and the number of
 * recorded projections.  Enabling clears the record. */
dflash_status dflash_profile(dflash_ctx *ctx, int32_t enable);
dflash_status dflash_profile_replay(dflash_ctx *ctx, hipStream_t stream, int32_t iters, double *ms, double *bytes,
                                    int32_t *launches);

/* Synchronise `stream` and report device-side errors raised since the last call (sticky flags). */
dflash_status dflash_device_status(dflash_ctx *ctx, hipStream_t stream);

/* Message of the last failed call on this thread ("" if none). */
const char *dflash_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* DFLASH_H */
