/*
 * gpt.h -- C ABI of the MI355X (gfx950) decoder-block forward library, libgpt.so.
 *
 * The library runs the forward pass of the nanochat-style GPT decoder block as
 * a full-sequence prefill and as a KV-cache decode step, ending in the LM-head
 * logits, the vocabulary softmax and token selection.  Every step runs in
 * hand-written HIP kernels; the host side only validates arguments, carves
 * the caller's workspace and enqueues kernels on the caller's stream.
 *
 * Sources of the method (titles of the pages; sections named per entry point):
 *   [nanochat-launch]  "復刻 ChatGPT 有多難？" news article on nanochat's launch,
 *                      section on Karpathy's tricks (為什么可以訓練如此之快).
 *   [nanochat-forum]   hongdingcd.com thread on nanochat, paragraphs on the model
 *                      architecture (rotary positions, QK norm, MQA, KV cache).
 *   [nanochat-csdn]    CSDN walkthrough of the nanochat speedrun (base-model
 *                      section: Engine class with KV cache, prefill and decode).
 *   [microgpt]         Hacker News summary of microgpt, sections "Tokenizer",
 *                      "Model parameters", "Core architecture", "Inference".
 *
 * Conventions
 *   - All device pointers are allocated and owned by the caller.  The library
 *     never allocates device memory; it owns only small host-side handles.
 *   - Linear weights are row-major [out, in] (y = W x), dtype per config:
 *     bf16 (GPT_DTYPE_BF16) or fp32 (GPT_DTYPE_F32).  The residual stream,
 *     every accumulator, the softmax and the logits are fp32.
 *   - Calls are asynchronous and stream-ordered: a call returns after
 *     enqueueing its kernels on `stream`.  Host arrays passed in (cu_seqlens)
 *     may be reused as soon as the call returns.  Device faults surface at the
 *     caller's next synchronisation.
 *   - Every call validates its arguments on the host before touching the
 *     device.  On failure it returns a non-zero gpt_status, enqueues nothing,
 *     and gpt_last_error() describes the problem.  No C++ exception crosses the
 *     ABI.  Calls that share one gpt_kv_cache are not thread-safe.
 */
#ifndef GPT_BLOCK_FWD_GPT_H
#define GPT_BLOCK_FWD_GPT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t *gpt_stream_t; /* a hipStream_t; NULL = default stream */

typedef enum {
  GPT_OK = 0,
  GPT_ERR_ARG = 1,         /* a pointer, size or layout argument is invalid */
  GPT_ERR_CAPACITY = 2,    /* a sequence would outgrow its KV-cache capacity */
  GPT_ERR_UNSUPPORTED = 3, /* a valid configuration the library has no kernels for */
  GPT_ERR_HIP = 4          /* the HIP runtime reported an error while enqueueing */
} gpt_status;

enum { GPT_POS_LEARNED = 0, GPT_POS_ROPE = 1 };
enum { GPT_ACT_RELU = 0, GPT_ACT_RELU2 = 1 };
enum { GPT_DTYPE_F32 = 0, GPT_DTYPE_BF16 = 1 };
enum { GPT_ROWS_ALL = 0, GPT_ROWS_LAST = 1 };

/* Text describing the last non-OK status returned on the calling thread. */
const char *gpt_last_error(void);

/*
 * Model shape.  [microgpt "Core architecture"]: pre-norm blocks with a
 * weightless RMSNorm (x / sqrt(mean(x^2) + norm_eps)), no biases, residual
 * connections, a two-layer MLP, an untied output projection.
 * [nanochat-launch tricks]: rotary positions, ReLU^2 MLP, separate Q/K/V.
 * [nanochat-forum]: QK normalisation and multi-query attention.
 * [microgpt "differences from production models", item 3]: grouped-query
 * attention.  n_kv_head K/V heads, each shared by n_head / n_kv_head
 * consecutive query heads: 1 is multi-query, n_head is multi-head.
 *
 *   pos_kind  GPT_POS_LEARNED: x = WTE[id] + WPE[t]  (microgpt layout)
 *             GPT_POS_ROPE:    x = WTE[id]; q, k rotated by half-split RoPE
 *   act       GPT_ACT_RELU (max(z,0)) or GPT_ACT_RELU2 (max(z,0)^2)
 *   qk_norm   1: weightless RMSNorm of every q and k head vector after RoPE
 *   max_seq   rows of the RoPE tables / WPE; upper bound on any position
 *
 * Supported: bf16 needs head_dim == 128, pos_kind ROPE, act RELU2,
 * n_head <= 16, d_model == n_head * head_dim, d_ff and vocab multiples of
 * 128; fp32 needs head_dim <= 64 and d_model % 4 == 0, <= 4096 (a small-model
 * path).  Both need n_head % n_kv_head == 0.  Anything else is
 * GPT_ERR_UNSUPPORTED.  A decode step handles at most 4096 sequences x
 * n_kv_head.
 */
typedef struct {
  int32_t vocab, n_layer, d_model, n_head, n_kv_head, head_dim, d_ff, max_seq;
  float rope_base, norm_eps;
  int32_t pos_kind, act, qk_norm, dtype;
} gpt_config;

/*
 * Weights.  wte [vocab, d_model]; wpe [max_seq, d_model] (NULL unless
 * pos_kind == GPT_POS_LEARNED); lm_head [vocab, d_model].  Per layer l
 * (host arrays of n_layer device pointers): wq[l] [n_head*head_dim, d_model],
 * wk[l], wv[l] [n_kv_head*head_dim, d_model], wo[l] [d_model, n_head*head_dim],
 * w1[l] [d_ff, d_model], w2[l] [d_model, d_ff].  All device, row-major, in
 * the config dtype, 16-byte aligned.
 */
typedef struct {
  const void *wte, *wpe, *lm_head;
  const void *const *wq, *const *wk, *const *wv, *const *wo, *const *w1, *const *w2;
} gpt_weights;

/*
 * rope_tables -- [nanochat-launch tricks]: rotary cos/sin values depend on no
 * trained parameter, so they are computed once and kept in GPU memory.
 * Writes cos_out[t*(head_dim/2) + i] = cos(t * base^(-2i/head_dim)) and the
 * same for sin, t < max_seq, i < head_dim/2, fp32 device arrays.  Angles and
 * cos/sin are evaluated in fp64 on the host and rounded once to fp32, then
 * copied with one stream-ordered transfer each.
 * Errors: GPT_ERR_ARG for max_seq <= 0, odd or non-positive head_dim,
 * base <= 0, NULL outputs; GPT_ERR_HIP if the copy cannot be enqueued.
 */
gpt_status rope_tables(int32_t max_seq, int32_t head_dim, float base, float *cos_out,
                       float *sin_out, gpt_stream_t stream);

/*
 * Paged KV cache -- [nanochat-launch tricks] and [microgpt "Core
 * architecture", item 7]: keys and values of earlier positions are kept so a
 * decode step only computes the new position.
 *
 * Layout of the caller's device buffer (offsets 256-byte aligned):
 *   pages   [n_layer][n_pages][2][page]   n_pages = n_seqs * ceil(capacity/page_size)
 *           K half: [page_size][n_kv_head*head_dim], row per position
 *           V half: bf16: [n_kv_head*head_dim][page_size] (transposed, so the
 *                   decode kernel's P*V operand is contiguous along positions;
 *                   within each 32-position half of a page, position
 *                   16a + 4q + b (a < 2, q < 4, b < 4) is stored at column
 *                   8q + 4a + b, the order the decode MFMA takes keys in);
 *                   fp32: [page_size][n_kv_head*head_dim]
 *           keys are stored after RoPE and QK-norm, as attention reads them.
 *   table   int32 [n_seqs][pages_per_seq]  page index of each logical page;
 *           sequence s owns pages s*pages_per_seq .. (s+1)*pages_per_seq-1.
 *   lens    int32 [n_seqs]  cached positions per sequence (device copy; the
 *           handle keeps a host mirror so capacity checks need no sync).
 *
 * kv_cache_alloc: with device_buf == NULL, stores the required byte count in
 * *bytes_inout and returns GPT_OK (out may be NULL).  With a buffer, checks
 * *bytes_inout >= required, writes the page table and zero lengths with
 * blocking copies, and returns a new handle in *out.  page_size must be 64.
 * Errors: GPT_ERR_ARG (NULL config/bytes_inout/out, n_seqs or capacity <= 0,
 * capacity > max_seq, buffer too small), GPT_ERR_UNSUPPORTED (page_size other
 * than 64, or a bf16 model with capacity above 16384 positions per sequence),
 * GPT_ERR_HIP.
 * kv_cache_free releases the handle only; the device buffer stays the
 * caller's.  kv_cache_lengths copies the host mirror of the lengths.
 */
typedef struct gpt_kv_cache gpt_kv_cache;
gpt_status kv_cache_alloc(const gpt_config *c, int32_t n_seqs, int32_t capacity_per_seq,
                          int32_t page_size, void *device_buf, size_t *bytes_inout,
                          gpt_kv_cache **out);
gpt_status kv_cache_free(gpt_kv_cache *kv);
gpt_status kv_cache_lengths(const gpt_kv_cache *kv, int32_t *lens_out);

/*
 * gpt_workspace_bytes -- bytes of device scratch that gpt_prefill and
 * gpt_decode_step need for up to max_tokens packed rows (prefill: total
 * prompt tokens; decode: number of sequences) and up to max_seqs sequences.
 * Returns 0 for an invalid or unsupported config.
 */
size_t gpt_workspace_bytes(const gpt_config *c, int32_t max_tokens, int32_t max_seqs);

/*
 * gpt_prefill -- full-sequence forward of packed, variable-length prompts.
 * [microgpt "Core architecture"], [nanochat-launch tricks], [nanochat-forum]:
 *   x = WTE[id] (+ WPE[t]); per layer: h = rms(x); q,k,v = Wq h, Wk h, Wv h;
 *   q,k rotated (RoPE) and normalised (QK-norm); causal attention of every
 *   query head against the K/V head floor(h*Hkv/H) with scale 1/sqrt(dh);
 *   x += Wo o; x += W2 act(W1 rms(x)).  logits = W_lm rms(x); lse = log sum
 *   exp(logits); probs = exp(logits - lse)  [microgpt "Core architecture" 2].
 *
 *   tokens      device int32 [total], sequences packed back to back
 *   cu_seqlens  HOST int32 [n_seqs+1], cu_seqlens[0] = 0, non-decreasing,
 *               every sequence non-empty, total = cu_seqlens[n_seqs] <= the
 *               workspace's max_tokens, every length <= max_seq
 *   kv          NULL: no cache.  Otherwise the sequences' K/V (positions
 *               0..len-1) are written into it and its lengths set to len
 *               (n_seqs must equal the handle's; GPT_ERR_CAPACITY if a length
 *               exceeds its capacity).  [nanochat-launch tricks]: the forward
 *               branches on whether a cache is present.
 *   logits_rows GPT_ROWS_ALL: logits/lse/probs have `total` rows in packed
 *               order; GPT_ROWS_LAST: one row per sequence (its last position)
 *   logits      device fp32 [rows, vocab] (required)
 *   lse, probs  device fp32 [rows] and [rows, vocab], each may be NULL
 *   rope_cos/rope_sin  tables from rope_tables() with >= max_seq rows
 *               (may be NULL when pos_kind == GPT_POS_LEARNED)
 *   workspace   device, >= gpt_workspace_bytes(c, total, n_seqs) bytes,
 *               256-byte aligned; clobbered
 */
gpt_status gpt_prefill(const gpt_config *c, const gpt_weights *w, const float *rope_cos,
                       const float *rope_sin, const int32_t *tokens, const int32_t *cu_seqlens,
                       int32_t n_seqs, gpt_kv_cache *kv, int32_t logits_rows, float *logits,
                       float *lse, float *probs, void *workspace, size_t workspace_bytes,
                       gpt_stream_t stream);

/*
 * gpt_prefill_loss -- next-token cross-entropy of packed prompts, without
 * materialising the logits.  [microgpt "Training process", item 2]: the
 * forward pass predicts each next token and the loss is the cross-entropy
 * between that prediction and the real token (how surprised the model is).
 * The forward is gpt_prefill's over every position; then, for row r with
 * t = targets[r] in [0, vocab):
 *   loss[r] = log sum_v exp(logits[r][v]) - logits[r][t]
 * A target outside [0, vocab) (e.g. -1 at a sequence's last position, which
 * has no next token) gives loss 0, and the row is left out of the mean.
 *   targets     device int32 [total], packed like tokens
 *   loss        device fp32 [total] (required)
 *   lse         device fp32 [total] or NULL
 *   mean        device fp32 [1] or NULL: the sum of the counted rows' losses
 *               over their number (0 if no row counts), summed in a fixed
 *               order so repeated calls agree bit for bit
 *   kv, tokens, cu_seqlens, rope tables, workspace: as gpt_prefill (the same
 *               gpt_workspace_bytes covers both calls)
 * bf16 models with more than 64 rows run the LM head with an epilogue that
 * keeps, per row, a (max, sum exp) pair for each 64 vocabulary columns and the
 * target's logit; the fp32 logits never reach device memory.  fp32 models and
 * prefills of at most 64 rows write the logits into the workspace first.
 * Errors: as gpt_prefill.
 */
gpt_status gpt_prefill_loss(const gpt_config *c, const gpt_weights *w, const float *rope_cos,
                            const float *rope_sin, const int32_t *tokens, const int32_t *targets,
                            const int32_t *cu_seqlens, int32_t n_seqs, gpt_kv_cache *kv,
                            float *loss, float *lse, float *mean, void *workspace,
                            size_t workspace_bytes, gpt_stream_t stream);

/*
 * gpt_decode_step -- one KV-cache decode step for every sequence of `kv`
 * ([nanochat-csdn] Engine with KV cache, prefill and decode; [microgpt
 * "Inference"] feed the previous token back).  Sequence s embeds
 * tokens_in[s] at position t = len_s, appends its K/V at t, attends over
 * positions 0..t, and its length becomes t+1.  Then the next token is chosen
 * from its logits:
 *   temperature <= 0: greedy, the lowest index among the maxima;
 *   temperature  > 0: p = softmax(logits / temperature), token = the smallest
 *                     i with sum_{j<=i} p_j > uniforms[s]; if rounding leaves
 *                     the total <= u, the last index with p > 0
 *                     ([microgpt "Inference"]: lower temperature sharpens).
 *   tokens_in   device int32 [n_seqs]; tokens_out device int32 [n_seqs]
 *               (may alias tokens_in)
 *   uniforms    device fp32 [n_seqs] in [0,1), required iff temperature > 0
 *   logits      device fp32 [n_seqs, vocab] or NULL (then kept in workspace)
 *   workspace   >= gpt_workspace_bytes(c, n_seqs, n_seqs) bytes
 * Errors: GPT_ERR_CAPACITY if some len_s + 1 > capacity (checked on the host
 * mirror, nothing enqueued), GPT_ERR_ARG, GPT_ERR_UNSUPPORTED, GPT_ERR_HIP.
 */
gpt_status gpt_decode_step(const gpt_config *c, const gpt_weights *w, const float *rope_cos,
                           const float *rope_sin, gpt_kv_cache *kv, const int32_t *tokens_in,
                           float temperature, const float *uniforms, int32_t *tokens_out,
                           float *logits, void *workspace, size_t workspace_bytes,
                           gpt_stream_t stream);

/*
 * gpt_decode_step_noalloc -- gpt_decode_step without a workspace argument,
 * for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.  The same
 * kernels run on a file-scope device scratch array of
 * GPT_NOALLOC_SCRATCH_BYTES (64 MiB) that each GPU the library runs on holds
 * until the process ends; its address on the current device is looked up
 * once, on the first call on that device.  The call allocates nothing and
 * records no profiling events.  Arguments, results and errors are those of
 * gpt_decode_step, plus GPT_ERR_CAPACITY (nothing enqueued) when the step
 * needs more scratch than that, i.e. gpt_workspace_bytes(c, n_seqs, n_seqs)
 * > GPT_NOALLOC_SCRATCH_BYTES.  Every call on a GPU shares its scratch:
 * calls that overlap on one GPU (other streams or threads) race; calls in
 * one stream are ordered and safe.  The scratch keeps the last call's
 * contents; what a step needs zeroed, its own kernels clear.
 */
#define GPT_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
gpt_status gpt_decode_step_noalloc(const gpt_config *c, const gpt_weights *w, const float *rope_cos,
                                   const float *rope_sin, gpt_kv_cache *kv, const int32_t *tokens_in,
                                   float temperature, const float *uniforms, int32_t *tokens_out,
                                   float *logits, gpt_stream_t stream);

/*
 * gpt_select_tokens -- token choice on rows of given logits, with the same
 * rule as gpt_decode_step (greedy or inverse-CDF temperature sampling).
 * Used for the first token after a prefill.  logits device fp32 [rows, vocab];
 * uniforms device fp32 [rows] (required iff temperature > 0); tokens_out
 * device int32 [rows].  No workspace.
 */
gpt_status gpt_select_tokens(const float *logits, int32_t rows, int32_t vocab, float temperature,
                             const float *uniforms, int32_t *tokens_out, gpt_stream_t stream);

/*
 * Gradients of the mean next-token loss, one fp32 device array per weight,
 * shaped like it: wte [vocab, d_model]; wpe [max_seq, d_model] (used only
 * with GPT_POS_LEARNED, else may be NULL); lm_head [vocab, d_model]; per
 * layer (host arrays of n_layer device pointers) wq, wk, wv, wo, w1, w2.
 */
typedef struct {
  float *wte, *wpe, *lm_head;
  float *const *wq, *const *wk, *const *wv, *const *wo, *const *w1, *const *w2;
} gpt_grads;

/* Bytes of device scratch gpt_loss_grads needs for up to max_tokens packed
 * rows and max_seqs sequences; 0 for an invalid or unsupported config.
 * bf16 models keep every layer's forward activations there for the
 * backward (about 2.5 GB at depth 12 with 16384 rows). */
size_t gpt_train_workspace_bytes(const gpt_config *c, int32_t max_tokens, int32_t max_seqs);

/*
 * gpt_loss_grads -- the mean next-token cross-entropy of packed sequences
 * and its gradient with respect to every weight.  [microgpt "Training
 * process", items 2 and 3]: the forward pass predicts each next token, the
 * loss is the cross-entropy against the real one, and back-propagation runs
 * the chain rule from the loss back to every parameter.
 *   loss = (1/n) sum over rows r with t = targets[r] in [0, vocab) of
 *          log sum_v exp(logits[r][v]) - logits[r][t],   n = their number
 * (rows whose target lies outside [0, vocab) count for nothing).  The
 * forward is gpt_prefill's (no cache).  The gradient of the loss with
 * respect to row r's logits is (softmax(logits[r]) - onehot(t)) / n; it is
 * carried back through the LM head, the final RMSNorm, each block (MLP,
 * RMSNorm, output projection, attention, QK-norm, RoPE, the Q/K/V
 * projections) and the embeddings.
 *   tokens, targets  device int32 [total], packed
 *   cu_seqlens, n_seqs, rope tables: as gpt_prefill
 *   grads       gradients, overwritten (not accumulated)
 *   loss        device fp32 [total] per-row losses (0 for skipped rows)
 *   mean        device fp32 [1] or NULL: the loss above
 *   workspace   >= gpt_train_workspace_bytes(c, total, n_seqs), 256-byte
 *               aligned; clobbered
 * bf16 models run every matrix product as a bf16 GEMM with fp32
 * accumulation (gradients rounded to bf16 where they are GEMM operands);
 * everything else is fp32.  The token-table gradient sums rows with fp32
 * atomics, so its last bits may differ from call to call.
 * Errors: GPT_ERR_ARG (NULL or inconsistent arguments, small workspace),
 * GPT_ERR_UNSUPPORTED (config), GPT_ERR_HIP.
 */
gpt_status gpt_loss_grads(const gpt_config *c, const gpt_weights *w, const float *rope_cos,
                          const float *rope_sin, const int32_t *tokens, const int32_t *targets,
                          const int32_t *cu_seqlens, int32_t n_seqs, const gpt_grads *grads,
                          float *loss, float *mean, void *workspace, size_t workspace_bytes,
                          gpt_stream_t stream);

/*
 * gpt_adam_step -- one Adam update of n fp32 parameters, in place.
 * [microgpt "Training process", item 4]: Adam keeps, per parameter, a
 * running mean of the gradient (momentum) and of its square (which scales
 * the step size), and moves the parameter by their ratio.  With
 * t = step >= 1:
 *   m = beta1 m + (1 - beta1) g
 *   v = beta2 v + (1 - beta2) g^2
 *   p = p - lr * (m / (1 - beta1^t)) / (sqrt(v / (1 - beta2^t)) + eps)
 * in fp32 (the bias corrections 1 / (1 - beta^t) are formed in fp64 on the
 * host and rounded once).  No weight decay.
 *   param, m, v  device fp32 [n], read and written; m and v start at 0
 *   grad         device fp32 [n]
 *   param_bf16   device bf16 [n] or NULL: receives the updated parameters
 *                rounded to bf16 (nearest even), the dtype the bf16 forward
 *                reads its weights in
 * param, grad, m, v must be 16-byte aligned and param_bf16 8-byte aligned;
 * the arrays must not overlap.  n == 0 enqueues nothing.
 * Errors: GPT_ERR_ARG for a NULL array, misalignment, n < 0, step < 1,
 * beta outside [0, 1), a negative or NaN eps, a non-finite lr;
 * GPT_ERR_HIP if the launch fails.
 */
gpt_status gpt_adam_step(float *param, const float *grad, float *m, float *v, void *param_bf16,
                         int64_t n, int32_t step, float lr, float beta1, float beta2, float eps,
                         gpt_stream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* GPT_BLOCK_FWD_GPT_H */
