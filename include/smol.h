/*
 * smol.h -- C ABI of libsmol: the forward pass of a LLaMA-style pre-norm decoder
 * stack (SmolLM2-135M shape and relatives) on AMD Instinct MI355X (gfx950).
 *
 * What is computed (sources are the pages on SmolLM2-135M / SmolLM3):
 *   embedding gather   -> abi96062 model.py, SmolLM2Model.forward
 *   per block          -> h = x + attn(RMSNorm_a(x)); out = h + mlp(RMSNorm_m(h))
 *                         (nnterp "SmolLM3", "The block, in order"; tohio block.py)
 *   RMSNorm            -> w * x / sqrt(mean(x^2) + eps) (abi96062 components.py, RMSNorm)
 *   RoPE               -> pairs (i, i + d/2) rotated by p * theta^(-2i/d), on q and k only
 *                         (Sualeh77 model.py, "3. RoPE"; rope_interleaved false in "1. Config")
 *   attention          -> causal softmax(q k^T / sqrt(d)) v, query head h reads kv head
 *                         h / (n_heads / n_kv_heads) (Sualeh77 model.py, "4. Attention";
 *                         abi96062 components.py, GroupedQueryAttention)
 *   MLP                -> down(silu(gate(x)) * up(x)) (abi96062 components.py, SwiGLU_FFN)
 *   head               -> logits = RMSNorm_f(x) E^T, lm_head tied to the embedding E
 *                         (abi96062 model.py, weight tying)
 *   decode             -> one new token per sequence at position cache_len[b]; its k (after
 *                         RoPE) and v are appended to the cache and it attends over keys
 *                         0 .. cache_len[b] (Sualeh77 model.py, "7. Top-level", forward with
 *                         past_key_values; the cache holds keys after RoPE)
 *
 * Conventions for every entry point
 *   - Pointers are DEVICE pointers unless marked "host". The caller owns every buffer
 *     (weights, ids, caches, logits, workspace); the library keeps no pointer after it
 *     returns, never allocates or frees device memory and never synchronises.
 *   - Work is enqueued on `stream` (a hipStream_t passed as void*; NULL = default
 *     stream) and is asynchronous. No memset nodes are recorded, so the calls may be
 *     captured into a HIP graph.
 *   - Arguments are checked on the host before anything is enqueued. A failed check
 *     returns a status and enqueues nothing; smol_last_error() then names the
 *     argument. SMOL_ERR_HIP reports a launch error (hipGetLastError after enqueue);
 *     faults during execution surface at the caller's next synchronisation.
 *   - Element types follow config.dtype: SMOL_F32 -> float, SMOL_BF16 -> bfloat16
 *     (weights, embedding, norm weights, caches, logits). The residual stream inside
 *     the library and the hidden states at the block interface are float32 for both.
 *   - Buffers of rows (weights, embedding, norm weights, hidden states, caches and
 *     the logits a forward call writes) must start on a 16-byte boundary: the
 *     kernels move rows in 16-byte vectors. A misaligned one returns
 *     SMOL_ERR_INVALID_ARG naming it. ids, cache_len and masks need only their
 *     element's alignment; smol_sample reads logits rows at any alignment.
 *   - Matrices are row-major. Linear weights are [out, in] (as nn.Linear stores them):
 *     wq [n_heads*d, H], wk/wv [n_kv*d, H], wo [H, n_heads*d], w_gate/w_up [I, H],
 *     w_down [H, I]; norm weights [H]; embedding [vocab, H].
 *   - Supported shapes: head_dim 64 or 128; hidden, intermediate and vocab multiples
 *     of 64; hidden at most 4096; hidden == n_heads*head_dim; n_heads divisible by n_kv_heads with 1 to 4
 *     query heads per kv head. Anything else returns SMOL_ERR_UNSUPPORTED or
 *     SMOL_ERR_INVALID_ARG. Batch and sequence length are arbitrary (>= 1).
 *   - Calls that share a workspace or a cache must not overlap.
 */
#ifndef SMOL_H
#define SMOL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SMOL_OK = 0,
  SMOL_ERR_INVALID_ARG = 1, /* null pointer, size out of range, inconsistent config */
  SMOL_ERR_UNSUPPORTED = 2, /* a valid shape this library does not implement */
  SMOL_ERR_WORKSPACE = 3,   /* ws_bytes smaller than smol_workspace_size() */
  SMOL_ERR_HIP = 4          /* the HIP runtime reported an error while enqueuing */
} smol_status;

typedef enum { SMOL_F32 = 0, SMOL_BF16 = 1 } smol_dtype;

typedef enum { SMOL_OP_BLOCK = 0, SMOL_OP_PREFILL = 1, SMOL_OP_DECODE = 2 } smol_op;

/* Model shape (host struct). SmolLM2-135M: hidden 576, n_heads 9, n_kv_heads 3,
 * head_dim 64, intermediate 1536, n_layers 30, vocab 49152, max_pos 8192,
 * rms_eps 1e-5, rope_theta 100000 (Sualeh77 model.py, "1. Config"). */
typedef struct {
  int32_t hidden, n_heads, n_kv_heads, head_dim, intermediate, n_layers, vocab, max_pos;
  float rms_eps, rope_theta;
  int32_t dtype; /* smol_dtype */
  /* SmolLM3 variants (nnterp "SmolLM3", NoPE blocks and sliding window): with
   * no_rope_interval k > 0, block l (0-based) applies no rotary to q and k when
   * (l + 1) % k == 0 (k = 4: blocks 3, 7, 11, ...); with sliding_window W > 0 those
   * blocks attend only to keys at positions p - W < pos <= p. 0 and 0: every block
   * rotary with full causal attention (SmolLM2). */
  int32_t no_rope_interval, sliding_window;
} smol_config;

/* One block's weights (host struct of device pointers), element type config.dtype. */
typedef struct {
  const void *attn_norm, *wq, *wk, *wv, *wo, *mlp_norm, *w_gate, *w_up, *w_down;
} smol_layer_weights;

/* The model (host struct): embed [vocab, H] is also the lm_head (tied); layers is a
 * HOST array of n_layers entries; final_norm [H]. */
typedef struct {
  const void *embed;
  const smol_layer_weights *layers;
  const void *final_norm;
} smol_model_weights;

/* Bytes of scratch device memory that `op` needs for this config, batch and seq;
 * for SMOL_OP_DECODE pass the cache capacity (cache_cap) as seq. Host-only;
 * writes *bytes. The workspace must be 256-byte aligned. */
smol_status smol_workspace_size(const smol_config *cfg, int op, int batch, int seq, size_t *bytes);

/* One decoder block on hidden states x_in [batch, seq, H] float32 -> x_out (same
 * shape, float32; may equal x_in). Token t sits at absolute position pos0 + t.
 * k_cache / v_cache: NULL, or [batch, n_kv, cache_cap, head_dim] caches that receive
 * the block's k (after RoPE) and v at indices pos0 .. pos0+seq-1; with a cache the
 * queries also attend to the cached keys 0 .. pos0-1. Without a cache they attend
 * only to the seq new tokens. Requires pos0 + seq <= max_pos (and <= cache_cap). */
smol_status smol_block_forward(const smol_config *cfg, const smol_layer_weights *w,
                               const float *x_in, float *x_out, int batch, int seq, int pos0,
                               void *k_cache, void *v_cache, int cache_cap,
                               void *ws, size_t ws_bytes, void *stream);

/* Whole-model prefill: ids [batch, seq] int32 at positions 0 .. seq-1 -> logits
 * [batch, seq, vocab]. k_cache / v_cache: NULL, or [n_layers, batch, n_kv, cache_cap,
 * head_dim] caches filled at indices 0 .. seq-1 for a later smol_decode_step.
 * Requires seq <= max_pos (and <= cache_cap). Ids must lie in [0, vocab): an id
 * outside it makes its sequence's logits NaN from that position on (earlier
 * positions of that sequence may turn NaN too; other sequences are unaffected). */
smol_status smol_model_prefill(const smol_config *cfg, const smol_model_weights *w,
                               const int32_t *ids, int batch, int seq, void *logits,
                               void *k_cache, void *v_cache, int cache_cap,
                               void *ws, size_t ws_bytes, void *stream);

/* One decode step: ids [batch] int32; cache_len [batch] int32 (device) = positions
 * already in the cache for each sequence. Sequence b's token sits at position
 * cache_len[b]: its k (after RoPE) and v are written to index cache_len[b] of every
 * layer's cache [n_layers, batch, n_kv, cache_cap, head_dim] and it attends to
 * indices 0 .. cache_len[b]. logits [batch, vocab]. cache_len is not advanced. A
 * sequence whose cache_len[b] is negative or leaves no room (cache_len[b] >=
 * min(cache_cap, max_pos)) writes nothing to the cache and gets NaN logits. */
smol_status smol_decode_step(const smol_config *cfg, const smol_model_weights *w,
                             const int32_t *ids, const int32_t *cache_len, int batch,
                             void *k_cache, void *v_cache, int cache_cap, void *logits,
                             void *ws, size_t ws_bytes, void *stream);

/* smol_decode_step without a workspace and without any allocation, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc. Arguments, results and errors as smol_decode_step
 * (no key mask). The scratch is a fixed device array of SMOL_STATIC_SCRATCH_MIB MiB
 * inside the library: each GPU the library runs on holds its own copy from the first
 * call on it until the process ends. A call whose decode workspace
 * (smol_workspace_size with SMOL_OP_DECODE and cache_cap) would exceed it returns
 * SMOL_ERR_WORKSPACE (batch 64 over a 2048-key cache of the SmolLM2-135M shape needs
 * about 3.7 MiB). Every call on a GPU shares that GPU's array and leaves its contents
 * behind; nothing in it needs to start at zero (each call writes every value it reads
 * before reading it), but calls that overlap on one GPU (different streams or host
 * threads without ordering) race on it: the caller must serialise them. */
#define SMOL_STATIC_SCRATCH_MIB 32
smol_status smol_decode_step_static(const smol_config *cfg, const smol_model_weights *w,
                                    const int32_t *ids, const int32_t *cache_len, int batch,
                                    void *k_cache, void *v_cache, int cache_cap, void *logits,
                                    void *stream);

/* Next token of each sequence from one row of logits per sequence (the generation
 * loop of Sualeh77 model.py, "7. Top-level SmolLM2-135M Model Architecture",
 * generate, and abi96062 model.py, SmolLM2Model.generate).
 *   logits: row b starts at logits + b * row_stride elements; vocab elements, of
 *     dtype (float or bfloat16). For the last position of a prefill [B, T, V] pass
 *     logits + (T-1)*V and row_stride T*V; for a decode step [B, V], 0 and V.
 *   temperature == 0: greedy, next_ids[b] = index of the largest logit (lowest index
 *     among equal maxima).
 *   temperature > 0: z = logit / temperature; top_k in 1 .. vocab-1 keeps the tokens
 *     whose logit is >= the k-th largest logit (0 or >= vocab: off); top_p < 1 then
 *     keeps, in descending logit order (equal logits by ascending index), every token
 *     up to and including the first at which the cumulative softmax probability of
 *     the tokens kept so far exceeds top_p (top_p >= 1: off). next_ids[b] is the first
 *     index, in vocabulary order, at which the cumulative softmax probability of the
 *     kept z exceeds uniforms[b] (inverse CDF).
 *   uniforms [batch] float in [0, 1) (device; read only when temperature > 0): the
 *     caller's random numbers, one per row.
 *   next_ids [batch] int32 (device, written): the chosen index, or -1 for a row that
 *     holds a NaN, or (when sampling) whose largest logit is infinite.
 * Errors: SMOL_ERR_INVALID_ARG for null pointers, batch < 1, vocab < 1, row_stride <
 * vocab when batch > 1, a negative or NaN temperature or top_p, top_k < 0 or an
 * unknown dtype. Every float sum is taken in a fixed order, so a call with the same
 * inputs returns the same ids. Uses no workspace. */
smol_status smol_sample(const void *logits, int dtype, int batch, int vocab, int64_t row_stride,
                        float temperature, int top_k, float top_p, const float *uniforms,
                        int32_t *next_ids, void *stream);

/* Generation (the loop of Sualeh77 model.py, "7. Top-level SmolLM2-135M Model
 * Architecture", generate: the prompt once, then one cached decode step per new
 * token). prompt_ids [batch, prompt_len] int32, right-padded when the prompts differ
 * in length: prompt_lens NULL (every prompt has prompt_len tokens) or int32 [batch]
 * (device), sequence b's length L_b = prompt_lens[b] clamped to [1, prompt_len]. The
 * prompt fills the caches [n_layers, batch, n_kv, cache_cap, head_dim] at
 * 0 .. prompt_len-1 (causality keeps the padding out of the real tokens) and the
 * logits of position L_b - 1 give token 0 through smol_sample's rule (temperature,
 * top_k, top_p; uniforms [max_new, batch] device, row j for token j, NULL when
 * temperature is 0). Token j >= 1 comes from a decode step that feeds token j-1 at
 * position L_b + j - 1 (overwriting the padding's cache entries). out_ids
 * [max_new, batch] int32 (device, written; token j of sequence b at j * batch + b). All max_new tokens are produced: a caller that stops
 * at an end-of-sequence id trims afterwards. Requires prompt_len + max_new - 1 <=
 * min(cache_cap, max_pos). ws: smol_generate_workspace_size() bytes, 256-byte
 * aligned. Everything is enqueued on `stream`; nothing synchronises, so the whole
 * call can be captured into one HIP graph. */
smol_status smol_generate_workspace_size(const smol_config *cfg, int batch, int prompt_len, int max_new,
                                         int cache_cap, size_t *bytes);
smol_status smol_generate(const smol_config *cfg, const smol_model_weights *w, const int32_t *prompt_ids,
                          const int32_t *prompt_lens, int batch, int prompt_len, int max_new,
                          float temperature, int top_k, float top_p, const float *uniforms,
                          int32_t *out_ids, void *k_cache, void *v_cache, int cache_cap, void *ws,
                          size_t ws_bytes, void *stream);

/* Prefill of a chunk, with an optional padding mask (Sualeh77 model.py, "4.
 * Attention": the attention_mask added to the scores as 0 / -inf per key).
 *   pos0: the chunk's tokens sit at positions pos0 .. pos0 + seq - 1. pos0 > 0
 *     needs k_cache / v_cache, whose indices 0 .. pos0 - 1 hold the earlier tokens
 *     (keys after RoPE); the chunk's k and v are written at pos0 .. pos0 + seq - 1
 *     and each query attends to every key index <= its own position (absolute-
 *     position causality; the pages leave T > 1 with a cache undefined).
 *   key_mask: NULL, or uint8 [batch, cache_cap] (with caches) / [batch, seq]
 *     (without), indexed by key position: 0 removes that key from every query of
 *     its sequence; a query that is left with no key gets NaN outputs (the softmax
 *     of all -inf), which then reach that sequence's later positions through the
 *     residual stream only where they attend to it.
 * Everything else as smol_model_prefill (which is this call with pos0 0 and no
 * mask); requires pos0 + seq <= max_pos and, with caches, <= cache_cap. */
smol_status smol_model_prefill_ex(const smol_config *cfg, const smol_model_weights *w,
                                  const int32_t *ids, int batch, int seq, int pos0,
                                  const uint8_t *key_mask, void *logits, void *k_cache,
                                  void *v_cache, int cache_cap, void *ws, size_t ws_bytes,
                                  void *stream);

/* A decode step with an optional padding mask: key_mask NULL or uint8
 * [batch, cache_cap] over key positions (0: the key is ignored by the new token).
 * Everything else as smol_decode_step (which is this call with no mask). */
smol_status smol_decode_step_ex(const smol_config *cfg, const smol_model_weights *w,
                                const int32_t *ids, const int32_t *cache_len, int batch,
                                const uint8_t *key_mask, void *k_cache, void *v_cache,
                                int cache_cap, void *logits, void *ws, size_t ws_bytes,
                                void *stream);

/* Gradient buffers of one block (host struct of device pointers, float32, shaped
 * like the weights of smol_layer_weights). */
typedef struct {
  float *attn_norm, *wq, *wk, *wv, *wo, *mlp_norm, *w_gate, *w_up, *w_down;
} smol_layer_grads;

/* Backward of one decoder block (the block of smol_block_forward, trained in the
 * pages: Sualeh77 model.py trains it on TinyShakespeare, abi96062 model.py sets it
 * up for training; the chain rule through nnterp "SmolLM3", "The block, in order",
 * and abi96062 components.py, RMSNorm / GroupedQueryAttention / SwiGLU_FFN).
 * For L = sum(dy * block(x)):
 *   x [batch, seq, H] float32: the block's input, tokens at positions pos0 .. pos0 +
 *     seq - 1 (RoPE angles; the queries attend to the seq tokens of the call only, as
 *     smol_block_forward without a cache);
 *   layer: the block's index in its model (decides the SmolLM3 NoPE rotary and the
 *     sliding window; 0 for a SmolLM2 block);
 *   key_mask: NULL or uint8 [batch, seq] by token index (0: the key is hidden from
 *     every query of its sequence; a query must keep at least one key);
 *   dy [batch, seq, H] float32: dL/d(block output);
 *   dx [batch, seq, H] float32 (written): dL/dx; may not alias x or dy;
 *   grads: the nine weight gradients, written (accumulate == 0) or added to what the
 *     buffers hold (accumulate == 1: gradient accumulation over micro-batches).
 * The forward is recomputed inside (activations are not taken from a forward call).
 * Every contraction is a float32 MFMA: with config.dtype SMOL_BF16 the bfloat16
 * weights (16-byte aligned) are first widened to float32 in the workspace (exact),
 * so a bf16 model gets the float32 gradients of its own weights. Requires pos0 >= 0,
 * pos0 + seq <= max_pos, 0 <= layer < n_layers. ws:
 * smol_block_backward_workspace_size() bytes, 256-byte aligned. Deterministic: no
 * atomics, every sum in a fixed order. */
smol_status smol_block_backward_workspace_size(const smol_config *cfg, int batch, int seq, size_t *bytes);
smol_status smol_block_backward(const smol_config *cfg, const smol_layer_weights *w, int layer,
                                const float *x, const float *dy, int batch, int seq, int pos0,
                                const uint8_t *key_mask, float *dx, const smol_layer_grads *grads,
                                int accumulate, void *ws, size_t ws_bytes, void *stream);

/* Static text for a status code. */
const char *smol_status_string(smol_status s);

/* Text of the last failed check on this thread ("" if none). */
const char *smol_last_error(void);

/* Kernel-duration measurement (diagnostic, not for captured streams). After
 * smol_timing_begin(kernel, max_launches) the next launches of that kernel class
 * (smol_kernel), up to max_launches, are timed by a start/stop event pair that the
 * HIP runtime records at the kernel's dispatch (hipExtLaunchKernelGGL): the kernel's
 * own execution time, as a kernel trace reports it. smol_timing_end() waits for
 * those events and returns the summed duration in milliseconds and the number of
 * launches timed (host pointers). SMOL_K_EMBED times
 * the kernel that starts the residual stream (embedding gather, or the copy of x_in
 * in smol_block_forward); SMOL_K_RMSNORM has no launches of its own, since every
 * RMSNorm is folded into the GEMMs around it. */
typedef enum {
  SMOL_K_EMBED = 0, SMOL_K_RMSNORM = 1, SMOL_K_QKV_ROPE = 2, SMOL_K_ATTENTION = 3,
  SMOL_K_O_PROJ = 4, SMOL_K_GATE_UP = 5, SMOL_K_DOWN = 6, SMOL_K_LM_HEAD = 7,
  SMOL_K_DECODE_ATTENTION = 8, SMOL_K_DECODE_COMBINE = 9, SMOL_K_SAMPLE = 10,
  /* smol_block_backward: its GEMMs, attention forward / dQ / dK-dV, row kernels */
  SMOL_K_BW_GEMM = 11, SMOL_K_BW_ATTN_FWD = 12, SMOL_K_BW_ATTN_DQ = 13, SMOL_K_BW_ATTN_DKDV = 14,
  SMOL_K_BW_ROWS = 15,
  /* the one-launch decode step of a bf16 model at head_dim 64 (every layer, up to the
   * final norm; smol_decode_step and the decode steps of smol_generate) */
  SMOL_K_DECODE_STEP = 16, SMOL_K_COUNT = 17
} smol_kernel;
smol_status smol_timing_begin(int kernel, int max_launches);
smol_status smol_timing_end(float *total_ms, int *launches);

#ifdef __cplusplus
}
#endif

#endif /* SMOL_H */
