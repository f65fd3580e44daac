/*
 * dflash.h: C ABI of the DFlash draft-proposal path for AMD MI355X (gfx950).
 *
 * DFlash drafts a whole block of tokens in one non-causal forward of a small Qwen3-style
 * drafter, attending to target hidden states injected into each draft layer's KV cache.
 * The method is described in "DFlash Speculative Decoding in the vLLM Neuron Framework"
 * (AWS Neuron design doc, cited below as [N]), "[Feat][Spec Decode] DFlash" (vLLM pull
 * request #36847, [V]) and "Dflash: Block Diffusion Speculative Decoding" (Qualcomm
 * efficient-transformers pull request #995, [Q]).
 *
 * Conventions for every entry point:
 *  - All tensors are device pointers to memory the caller allocated and owns: weights,
 *    caches, inputs, outputs and workspace. The library allocates and frees nothing and keeps
 *    no pointer after a call returns. Host arrays of device pointers (per-layer weights,
 *    caches, aux inputs) are read during the call only.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) with no host
 *    synchronisation. Ordering between calls (e.g. inject before propose on the same cache)
 *    follows stream order and is the caller's job. Calls sharing a workspace must not overlap.
 *  - Dense weights are row-major [out_features, in_features] (y = W x). Weights, auxiliary
 *    states and KV caches use the config's storage dtype: bfloat16 (raw 16-bit bf16 values)
 *    or fp32. Activations stay fp32 inside the library; a bf16 GEMM takes each fp32
 *    activation f as two bf16 values, hi = bf16(f) and lo = bf16(f - hi), whose sum keeps 17
 *    significant bits of f (relative error at most 2^-17, about 7.6e-6), except the LM head
 *    and the gate|up projection of a proposal with more than 64 block rows, which take hi
 *    alone (bf16(f), relative error at most 2^-9). The block's q/k/v are rounded to the
 *    storage type like cached K/V. The RoPE table and hidden_out are fp32. Token ids and
 *    positions are int32; slots are int64.
 *  - Host-side validation covers pointers and scalars only. A call that fails validation
 *    (DFLASH_ERR_INVALID_ARGUMENT, DFLASH_ERR_UNSUPPORTED, DFLASH_ERR_WORKSPACE_TOO_SMALL)
 *    returns before enqueuing anything; every chunk and workspace carve-up of the call is
 *    planned before its first launch. A DFLASH_ERR_HIP status (a launch the runtime refused)
 *    can come part-way through a call, after earlier kernels of the same call were enqueued:
 *    the outputs are then unspecified. dflash_last_error() (thread-local) explains any
 *    failure. Values in
 *    device memory (positions, sequence lengths, block tables, slots, token ids) are not
 *    validated: out-of-range values are clamped or skipped as each call states, and give
 *    unspecified results but never an out-of-bounds access.
 *  - No entry point throws; nothing but status codes crosses the ABI.
 */
#ifndef DFLASH_H_
#define DFLASH_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum dflash_status {
  DFLASH_OK = 0,
  DFLASH_ERR_INVALID_ARGUMENT = -1,
  DFLASH_ERR_UNSUPPORTED = -2,
  DFLASH_ERR_WORKSPACE_TOO_SMALL = -3,
  DFLASH_ERR_HIP = -4
} dflash_status;

typedef enum dflash_dtype { DFLASH_F32 = 0, DFLASH_BF16 = 1 } dflash_dtype;

typedef enum dflash_op { DFLASH_OP_INJECT = 0, DFLASH_OP_PROPOSE = 1 } dflash_op;

/* Drafter shape ([N] "Draft Model": a small Qwen3 decoder stack, an fc layer over the
 * concatenated auxiliary states, target embedding and LM head; the DFlashConfig fields
 * block size and mask token id). Every dimension must be positive (n_layers may be 0) and
 * n_q_heads a multiple of n_kv_heads; mask_token_id in [0, vocab); rms_eps >= 0; dtype
 * DFLASH_F32 or DFLASH_BF16 (else DFLASH_ERR_INVALID_ARGUMENT). Supported shapes (else
 * DFLASH_ERR_UNSUPPORTED):
 *   head_dim 64 or 128;
 *   hidden, intermediate and n_aux*target_hidden multiples of 128, target_hidden of 32;
 *   n_q_heads*head_dim a multiple of 128;  hidden <= 16384;  vocab a multiple of 16;
 *   2 <= block_size <= 64 and block_size*n_q_heads/n_kv_heads <= 64 (so at most 63 drafts);
 *   n_layers <= 64;  n_aux <= 8. */
typedef struct dflash_config {
  int32_t hidden;         /* H */
  int32_t n_layers;       /* L */
  int32_t n_q_heads;      /* QH */
  int32_t n_kv_heads;     /* KVH */
  int32_t head_dim;       /* D */
  int32_t intermediate;   /* I (SwiGLU) */
  int32_t vocab;          /* V (target vocabulary) */
  int32_t n_aux;          /* number of concatenated target layers */
  int32_t target_hidden;  /* Ht; fc in-features = n_aux * Ht */
  int32_t block_size;     /* bs; K = bs - 1 drafts */
  int32_t mask_token_id;
  float rms_eps;
  int32_t dtype;          /* dflash_dtype: storage type of weights, aux states and KV */
} dflash_config;

/* Drafter weights. Single tensors are device pointers; per-layer tensors are host arrays of
 * n_layers device pointers. Norm weights are [H] or [D] vectors of the storage dtype. */
typedef struct dflash_weights {
  const void *fc;           /* [H, n_aux*Ht] */
  const void *hidden_norm;  /* [H] */
  const void *embed;        /* [V, H] the target's token embedding */
  const void *lm_head;      /* [V, H] the target's LM head */
  const void *final_norm;   /* [H] */
  const void *kv_fused;     /* [L*2*KVH*D, H], built by dflash_build_fused_kv_weight */
  const void *const *in_norm;    /* [L] x [H]   input_layernorm */
  const void *const *wq;         /* [L] x [QH*D, H] */
  const void *const *wk;         /* [L] x [KVH*D, H] */
  const void *const *wv;         /* [L] x [KVH*D, H] */
  const void *const *q_norm;     /* [L] x [D]   per-head RMSNorm weight, shared by heads */
  const void *const *k_norm;     /* [L] x [D] */
  const void *const *wo;         /* [L] x [H, QH*D] */
  const void *const *post_norm;  /* [L] x [H]   post_attention_layernorm */
  const void *const *w_gate;     /* [L] x [I, H] */
  const void *const *w_up;       /* [L] x [I, H] */
  const void *const *w_down;     /* [L] x [H, I] */
  const float *rope_cos;         /* [rope_max_pos, D/2], built by dflash_build_rope_table */
  const float *rope_sin;         /* [rope_max_pos, D/2] */
  int32_t rope_max_pos;          /* positions are clamped to rope_max_pos - 1 */
} dflash_weights;

/* Paged KV cache of every draft layer ([N] "Paged KV Integration"). Each layer's K and V are
 * [num_pages, page_size, KVH, D]: slot s = page * page_size + offset holds the KVH x D
 * values of one token. block_table is a device [batch, max_blocks_per_seq] int32 array of
 * physical page ids (row b serves sequence b of a propose call); inject uses slots directly
 * and ignores it. */
typedef struct dflash_kv_cache {
  void *const *k;  /* host array [L] of device pointers */
  void *const *v;  /* host array [L] of device pointers */
  int32_t num_pages;
  int32_t page_size;
  const int32_t *block_table;
  int32_t max_blocks_per_seq;
} dflash_kv_cache;

/* RoPE table: cos/sin[p][i] = cos/sin(p * theta^(-2i/D)) for p < max_pos, i < D/2, computed
 * in fp64 on the device and rounded to fp32. Rotate-half pairing (element i with i + D/2),
 * absolute positions, no scaling: the model-level rotary table of [Q] (commit moving the
 * rotary embedding to the model level) gathered by absolute position. cos_out and sin_out
 * are device arrays of max_pos * D/2 floats. */
dflash_status dflash_build_rope_table(int32_t head_dim, double theta, int32_t max_pos,
                                      float *cos_out, float *sin_out, void *stream);

/* Stack every layer's K and V projection into the fused KV weight ([N] "Context KV
 * Injection" step 2: built once at bind time from this rank's KV heads). Row blocks of
 * out [L*2*KVH*D, H] are, in order, wk[0], wv[0], wk[1], wv[1], ... Only wk and wv of
 * `w` are read. */
dflash_status dflash_build_fused_kv_weight(const dflash_config *cfg, const dflash_weights *w,
                                           void *out, void *stream);

/* Workspace bytes that a call of `op` needs: for DFLASH_OP_INJECT, max_rows_or_batch is
 * the largest n_rows (rows are processed in bounded chunks, so the size stops growing);
 * for DFLASH_OP_PROPOSE it is the largest batch and max_context the largest sequence
 * length. Returns 0 for an invalid config or op. */
size_t dflash_workspace_bytes(const dflash_config *cfg, int32_t op, int32_t max_rows_or_batch,
                              int32_t max_context);

/* KV injection ([N] "Context KV Injection (Precompute)"). For each row r < n_rows:
 * x = concat(aux[0][r], ..., aux[n_aux-1][r]) (ascending target-layer order, [N] "Target
 * Auxiliary Hidden State Extraction"); ctx = hidden_norm(fc(x)); for every layer l and kv
 * head g: K_l[slot_mapping[r], g] = RoPE(k_norm_l(W_k^l ctx)_g, positions[r]) and
 * V_l[slot_mapping[r], g] = (W_v^l ctx)_g. Rows with slot_mapping[r] < 0 (padding) or
 * >= num_pages*page_size are skipped, and no other cache entry is touched. Each call writes
 * only its own rows, so injecting incrementally equals injecting everything at once.
 *   aux: host array of n_aux device pointers, each [n_rows, Ht] with row stride
 *        aux_row_stride elements (>= Ht).
 *   positions: device [n_rows] int32 absolute positions.  slot_mapping: device [n_rows].
 * n_rows == 0 returns DFLASH_OK and does nothing. */
dflash_status dflash_inject_context_kv(const dflash_config *cfg, const dflash_weights *w,
                                       const dflash_kv_cache *cache, const void *const *aux,
                                       int64_t aux_row_stride, int32_t n_rows,
                                       const int32_t *positions, const int64_t *slot_mapping,
                                       void *workspace, size_t workspace_bytes, void *stream);

/* Block proposal ([N] "DFlash Draft Model Architecture", forward(); "Draft Block
 * Construction"). For each sequence b < batch, the block [bonus_tokens[b], mask x K] sits
 * at positions seq_lens[b] + j. It is embedded with the target embedding, then goes through
 * L decoder layers. Each layer runs RMSNorm, QKV, q/k RMSNorm + RoPE, attention, O projection
 * and residual, RMSNorm, SwiGLU MLP and residual. Attention is non-causal: every block query
 * sees the seq_lens[b] context keys of the paged cache (positions [0, seq_lens[b])) and all
 * block_size block keys ([V] test of the first pass: causal is False). The block's own K/V
 * are not written to the cache. Rows 1..K get the final RMSNorm and the LM head; the greedy
 * argmax (lowest index on ties) gives the drafts.
 *   seq_lens: device [batch] int32, clamped to [0, max_context].  bonus_tokens: device
 *   [batch], clamped to [0, V).  Outputs: draft_token_ids [batch, bs] = [bonus, drafts],
 *   drafts_only [batch, K], and optionally hidden_out [batch*K, H] (fp32): the
 *   final-norm rows fed to the LM head (NULL skips it).
 * batch == 0 returns DFLASH_OK and does nothing.
 * With DFLASH_PERSISTENT_LAYERS=1 in the environment at the call, a batch-1 bf16 proposal
 * (head_dim 128, hidden, n_q_heads * 128 and intermediate multiples of 256, at most 8 layers,
 * block_size <= 16) runs the layer stack as one persistent launch in place of a launch per
 * projection: the same computation within the same tolerances, off by default (on MI355X it
 * measured slower than the per-projection launches at the Qwen3-8B shape). Its work-groups
 * wait for each other with bounded waits; if one gives up (about a second), every draft is -1. */
dflash_status dflash_propose_block(const dflash_config *cfg, const dflash_weights *w,
                                   const dflash_kv_cache *cache, int32_t batch,
                                   const int32_t *bonus_tokens, const int32_t *seq_lens,
                                   int32_t max_context, int32_t *draft_token_ids,
                                   int32_t *drafts_only, float *hidden_out, void *workspace,
                                   size_t workspace_bytes, void *stream);

/* Block proposal overlapped with the step's injection ([N] "Context KV Injection" and
 * "DFlashProposer": the injected rows are context for the block that follows). The same
 * computation, arguments, outputs and errors as dflash_propose_block, plus `cache_ready`: a
 * hipEvent_t (NULL: none), recorded by the caller after the injection of this step's rows,
 * on any stream of the same device. The embedding and the first layer's QKV projection read
 * no cache and are enqueued first; the stream waits for the event before the first launch
 * that reads the cache (the first layer's attention; with no layer, after the last launch),
 * so an injection running on another stream overlaps with them, and the proposal's completion
 * on `stream` implies the event's. The two calls must use different workspaces. The event is
 * only waited on, never recorded or destroyed; under stream capture it must be recorded in
 * the same capture. */
dflash_status dflash_propose_block_after(const dflash_config *cfg, const dflash_weights *w,
                                         const dflash_kv_cache *cache, int32_t batch,
                                         const int32_t *bonus_tokens, const int32_t *seq_lens,
                                         int32_t max_context, int32_t *draft_token_ids,
                                         int32_t *drafts_only, float *hidden_out, void *workspace,
                                         size_t workspace_bytes, void *cache_ready, void *stream);

/* Bytes of the static device scratch that dflash_propose_block_noalloc uses (per GPU). */
#define DFLASH_STATIC_SCRATCH_BYTES (64u << 20)

/* Block proposal for callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc. The same computation, arguments,
 * outputs and errors as dflash_propose_block, without the workspace: the call runs on the
 * library's static device scratch of DFLASH_STATIC_SCRATCH_BYTES, one copy per GPU, held from
 * the first call on that GPU until the process ends. It allocates nothing and calls no
 * allocating routine. A call whose workspace would exceed the scratch (dflash_workspace_bytes
 * of DFLASH_OP_PROPOSE for this batch and max_context) returns DFLASH_ERR_WORKSPACE_TOO_SMALL
 * before enqueuing anything; 64 MiB holds a Qwen3-8B-shaped batch-1 proposal up to a
 * 32768-token context. `stream` must belong to the calling thread's current device. Every
 * call on a GPU shares that GPU's scratch, and the kernels clear what must start at zero, so
 * calls in stream order need nothing between them; calls that overlap on one GPU (other
 * streams, other threads) race on the scratch and give unspecified results. */
dflash_status dflash_propose_block_noalloc(const dflash_config *cfg, const dflash_weights *w,
                                           const dflash_kv_cache *cache, int32_t batch,
                                           const int32_t *bonus_tokens, const int32_t *seq_lens,
                                           int32_t max_context, int32_t *draft_token_ids,
                                           int32_t *drafts_only, float *hidden_out, void *stream);

/* Greedy verification ([N] "Async Rejection and Position Correction": rejected entries are
 * -1; [Q]: verification by the frozen target gives output identical to standard decoding).
 * target_tokens[b, i] is the target's argmax after the context and draft_tokens[b, :i].
 * accepted_len[b] = a = 1 + the length of the longest prefix where draft == target, so
 * 1 <= a <= K+1; output_tokens[b] = target[b, :a] followed by -1; next_bonus[b] =
 * target[b, a-1]. Shapes: draft_tokens [batch, K], target_tokens and output_tokens
 * [batch, K+1], accepted_len and next_bonus [batch], all int32 device arrays.
 * Requires 1 <= num_drafts <= 63. */
dflash_status dflash_greedy_verify(int32_t batch, int32_t num_drafts,
                                   const int32_t *draft_tokens, const int32_t *target_tokens,
                                   int32_t *accepted_len, int32_t *output_tokens,
                                   int32_t *next_bonus, void *stream);

/* Greedy verification with the acceptance counters of [V]'s spec-decode metrics fused in:
 * the same outputs as dflash_greedy_verify, and the int64 device array stats[3] is
 * incremented by this call's num_drafts (batch: one draft block per sequence),
 * num_draft_tokens (batch * num_drafts) and num_accepted_tokens (sum of accepted_len - 1).
 * The caller zeroes stats once; acceptance rate = stats[2] / stats[1] and acceptance length
 * = 1 + stats[2] / stats[0]. Increments are integer atomics, so the totals do not depend on
 * scheduling. stats must not be NULL. */
dflash_status dflash_greedy_verify_stats(int32_t batch, int32_t num_drafts,
                                         const int32_t *draft_tokens, const int32_t *target_tokens,
                                         int32_t *accepted_len, int32_t *output_tokens,
                                         int32_t *next_bonus, int64_t *stats, void *stream);

/* Proposal-input preparation ([N] "Async Rejection and Position Correction", "Paged KV
 * Integration", "Draft Block Construction"): corrects a step that was scheduled as if every
 * draft of the previous step had been accepted. For request b, prev_out[b] is the previous
 * step's rejection-sampler output [prev_num_drafts + 1] (emitted tokens, -1 for rejected):
 *   valid_b = entries that are not -1 and lie in [0, vocab); rejected_b = prev_num_drafts + 1
 *   - valid_b;
 *   seq_lens[b] = opt_seq_lens[b] - rejected_b (post-verification length);
 *   positions[r] = opt_positions[r] - rejected_{row_req[r]} for the n_rows context rows;
 *   slot_mapping[r] = block_table[req][min(pos / page_size, max_blocks_per_seq - 1)] *
 *     page_size + pos % page_size, or -1 when the corrected position is negative (injection
 *     skips it);
 *   bonus[b] = the last valid entry of prev_out[b] (0 if none), the block's slot-0 token.
 * row_req values are clamped to [0, batch). Shapes: prev_out [batch, prev_num_drafts + 1];
 * opt_seq_lens, seq_lens, bonus [batch]; row_req, opt_positions, positions [n_rows] int32;
 * slot_mapping [n_rows] int64; block_table [batch, max_blocks_per_seq] int32. All device
 * arrays. Requires 0 <= prev_num_drafts <= 63, page_size > 0, max_blocks_per_seq > 0. */
dflash_status dflash_prepare_proposal_inputs(int32_t batch, int32_t prev_num_drafts,
                                             const int32_t *prev_out, int32_t vocab,
                                             const int32_t *opt_seq_lens, int32_t n_rows,
                                             const int32_t *row_req, const int32_t *opt_positions,
                                             const int32_t *block_table,
                                             int32_t max_blocks_per_seq, int32_t page_size,
                                             int32_t *seq_lens, int32_t *positions,
                                             int64_t *slot_mapping, int32_t *bonus, void *stream);

/* Per-kernel timing, for measurement tools. While enabled, every kernel the library launches
 * is bracketed by two hipEvents recorded on the launch's stream. dflash_profile_collect
 * waits for the recorded events and adds each launch's duration to the totals of its kernel
 * (by kernel name). Disabled by default, when no event is recorded. Process-wide and
 * thread-safe. Enabling creates events (host-side runtime objects); the drafting calls still
 * allocate no device memory. */
dflash_status dflash_profile_enable(int32_t on);
/* Restricts the timing to launches whose kernel name is in `names` (comma-separated, copied),
 * so that a timed loop carries events only around the kernels of interest. NULL or ""
 * times every launch (the default). */
dflash_status dflash_profile_filter(const char *names);
dflash_status dflash_profile_collect(void);
void dflash_profile_reset(void);
int32_t dflash_profile_count(void); /* number of distinct kernel names with totals */
/* Totals of entry i < dflash_profile_count(): name (static string), launches, milliseconds. */
dflash_status dflash_profile_entry(int32_t i, const char **name, int64_t *launches, double *total_ms);

const char *dflash_status_string(int32_t status);
const char *dflash_last_error(void); /* thread-local; "" when the last call succeeded */

#ifdef __cplusplus
}
#endif
#endif /* DFLASH_H_ */
