/*
 * hs2.h - C ABI of libhs2.so: the HySparse2 hybrid-block decode path and the
 * KV-Bridging projection on one MI355X (gfx950).
 *
 * The operations (the pages are news reports of arXiv 2609.26368):
 *  - A hybrid block is one full-attention layer followed by several sparse-
 *    attention layers; the full layer picks positions from its attention
 *    scores and the sparse layers reuse its KV cache and its selection
 *    (toolnavs.com article 2080, section "Ce que fait HySparse2" (fr) /
 *    "HySparse2가 한 일" (ko); "Luo Fuli Teases Xiaomi MiMo-V3 Architecture"
 *    (ai.synthepulse.app), paragraphs on KV Reuse and on token selection).
 *  - The selection is token-level: the 128 most recent positions always, plus
 *    1024 positions from before that window (readaitime.com news of
 *    2026-09-24, paragraph on dropping the separate SWA branch; the toolnavs
 *    sections above).
 *  - KV Bridging: each bridged full-attention layer builds its own K and V
 *    from one shared self-decoder hidden state with its own projections
 *    (toolnavs.com (ko), section "HySparse2가 한 일").
 *
 * Readings taken where the pages are silent: softmax scale 1/sqrt(head_dim);
 * per-token score = sum over query heads of the softmax probability over the
 * whole context; window = the last 128 positions, current token included;
 * top-k taken from the positions before the window; ties to the lower
 * position; a context of at most window + top_k tokens selects every token;
 * one selection per sequence (MQA: one KV head).
 *
 * Conventions for every call:
 *  - Pointers marked (device) are device memory on the current HIP device;
 *    pointers marked (host) are host memory read during the call only.
 *  - The caller owns every buffer.  The library allocates no device memory,
 *    keeps no pointer after returning, and never synchronises: work is
 *    enqueued on `stream` (a hipStream_t passed as void*, NULL = the null
 *    stream) and buffers must stay alive until that stream has run it.
 *  - Every argument is validated before any HIP call; a failed check returns
 *    HS2_ERR_INVALID_ARGUMENT, HS2_ERR_UNSUPPORTED or
 *    HS2_ERR_WORKSPACE_TOO_SMALL and enqueues nothing.  A failed launch
 *    returns HS2_ERR_HIP.  hs2_last_error_message() (thread-local) explains
 *    the last non-OK status.  No C++ exception crosses the ABI.
 *  - Identical inputs give bitwise-identical outputs (fixed reduction order).
 *  - Calls that share a workspace must not overlap in time.
 */
#ifndef HS2_H
#define HS2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  HS2_OK = 0,
  HS2_ERR_INVALID_ARGUMENT = 1,
  HS2_ERR_UNSUPPORTED = 2,
  HS2_ERR_WORKSPACE_TOO_SMALL = 3,
  HS2_ERR_HIP = 4
} hs2_status;

typedef enum {
  HS2_KV_BF16 = 0,     /* bfloat16 rows, 2 bytes per element                     */
  HS2_KV_FP8_E4M3 = 1  /* OCP E4M3 codes, 1 byte per element, with per-token fp32
                          scales: value = E4M3(code) * scale[token]             */
} hs2_kv_dtype;

/* Shape of one decode call (host struct, passed by pointer).
 * Supported: n_q_heads 16, head_dim 128, window 128, top_k 1024,
 * n_sparse_layers 0..8, batch >= 0, max_context <= 2^24.                     */
typedef struct {
  int32_t batch;            /* B sequences                                       */
  int32_t n_q_heads;        /* query heads sharing the one KV head (16)          */
  int32_t head_dim;         /* D (128)                                           */
  int32_t window;           /* recent positions always selected (128)            */
  int32_t top_k;            /* positions selected before the window (1024)       */
  int32_t n_sparse_layers;  /* n_s sparse layers reusing the selection (0..8)    */
  int32_t kv_dtype;         /* hs2_kv_dtype                                      */
  float softmax_scale;      /* multiplies q.k; 1/sqrt(head_dim) in the workloads */
  int64_t total_tokens;     /* N = seq_offsets[B] (host-known; sizes buffers)    */
  int64_t max_context;      /* >= every L_b (host-known; sizes the grids)        */
} hs2_decode_desc;

/* Bytes of workspace for `desc` (0 when desc is invalid):
 *  - hs2_decode_workspace_bytes: hs2_decode_block with score_out == NULL, and
 *    hs2_decode_block_gen1, hs2_topk_select, hs2_block_select,
 *    hs2_sparse_decode, hs2_full_decode;
 *  - hs2_decode_score_workspace_bytes: the calls that return per-token scores,
 *    hs2_decode_block with score_out != NULL and hs2_full_decode_score; it adds
 *    64 bytes a token (every logit of the full layer) to the first size.
 * A workspace of the larger size serves every call.                          */
size_t hs2_decode_workspace_bytes(const hs2_decode_desc* desc);
size_t hs2_decode_score_workspace_bytes(const hs2_decode_desc* desc);

/* One decode step of one hybrid block for a packed batch.
 *
 * seq_offsets (device) int64 [B+1]: sequence b owns cache rows
 *   [seq_offsets[b], seq_offsets[b+1]); L_b = their difference, 0 <= L_b <=
 *   max_context; seq_offsets[B] == total_tokens; the current token's K/V is
 *   already stored at position L_b - 1.
 * k_cache, v_cache (device): [N][head_dim] rows, bf16 or E4M3 per kv_dtype,
 *   16-byte aligned.  This is the shared MQA cache of the block's full layer.
 * k_scale, v_scale (device) fp32 [N]: per-token scales (E4M3 only, else NULL).
 * q_full (device) fp32 [B][n_q_heads][head_dim]: the full layer's query.
 * q_sparse (device) fp32 [n_s][B][n_q_heads][head_dim]: each sparse layer's
 *   query (NULL when n_s == 0).
 * o_full (device) fp32 [B][n_q_heads][head_dim]: full-attention output.
 * o_sparse (device) fp32 [n_s][B][n_q_heads][head_dim]: each sparse layer's
 *   attention over the selected rows of the shared cache.
 * sel_idx (device) int32 [B][window + top_k]: selected positions within the
 *   sequence, ascending, padded with -1.
 * sel_count (device) int32 [B]: min(L_b, window + top_k).
 * score_out (device) fp32 [N] or NULL: per-token score (sum over heads of the
 *   softmax probability), for every position of every sequence.
 * workspace (device), workspace_bytes >= hs2_decode_workspace_bytes(desc)
 *   (hs2_decode_score_workspace_bytes(desc) when score_out != NULL), 256-byte
 *   aligned; its contents on entry do not matter.
 * A sequence with L_b == 0 yields zero outputs, sel_count 0 and all -1.      */
hs2_status hs2_decode_block(const hs2_decode_desc* desc, const int64_t* seq_offsets,
                            const void* k_cache, const void* v_cache,
                            const float* k_scale, const float* v_scale,
                            const float* q_full, const float* q_sparse,
                            float* o_full, float* o_sparse,
                            int32_t* sel_idx, int32_t* sel_count, float* score_out,
                            void* workspace, size_t workspace_bytes, void* stream);

/* hs2_decode_block (score_out NULL) for callers that cannot allocate device
 * memory, such as code under HIP graph capture, tight serving loops or
 * harnesses that forbid allocation: the workspace is a device array of the
 * library's own, HS2_NOALLOC_SCRATCH_BYTES long, which each GPU the library
 * runs on holds until the process ends (looked up on the first call on that
 * device).  Arguments, outputs, errors and results (bit for bit) as
 * hs2_decode_block with score_out == NULL.  A shape whose
 * hs2_decode_workspace_bytes exceeds HS2_NOALLOC_SCRATCH_BYTES is rejected
 * with HS2_ERR_UNSUPPORTED before any HIP call (96 MiB covers, with 4 sparse
 * layers, 32 sequences of 131072 tokens (bf16) or 4 of 1048576 (E4M3), and
 * 8 of 32768).  Every call on one GPU shares that GPU's array: calls
 * that overlap in time on one GPU (other streams, other threads) race and
 * must not be made.  The array's contents on entry do not matter.           */
#define HS2_NOALLOC_SCRATCH_BYTES (96u << 20)
hs2_status hs2_decode_block_noalloc(const hs2_decode_desc* desc, const int64_t* seq_offsets,
                                    const void* k_cache, const void* v_cache,
                                    const float* k_scale, const float* v_scale,
                                    const float* q_full, const float* q_sparse,
                                    float* o_full, float* o_sparse,
                                    int32_t* sel_idx, int32_t* sel_count, void* stream);

/* One decode step of the hybrid block with gen-1 (block-level) selection in
 * place of the token-level one, without per-token scores: the comparator
 * the pages' ablation sets against the token-level selection at the same
 * attention budget ("Luo Fuli Teases Xiaomi MiMo-V3 Architecture",
 * paragraphs on how the sparse layers select and on the ablation;
 * readaitime.com news of 2026-09-24, paragraph on block versus token
 * selection).  Sequence b selects the last `window` positions plus the
 * top_k / 64 = 16 complete 64-token blocks [64 i, 64 i + 64) that end before
 * the window, ranked by the sum of their positions' scores (descending; ties
 * to the lower block), as hs2_full_decode_score, hs2_block_select and
 * hs2_sparse_decode do in three calls; a context of at most window + top_k
 * positions selects every position.  Here the full layer keeps, per 16-token
 * tile and head, the sum of its softmax weights instead of every logit, and
 * the block sums are formed from those after the merge; they agree with the
 * per-token route's up to fp32 rounding order (relative ~1e-6), so the two
 * lists can differ only between blocks whose sums tie that closely.
 * Arguments, outputs (o_full, o_sparse, sel_idx, sel_count), workspace
 * (hs2_decode_workspace_bytes(desc)) and errors as hs2_decode_block with
 * score_out == NULL.  Stage timing records all four stages (2: the block
 * ranking).                                                                  */
hs2_status hs2_decode_block_gen1(const hs2_decode_desc* desc, const int64_t* seq_offsets,
                                 const void* k_cache, const void* v_cache,
                                 const float* k_scale, const float* v_scale,
                                 const float* q_full, const float* q_sparse,
                                 float* o_full, float* o_sparse,
                                 int32_t* sel_idx, int32_t* sel_count,
                                 void* workspace, size_t workspace_bytes, void* stream);

/* Multi-token decode (speculative verification): n_query = T query tokens
 * per sequence in one step.  The pages give no multi-token rule for
 * HySparse2; the reading taken: the T tokens are the sequence's last T cache
 * rows (already stored), and token t, at position L_b - T + t, is a decode
 * step of its own over the causal prefix [0, L_b - T + t], with its own
 * selection (window and top-k as hs2_decode_block).  Arguments as
 * hs2_decode_block with the token index after the sequence index:
 *   q_full, o_full fp32 [B][T][16][128]; q_sparse, o_sparse fp32
 *   [n_s][B][T][16][128]; sel_idx int32 [B][T][window + top_k];
 *   sel_count int32 [B][T].
 * A token whose position would be below 0 (L_b < T) gets zero outputs and
 * sel_count 0.  Supported: 1 <= n_query <= 16, batch * n_query <= 2^24.
 * workspace >= hs2_decode_multi_workspace_bytes(desc, n_query) (it grows
 * with T: each token keeps its own scores and candidates).  Every token
 * streams its prefix's K/V rows (T x the full layer's bytes at most).      */
size_t hs2_decode_multi_workspace_bytes(const hs2_decode_desc* desc, int32_t n_query);
hs2_status hs2_decode_multi(const hs2_decode_desc* desc, int32_t n_query, const int64_t* seq_offsets,
                            const void* k_cache, const void* v_cache,
                            const float* k_scale, const float* v_scale,
                            const float* q_full, const float* q_sparse,
                            float* o_full, float* o_sparse,
                            int32_t* sel_idx, int32_t* sel_count,
                            void* workspace, size_t workspace_bytes, void* stream);

/* Stage call: the full-attention layer alone.  Same arguments as
 * hs2_decode_block; writes o_full and score_out (required here).  workspace
 * >= hs2_decode_score_workspace_bytes(desc).                                 */
hs2_status hs2_full_decode_score(const hs2_decode_desc* desc, const int64_t* seq_offsets,
                                 const void* k_cache, const void* v_cache,
                                 const float* k_scale, const float* v_scale,
                                 const float* q_full, float* o_full, float* score_out,
                                 void* workspace, size_t workspace_bytes, void* stream);

/* Stage call: token selection from given scores.  score (device) fp32 [N]
 * non-negative (-0.0, negative values and NaN are ranked as +0.0); writes
 * sel_idx and sel_count as hs2_decode_block does: the last `window` positions
 * plus the top_k positions before them by (score descending, position
 * ascending).  seq_offsets 8-byte aligned.                                    */
hs2_status hs2_topk_select(const hs2_decode_desc* desc, const int64_t* seq_offsets,
                           const float* score, int32_t* sel_idx, int32_t* sel_count,
                           void* workspace, size_t workspace_bytes, void* stream);

/* Stage call: gen-1 (block-level) selection from given scores, the
 * comparator the pages' ablation sets against the token-level selection at
 * the same attention budget ("Luo Fuli Teases Xiaomi MiMo-V3 Architecture",
 * paragraphs on how the sparse layers select and on the ablation;
 * readaitime.com news of 2026-09-24, paragraph on block versus token
 * selection).  Sequence b selects the last `window` positions plus the
 * top_k / 64 = 16 complete 64-token blocks [64 i, 64 i + 64) that end before
 * the window, ranked by the sum of their positions' scores (descending;
 * ties to the lower block); a context of at most window + top_k positions
 * selects every position.  Arguments, workspace, errors and output format
 * (ascending, -1 padded, sel_count = min(L_b, window + top_k)) as
 * hs2_topk_select.  hs2_full_decode_score, then this, then
 * hs2_sparse_decode is the hybrid block with gen-1 selection.               */
hs2_status hs2_block_select(const hs2_decode_desc* desc, const int64_t* seq_offsets,
                            const float* score, int32_t* sel_idx, int32_t* sel_count,
                            void* workspace, size_t workspace_bytes, void* stream);

/* Stage call: the sparse layers over a given selection.  desc->n_sparse_layers
 * queries in q_sparse; sel_idx/sel_count as written by hs2_topk_select (the
 * caller may keep them across calls: one selection serves every layer).
 * With n_sparse_layers == 1 this is one sparse layer at a time.              */
hs2_status hs2_sparse_decode(const hs2_decode_desc* desc, const int64_t* seq_offsets,
                             const void* k_cache, const void* v_cache,
                             const float* k_scale, const float* v_scale,
                             const float* q_sparse, const int32_t* sel_idx,
                             const int32_t* sel_count, float* o_sparse,
                             void* workspace, size_t workspace_bytes, void* stream);

/* KV-Bridging projection: for l in [0, n_bridged):
 *   k_out[l] = hidden . w_k[l],  v_out[l] = hidden . w_v[l]
 * hidden (device) bf16 [n_tokens][d_model] row-major;
 * w_k, w_v (host arrays of n_bridged device pointers) bf16 [d_model][head_dim];
 * k_out, v_out (host arrays of n_bridged device pointers) bf16
 *   [n_tokens][head_dim]; fp32 accumulation, round-to-nearest-even output.
 * Supported: head_dim 128, d_model a positive multiple of 64,
 * 1 <= n_bridged <= 4, n_tokens >= 0.  All device pointers 16-byte aligned.
 * workspace (device) >= hs2_bridge_workspace_bytes(...), 256-byte aligned.  */
size_t hs2_bridge_workspace_bytes(int64_t n_tokens, int32_t d_model, int32_t head_dim,
                                  int32_t n_bridged);
hs2_status hs2_bridge_kv(int64_t n_tokens, int32_t d_model, int32_t head_dim, int32_t n_bridged,
                         const void* hidden, const void* const* w_k, const void* const* w_v,
                         void* const* k_out, void* const* v_out,
                         void* workspace, size_t workspace_bytes, void* stream);

/* KV-Bridging projection writing the FP8 cache the pages' 1M-token
 * footprints assume ([en] paragraph on cost; [pt]): the same products as
 * hs2_bridge_kv, each output row (one token of one matrix) stored as OCP
 * E4M3 codes with an fp32 scale: scale = (largest |value| of the row) / 448
 * (1 for an all-zero row), code = E4M3(value / scale), round to nearest,
 * ties to even, saturating at +-448; values from the fp32 products.
 * k_out, v_out (host arrays of n_bridged device pointers) uint8
 *   [n_tokens][head_dim]; k_scale, v_scale (host arrays of n_bridged device
 *   pointers) fp32 [n_tokens], 4-byte aligned.  These are the cache and
 *   scale arrays hs2_decode_block reads with kv_dtype HS2_KV_FP8_E4M3.
 * Same support, workspace and errors as hs2_bridge_kv; NULL scale arrays:
 * HS2_ERR_INVALID_ARGUMENT.                                                   */
hs2_status hs2_bridge_kv_fp8(int64_t n_tokens, int32_t d_model, int32_t head_dim, int32_t n_bridged,
                             const void* hidden, const void* const* w_k, const void* const* w_v,
                             void* const* k_out, float* const* k_scale,
                             void* const* v_out, float* const* v_scale,
                             void* workspace, size_t workspace_bytes, void* stream);

/* The bridge projection with its weights packed once per weight set, for a
 * caller that runs it on many hidden-state batches with the same W_k, W_v
 * (the pages' prefill computes every bridged layer's K and V from one
 * hidden state: [ko] "HySparse2가 한 일"; [fr] "Le Prefill s'arrête à
 * mi-chemin").  hs2_bridge_kv and hs2_bridge_kv_fp8 pack the weights into
 * their workspace on every call; these entry points split that step off.
 *
 * hs2_bridge_pack_weights: writes the 2 * n_bridged matrices w_k[0], w_v[0],
 * w_k[1], ... (host arrays of device pointers, bf16 [d_model][head_dim],
 * 16-byte aligned) into packed (device, 256-byte aligned, caller-owned,
 * >= hs2_bridge_packed_weight_bytes(...) bytes) in the layout the GEMM
 * reads: [2 * n_bridged * head_dim][d_model], the reduction dimension
 * contiguous.  Asynchronous on stream.  Same support and errors as
 * hs2_bridge_kv; a short buffer: HS2_ERR_WORKSPACE_TOO_SMALL.
 *
 * hs2_bridge_kv_packed: the projection from packed weights, no workspace.
 * kv_dtype HS2_KV_BF16: the outputs of hs2_bridge_kv (k_scale and v_scale
 * unused, may be NULL); HS2_KV_FP8_E4M3: those of hs2_bridge_kv_fp8.  The
 * results are bit-identical to those entry points'.  packed must hold the
 * packing of the weights for this d_model and n_bridged; nothing checks
 * that.                                                                       */
size_t hs2_bridge_packed_weight_bytes(int32_t d_model, int32_t head_dim, int32_t n_bridged);
hs2_status hs2_bridge_pack_weights(int32_t d_model, int32_t head_dim, int32_t n_bridged,
                                   const void* const* w_k, const void* const* w_v,
                                   void* packed, size_t packed_bytes, void* stream);
hs2_status hs2_bridge_kv_packed(int64_t n_tokens, int32_t d_model, int32_t head_dim, int32_t n_bridged,
                                int32_t kv_dtype, const void* hidden, const void* packed,
                                void* const* k_out, float* const* k_scale,
                                void* const* v_out, float* const* v_scale, void* stream);

/* Self-Decoder layers at decode.  The model's front half (the Self-Decoder)
 * mixes full-attention and sliding-window layers; in the pages' 49-layer
 * model the first 25 layers hold one full-attention layer, whose input hidden
 * state is the bridge source ([fr] "Ce que fait HySparse2" and "Le Prefill
 * s'arrête à mi-chemin"; [en] paragraphs on the self-decoder split and on
 * early prefill exit).
 *
 * hs2_full_decode: the Self-Decoder's full-attention layer: full attention
 * alone (o_full), no score and no selection: the workspace receives the
 * split-K partials only.  Arguments, workspace and errors as
 * hs2_decode_block.  Stage timing records stages 0 and 1.
 *
 * hs2_swa_decode: one sliding-window layer for a batch: each sequence's
 * query attends to its `window` most recent positions, the current token
 * included (the pages give no window size; the workloads use 128, the local
 * window the pages do give).  The layer's cache is a ring per sequence:
 *   ring_k, ring_v (device) [batch][window][128] rows, bf16 or E4M3 codes per
 *     kv_dtype, 16-byte aligned; position p lives in slot p mod window;
 *   ring_k_scale, ring_v_scale (device) fp32 [batch][window] (E4M3), else NULL;
 *   lengths (device) int64 [batch]: positions so far, the current one
 *     included (0: zero output);
 *   k_new, v_new (device, 16-byte aligned) [batch][128] the current token's
 *     rows (with k_new_scale, v_new_scale fp32 [batch] for E4M3): attended in
 *     place of slot (lengths[b] - 1) mod window and stored there, by the same
 *     launch; NULL when the caller has already written them into the ring;
 *   q (device) fp32 [batch][16][128]; o (device) fp32 [batch][16][128];
 *   softmax_scale multiplies q.k (1/sqrt(128) in the workloads).
 * Supported: 1 <= window <= 1152, 16 query heads, head_dim 128.  No
 * workspace.  Calls on the same ring must not overlap.                      */
hs2_status hs2_full_decode(const hs2_decode_desc* desc, const int64_t* seq_offsets,
                           const void* k_cache, const void* v_cache,
                           const float* k_scale, const float* v_scale,
                           const float* q_full, float* o_full,
                           void* workspace, size_t workspace_bytes, void* stream);
hs2_status hs2_swa_decode(int32_t batch, int32_t window, int32_t kv_dtype, float softmax_scale,
                          const int64_t* lengths, void* ring_k, void* ring_v,
                          float* ring_k_scale, float* ring_v_scale,
                          const void* k_new, const void* v_new,
                          const float* k_new_scale, const float* v_new_scale,
                          const float* q, float* o, void* stream);

/* Decode-time KV Bridging: each decode step, the current token's hidden
 * state is projected by every bridged layer's W_k and W_v (the products of
 * hs2_bridge_kv, one row per sequence) and written into that layer's cache at
 * the current token's row, seq_offsets[b + 1] - 1, where hs2_decode_block
 * reads it (toolnavs.com (ko), section "HySparse2가 한 일"; [en] paragraph on
 * KV Bridging).  Sequences with L_b == 0 are skipped; no other row changes.
 * hidden (device) bf16 [batch][d_model]; w_k, w_v (host arrays of n_bridged
 *   device pointers) bf16 [d_model][head_dim];
 * k_cache, v_cache (host arrays of n_bridged device pointers, 16-byte
 *   aligned) [total_tokens]
 *   [head_dim] rows, bf16 or E4M3 codes per kv_dtype (hs2_kv_dtype);
 * k_scale, v_scale (host arrays of device pointers) fp32 [total_tokens] for
 *   E4M3 (the row's scale is written: row max |value| / 448, 1 for a zero
 *   row, codes rounded to nearest even and saturated, as hs2_bridge_kv_fp8),
 *   NULL for bf16 (round to nearest even).
 * seq_offsets (device) int64 [batch + 1], as in hs2_decode_block.
 * Supported: head_dim 128, d_model a multiple of 128 up to 16384,
 * 1 <= n_bridged <= 4, batch >= 0.  workspace (device) >=
 * hs2_bridge_append_workspace_bytes(...), 256-byte aligned.  fp32
 * accumulation; the summation order differs from hs2_bridge_kv's, so a row
 * can differ from the prefill bridge's in the last bit.                     */
size_t hs2_bridge_append_workspace_bytes(int32_t batch, int32_t d_model, int32_t head_dim,
                                         int32_t n_bridged);
hs2_status hs2_bridge_append(int32_t batch, int32_t d_model, int32_t head_dim, int32_t n_bridged,
                             int32_t kv_dtype, const int64_t* seq_offsets, int64_t total_tokens,
                             const void* hidden, const void* const* w_k, const void* const* w_v,
                             void* const* k_cache, void* const* v_cache,
                             float* const* k_scale, float* const* v_scale,
                             void* workspace, size_t workspace_bytes, void* stream);

/* Per-stage kernel timing of hs2_decode_block and hs2_full_decode_score, for
 * benchmarks.  Mode 1: each call records HIP events around its stages on its
 * stream (HS2_N_STAGES stages: 0 full-attention partial pass, 1 full-attention
 * merge (with the selection's first pass when no score is returned), 2 score
 * and selection (hs2_full_decode_score: the score pass), 3 sparse layers
 * (hs2_full_decode_score: none)).  Mode 2: only the events around stages 0 and
 * 1 (each marker costs the step about 1.5 us).  Mode 0: off.  Other modes:
 * HS2_ERR_INVALID_ARGUMENT.  The events are timing-only (no system-scope
 * fence).  At most 1024 calls are recorded between reads.
 * Process-global state: the mode and the record are shared by every thread
 * and device (guarded by a mutex); with timing on, calls from several threads
 * land in one record in the order they take it.  With timing off (the
 * default) the calls keep no state (hs2_decode_block_noalloc aside, which
 * keeps its scratch array's address per device).
 * hs2_stage_timing_read waits for the recorded events and returns, per stage,
 * the mean duration in milliseconds over the calls recorded since the last
 * read (a stage a call did not record counts as 0), and the number of calls
 * in *n_calls; it then clears the record.  hs2_stage_timing_read_calls does
 * the same but writes each call's durations, ms[r * HS2_N_STAGES + stage] for
 * the first max_calls calls r (host array), instead of the means.           */
#define HS2_N_STAGES 4
hs2_status hs2_stage_timing_enable(int32_t mode);
hs2_status hs2_stage_timing_read(float* mean_ms /* [HS2_N_STAGES] (host) */, int32_t* n_calls);
hs2_status hs2_stage_timing_read_calls(float* ms /* [max_calls][HS2_N_STAGES] (host) */, int32_t max_calls,
                                       int32_t* n_calls);

const char* hs2_status_string(hs2_status status);
const char* hs2_last_error_message(void);

#ifdef __cplusplus
}
#endif

#endif /* HS2_H */
