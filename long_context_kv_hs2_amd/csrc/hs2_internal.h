// Internal launch interface between the C ABI (hs2_api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace hs2 {

// ---- full-attention layer: split-K partial pass and merge -------------------
// Most tokens one full-attention workgroup takes (its bound-mode LDS is sized
// by this), and the multiple a chunk is rounded to: one 16-token tile per
// tile stream (4 streams for bf16, 28 for E4M3).
constexpr int kMaxChunkBf16 = 16384;
constexpr int kMaxChunkFp8 = 39 * 448;
constexpr int max_chunk(bool fp8) { return fp8 ? kMaxChunkFp8 : kMaxChunkBf16; }
// bf16 full pass with one wave per SIMD over a batch of equal lengths, a
// sequence with an even number of chunks: the last 1/kEvenXcdDen of its
// tiles go to the workgroups on even XCDs only (they stream faster), which
// thus take (D + 1) tiles for every (D - 1) of the others.
constexpr int kEvenXcdDen = 21;
constexpr int chunk_quantum(bool fp8) { return fp8 ? 448 : 64; }
struct FullParams {
  const int64_t* seq_offsets;
  int64_t total_tokens;
  int64_t max_context;
  const uint8_t* k;          // [N][128] bf16 or E4M3
  const uint8_t* v;
  const float* k_scale;      // [N] (E4M3) or nullptr
  const float* v_scale;
  const float* q;            // [B][16][128]
  float qscale;              // softmax_scale * log2(e)
  int batch;
  int chunk;                 // tokens per workgroup, multiple of 64
  int chunks_per_seq;
  float* partials;           // [B][chunks_per_seq][kPartialFloats]
  float* pstats;             // [B][chunks_per_seq][32]: each partial's (m[16], z[16]) again, packed
  float* spill;              // spill mode: [N][16] log2-domain logits
  uint16_t* shat;            // bound mode: [N] per-token sum over heads of the running-normalised weights, bf16 (RNE)
  float* tile_stats;         // bound mode: [tile_slots][16] per head after each tile: running max - log2(~1/running sum);
                             // tile-sum mode: the running max m_h the tile's weights are taken against
  float* tile_sums;          // tile-sum mode: [tile_slots][16] per head: sum over the tile's tokens of exp2(l_hj - m_h)
  uint32_t* hist0;           // [B][kRadixBins] selection histogram, cleared here
  uint32_t* counters;        // [B][4] selection counters, cleared here
  const int64_t* kv_start;   // [B] first K/V row of each sequence, or nullptr: the row seq_offsets[b]
  int xcd_split;             // 1: bf16 and every sequence of the batch the same length (the even-XCD share)
};
// Slot of tile t (tokens [16t, 16t + 16)) of the sequence starting at row `base`:
// unique over all sequences, at most N/16 + B.
__host__ __device__ inline int64_t tile_slot(int64_t base, int b, int t) { return (base >> 4) + b + t; }
// What the partial pass keeps beside its partials: score bounds (the default
// selection path), every logit (the score path), nothing (full attention
// alone), or per tile and head the sum of the weights (gen-1 block selection
// without per-token scores: a 64-token block is four whole tiles).
enum FullMode { kFullBound = 0, kFullSpill = 1, kFullPlain = 2, kFullTileSums = 3 };
hipError_t launch_full_partial(const FullParams& p, int batch, bool fp8, int mode, hipStream_t s);

struct MergeParams {
  const int64_t* seq_offsets;
  int64_t total_tokens;
  int64_t max_context;
  int budget;
  const float* partials;     // [B][chunks_per_seq][kPartialFloats]
  int chunk;                 // tokens per partial
  int chunks_per_seq;
  int stride_seq;            // floats between sequences' partial blocks
  int stride_chunk;          // floats between partials of one sequence
  int count_from_sel;        // 0: partial count = ceil(L_b / chunk); 1: ceil(sel_count[b] / chunk)
  const int32_t* sel_count;
  float* out;                // [B][16][128] (row b at out + b * out_stride_seq)
  int64_t out_stride_seq;
  float* stats;              // [B][16][2] (m, z) or nullptr
};
hipError_t launch_merge(const MergeParams& p, int batch, hipStream_t s);

// ---- score and token selection ---------------------------------------------
// Gen-1 block-level selection (the ablation comparator): 64-token blocks.
constexpr int kSelectBlock = 64;
constexpr int kTopBlocks = kTopK / kSelectBlock;
struct BlockParams {
  const int64_t* seq_offsets;
  int64_t total_tokens;
  int64_t max_context;
  int batch;
  const float* score;         // [N] per-token scores
  float* block_scores;        // [N / 64 + B]: block i of the sequence at row base_b in slot (base_b >> 6) + b + i
  unsigned long long* group_keys;  // [N / 1024 + B]: largest key of blocks [16 g, 16 g + 16), slot (base_b >> 10) + b + g
  int32_t* sel_idx;           // [B][window + top_k]
  int32_t* sel_count;         // [B]
  // Block sums from the full pass's tile sums (no per-token scores): the
  // pass's pstats give each head's (M, Z); score unused.
  const float* tile_stats;    // [tile_slots][16] m_h of each tile
  const float* tile_sums;     // [tile_slots][16] sum of exp2(l - m_h) over the tile
  const float* pstats;        // [B][chunks_per_seq][32] (m[16], z[16]) per partial
  int chunk;
  int chunks_per_seq;
};
// From given scores: the pool launch, then the selection launch.
hipError_t launch_block_select(const BlockParams& p, hipStream_t s);
// From the tile-sum pass: the full layer's merge and the block sums in one
// launch (mp: the merge); then launch_block_rank, the selection launch.
hipError_t launch_merge_block_pool(const MergeParams& mp, const BlockParams& p, hipStream_t s);
hipError_t launch_block_rank(const BlockParams& p, hipStream_t s);

struct SelectParams {
  const int64_t* seq_offsets;
  int64_t total_tokens;
  int64_t max_context;
  int batch;
  int window, top_k, budget;
  const float* spill;         // [N][16] (spill mode)
  const float* stats;         // [B][16][2] global (max, sum) per head
  const float* pstats;        // [B][chunks_per_seq][32] the full pass's partial (m, z)
  int chunks_per_seq;
  const uint16_t* shat;       // [N] bf16 (bound mode)
  const float* tile_stats;    // [tile_slots][16] (bound mode)
  float* tile_ub;             // [tile_slots][2] (bound mode): max over the tile of shat * max_h F_h, and max_h F_h
  float* score;               // [N]
  uint32_t* hist0;            // [B][kRadixBins]: first-digit histogram
  uint32_t* counters;         // [B][4]: winners emitted, candidates seen
  int32_t* selbuf;            // [B][top_k]: positions emitted so far
  unsigned long long* cand;   // spill mode: [B][kCandCap] threshold-bin keys; bound mode: [N + B * kBoundBlockTokens]
                              // exact candidate keys, one list per sequence or one segment per candidate workgroup
  uint32_t* cand_cnt;         // bound mode: [B][cand_blocks] candidates per candidate workgroup (segmented lists)
  int cand_blocks;            // ceil(longest context / kBoundBlockTokens)
  int32_t* sel_idx;           // [B][budget]
  int32_t* sel_count;         // [B]
  // exact rescoring of candidates (bound mode)
  const uint8_t* k;
  const float* k_scale;
  const float* q;             // [B][16][128]
  float qscale;
  const int64_t* kv_start;    // [B] first K/V row of each sequence, or nullptr: the row seq_offsets[b]
};
constexpr int kRadixBins = 2048;
constexpr int kScoreBlockTokens = 2048;   // tokens per score-pass workgroup
constexpr int kCollectBlockTokens = 8192; // tokens per collect workgroup
constexpr int kBoundBlockTokens = 4096;   // tokens per collect workgroup (one 16-token tile per thread)
constexpr int kMaxCollectBlocks = (1 << 24) / kBoundBlockTokens;  // collect workgroups of the longest context
constexpr int kSharedListBlocks = 128;    // more collect workgroups per sequence: per-workgroup candidate segments
constexpr int64_t kHistLongContext = 1 << 19;  // longer: two tiles per thread in the lower-bound histogram
constexpr int kMinCollectBlocks = 32;     // candidate workgroups per sequence, at least (from 8K tokens on)
constexpr int kCandCap = 32768;           // threshold-bin keys kept per sequence (spill mode)
hipError_t launch_select_init(const SelectParams& p, int batch, hipStream_t s);
// Spill mode: score_j from the spilled logits (compute_score) or read from
// p.score, and the first-digit histogram.
hipError_t launch_score_hist(const SelectParams& p, int batch, int64_t max_context, bool compute_score,
                             bool histogram, hipStream_t s);
hipError_t launch_collect_finish(const SelectParams& p, int batch, int64_t max_context, hipStream_t s);
// Bound mode: the full layer's merge fused with the histogram of the lower
// bounds; then the candidates by upper bound with their exact keys, and the
// exact top-k among them.
hipError_t launch_merge_bound_hist(const MergeParams& mp, const SelectParams& p, int batch, int64_t max_context,
                                   hipStream_t s);
hipError_t launch_bound_select(const SelectParams& p, int batch, int64_t max_context, bool fp8, hipStream_t s);

// ---- sparse layers -----------------------------------------------------------
struct SparseParams {
  const int64_t* seq_offsets;
  int64_t total_tokens;
  int64_t max_context;
  const uint8_t* k;
  const uint8_t* v;
  const float* k_scale;
  const float* v_scale;
  const float* q_sparse;      // [n_s][B][16][128]
  float qscale;
  int batch;
  int n_layers;
  int budget;
  const int32_t* sel_idx;     // [B][budget]
  const int32_t* sel_count;   // [B]
  float* out;                 // [n_layers][B][16][128]
  float* partials;            // [n_layers][B][slices][kPartialFloats] when the selection is sliced
  const int64_t* kv_start;    // [B] first K/V row of each sequence, or nullptr: the row seq_offsets[b]
  // Window mode (sliding-window layers; launch_sparse_window): k, v, k_scale,
  // v_scale are rings of `budget` rows per sequence, position p in slot
  // p mod budget; the window covers min(lengths[b], budget) slots (all once the
  // ring is full, else slots 0 .. L-1); seq_offsets, sel_idx, sel_count unused.
  const int64_t* lengths;     // [B] positions so far, the current token included
  const uint8_t* k_new;       // [B][128] the current token's rows (read in place of its slot), or nullptr
  const uint8_t* v_new;
  const float* k_new_scale;   // [B] (E4M3)
  const float* v_new_scale;
  uint8_t* ring_k;            // writable aliases of k, v, k_scale, v_scale: the current rows are stored there
  uint8_t* ring_v;
  float* ring_ks;
  float* ring_vs;
};
// Slices of each sequence's selection the sparse pass cuts (1: no partials,
// no merge); depends on the batch size only.
int sparse_slices(int batch);
// Attention of every sparse layer over the selected rows, each row gathered
// once for all layers: one launch, plus a merge of the slices when sliced.
hipError_t launch_sparse_attend(const SparseParams& p, bool fp8, hipStream_t s);
// Window mode: one sliding-window layer over ring caches of p.budget (<= 1152)
// rows per sequence, in one unsliced launch that also stores the current rows.
hipError_t launch_sparse_window(const SparseParams& p, bool fp8, hipStream_t s);


// ---- KV bridging ---------------------------------------------------------------
struct BridgeParams {
  int64_t n_tokens;
  int d_model;
  int n_out;                  // 2 * n_bridged column blocks of 128
  const uint16_t* hidden;     // [T][d_model]
  const uint16_t* w_t;        // workspace: [n_out * 128][d_model] (W transposed)
  void* out[8];               // [T][128] each: bf16, or E4M3 codes when fp8
  float* scale[8];            // fp8: [T] per-token scale of each output
  int fp8;                    // 1: E4M3 output with per-token scales
};
hipError_t launch_bridge_transpose_w(const uint16_t* const* w, int n_out, int d_model, uint16_t* w_t,
                                     hipStream_t s);
hipError_t launch_bridge_gemm(const BridgeParams& p, hipStream_t s);

// Decode-time bridging: one hidden row per sequence, appended at its last row.
constexpr int kAppendSliceK = 128;  // d_model rows per split-K slice
constexpr int kMaxAppendDModel = 16384;
struct AppendParams {
  const int64_t* seq_offsets;  // [B + 1]: row seq_offsets[b + 1] - 1 takes sequence b's projection
  int64_t total_tokens;
  int batch;
  int d_model;                 // multiple of kAppendSliceK
  int n_out;                   // 2 * n_bridged output matrices (K0, V0, K1, ...)
  const uint16_t* hidden;      // [B][d_model] bf16
  const uint16_t* w[8];        // [d_model][128] bf16 each
  void* out[8];                // caches [N][128]: bf16, or E4M3 codes when fp8
  float* scale[8];             // fp8: [N] per-token scales
  int fp8;
  float* partials;             // workspace: [d_model / kAppendSliceK][B][n_out * 128]
};
hipError_t launch_bridge_append(const AppendParams& p, hipStream_t s);

// Multi-token decode: T query tokens per sequence, token t a decode step of
// its own over the causal prefix [0, L_b - T + t]; run as a batch of B * T
// virtual sequences whose workspace ranges are disjoint and whose K/V rows
// start at their real sequence's first row.
constexpr int kMaxQueryTokens = 16;
struct MultiParams {
  const int64_t* seq_offsets;  // [B + 1] real sequences
  int64_t total_tokens;
  int64_t max_context;
  int batch;
  int n_query;                 // T
  int64_t* voffs;              // [B * T + 1] virtual offsets (prefix lengths, packed)
  int64_t* kv_start;           // [B * T] real first row of each virtual sequence
};
hipError_t launch_multi_prep(const MultiParams& p, hipStream_t s);
// The bound-mode full pass for a group of up to kMultiQ of the T tokens of
// every sequence, reading each K/V row once for the group.  f holds the real
// batch (seq_offsets, batch, total_tokens, max_context, k, v, scales) and the
// virtual batch's outputs (q [B T][16][128], partials, pstats, shat,
// tile_stats, hist0, counters, chunks_per_seq); f.chunk is the real batch's.
constexpr int kMultiQ = 4;
struct MultiFullParams {
  FullParams f;
  const int64_t* voffs;  // [B T + 1] virtual offsets (multi_prep_kernel)
  int n_query;           // T
  int t_first;           // the group's first token
  int nq;                // tokens in the group, 1..kMultiQ
  int fp8;
};
hipError_t launch_full_multi(const MultiFullParams& p, hipStream_t s);

}  // namespace hs2
