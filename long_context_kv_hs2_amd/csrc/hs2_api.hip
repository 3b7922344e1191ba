// C ABI of libhs2.so: argument validation (before any HIP call), workspace
// layout, and the launch sequence of each entry point.  See include/hs2.h.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include "hs2.h"
#include "hs2_device.h"
#include "hs2_internal.h"

namespace {

using namespace hs2;

thread_local char g_err[512] = "";

hs2_status fail(hs2_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
hs2_status fail(hs2_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

hs2_status hip_fail(hipError_t e, const char* what) {
  return fail(HS2_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr double kLog2e = 1.4426950408889634;
constexpr int64_t kMaxContext = int64_t(1) << 24;

size_t align_up(size_t x) { return (x + 255) & ~size_t(255); }
bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Tokens per full-attention workgroup.  The pass runs best as one round of
// workgroups, one per CU of a 256-CU part: a workgroup's end (writing its
// per-tile outputs, merging its waves) overlaps no streaming, so it should
// happen once, and a partly filled second round would leave CUs idle.  (Two
// co-resident workgroups progress unevenly: on each SIMD the older wave's
// loads are served first, so the younger workgroup streams the last part of
// the pass alone at a lower rate.  Within one workgroup the kernel deals the
// tiles to match.)  A batch takes sum_b ceil(L_b / chunk) < N / chunk + B
// workgroups, so chunk >= N / (256 - B) keeps them within the round.  Chunks
// are multiples of chunk_quantum in [256, max_chunk].  The choice affects
// speed, and the rounding of the outputs (never the selection), and depends
// on nothing but N, B and the cache type.
int choose_chunk(int64_t total_tokens, int64_t max_context, int batch, bool fp8) {
  constexpr int64_t kSlots = 256;
  const int64_t denom = std::max<int64_t>(kSlots - batch, kSlots / 4);
  const int64_t quantum = chunk_quantum(fp8);
  auto round_up = [&](int64_t c) { return (c + quantum - 1) / quantum * quantum; };
  int64_t c = round_up((total_tokens + denom - 1) / denom);
  // Every sequence the same length (total = batch x longest, known here): the
  // smallest chunk that still gives each sequence at most kSlots / batch items
  // fills the slots exactly, where the rule above leaves room for a ragged tail
  // per sequence (4 x 1M tokens: 256 items of 16576 tokens, not 248 of 17024).
  if (batch > 0 && batch <= kSlots && max_context > 0 && total_tokens == static_cast<int64_t>(batch) * max_context) {
    const int64_t per = kSlots / batch;
    c = std::min(c, round_up((max_context + per - 1) / per));
  }
  return static_cast<int>(std::min<int64_t>(std::max<int64_t>(c, 256), max_chunk(fp8)));
}

struct DecodeLayout {
  int chunk = 0;
  int chunks_per_seq = 0;
  size_t partials = 0, stats = 0, pstats = 0, spill = 0, hist0 = 0, counters = 0, selbuf = 0, cand = 0, shat = 0,
         tile_stats = 0, tile_ub = 0, cand_cnt = 0, sparse = 0, blocks = 0, groups = 0, tile_sums = 0, total = 0;
  int cand_blocks = 0;
};

// with_spill: room for the score path's logits ([N][16] fp32, 64 bytes a
// token), only for calls that return per-token scores.  It comes last, so the
// layout without it is a prefix of the layout with it.
// chunk: the full pass's chunk when another batch sets it (multi-token
// decode: the real batch's), else 0 for this batch's own.
DecodeLayout decode_layout(const hs2_decode_desc& d, bool with_spill, int chunk = 0) {
  DecodeLayout L;
  const size_t B = static_cast<size_t>(d.batch);
  const size_t N = static_cast<size_t>(d.total_tokens);
  L.chunk = chunk > 0 ? chunk : choose_chunk(d.total_tokens, d.max_context, d.batch, d.kv_dtype == HS2_KV_FP8_E4M3);
  L.chunks_per_seq = static_cast<int>((d.max_context + L.chunk - 1) / L.chunk);
  if (L.chunks_per_seq < 1) L.chunks_per_seq = 1;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes);
    return at;
  };
  L.partials = take(B * L.chunks_per_seq * kPartialFloats * sizeof(float));
  L.stats = take(B * kHeads * 2 * sizeof(float));
  L.pstats = take(B * L.chunks_per_seq * 2 * kHeads * sizeof(float));
  L.hist0 = take(B * kRadixBins * sizeof(uint32_t));
  L.counters = take(B * 4 * sizeof(uint32_t));
  L.selbuf = take(B * kTopK * sizeof(int32_t));
  // spill mode: [B][kCandCap] keys of the threshold bin; bound mode: one slot
  // per position (every candidate's exact key, sequence b's from row base_b)
  L.cand = take(std::max(B * kCandCap, N + B * kBoundBlockTokens) * sizeof(unsigned long long));
  L.cand_blocks = static_cast<int>(std::max<int64_t>((d.max_context + kBoundBlockTokens - 1) / kBoundBlockTokens, 1));
  L.cand_cnt = take(B * static_cast<size_t>(L.cand_blocks) * sizeof(uint32_t));
  // gen-1 selection from the tile-sum pass: the per-tile head sums,
  // ((N >> 4) + B + 1) x 16 floats (<= 4 N + 64 (B + 1) bytes), live in the
  // candidate slots (>= 8 N + 8 * 4096 B bytes), which that path leaves unused
  L.tile_sums = L.cand;
  L.shat = take(N * sizeof(uint16_t));
  L.tile_stats = take(((N >> 4) + B + 1) * kHeads * sizeof(float));
  L.tile_ub = take(((N >> 4) + B + 1) * 2 * sizeof(float));
  const int n_sparse = d.n_sparse_layers > 0 ? d.n_sparse_layers : 1;
  const int slices = sparse_slices(d.batch);
  L.sparse = take(slices > 1 ? B * n_sparse * static_cast<size_t>(slices) * kPartialFloats * sizeof(float) : 0);
  L.blocks = take(((N >> 6) + B + 1) * sizeof(float));  // gen-1 block selection: per-block score sums
  L.groups = take(((N >> 10) + B + 1) * sizeof(unsigned long long));  // and each 16-block group's largest key
  L.spill = with_spill ? take(N * kHeads * sizeof(float)) : off;
  L.total = off;
  return L;
}

hs2_status check_desc(const hs2_decode_desc* d) {
  if (!d) return fail(HS2_ERR_INVALID_ARGUMENT, "desc is NULL");
  if (d->batch < 0) return fail(HS2_ERR_INVALID_ARGUMENT, "batch %d < 0", d->batch);
  if (d->n_q_heads != kHeads) return fail(HS2_ERR_UNSUPPORTED, "n_q_heads %d (only 16 is supported)", d->n_q_heads);
  if (d->head_dim != kDim) return fail(HS2_ERR_UNSUPPORTED, "head_dim %d (only 128 is supported)", d->head_dim);
  if (d->window != kWindow) return fail(HS2_ERR_UNSUPPORTED, "window %d (only 128 is supported)", d->window);
  if (d->top_k != kTopK) return fail(HS2_ERR_UNSUPPORTED, "top_k %d (only 1024 is supported)", d->top_k);
  if (d->n_sparse_layers < 0 || d->n_sparse_layers > 8)
    return fail(HS2_ERR_UNSUPPORTED, "n_sparse_layers %d (0..8 supported)", d->n_sparse_layers);
  if (d->kv_dtype != HS2_KV_BF16 && d->kv_dtype != HS2_KV_FP8_E4M3)
    return fail(HS2_ERR_INVALID_ARGUMENT, "kv_dtype %d unknown", d->kv_dtype);
  if (!(d->softmax_scale > 0.f) || !isfinite(d->softmax_scale))
    return fail(HS2_ERR_INVALID_ARGUMENT, "softmax_scale must be finite and > 0");
  if (d->total_tokens < 0) return fail(HS2_ERR_INVALID_ARGUMENT, "total_tokens < 0");
  if (d->max_context < 0 || d->max_context > kMaxContext)
    return fail(HS2_ERR_UNSUPPORTED, "max_context %lld outside [0, 2^24]", static_cast<long long>(d->max_context));
  if (d->total_tokens > static_cast<int64_t>(d->batch) * d->max_context)
    return fail(HS2_ERR_INVALID_ARGUMENT, "total_tokens exceeds batch * max_context");
  return HS2_OK;
}

hs2_status check_kv(const hs2_decode_desc& d, const int64_t* offs, const void* k, const void* v, const float* ks,
                    const float* vs) {
  if (d.batch > 0 && !offs) return fail(HS2_ERR_INVALID_ARGUMENT, "seq_offsets is NULL");
  if (offs && !aligned(offs, 8)) return fail(HS2_ERR_INVALID_ARGUMENT, "seq_offsets not 8-byte aligned");
  if (d.total_tokens > 0) {
    if (!k || !v) return fail(HS2_ERR_INVALID_ARGUMENT, "k_cache/v_cache is NULL");
    if (!aligned(k, 16) || !aligned(v, 16)) return fail(HS2_ERR_INVALID_ARGUMENT, "k_cache/v_cache not 16-byte aligned");
    if (d.kv_dtype == HS2_KV_FP8_E4M3) {
      if (!ks || !vs) return fail(HS2_ERR_INVALID_ARGUMENT, "E4M3 cache needs k_scale and v_scale");
      if (!aligned(ks, 4) || !aligned(vs, 4)) return fail(HS2_ERR_INVALID_ARGUMENT, "scales not 4-byte aligned");
    }
  }
  if (d.kv_dtype == HS2_KV_BF16 && (ks || vs))
    return fail(HS2_ERR_INVALID_ARGUMENT, "bf16 cache takes no scales (pass NULL)");
  return HS2_OK;
}

hs2_status check_ptr(const void* p, bool needed, size_t align, const char* name) {
  if (!needed) return HS2_OK;
  if (!p) return fail(HS2_ERR_INVALID_ARGUMENT, "%s is NULL", name);
  if (!aligned(p, align)) return fail(HS2_ERR_INVALID_ARGUMENT, "%s not %zu-byte aligned", name, align);
  return HS2_OK;
}

hs2_status check_workspace(const hs2_decode_desc& d, const void* ws, size_t bytes, DecodeLayout& L,
                           bool with_spill = false) {
  L = decode_layout(d, with_spill);
  if (bytes < L.total)
    return fail(HS2_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu needed", bytes, L.total);
  if (L.total > 0 && !ws) return fail(HS2_ERR_INVALID_ARGUMENT, "workspace is NULL");
  if (ws && !aligned(ws, 256)) return fail(HS2_ERR_INVALID_ARGUMENT, "workspace not 256-byte aligned");
  return HS2_OK;
}

#define HS2_TRY(expr)                 \
  do {                                \
    const hs2_status _s = (expr);     \
    if (_s != HS2_OK) return _s;      \
  } while (0)

#define HS2_HIP(expr, what)                       \
  do {                                            \
    const hipError_t _e = (expr);                 \
    if (_e != hipSuccess) return hip_fail(_e, what); \
  } while (0)

uint8_t* ws_at(void* ws, size_t off) { return static_cast<uint8_t*>(ws) + off; }

// ---- stage timing -------------------------------------------------------------
struct TimingRecord {
  hipEvent_t ev[HS2_N_STAGES + 1];
  int last;  // events ev[0 .. last] are recorded
};
std::mutex g_timing_mu;
int32_t g_timing_mode = 0;  // 0 off, 1 every stage, 2 the full-attention partial pass only
std::vector<TimingRecord> g_records;
int g_records_used = 0;
constexpr int kMaxRecords = 1024;

// Returns the record to fill for this call, or nullptr when timing is off.
hs2_status timing_begin(TimingRecord** out) {
  *out = nullptr;
  std::lock_guard<std::mutex> lock(g_timing_mu);
  if (g_timing_mode == 0 || g_records_used >= kMaxRecords) return HS2_OK;
  // Room for every record up front: a later push_back must not move the
  // records that calls in flight on other threads are filling.
  if (g_records.capacity() < static_cast<size_t>(kMaxRecords)) g_records.reserve(kMaxRecords);
  if (g_records_used == static_cast<int>(g_records.size())) {
    TimingRecord r;
    // Timing-only events: no system-scope fence (a cache writeback and
    // invalidate) when each is recorded, so the markers neither slow the step
    // nor add that writeback to the stage before them.
    for (int i = 0; i <= HS2_N_STAGES; ++i)
      HS2_HIP(hipEventCreateWithFlags(&r.ev[i], hipEventDisableSystemFence), "hipEventCreateWithFlags");
    g_records.push_back(r);
  }
  *out = &g_records[g_records_used++];
  (*out)->last = g_timing_mode == 2 ? 2 : HS2_N_STAGES;
  return HS2_OK;
}

hs2_status mark(TimingRecord* rec, int i, hipStream_t s) {
  if (rec && i <= rec->last) HS2_HIP(hipEventRecord(rec->ev[i], s), "hipEventRecord");
  return HS2_OK;
}

// ---- the decode sequence ----------------------------------------------------------
struct DecodeArgs {
  const hs2_decode_desc* d;
  const int64_t* offs;
  const void* k;
  const void* v;
  const float* ks;
  const float* vs;
  const float* q_full;
  const float* q_sparse;
  float* o_full;
  float* o_sparse;
  int32_t* sel_idx;
  int32_t* sel_count;
  float* score_out;
  void* ws;
  hipStream_t stream;
  const int64_t* kv_start = nullptr;  // multi-token decode: real first K/V row of each virtual sequence
  const MultiFullParams* multi = nullptr;  // multi-token decode: the shared-stream full pass (real batch)
};

// The full pass's even-XCD share (bf16 tiles dealt 22:20 to the workgroups
// on even XCDs) pays when every workgroup streams the same amount; a ragged
// batch leaves CUs idle and its longest sequences set the end.
int even_xcd_split(const hs2_decode_desc& d) {
  return d.kv_dtype == HS2_KV_BF16 && d.batch > 0 && d.total_tokens == static_cast<int64_t>(d.batch) * d.max_context;
}

FullParams full_params(const DecodeArgs& a, const DecodeLayout& L) {
  FullParams p{};
  p.kv_start = a.kv_start;
  p.seq_offsets = a.offs;
  p.total_tokens = a.d->total_tokens;
  p.max_context = a.d->max_context;
  p.k = static_cast<const uint8_t*>(a.k);
  p.v = static_cast<const uint8_t*>(a.v);
  p.k_scale = a.ks;
  p.v_scale = a.vs;
  p.q = a.q_full;
  p.qscale = static_cast<float>(static_cast<double>(a.d->softmax_scale) * kLog2e);
  p.batch = a.d->batch;
  p.xcd_split = even_xcd_split(*a.d);
  p.chunk = L.chunk;
  p.chunks_per_seq = L.chunks_per_seq;
  p.partials = reinterpret_cast<float*>(ws_at(a.ws, L.partials));
  p.pstats = reinterpret_cast<float*>(ws_at(a.ws, L.pstats));
  p.spill = reinterpret_cast<float*>(ws_at(a.ws, L.spill));
  p.shat = reinterpret_cast<uint16_t*>(ws_at(a.ws, L.shat));
  p.tile_stats = reinterpret_cast<float*>(ws_at(a.ws, L.tile_stats));
  p.tile_sums = reinterpret_cast<float*>(ws_at(a.ws, L.tile_sums));
  p.hist0 = reinterpret_cast<uint32_t*>(ws_at(a.ws, L.hist0));
  p.counters = reinterpret_cast<uint32_t*>(ws_at(a.ws, L.counters));
  return p;
}

SelectParams select_params(const DecodeArgs& a, const DecodeLayout& L, float* score) {
  SelectParams p{};
  p.kv_start = a.kv_start;
  p.seq_offsets = a.offs;
  p.total_tokens = a.d->total_tokens;
  p.max_context = a.d->max_context;
  p.batch = a.d->batch;
  p.window = a.d->window;
  p.top_k = a.d->top_k;
  p.budget = a.d->window + a.d->top_k;
  p.spill = reinterpret_cast<const float*>(ws_at(a.ws, L.spill));
  p.stats = reinterpret_cast<const float*>(ws_at(a.ws, L.stats));
  p.pstats = reinterpret_cast<const float*>(ws_at(a.ws, L.pstats));
  p.chunks_per_seq = L.chunks_per_seq;
  p.score = score;
  p.hist0 = reinterpret_cast<uint32_t*>(ws_at(a.ws, L.hist0));
  p.counters = reinterpret_cast<uint32_t*>(ws_at(a.ws, L.counters));
  p.selbuf = reinterpret_cast<int32_t*>(ws_at(a.ws, L.selbuf));
  p.cand = reinterpret_cast<unsigned long long*>(ws_at(a.ws, L.cand));
  p.shat = reinterpret_cast<const uint16_t*>(ws_at(a.ws, L.shat));
  p.tile_stats = reinterpret_cast<const float*>(ws_at(a.ws, L.tile_stats));
  p.tile_ub = reinterpret_cast<float*>(ws_at(a.ws, L.tile_ub));
  p.cand_cnt = reinterpret_cast<uint32_t*>(ws_at(a.ws, L.cand_cnt));
  p.cand_blocks = L.cand_blocks;
  p.k = static_cast<const uint8_t*>(a.k);
  p.k_scale = a.ks;
  p.q = a.q_full;
  p.qscale = static_cast<float>(static_cast<double>(a.d->softmax_scale) * kLog2e);
  p.sel_idx = a.sel_idx;
  p.sel_count = a.sel_count;
  return p;
}

// Full-attention pass and merge.  `mode`: kFullBound (the merge launch also
// runs the selection's first pass, with `bound_sel`), kFullSpill (every logit
// kept for the score pass), kFullPlain (full attention alone: partials and
// o_full only) or kFullTileSums (the merge launch also computes the gen-1
// block sums, with `block_sel`).
hs2_status run_full(const DecodeArgs& a, const DecodeLayout& L, int mode, const SelectParams* bound_sel,
                    TimingRecord* rec, const BlockParams* block_sel = nullptr) {
  const bool bound_mode = mode == kFullBound;
  const hs2_decode_desc& d = *a.d;
  const FullParams fp = full_params(a, L);
  if (a.multi && bound_mode) {
    // Multi-token decode: the tokens of a sequence share its K/V stream, in
    // groups of kMultiQ tokens (one launch per group).
    MultiFullParams m = *a.multi;
    const FullParams real = m.f;
    m.f = fp;
    m.f.seq_offsets = real.seq_offsets;
    m.f.batch = real.batch;
    m.f.total_tokens = real.total_tokens;
    m.f.max_context = real.max_context;
    m.f.kv_start = nullptr;
    m.f.xcd_split = real.xcd_split;
    m.fp8 = d.kv_dtype == HS2_KV_FP8_E4M3;
    for (int t = 0; t < m.n_query; t += kMultiQ) {
      m.t_first = t;
      m.nq = std::min(kMultiQ, m.n_query - t);
      HS2_HIP(launch_full_multi(m, a.stream), "multi-token full-attention pass");
    }
  } else {
    HS2_HIP(launch_full_partial(fp, d.batch, d.kv_dtype == HS2_KV_FP8_E4M3, mode, a.stream),
            "full-attention partial pass");
  }
  HS2_TRY(mark(rec, 1, a.stream));
  MergeParams mp;
  mp.seq_offsets = a.offs;
  mp.total_tokens = d.total_tokens;
  mp.max_context = d.max_context;
  mp.budget = d.window + d.top_k;
  mp.partials = fp.partials;
  mp.chunk = L.chunk;
  mp.chunks_per_seq = L.chunks_per_seq;
  mp.stride_seq = L.chunks_per_seq * kPartialFloats;
  mp.stride_chunk = kPartialFloats;
  mp.count_from_sel = 0;
  mp.sel_count = nullptr;
  mp.out = a.o_full;
  mp.out_stride_seq = kHeads * kDim;
  mp.stats = mode == kFullPlain ? nullptr : reinterpret_cast<float*>(ws_at(a.ws, L.stats));
  if (bound_mode) {
    HS2_HIP(launch_merge_bound_hist(mp, *bound_sel, d.batch, d.max_context, a.stream), "merge and bound histogram");
  } else if (mode == kFullTileSums) {
    HS2_HIP(launch_merge_block_pool(mp, *block_sel, a.stream), "merge and block sums");
  } else {
    HS2_HIP(launch_merge(mp, d.batch, a.stream), "full-attention merge");
  }
  HS2_TRY(mark(rec, 2, a.stream));
  return HS2_OK;
}

hs2_status run_sparse(const DecodeArgs& a, const DecodeLayout& L, const int32_t* sel_idx, const int32_t* sel_count) {
  const hs2_decode_desc& d = *a.d;
  if (d.n_sparse_layers == 0 || d.batch == 0) return HS2_OK;
  SparseParams sp{};
  sp.seq_offsets = a.offs;
  sp.total_tokens = d.total_tokens;
  sp.max_context = d.max_context;
  sp.k = static_cast<const uint8_t*>(a.k);
  sp.v = static_cast<const uint8_t*>(a.v);
  sp.k_scale = a.ks;
  sp.v_scale = a.vs;
  sp.q_sparse = a.q_sparse;
  sp.qscale = static_cast<float>(static_cast<double>(d.softmax_scale) * kLog2e);
  sp.batch = d.batch;
  sp.n_layers = d.n_sparse_layers;
  sp.budget = d.window + d.top_k;
  sp.sel_idx = sel_idx;
  sp.sel_count = sel_count;
  sp.out = a.o_sparse;
  sp.partials = reinterpret_cast<float*>(ws_at(a.ws, L.sparse));
  sp.kv_start = a.kv_start;
  HS2_HIP(launch_sparse_attend(sp, d.kv_dtype == HS2_KV_FP8_E4M3, a.stream), "sparse layers");
  return HS2_OK;
}

hs2_status run_block(const DecodeArgs& a, const DecodeLayout& L);
hs2_status run_block_gen1(const DecodeArgs& a, const DecodeLayout& L);

// The arguments of a decode step other than its workspace.
hs2_status check_decode_args(const hs2_decode_desc* desc, const int64_t* seq_offsets, const void* k_cache,
                             const void* v_cache, const float* k_scale, const float* v_scale, const float* q_full,
                             const float* q_sparse, const float* o_full, const float* o_sparse,
                             const int32_t* sel_idx, const int32_t* sel_count, const float* score_out) {
  HS2_TRY(check_desc(desc));
  const hs2_decode_desc& d = *desc;
  HS2_TRY(check_kv(d, seq_offsets, k_cache, v_cache, k_scale, v_scale));
  const bool any = d.batch > 0;
  const bool sparse = any && d.n_sparse_layers > 0;
  HS2_TRY(check_ptr(q_full, any, 16, "q_full"));
  HS2_TRY(check_ptr(o_full, any, 16, "o_full"));
  HS2_TRY(check_ptr(q_sparse, sparse, 16, "q_sparse"));
  HS2_TRY(check_ptr(o_sparse, sparse, 16, "o_sparse"));
  HS2_TRY(check_ptr(sel_idx, any, 4, "sel_idx"));
  HS2_TRY(check_ptr(sel_count, any, 4, "sel_count"));
  if (score_out && !aligned(score_out, 4)) return fail(HS2_ERR_INVALID_ARGUMENT, "score_out not 4-byte aligned");
  return HS2_OK;
}

}  // namespace

extern "C" {

size_t hs2_decode_workspace_bytes(const hs2_decode_desc* desc) {
  if (check_desc(desc) != HS2_OK) return 0;
  return decode_layout(*desc, false).total;
}

size_t hs2_decode_score_workspace_bytes(const hs2_decode_desc* desc) {
  if (check_desc(desc) != HS2_OK) return 0;
  return decode_layout(*desc, true).total;
}

hs2_status hs2_decode_block(const hs2_decode_desc* desc, const int64_t* seq_offsets, const void* k_cache,
                            const void* v_cache, const float* k_scale, const float* v_scale, const float* q_full,
                            const float* q_sparse, float* o_full, float* o_sparse, int32_t* sel_idx,
                            int32_t* sel_count, float* score_out, void* workspace, size_t workspace_bytes,
                            void* stream) {
  HS2_TRY(check_decode_args(desc, seq_offsets, k_cache, v_cache, k_scale, v_scale, q_full, q_sparse, o_full,
                            o_sparse, sel_idx, sel_count, score_out));
  const hs2_decode_desc& d = *desc;
  DecodeLayout L;
  HS2_TRY(check_workspace(d, workspace, workspace_bytes, L, score_out != nullptr));
  if (d.batch == 0) return HS2_OK;

  DecodeArgs a{desc, seq_offsets, k_cache, v_cache, k_scale, v_scale, q_full, q_sparse, o_full, o_sparse,
               sel_idx, sel_count, score_out, workspace, static_cast<hipStream_t>(stream)};
  return run_block(a, L);
}

hs2_status hs2_decode_block_gen1(const hs2_decode_desc* desc, const int64_t* seq_offsets, const void* k_cache,
                                 const void* v_cache, const float* k_scale, const float* v_scale,
                                 const float* q_full, const float* q_sparse, float* o_full, float* o_sparse,
                                 int32_t* sel_idx, int32_t* sel_count, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  HS2_TRY(check_decode_args(desc, seq_offsets, k_cache, v_cache, k_scale, v_scale, q_full, q_sparse, o_full,
                            o_sparse, sel_idx, sel_count, nullptr));
  const hs2_decode_desc& d = *desc;
  DecodeLayout L;
  HS2_TRY(check_workspace(d, workspace, workspace_bytes, L, false));
  if (d.batch == 0) return HS2_OK;
  DecodeArgs a{desc, seq_offsets, k_cache, v_cache, k_scale, v_scale, q_full, q_sparse, o_full, o_sparse,
               sel_idx, sel_count, nullptr, workspace, static_cast<hipStream_t>(stream)};
  return run_block_gen1(a, L);
}

}  // extern "C"

// ---- the decode step without an allocation ------------------------------------
// hs2_decode_block_noalloc runs hs2_decode_block (no score output) with its
// workspace in `scratch`, a device array of the library's own: each GPU the
// library runs on holds one copy for the life of the process.  The array's
// device address is looked up once per device (hipGetSymbolAddress, with the
// device current) and kept; host code uses that address, never the symbol.
namespace {
__device__ __align__(256) uint8_t scratch[HS2_NOALLOC_SCRATCH_BYTES];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

hs2_status scratch_address(void** out) {
  int dev = -1;
  HS2_HIP(hipGetDevice(&dev), "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(HS2_ERR_UNSUPPORTED, "device %d (0..%d supported)", dev, kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    HS2_HIP(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
    if (!ptr) return fail(HS2_ERR_HIP, "hipGetSymbolAddress(scratch) gave NULL");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return HS2_OK;
}
}  // namespace

extern "C" hs2_status hs2_decode_block_noalloc(const hs2_decode_desc* desc, const int64_t* seq_offsets,
                                               const void* k_cache, const void* v_cache, const float* k_scale,
                                               const float* v_scale, const float* q_full, const float* q_sparse,
                                               float* o_full, float* o_sparse, int32_t* sel_idx,
                                               int32_t* sel_count, void* stream) {
  HS2_TRY(check_decode_args(desc, seq_offsets, k_cache, v_cache, k_scale, v_scale, q_full, q_sparse, o_full,
                            o_sparse, sel_idx, sel_count, nullptr));
  const DecodeLayout L = decode_layout(*desc, false);
  if (L.total > static_cast<size_t>(HS2_NOALLOC_SCRATCH_BYTES))
    return fail(HS2_ERR_UNSUPPORTED, "this shape needs %zu bytes of workspace; the library's scratch holds %zu",
                L.total, static_cast<size_t>(HS2_NOALLOC_SCRATCH_BYTES));
  if (desc->batch == 0) return HS2_OK;
  void* ws = nullptr;
  HS2_TRY(scratch_address(&ws));
  DecodeArgs a{desc, seq_offsets, k_cache, v_cache, k_scale, v_scale, q_full, q_sparse, o_full, o_sparse,
               sel_idx, sel_count, nullptr, ws, static_cast<hipStream_t>(stream)};
  return run_block(a, L);
}

namespace {
// One hybrid block for the (validated) batch in `a`.
hs2_status run_block(const DecodeArgs& a, const DecodeLayout& L) {
  const hs2_decode_desc& d = *a.d;
  void* workspace = a.ws;
  float* score_out = a.score_out;
  TimingRecord* rec = nullptr;
  HS2_TRY(timing_begin(&rec));
  // Without a score output the full pass keeps only score bounds (2 + 4 bytes
  // per token instead of 64 bytes of logits) and the selection rescores the
  // few positions the bounds cannot rule out; with it, every logit is kept and
  // every score computed.  Both give the same scores for the positions that
  // matter, hence the same selection.
  const bool bound_mode = score_out == nullptr;
  const SelectParams sp = select_params(a, L, score_out);  // bound mode reads no score array
  // (bound mode: the full pass itself clears the selection's histogram and counters)
  if (!bound_mode) HS2_HIP(launch_select_init(sp, d.batch, a.stream), "selection init");
  HS2_TRY(mark(rec, 0, a.stream));
  HS2_TRY(run_full(a, L, bound_mode ? kFullBound : kFullSpill, bound_mode ? &sp : nullptr, rec));
  if (bound_mode) {
    HS2_HIP(launch_bound_select(sp, d.batch, d.max_context, d.kv_dtype == HS2_KV_FP8_E4M3, a.stream), "selection");
  } else {
    HS2_HIP(launch_score_hist(sp, d.batch, d.max_context, true, true, a.stream), "score pass");
    HS2_HIP(launch_collect_finish(sp, d.batch, d.max_context, a.stream), "selection");
  }
  HS2_TRY(mark(rec, 3, a.stream));
  HS2_TRY(run_sparse(a, L, a.sel_idx, a.sel_count));
  HS2_TRY(mark(rec, 4, a.stream));
  return HS2_OK;
}

// The hybrid block with gen-1 selection and no per-token scores: the full
// pass keeps per-tile head sums of its weights (8 bytes a token), the merge
// launch turns them into block sums, then the block ranking and the sparse
// layers.  Stages as run_block.
hs2_status run_block_gen1(const DecodeArgs& a, const DecodeLayout& L) {
  const hs2_decode_desc& d = *a.d;
  TimingRecord* rec = nullptr;
  HS2_TRY(timing_begin(&rec));
  BlockParams bp{};
  bp.seq_offsets = a.offs;
  bp.total_tokens = d.total_tokens;
  bp.max_context = d.max_context;
  bp.batch = d.batch;
  bp.block_scores = reinterpret_cast<float*>(ws_at(a.ws, L.blocks));
  bp.group_keys = reinterpret_cast<unsigned long long*>(ws_at(a.ws, L.groups));
  bp.sel_idx = a.sel_idx;
  bp.sel_count = a.sel_count;
  bp.tile_stats = reinterpret_cast<const float*>(ws_at(a.ws, L.tile_stats));
  bp.tile_sums = reinterpret_cast<const float*>(ws_at(a.ws, L.tile_sums));
  bp.pstats = reinterpret_cast<const float*>(ws_at(a.ws, L.pstats));
  bp.chunk = L.chunk;
  bp.chunks_per_seq = L.chunks_per_seq;
  HS2_TRY(mark(rec, 0, a.stream));
  HS2_TRY(run_full(a, L, kFullTileSums, nullptr, rec, &bp));
  HS2_HIP(launch_block_rank(bp, a.stream), "block selection");
  HS2_TRY(mark(rec, 3, a.stream));
  HS2_TRY(run_sparse(a, L, a.sel_idx, a.sel_count));
  HS2_TRY(mark(rec, 4, a.stream));
  return HS2_OK;
}
}  // namespace

extern "C" {

// Multi-token decode: the virtual batch's descriptor, and its layout followed
// by the virtual offsets and K/V starts.
static hs2_decode_desc multi_desc(const hs2_decode_desc& d, int32_t n_query) {
  hs2_decode_desc v = d;
  v.batch = d.batch * n_query;
  v.total_tokens = d.total_tokens * n_query;  // bounds the packed prefix lengths
  return v;
}

// The full pass of multi-token decode runs on the real batch (its tokens
// share each sequence's K/V stream), with the real batch's chunk.
static int multi_chunk(const hs2_decode_desc& d) {
  return choose_chunk(d.total_tokens, d.max_context, d.batch, d.kv_dtype == HS2_KV_FP8_E4M3);
}

size_t hs2_decode_multi_workspace_bytes(const hs2_decode_desc* desc, int32_t n_query) {
  if (check_desc(desc) != HS2_OK || n_query < 1 || n_query > kMaxQueryTokens) return 0;
  const hs2_decode_desc v = multi_desc(*desc, n_query);
  if (check_desc(&v) != HS2_OK) return 0;
  const size_t n = static_cast<size_t>(v.batch);
  return align_up(decode_layout(v, false, multi_chunk(*desc)).total) + align_up((n + 1) * sizeof(int64_t)) +
         align_up(n * sizeof(int64_t));
}

hs2_status hs2_decode_multi(const hs2_decode_desc* desc, int32_t n_query, const int64_t* seq_offsets,
                            const void* k_cache, const void* v_cache, const float* k_scale, const float* v_scale,
                            const float* q_full, const float* q_sparse, float* o_full, float* o_sparse,
                            int32_t* sel_idx, int32_t* sel_count, void* workspace, size_t workspace_bytes,
                            void* stream) {
  HS2_TRY(check_desc(desc));
  const hs2_decode_desc& d = *desc;
  if (n_query < 1 || n_query > kMaxQueryTokens)
    return fail(HS2_ERR_UNSUPPORTED, "n_query %d (1..%d supported)", n_query, kMaxQueryTokens);
  if (static_cast<int64_t>(d.batch) * n_query > (1 << 24))
    return fail(HS2_ERR_UNSUPPORTED, "batch * n_query above 2^24");
  HS2_TRY(check_kv(d, seq_offsets, k_cache, v_cache, k_scale, v_scale));
  const hs2_decode_desc v = multi_desc(d, n_query);
  HS2_TRY(check_desc(&v));
  const bool any = d.batch > 0;
  const bool sparse = any && d.n_sparse_layers > 0;
  HS2_TRY(check_ptr(q_full, any, 16, "q_full"));
  HS2_TRY(check_ptr(o_full, any, 16, "o_full"));
  HS2_TRY(check_ptr(q_sparse, sparse, 16, "q_sparse"));
  HS2_TRY(check_ptr(o_sparse, sparse, 16, "o_sparse"));
  HS2_TRY(check_ptr(sel_idx, any, 4, "sel_idx"));
  HS2_TRY(check_ptr(sel_count, any, 4, "sel_count"));
  const size_t need = hs2_decode_multi_workspace_bytes(desc, n_query);
  if (workspace_bytes < need) return fail(HS2_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu needed", workspace_bytes, need);
  HS2_TRY(check_ptr(workspace, true, 256, "workspace"));
  if (!any) return HS2_OK;
  const DecodeLayout L = decode_layout(v, false, multi_chunk(d));
  const size_t n = static_cast<size_t>(v.batch);
  MultiParams mp{};
  mp.seq_offsets = seq_offsets;
  mp.total_tokens = d.total_tokens;
  mp.max_context = d.max_context;
  mp.batch = d.batch;
  mp.n_query = n_query;
  mp.voffs = reinterpret_cast<int64_t*>(ws_at(workspace, align_up(L.total)));
  mp.kv_start = reinterpret_cast<int64_t*>(ws_at(workspace, align_up(L.total) + align_up((n + 1) * sizeof(int64_t))));
  HS2_HIP(launch_multi_prep(mp, static_cast<hipStream_t>(stream)), "multi-token offsets");
  MultiFullParams mf{};
  mf.f.seq_offsets = seq_offsets;
  mf.f.batch = d.batch;
  mf.f.total_tokens = d.total_tokens;
  mf.f.max_context = d.max_context;
  mf.f.xcd_split = even_xcd_split(d);  // the real batch's, as hs2_decode_block's
  mf.voffs = mp.voffs;
  mf.n_query = n_query;
  DecodeArgs a{&v, mp.voffs, k_cache, v_cache, k_scale, v_scale, q_full, q_sparse, o_full, o_sparse,
               sel_idx, sel_count, nullptr, workspace, static_cast<hipStream_t>(stream), mp.kv_start, &mf};
  return run_block(a, L);
}

hs2_status hs2_full_decode_score(const hs2_decode_desc* desc, const int64_t* seq_offsets, const void* k_cache,
                                 const void* v_cache, const float* k_scale, const float* v_scale,
                                 const float* q_full, float* o_full, float* score_out, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  HS2_TRY(check_desc(desc));
  const hs2_decode_desc& d = *desc;
  HS2_TRY(check_kv(d, seq_offsets, k_cache, v_cache, k_scale, v_scale));
  const bool any = d.batch > 0;
  HS2_TRY(check_ptr(q_full, any, 16, "q_full"));
  HS2_TRY(check_ptr(o_full, any, 16, "o_full"));
  HS2_TRY(check_ptr(score_out, d.total_tokens > 0, 4, "score_out"));
  DecodeLayout L;
  HS2_TRY(check_workspace(d, workspace, workspace_bytes, L, true));
  if (!any) return HS2_OK;
  DecodeArgs a{desc, seq_offsets, k_cache, v_cache, k_scale, v_scale, q_full, nullptr, o_full, nullptr,
               nullptr, nullptr, score_out, workspace, static_cast<hipStream_t>(stream)};
  TimingRecord* rec = nullptr;
  HS2_TRY(timing_begin(&rec));
  if (rec && rec->last > 3) rec->last = 3;  // stages 0 partial pass, 1 merge, 2 score pass
  HS2_TRY(mark(rec, 0, a.stream));
  HS2_TRY(run_full(a, L, kFullSpill, nullptr, rec));
  const SelectParams sp = select_params(a, L, score_out);
  HS2_HIP(launch_score_hist(sp, d.batch, d.max_context, true, false, a.stream), "score pass");
  HS2_TRY(mark(rec, 3, a.stream));
  return HS2_OK;
}

hs2_status hs2_topk_select(const hs2_decode_desc* desc, const int64_t* seq_offsets, const float* score,
                           int32_t* sel_idx, int32_t* sel_count, void* workspace, size_t workspace_bytes,
                           void* stream) {
  HS2_TRY(check_desc(desc));
  const hs2_decode_desc& d = *desc;
  const bool any = d.batch > 0;
  if (any && !seq_offsets) return fail(HS2_ERR_INVALID_ARGUMENT, "seq_offsets is NULL");
  if (seq_offsets && !aligned(seq_offsets, 8)) return fail(HS2_ERR_INVALID_ARGUMENT, "seq_offsets not 8-byte aligned");
  HS2_TRY(check_ptr(score, d.total_tokens > 0, 4, "score"));
  HS2_TRY(check_ptr(sel_idx, any, 4, "sel_idx"));
  HS2_TRY(check_ptr(sel_count, any, 4, "sel_count"));
  DecodeLayout L;
  HS2_TRY(check_workspace(d, workspace, workspace_bytes, L));
  if (!any) return HS2_OK;
  DecodeArgs a{desc, seq_offsets, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
               sel_idx, sel_count, nullptr, workspace, static_cast<hipStream_t>(stream)};
  const SelectParams sp = select_params(a, L, const_cast<float*>(score));
  HS2_HIP(launch_select_init(sp, d.batch, a.stream), "selection init");
  HS2_HIP(launch_score_hist(sp, d.batch, d.max_context, false, true, a.stream), "score histogram");
  HS2_HIP(launch_collect_finish(sp, d.batch, d.max_context, a.stream), "selection");
  return HS2_OK;
}

hs2_status hs2_block_select(const hs2_decode_desc* desc, const int64_t* seq_offsets, const float* score,
                            int32_t* sel_idx, int32_t* sel_count, void* workspace, size_t workspace_bytes,
                            void* stream) {
  HS2_TRY(check_desc(desc));
  const hs2_decode_desc& d = *desc;
  const bool any = d.batch > 0;
  if (any && !seq_offsets) return fail(HS2_ERR_INVALID_ARGUMENT, "seq_offsets is NULL");
  if (seq_offsets && !aligned(seq_offsets, 8)) return fail(HS2_ERR_INVALID_ARGUMENT, "seq_offsets not 8-byte aligned");
  HS2_TRY(check_ptr(score, d.total_tokens > 0, 4, "score"));
  HS2_TRY(check_ptr(sel_idx, any, 4, "sel_idx"));
  HS2_TRY(check_ptr(sel_count, any, 4, "sel_count"));
  DecodeLayout L;
  HS2_TRY(check_workspace(d, workspace, workspace_bytes, L));
  if (!any) return HS2_OK;
  BlockParams p{};
  p.seq_offsets = seq_offsets;
  p.total_tokens = d.total_tokens;
  p.max_context = d.max_context;
  p.batch = d.batch;
  p.score = score;
  p.block_scores = reinterpret_cast<float*>(ws_at(workspace, L.blocks));
  p.group_keys = reinterpret_cast<unsigned long long*>(ws_at(workspace, L.groups));
  p.sel_idx = sel_idx;
  p.sel_count = sel_count;
  HS2_HIP(launch_block_select(p, static_cast<hipStream_t>(stream)), "block selection");
  return HS2_OK;
}

hs2_status hs2_sparse_decode(const hs2_decode_desc* desc, const int64_t* seq_offsets, const void* k_cache,
                             const void* v_cache, const float* k_scale, const float* v_scale,
                             const float* q_sparse, const int32_t* sel_idx, const int32_t* sel_count,
                             float* o_sparse, void* workspace, size_t workspace_bytes, void* stream) {
  HS2_TRY(check_desc(desc));
  const hs2_decode_desc& d = *desc;
  HS2_TRY(check_kv(d, seq_offsets, k_cache, v_cache, k_scale, v_scale));
  const bool sparse = d.batch > 0 && d.n_sparse_layers > 0;
  HS2_TRY(check_ptr(q_sparse, sparse, 16, "q_sparse"));
  HS2_TRY(check_ptr(o_sparse, sparse, 16, "o_sparse"));
  HS2_TRY(check_ptr(sel_idx, sparse, 4, "sel_idx"));
  HS2_TRY(check_ptr(sel_count, sparse, 4, "sel_count"));
  DecodeLayout L;
  HS2_TRY(check_workspace(d, workspace, workspace_bytes, L));
  if (!sparse) return HS2_OK;
  DecodeArgs a{desc, seq_offsets, k_cache, v_cache, k_scale, v_scale, nullptr, q_sparse, nullptr, o_sparse,
               nullptr, nullptr, nullptr, workspace, static_cast<hipStream_t>(stream)};
  return run_sparse(a, L, sel_idx, sel_count);
}

size_t hs2_bridge_workspace_bytes(int64_t n_tokens, int32_t d_model, int32_t head_dim, int32_t n_bridged) {
  if (n_tokens < 0 || d_model <= 0 || d_model % 64 || head_dim != kDim || n_bridged < 1 || n_bridged > 4) return 0;
  return align_up(static_cast<size_t>(2 * n_bridged) * kDim * d_model * sizeof(uint16_t));
}

// Checks shared by every bridge entry point.
static hs2_status check_bridge_shape(int64_t n_tokens, int32_t d_model, int32_t head_dim, int32_t n_bridged) {
  if (n_tokens < 0) return fail(HS2_ERR_INVALID_ARGUMENT, "n_tokens < 0");
  if (head_dim != kDim) return fail(HS2_ERR_UNSUPPORTED, "head_dim %d (only 128 is supported)", head_dim);
  if (d_model <= 0 || d_model % 64) return fail(HS2_ERR_UNSUPPORTED, "d_model %d must be a positive multiple of 64", d_model);
  if (n_bridged < 1 || n_bridged > 4) return fail(HS2_ERR_UNSUPPORTED, "n_bridged %d (1..4 supported)", n_bridged);
  if (n_tokens > (int64_t(1) << 31)) return fail(HS2_ERR_UNSUPPORTED, "n_tokens above 2^31");
  return HS2_OK;
}

// Interleaves the per-layer weight and output arrays into the GEMM's column
// blocks (W_k0, W_v0, W_k1, ...) and checks every pointer.
static hs2_status bridge_columns(int64_t n_tokens, int32_t n_bridged, const void* const* w_k, const void* const* w_v,
                                 void* const* k_out, void* const* v_out, float* const* k_scale,
                                 float* const* v_scale, bool fp8, const uint16_t** ws, void** outs, float** scales) {
  if ((w_k || w_v) && (!w_k || !w_v)) return fail(HS2_ERR_INVALID_ARGUMENT, "weight pointer array is NULL");
  if (!k_out || !v_out) return fail(HS2_ERR_INVALID_ARGUMENT, "output pointer array is NULL");
  if (fp8 && (!k_scale || !v_scale)) return fail(HS2_ERR_INVALID_ARGUMENT, "scale pointer array is NULL");
  for (int l = 0; l < n_bridged; ++l) {
    if (w_k) {
      ws[2 * l] = static_cast<const uint16_t*>(w_k[l]);
      ws[2 * l + 1] = static_cast<const uint16_t*>(w_v[l]);
    }
    outs[2 * l] = k_out[l];
    outs[2 * l + 1] = v_out[l];
    if (fp8) {
      scales[2 * l] = k_scale[l];
      scales[2 * l + 1] = v_scale[l];
    }
  }
  for (int i = 0; i < 2 * n_bridged; ++i) {
    if (w_k) HS2_TRY(check_ptr(ws[i], true, 16, "w_k/w_v entry"));
    HS2_TRY(check_ptr(outs[i], n_tokens > 0, 16, "k_out/v_out entry"));
    if (fp8) HS2_TRY(check_ptr(scales[i], n_tokens > 0, 4, "k_scale/v_scale entry"));
  }
  return HS2_OK;
}

static hipError_t bridge_gemm(int64_t n_tokens, int32_t d_model, int32_t n_bridged, const void* hidden,
                              const uint16_t* w_t, void* const* outs, float* const* scales, bool fp8, hipStream_t s) {
  BridgeParams p;
  p.n_tokens = n_tokens;
  p.d_model = d_model;
  p.n_out = 2 * n_bridged;
  p.hidden = static_cast<const uint16_t*>(hidden);
  p.w_t = w_t;
  p.fp8 = fp8 ? 1 : 0;
  for (int i = 0; i < 8; ++i) {
    p.out[i] = i < 2 * n_bridged ? outs[i] : nullptr;
    p.scale[i] = i < 2 * n_bridged ? scales[i] : nullptr;
  }
  return launch_bridge_gemm(p, s);
}

// The bridge projection, with bf16 or E4M3 (per-token scales) outputs.
static hs2_status bridge_run(int64_t n_tokens, int32_t d_model, int32_t head_dim, int32_t n_bridged,
                             const void* hidden, const void* const* w_k, const void* const* w_v,
                             void* const* k_out, void* const* v_out, float* const* k_scale, float* const* v_scale,
                             bool fp8, void* workspace, size_t workspace_bytes, void* stream) {
  HS2_TRY(check_bridge_shape(n_tokens, d_model, head_dim, n_bridged));
  if (!w_k || !w_v) return fail(HS2_ERR_INVALID_ARGUMENT, "weight pointer array is NULL");
  const uint16_t* ws[8] = {};
  void* outs[8] = {};
  float* scales[8] = {};
  HS2_TRY(bridge_columns(n_tokens, n_bridged, w_k, w_v, k_out, v_out, k_scale, v_scale, fp8, ws, outs, scales));
  HS2_TRY(check_ptr(hidden, n_tokens > 0, 16, "hidden"));
  const size_t need = hs2_bridge_workspace_bytes(n_tokens, d_model, head_dim, n_bridged);
  if (workspace_bytes < need) return fail(HS2_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu needed", workspace_bytes, need);
  HS2_TRY(check_ptr(workspace, true, 256, "workspace"));
  if (n_tokens == 0) return HS2_OK;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  uint16_t* w_t = static_cast<uint16_t*>(workspace);
  HS2_HIP(launch_bridge_transpose_w(ws, 2 * n_bridged, d_model, w_t, s), "bridge weight transpose");
  HS2_HIP(bridge_gemm(n_tokens, d_model, n_bridged, hidden, w_t, outs, scales, fp8, s), "bridge GEMM");
  return HS2_OK;
}

hs2_status hs2_bridge_kv(int64_t n_tokens, int32_t d_model, int32_t head_dim, int32_t n_bridged, const void* hidden,
                         const void* const* w_k, const void* const* w_v, void* const* k_out, void* const* v_out,
                         void* workspace, size_t workspace_bytes, void* stream) {
  return bridge_run(n_tokens, d_model, head_dim, n_bridged, hidden, w_k, w_v, k_out, v_out, nullptr, nullptr, false,
                    workspace, workspace_bytes, stream);
}

hs2_status hs2_bridge_kv_fp8(int64_t n_tokens, int32_t d_model, int32_t head_dim, int32_t n_bridged,
                             const void* hidden, const void* const* w_k, const void* const* w_v, void* const* k_out,
                             float* const* k_scale, void* const* v_out, float* const* v_scale, void* workspace,
                             size_t workspace_bytes, void* stream) {
  return bridge_run(n_tokens, d_model, head_dim, n_bridged, hidden, w_k, w_v, k_out, v_out, k_scale, v_scale, true,
                    workspace, workspace_bytes, stream);
}

size_t hs2_bridge_packed_weight_bytes(int32_t d_model, int32_t head_dim, int32_t n_bridged) {
  return hs2_bridge_workspace_bytes(0, d_model, head_dim, n_bridged);
}

hs2_status hs2_bridge_pack_weights(int32_t d_model, int32_t head_dim, int32_t n_bridged, const void* const* w_k,
                                   const void* const* w_v, void* packed, size_t packed_bytes, void* stream) {
  HS2_TRY(check_bridge_shape(0, d_model, head_dim, n_bridged));
  if (!w_k || !w_v) return fail(HS2_ERR_INVALID_ARGUMENT, "weight pointer array is NULL");
  const uint16_t* ws[8] = {};
  for (int l = 0; l < n_bridged; ++l) {
    ws[2 * l] = static_cast<const uint16_t*>(w_k[l]);
    ws[2 * l + 1] = static_cast<const uint16_t*>(w_v[l]);
  }
  for (int i = 0; i < 2 * n_bridged; ++i) HS2_TRY(check_ptr(ws[i], true, 16, "w_k/w_v entry"));
  const size_t need = hs2_bridge_packed_weight_bytes(d_model, head_dim, n_bridged);
  if (packed_bytes < need) return fail(HS2_ERR_WORKSPACE_TOO_SMALL, "packed buffer %zu bytes < %zu needed", packed_bytes, need);
  HS2_TRY(check_ptr(packed, true, 256, "packed"));
  HS2_HIP(launch_bridge_transpose_w(ws, 2 * n_bridged, d_model, static_cast<uint16_t*>(packed),
                                    static_cast<hipStream_t>(stream)),
          "bridge weight packing");
  return HS2_OK;
}

hs2_status hs2_bridge_kv_packed(int64_t n_tokens, int32_t d_model, int32_t head_dim, int32_t n_bridged,
                                int32_t kv_dtype, const void* hidden, const void* packed, void* const* k_out,
                                float* const* k_scale, void* const* v_out, float* const* v_scale, void* stream) {
  HS2_TRY(check_bridge_shape(n_tokens, d_model, head_dim, n_bridged));
  if (kv_dtype != HS2_KV_BF16 && kv_dtype != HS2_KV_FP8_E4M3) return fail(HS2_ERR_UNSUPPORTED, "kv_dtype %d", kv_dtype);
  const bool fp8 = kv_dtype == HS2_KV_FP8_E4M3;
  const uint16_t* ws[8] = {};
  void* outs[8] = {};
  float* scales[8] = {};
  HS2_TRY(bridge_columns(n_tokens, n_bridged, nullptr, nullptr, k_out, v_out, k_scale, v_scale, fp8, ws, outs, scales));
  HS2_TRY(check_ptr(hidden, n_tokens > 0, 16, "hidden"));
  HS2_TRY(check_ptr(packed, true, 256, "packed"));
  if (n_tokens == 0) return HS2_OK;
  HS2_HIP(bridge_gemm(n_tokens, d_model, n_bridged, hidden, static_cast<const uint16_t*>(packed), outs, scales, fp8,
                      static_cast<hipStream_t>(stream)),
          "bridge GEMM");
  return HS2_OK;
}

size_t hs2_bridge_append_workspace_bytes(int32_t batch, int32_t d_model, int32_t head_dim, int32_t n_bridged) {
  if (batch < 0 || d_model < kAppendSliceK || d_model > kMaxAppendDModel || d_model % kAppendSliceK ||
      head_dim != kDim || n_bridged < 1 || n_bridged > 4)
    return 0;
  const size_t partials = static_cast<size_t>(d_model / kAppendSliceK) * batch * 2 * n_bridged * kDim * sizeof(float);
  return std::max<size_t>(align_up(partials), 256);
}

hs2_status hs2_bridge_append(int32_t batch, int32_t d_model, int32_t head_dim, int32_t n_bridged, int32_t kv_dtype,
                             const int64_t* seq_offsets, int64_t total_tokens, const void* hidden,
                             const void* const* w_k, const void* const* w_v, void* const* k_cache,
                             void* const* v_cache, float* const* k_scale, float* const* v_scale, void* workspace,
                             size_t workspace_bytes, void* stream) {
  if (batch < 0) return fail(HS2_ERR_INVALID_ARGUMENT, "batch %d < 0", batch);
  if (total_tokens < 0) return fail(HS2_ERR_INVALID_ARGUMENT, "total_tokens < 0");
  if (head_dim != kDim) return fail(HS2_ERR_UNSUPPORTED, "head_dim %d (only 128 is supported)", head_dim);
  if (d_model < kAppendSliceK || d_model > kMaxAppendDModel || d_model % kAppendSliceK)
    return fail(HS2_ERR_UNSUPPORTED, "d_model %d must be a multiple of 128 in [128, 16384]", d_model);
  if (n_bridged < 1 || n_bridged > 4) return fail(HS2_ERR_UNSUPPORTED, "n_bridged %d (1..4 supported)", n_bridged);
  if (kv_dtype != HS2_KV_BF16 && kv_dtype != HS2_KV_FP8_E4M3)
    return fail(HS2_ERR_INVALID_ARGUMENT, "kv_dtype %d unknown", kv_dtype);
  const bool fp8 = kv_dtype == HS2_KV_FP8_E4M3;
  const bool any = batch > 0;
  if (any && !seq_offsets) return fail(HS2_ERR_INVALID_ARGUMENT, "seq_offsets is NULL");
  if (seq_offsets && !aligned(seq_offsets, 8)) return fail(HS2_ERR_INVALID_ARGUMENT, "seq_offsets not 8-byte aligned");
  if (!w_k || !w_v || !k_cache || !v_cache) return fail(HS2_ERR_INVALID_ARGUMENT, "weight/cache pointer array is NULL");
  if (fp8 && (!k_scale || !v_scale)) return fail(HS2_ERR_INVALID_ARGUMENT, "E4M3 caches need k_scale and v_scale");
  if (!fp8 && (k_scale || v_scale)) return fail(HS2_ERR_INVALID_ARGUMENT, "bf16 caches take no scales (pass NULL)");
  AppendParams p{};
  for (int l = 0; l < n_bridged; ++l) {
    p.w[2 * l] = static_cast<const uint16_t*>(w_k[l]);
    p.w[2 * l + 1] = static_cast<const uint16_t*>(w_v[l]);
    p.out[2 * l] = k_cache[l];
    p.out[2 * l + 1] = v_cache[l];
    if (fp8) {
      p.scale[2 * l] = k_scale[l];
      p.scale[2 * l + 1] = v_scale[l];
    }
  }
  const bool rows = any && total_tokens > 0;
  for (int i = 0; i < 2 * n_bridged; ++i) {
    HS2_TRY(check_ptr(p.w[i], true, 16, "w_k/w_v entry"));
    HS2_TRY(check_ptr(p.out[i], rows, 16, "k_cache/v_cache entry"));
    if (fp8) HS2_TRY(check_ptr(p.scale[i], rows, 4, "k_scale/v_scale entry"));
  }
  HS2_TRY(check_ptr(hidden, any, 16, "hidden"));
  const size_t need = hs2_bridge_append_workspace_bytes(batch, d_model, head_dim, n_bridged);
  if (workspace_bytes < need) return fail(HS2_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu needed", workspace_bytes, need);
  HS2_TRY(check_ptr(workspace, true, 256, "workspace"));
  if (!any || total_tokens == 0) return HS2_OK;
  p.seq_offsets = seq_offsets;
  p.total_tokens = total_tokens;
  p.batch = batch;
  p.d_model = d_model;
  p.n_out = 2 * n_bridged;
  p.hidden = static_cast<const uint16_t*>(hidden);
  p.fp8 = fp8 ? 1 : 0;
  p.partials = static_cast<float*>(workspace);
  HS2_HIP(launch_bridge_append(p, static_cast<hipStream_t>(stream)), "bridge append");
  return HS2_OK;
}

hs2_status hs2_swa_decode(int32_t batch, int32_t window, int32_t kv_dtype, float softmax_scale,
                          const int64_t* lengths, void* ring_k, void* ring_v, float* ring_k_scale,
                          float* ring_v_scale, const void* k_new, const void* v_new, const float* k_new_scale,
                          const float* v_new_scale, const float* q, float* o, void* stream) {
  if (batch < 0) return fail(HS2_ERR_INVALID_ARGUMENT, "batch %d < 0", batch);
  if (window < 1 || window > kBudget) return fail(HS2_ERR_UNSUPPORTED, "window %d (1..1152 supported)", window);
  if (kv_dtype != HS2_KV_BF16 && kv_dtype != HS2_KV_FP8_E4M3)
    return fail(HS2_ERR_INVALID_ARGUMENT, "kv_dtype %d unknown", kv_dtype);
  if (!(softmax_scale > 0.f) || !isfinite(softmax_scale))
    return fail(HS2_ERR_INVALID_ARGUMENT, "softmax_scale must be finite and > 0");
  const bool fp8 = kv_dtype == HS2_KV_FP8_E4M3;
  const bool any = batch > 0;
  HS2_TRY(check_ptr(lengths, any, 8, "lengths"));
  HS2_TRY(check_ptr(ring_k, any, 16, "ring_k"));
  HS2_TRY(check_ptr(ring_v, any, 16, "ring_v"));
  HS2_TRY(check_ptr(q, any, 16, "q"));
  HS2_TRY(check_ptr(o, any, 16, "o"));
  if (fp8) {
    HS2_TRY(check_ptr(ring_k_scale, any, 4, "ring_k_scale"));
    HS2_TRY(check_ptr(ring_v_scale, any, 4, "ring_v_scale"));
  } else if (ring_k_scale || ring_v_scale || k_new_scale || v_new_scale) {
    return fail(HS2_ERR_INVALID_ARGUMENT, "bf16 rings take no scales (pass NULL)");
  }
  if ((k_new == nullptr) != (v_new == nullptr)) return fail(HS2_ERR_INVALID_ARGUMENT, "k_new and v_new: both or neither");
  if (k_new) {
    HS2_TRY(check_ptr(k_new, any, 16, "k_new"));
    HS2_TRY(check_ptr(v_new, any, 16, "v_new"));
    if (fp8) {
      HS2_TRY(check_ptr(k_new_scale, any, 4, "k_new_scale"));
      HS2_TRY(check_ptr(v_new_scale, any, 4, "v_new_scale"));
    }
  }
  if (!any) return HS2_OK;
  SparseParams sp{};
  sp.total_tokens = static_cast<int64_t>(batch) * window;
  sp.max_context = window;
  sp.k = static_cast<const uint8_t*>(ring_k);
  sp.v = static_cast<const uint8_t*>(ring_v);
  sp.k_scale = ring_k_scale;
  sp.v_scale = ring_v_scale;
  sp.q_sparse = q;
  sp.qscale = static_cast<float>(static_cast<double>(softmax_scale) * kLog2e);
  sp.batch = batch;
  sp.n_layers = 1;
  sp.budget = window;
  sp.out = o;
  sp.lengths = lengths;
  sp.k_new = static_cast<const uint8_t*>(k_new);
  sp.v_new = static_cast<const uint8_t*>(v_new);
  sp.k_new_scale = k_new_scale;
  sp.v_new_scale = v_new_scale;
  sp.ring_k = static_cast<uint8_t*>(ring_k);
  sp.ring_v = static_cast<uint8_t*>(ring_v);
  sp.ring_ks = ring_k_scale;
  sp.ring_vs = ring_v_scale;
  HS2_HIP(launch_sparse_window(sp, fp8, static_cast<hipStream_t>(stream)), "sliding-window attention");
  return HS2_OK;
}

hs2_status hs2_full_decode(const hs2_decode_desc* desc, const int64_t* seq_offsets, const void* k_cache,
                           const void* v_cache, const float* k_scale, const float* v_scale, const float* q_full,
                           float* o_full, void* workspace, size_t workspace_bytes, void* stream) {
  HS2_TRY(check_desc(desc));
  const hs2_decode_desc& d = *desc;
  HS2_TRY(check_kv(d, seq_offsets, k_cache, v_cache, k_scale, v_scale));
  const bool any = d.batch > 0;
  HS2_TRY(check_ptr(q_full, any, 16, "q_full"));
  HS2_TRY(check_ptr(o_full, any, 16, "o_full"));
  DecodeLayout L;
  HS2_TRY(check_workspace(d, workspace, workspace_bytes, L));
  if (!any) return HS2_OK;
  DecodeArgs a{desc, seq_offsets, k_cache, v_cache, k_scale, v_scale, q_full, nullptr, o_full, nullptr,
               nullptr, nullptr, nullptr, workspace, static_cast<hipStream_t>(stream)};
  TimingRecord* rec = nullptr;
  HS2_TRY(timing_begin(&rec));
  if (rec && rec->last > 2) rec->last = 2;  // stages 0 partial pass, 1 merge
  // The plain pass: partials only, then the merge into o_full; no score
  // bounds, statistics or selection state.
  HS2_TRY(mark(rec, 0, a.stream));
  HS2_TRY(run_full(a, L, kFullPlain, nullptr, rec));
  return HS2_OK;
}

hs2_status hs2_stage_timing_enable(int32_t mode) {
  if (mode < 0 || mode > 2) return fail(HS2_ERR_INVALID_ARGUMENT, "timing mode %d (0, 1 or 2)", mode);
  std::lock_guard<std::mutex> lock(g_timing_mu);
  g_timing_mode = mode;
  return HS2_OK;
}

namespace {
// Waits for the recorded calls and writes each call's stage durations (0 for
// stages it did not record) to per_call[r][stage] for r < max_calls (when
// per_call is not NULL) and their means to mean_ms (when not NULL); clears the
// record.  Caller holds g_timing_mu.
hs2_status read_records(float* mean_ms, float* per_call, int32_t max_calls, int32_t* n_calls) {
  double sum[HS2_N_STAGES] = {0, 0, 0, 0};
  for (int r = 0; r < g_records_used; ++r) {
    const int last = g_records[r].last;
    HS2_HIP(hipEventSynchronize(g_records[r].ev[last]), "hipEventSynchronize");
    for (int sidx = 0; sidx < HS2_N_STAGES; ++sidx) {
      float ms = 0.f;
      if (sidx < last)
        HS2_HIP(hipEventElapsedTime(&ms, g_records[r].ev[sidx], g_records[r].ev[sidx + 1]), "hipEventElapsedTime");
      sum[sidx] += ms;
      if (per_call && r < max_calls) per_call[static_cast<size_t>(r) * HS2_N_STAGES + sidx] = ms;
    }
  }
  if (mean_ms)
    for (int sidx = 0; sidx < HS2_N_STAGES; ++sidx)
      mean_ms[sidx] = g_records_used ? static_cast<float>(sum[sidx] / g_records_used) : 0.f;
  *n_calls = g_records_used;
  g_records_used = 0;
  return HS2_OK;
}
}  // namespace

hs2_status hs2_stage_timing_read(float* mean_ms, int32_t* n_calls) {
  if (!mean_ms || !n_calls) return fail(HS2_ERR_INVALID_ARGUMENT, "NULL output");
  std::lock_guard<std::mutex> lock(g_timing_mu);
  return read_records(mean_ms, nullptr, 0, n_calls);
}

hs2_status hs2_stage_timing_read_calls(float* ms, int32_t max_calls, int32_t* n_calls) {
  if (!ms || !n_calls || max_calls < 0) return fail(HS2_ERR_INVALID_ARGUMENT, "NULL output or max_calls < 0");
  std::lock_guard<std::mutex> lock(g_timing_mu);
  return read_records(nullptr, ms, max_calls, n_calls);
}

const char* hs2_status_string(hs2_status status) {
  switch (status) {
    case HS2_OK: return "HS2_OK";
    case HS2_ERR_INVALID_ARGUMENT: return "HS2_ERR_INVALID_ARGUMENT";
    case HS2_ERR_UNSUPPORTED: return "HS2_ERR_UNSUPPORTED";
    case HS2_ERR_WORKSPACE_TOO_SMALL: return "HS2_ERR_WORKSPACE_TOO_SMALL";
    case HS2_ERR_HIP: return "HS2_ERR_HIP";
  }
  return "HS2_UNKNOWN_STATUS";
}

const char* hs2_last_error_message(void) { return g_err; }

}  // extern "C"
