// Per-token score and token-level selection for one hybrid block.
//
// Score: score_j = sum over the 16 query heads of head h's softmax
// probability of token j over the whole context (the full layer's attention
// scores pick the positions: "Luo Fuli Teases Xiaomi MiMo-V3 Architecture",
// paragraph on keeping a few full-attention layers; toolnavs.com article
// 2080, section "Ce que fait HySparse2").
//
// Selection: the last `window` positions always, plus the `top_k` positions
// before them with the largest score, ties to the lower position (readaitime.com
// news of 2026-09-24, paragraph on dropping the separate SWA branch; toolnavs.com
// (fr/ko), sections "Ce que fait HySparse2" / "HySparse2가 한 일").
//
// Exact radix select on a 64-bit key per token: the fp32 score bits (scores are
// >= 0, so their bit patterns order like the values) above the complement of the
// position, so larger keys win and equal scores go to the lower position; keys
// are distinct and the selection is exactly "the top_k largest keys".
//
// Two ways to the scores, one selection, and no cross-workgroup fence (on a
// multi-XCD part an agent-scope fence writes back the XCD's L2):
//
// Spill mode (every score is wanted): the full pass kept all logits.
//  1. score pass: score_j for every position, and the histogram of the first
//     11-bit digit (score bits 30..20), per workgroup in LDS, merged by
//     global atomics;
//  2. collect: every workgroup resolves the first digit D0 from the finished
//     histogram (the same result in all of them), sends the positions whose
//     digit is above D0 (all selected) to selbuf and the keys of the D0 bin to
//     a candidate list; each list is gathered in LDS and placed with one
//     atomic per workgroup;
//  3. finish, one workgroup per sequence: radix passes over the candidates in
//     LDS until the threshold key is fixed (over the sequence's scores if the
//     list overflowed), emit the rest, sort the positions ascending (bitonic)
//     and append the window.
//
// Bound mode (no score output): the full pass kept per token
// shat_j = sum_h a_hj (bf16) and per 16-token tile and head
// u_h = m_h - log2 c_h (its running max and approximate reciprocal running
// sum), which bound score_j within shat_j * [min_h F_h, max_h F_h].
//  1. histogram of the lower bounds' first digit (fused with the merge);
//  2. collect the positions whose upper bound reaches the lower edge of the bin
//     holding the k-th largest lower bound, less the slack: at least k
//     positions have a score at or above that edge, so every position of the
//     exact top-k (ties included) is collected;
//  3. rescore the candidates exactly, with the same arithmetic as the spill
//     path;
//  4. finish as above over the exact candidate keys.
#include "hs2_device.h"
#include "hs2_internal.h"
#include "merge.h"

namespace hs2 {

namespace {

constexpr int kCollectLds = 2048;  // tokens a collect workgroup stages per round

__device__ __forceinline__ unsigned long long select_key(float score, int pos) {
  return (static_cast<unsigned long long>(__float_as_uint(score)) << 32) |
         static_cast<unsigned long long>(0xFFFFFFFFu - static_cast<uint32_t>(pos));
}

__device__ __forceinline__ int key_pos(unsigned long long key) {
  return static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(key));
}

__device__ __forceinline__ uint32_t digit0(float score) { return (__float_as_uint(score) >> 20) & (kRadixBins - 1); }

// A caller-given score as the selection ranks it: -0.0, negative values and
// NaN count as +0.0, so the first digit and the 64-bit key of a score always
// agree (both read the bit pattern with the sign bit clear).
__device__ __forceinline__ float canon_score(float score) {
  const uint32_t u = __float_as_uint(score);
  return (u & 0x80000000u) || u > 0x7F800000u ? 0.f : score;
}

struct Resolved {
  int digit;        // the bin holding the rank-th largest key
  uint32_t above;   // keys in higher bins
  uint32_t count;   // keys in that bin
};

// Block-wide: find the bin where the count from the top reaches `rank`.
// Thread t owns bins [t * per, (t + 1) * per); suffix sums run within each
// wave by lane shuffles, and across the waves through NT / 64 totals in
// s_scan, so the whole search takes three barriers.
template <int NT>
__device__ Resolved block_resolve(const uint32_t* hist, int nbins, uint32_t rank, uint32_t* s_scan, Resolved* s_out) {
  constexpr int kWaves = NT / 64;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = t >> 6;
  const int per = nbins >= NT ? nbins / NT : 1;
  const int lo = t * per;
  uint32_t sum = 0;
  for (int i = 0; i < per; ++i)
    if (lo + i < nbins) sum += hist[lo + i];
  uint32_t suf = sum;  // keys in this lane's bins and in those of the lanes above it
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t o = __shfl_down(suf, d);
    if (lane + d < 64) suf += o;
  }
  if (lane == 0) s_scan[w] = suf;  // the wave's total
  __syncthreads();
  uint32_t above = suf - sum;  // keys in bins above this thread's range
  for (int w2 = w + 1; w2 < kWaves; ++w2) above += s_scan[w2];
  if (above < rank && rank <= above + sum) {
    uint32_t acc = above;
    for (int i = lo + per - 1; i >= lo; --i) {
      if (i >= nbins) continue;
      const uint32_t c = hist[i];
      if (acc + c >= rank) {
        s_out->digit = i;
        s_out->above = acc;
        s_out->count = c;
        break;
      }
      acc += c;
    }
  }
  __syncthreads();
  const Resolved r = *s_out;
  __syncthreads();
  return r;
}

// Block-wide exclusive prefix sum of one value per thread (NT threads):
// lane shuffles within each wave, NT / 64 wave totals through s_scan.
template <int NT>
__device__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* s_scan) {
  constexpr int kWaves = NT / 64;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = t >> 6;
  uint32_t incl = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t o = __shfl_up(incl, d);
    if (lane >= d) incl += o;
  }
  if (lane == 63) s_scan[w] = incl;
  __syncthreads();
  uint32_t before = incl - v;
  for (int w2 = 0; w2 < w; ++w2) before += s_scan[w2];
  return before;  // s_scan[0 .. NT/64) keeps the wave totals: sync before reusing it
}

}  // namespace

__global__ __launch_bounds__(256) void select_init_kernel(SelectParams p) {
  const int b = blockIdx.x;
  uint32_t* h = p.hist0 + static_cast<size_t>(b) * kRadixBins;
  for (int i = threadIdx.x; i < kRadixBins; i += blockDim.x) h[i] = 0;
  if (threadIdx.x < 4) p.counters[b * 4 + threadIdx.x] = 0;
}

hipError_t launch_select_init(const SelectParams& p, int batch, hipStream_t s) {
  if (batch == 0) return hipSuccess;
  hipLaunchKernelGGL(select_init_kernel, dim3(batch), dim3(256), 0, s, p);
  return hipGetLastError();
}

// Score pass (COMPUTE: score_j from the spilled log2-domain logits and each
// head's global max and sum; else read the given scores) with the first-digit
// histogram of the out-of-window positions.
template <bool COMPUTE>
__global__ __launch_bounds__(256) void score_hist_kernel(SelectParams p, int histogram) {
  __shared__ uint32_t s_hist[kRadixBins];
  const int b = blockIdx.y;
  int64_t base;
  int len;
  seq_bounds(p.seq_offsets, b, p.total_tokens, p.max_context, base, len);
  const int j0 = blockIdx.x * kScoreBlockTokens;
  const int limit = COMPUTE ? len : len - p.window;
  if (j0 >= limit) return;
  const int j1 = min(limit, j0 + kScoreBlockTokens);
  const bool selecting = histogram && len > p.budget;
  const int dom = len - p.window;
  float mx[kHeads], iz[kHeads];
  if constexpr (COMPUTE) {
    const float* st = p.stats + static_cast<int64_t>(b) * kHeads * 2;
#pragma unroll
    for (int h = 0; h < kHeads; ++h) {
      mx[h] = st[2 * h];
      iz[h] = 1.f / st[2 * h + 1];
    }
  }
  if (selecting)
    for (int i = threadIdx.x; i < kRadixBins; i += blockDim.x) s_hist[i] = 0;
  __syncthreads();
  constexpr int kPer = kScoreBlockTokens / 256;  // tokens per thread
  constexpr int kBatch = COMPUTE ? 2 : 8;       // tokens whose loads are in flight together
#pragma unroll
  for (int i0 = 0; i0 < kPer; i0 += kBatch) {
    float sc[kBatch];
    if constexpr (COMPUTE) {
      float4 l[kBatch][4];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int j = min(j0 + (i0 + u) * 256 + static_cast<int>(threadIdx.x), j1 - 1);
        const float4* lp = reinterpret_cast<const float4*>(p.spill + (base + j) * kHeads);
#pragma unroll
        for (int q = 0; q < 4; ++q) l[u][q] = lp[q];
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const float x[16] = {l[u][0].x, l[u][0].y, l[u][0].z, l[u][0].w, l[u][1].x, l[u][1].y, l[u][1].z, l[u][1].w,
                             l[u][2].x, l[u][2].y, l[u][2].z, l[u][2].w, l[u][3].x, l[u][3].y, l[u][3].z, l[u][3].w};
        float acc = 0.f;
#pragma unroll
        for (int h = 0; h < kHeads; ++h) acc = __builtin_fmaf(exp2f(x[h] - mx[h]), iz[h], acc);
        sc[u] = acc;
      }
    } else {
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int j = min(j0 + (i0 + u) * 256 + static_cast<int>(threadIdx.x), j1 - 1);
        sc[u] = canon_score(p.score[base + j]);
      }
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int j = j0 + (i0 + u) * 256 + static_cast<int>(threadIdx.x);
      if (j >= j1) continue;
      if constexpr (COMPUTE) p.score[base + j] = sc[u];
      if (selecting && j < dom) atomicAdd(&s_hist[digit0(sc[u])], 1u);
    }
  }
  if (!selecting) return;
  __syncthreads();
  uint32_t* gh = p.hist0 + static_cast<size_t>(b) * kRadixBins;
  for (int i = threadIdx.x; i < kRadixBins; i += blockDim.x) {
    const uint32_t c = s_hist[i];
    if (c) atomicAdd(gh + i, c);
  }
}

hipError_t launch_score_hist(const SelectParams& p, int batch, int64_t max_context, bool compute_score,
                             bool histogram, hipStream_t s) {
  if (batch == 0 || max_context == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((max_context + kScoreBlockTokens - 1) / kScoreBlockTokens), batch);
  if (compute_score)
    hipLaunchKernelGGL(score_hist_kernel<true>, grid, dim3(256), 0, s, p, histogram ? 1 : 0);
  else
    hipLaunchKernelGGL(score_hist_kernel<false>, grid, dim3(256), 0, s, p, histogram ? 1 : 0);
  return hipGetLastError();
}

// Collect: winners (digit above D0) straight into selbuf, the D0 bin's keys
// into the candidate list.  Each workgroup gathers both lists in LDS and
// reserves room in the sequence's lists with one atomic each.
__global__ __launch_bounds__(256) void collect_kernel(SelectParams p) {
  __shared__ uint32_t s_hist[kRadixBins];
  __shared__ uint32_t s_scan[256];
  __shared__ Resolved s_res;
  __shared__ int32_t s_win[kTopK];
  __shared__ unsigned long long s_cand[kCollectLds];
  __shared__ uint32_t s_nwin, s_ncand, s_bwin, s_bcand;
  const int b = blockIdx.y;
  int64_t base;
  int len;
  seq_bounds(p.seq_offsets, b, p.total_tokens, p.max_context, base, len);
  if (len <= p.budget) return;
  const int dom = len - p.window;
  const int j0 = blockIdx.x * kCollectBlockTokens;
  if (j0 >= dom) return;
  const int j1 = min(dom, j0 + kCollectBlockTokens);
  const uint32_t* gh = p.hist0 + static_cast<size_t>(b) * kRadixBins;
  for (int i = threadIdx.x; i < kRadixBins; i += blockDim.x) s_hist[i] = gh[i];
  if (threadIdx.x == 0) {
    s_nwin = 0;
    s_ncand = 0;
  }
  __syncthreads();
  const Resolved r0 = block_resolve<256>(s_hist, kRadixBins, static_cast<uint32_t>(p.top_k), s_scan, &s_res);
  const uint32_t d0 = static_cast<uint32_t>(r0.digit);
  uint32_t* wins = p.counters + b * 4;
  uint32_t* cands = p.counters + b * 4 + 1;
  int32_t* selbuf = p.selbuf + static_cast<size_t>(b) * p.top_k;
  unsigned long long* cand = p.cand + static_cast<size_t>(b) * kCandCap;
  for (int c0 = j0; c0 < j1; c0 += kCollectLds) {
    const int c1 = min(j1, c0 + kCollectLds);
    constexpr int kBatch = 8;
    for (int i0 = c0; i0 < c1; i0 += kBatch * 256) {
      float sc[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u)
        sc[u] = canon_score(p.score[base + min(i0 + u * 256 + static_cast<int>(threadIdx.x), c1 - 1)]);
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int j = i0 + u * 256 + static_cast<int>(threadIdx.x);
        if (j >= c1) continue;
        const uint32_t dg = digit0(sc[u]);
        if (dg > d0) {
          const uint32_t w = atomicAdd(&s_nwin, 1u);
          if (w < static_cast<uint32_t>(kTopK)) s_win[w] = j;
        } else if (dg == d0) {
          s_cand[atomicAdd(&s_ncand, 1u)] = select_key(sc[u], j);
        }
      }
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      s_bwin = s_nwin ? atomicAdd(wins, s_nwin) : 0u;
      s_bcand = s_ncand ? atomicAdd(cands, s_ncand) : 0u;
    }
    __syncthreads();
    for (uint32_t i = threadIdx.x; i < s_nwin; i += blockDim.x)
      if (s_bwin + i < static_cast<uint32_t>(p.top_k)) selbuf[s_bwin + i] = s_win[i];
    for (uint32_t i = threadIdx.x; i < s_ncand; i += blockDim.x)
      if (s_bcand + i < static_cast<uint32_t>(kCandCap)) cand[s_bcand + i] = s_cand[i];
    __syncthreads();
    if (threadIdx.x == 0) {
      s_nwin = 0;
      s_ncand = 0;
    }
    __syncthreads();
  }
}

// Finish one sequence with one workgroup.  Spill mode: resolve the threshold
// inside the D0 bin (winners above it are already in selbuf).  Bound mode: the
// candidate list holds exact keys of every position that can be selected;
// resolve the threshold over all of them.  Emit, sort ascending, add the window.
// The radix passes read the candidates from LDS when they fit there.
constexpr int kFinishLdsKeys = 16384;

// Keys of sequence b (base: its first row) in the key room: its region starts
// at row base + b * kBoundBlockTokens and holds len + kBoundBlockTokens
// slots, so the regions of consecutive sequences do not overlap.  A
// sequence's one list starts at the region's start (at most len - window
// keys); past kSharedListBlocks candidate workgroups, workgroup j's segment
// starts kBoundBlockTokens * j further in (nb = ceil((len - window) /
// kBoundBlockTokens) segments of at most kBoundBlockTokens keys each).
__device__ __forceinline__ int64_t key_segment(int64_t base, int b, int j) {
  return base + static_cast<int64_t>(b + j) * kBoundBlockTokens;
}

template <bool BOUND>
__global__ __launch_bounds__(1024) void finish_kernel(SelectParams p) {
  __shared__ uint32_t s_hist[kRadixBins];
  __shared__ uint32_t s_scan[16];
  // bound mode, keys in per-workgroup segments: exclusive prefix of the counts
  __shared__ uint32_t s_pre[BOUND ? kMaxCollectBlocks + 1 : 1];
  __shared__ Resolved s_res;
  __shared__ int32_t s_sel[kTopK];
  __shared__ uint32_t s_n, s_nst;
  __shared__ unsigned long long s_keys[kFinishLdsKeys];
  const int b = blockIdx.x;
  const int t = threadIdx.x;
  int64_t base;
  int len;
  seq_bounds(p.seq_offsets, b, p.total_tokens, p.max_context, base, len);
  int32_t* out = p.sel_idx + static_cast<size_t>(b) * p.budget;
  if (len <= p.budget) {
    for (int i = t; i < p.budget; i += blockDim.x) out[i] = i < len ? i : -1;
    if (t == 0) p.sel_count[b] = len;
    return;
  }
  const int dom = len - p.window;
  s_sel[t] = -1;  // a slot no emission fills stays out of the bitmap below (blockDim.x == kTopK)
  // Bound mode: the keys fill the start of the sequence's region, which has
  // room for every position, or (past kSharedListBlocks candidate
  // workgroups) one segment per workgroup, key i in the segment of the
  // workgroup j with s_pre[j] <= i < s_pre[j + 1].  Spill mode:
  // cand[b][0, kCandCap), and a scan of the D0 bin's scores when that
  // overflowed.
  const int nseg = (dom + kBoundBlockTokens - 1) / kBoundBlockTokens;
  const bool segmented = BOUND && nseg > kSharedListBlocks;  // uniform
  uint32_t ncand;
  if (segmented) {
    const uint32_t* cnt = p.cand_cnt + static_cast<size_t>(b) * p.cand_blocks;
    const int per = (nseg + 1023) / 1024;
    const int j0 = t * per;
    uint32_t sum = 0;
    for (int jj = j0; jj < min(j0 + per, nseg); ++jj) sum += cnt[jj];
    uint32_t run = block_exclusive_scan<1024>(sum, s_scan);
    for (int jj = j0; jj < min(j0 + per, nseg); ++jj) {
      s_pre[jj] = run;
      run += cnt[jj];
    }
    if (j0 < nseg && j0 + per >= nseg) s_pre[nseg] = run;  // the thread holding the last workgroup
    __syncthreads();
    ncand = s_pre[nseg];
  } else {
    ncand = p.counters[b * 4 + 1];
  }
  if (BOUND) ncand = min(ncand, static_cast<uint32_t>(dom));
  const bool overflow = !BOUND && ncand > static_cast<uint32_t>(kCandCap);
  const unsigned long long* cand = BOUND ? p.cand + key_segment(base, b, 0) : p.cand + static_cast<size_t>(b) * kCandCap;
  auto key_at = [&](uint32_t i) {  // key i of the candidate list, i < ncand
    if (!segmented) return cand[i];
    int lo = 0, hi = nseg - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_pre[mid] <= i) lo = mid; else hi = mid - 1;
    }
    return p.cand[key_segment(base, b, lo) + (i - s_pre[lo])];
  };
  const float* score = p.score ? p.score + base : nullptr;  // spill mode only
  bool staged = !overflow && ncand <= static_cast<uint32_t>(kFinishLdsKeys);
  if (staged) {
    constexpr int kBatch = 8;  // loads in flight per thread
    for (uint32_t i0 = 0; i0 < ncand; i0 += kBatch * 1024) {
      unsigned long long k8[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const uint32_t i = i0 + u * 1024 + t;
        k8[u] = i < ncand ? key_at(i) : 0ull;
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const uint32_t i = i0 + u * 1024 + t;
        if (i < ncand) s_keys[i] = k8[u];
      }
    }
  }
  uint32_t d0 = 0;
  uint32_t nwin = 0;
  uint32_t rank = static_cast<uint32_t>(p.top_k);
  unsigned long long prefix = 0;
  int pshift = 63;
  int first_pass = 0;
  bool done = false;
  if constexpr (!BOUND) {
    const uint32_t* gh = p.hist0 + static_cast<size_t>(b) * kRadixBins;
    for (int i = t; i < kRadixBins; i += blockDim.x) s_hist[i] = gh[i];
    __syncthreads();
    const Resolved r0 = block_resolve<1024>(s_hist, kRadixBins, rank, s_scan, &s_res);
    d0 = static_cast<uint32_t>(r0.digit);
    nwin = r0.above;  // positions already in selbuf
    rank -= nwin;
    prefix = d0;
    pshift = 52;
    first_pass = 1;
    done = r0.count == rank;
  }

  // Visit every key that can still be selected: the candidate list, or a scan
  // of the sequence's scores (spill mode: the D0 bin only) when it overflowed.
  auto for_each_key = [&](auto&& fn) {
    if (staged) {
      for (uint32_t i = t; i < ncand; i += blockDim.x) fn(s_keys[i]);
    } else if (!overflow) {
      constexpr int kBatch = 8;  // loads in flight per thread
      for (uint32_t i0 = 0; i0 < ncand; i0 += kBatch * 1024) {
        unsigned long long k8[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const uint32_t i = i0 + u * 1024 + t;
          k8[u] = i < ncand ? key_at(i) : 0ull;
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u)
          if (i0 + u * 1024 + t < ncand) fn(k8[u]);
      }
    } else {
      for (int j = t; j < dom; j += blockDim.x) {
        const float sc = canon_score(score[j]);
        if (BOUND || digit0(sc) == d0) fn(select_key(sc, j));
      }
    }
  };

  // The digits run over key - kmin, 11 bits at a time from bit top_bits down.
  // Normally kmin = 0 and top_bits = 63 (the bits below the sign: 11, 11, 11,
  // 11, 11, 8).  A large candidate list read from global memory (near-uniform
  // attention, where the bounds prune little) takes its range first: keys
  // that share an exponent would pile into one or two bins of the first digit,
  // and a wave's 64 atomic adds to one LDS word serialise; over the span's bits
  // the first digit spreads them.
  unsigned long long kmin = 0;
  int top_bits = 63;
  if (BOUND && !staged && ncand > 1u) {
    __shared__ unsigned long long s_lo[16], s_hi[16];
    unsigned long long lo = ~0ull, hi = 0ull;
    for_each_key([&](unsigned long long key) {
      lo = min(lo, key);
      hi = max(hi, key);
    });
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      lo = min(lo, shfl_xor_u64(lo, off));
      hi = max(hi, shfl_xor_u64(hi, off));
    }
    if ((t & 63) == 0) {
      s_lo[t >> 6] = lo;
      s_hi[t >> 6] = hi;
    }
    __syncthreads();
    lo = s_lo[0];
    hi = s_hi[0];
    for (int w = 1; w < 16; ++w) {
      lo = min(lo, s_lo[w]);
      hi = max(hi, s_hi[w]);
    }
    kmin = lo;
    top_bits = 64 - __clzll(hi - lo);  // keys are distinct, so hi > lo; hi - lo < 2^63
    pshift = top_bits;
  }
  for (int pass = first_pass; !done; ++pass) {
    const int top = top_bits - 11 * pass;
    if (top <= 0) break;
    const int bits = min(11, top);
    const int shift = top - bits;
    const uint32_t mask = (1u << bits) - 1u;
    for (int i = t; i < kRadixBins; i += blockDim.x) s_hist[i] = 0;
    __syncthreads();
    for_each_key([&](unsigned long long key) {
      const unsigned long long rk = key - kmin;
      if ((rk >> pshift) == prefix) atomicAdd(&s_hist[static_cast<uint32_t>(rk >> shift) & mask], 1u);
    });
    __syncthreads();
    const Resolved r = block_resolve<1024>(s_hist, 1 << bits, rank, s_scan, &s_res);
    rank -= r.above;
    prefix = (prefix << bits) | static_cast<unsigned long long>(r.digit);
    pshift = shift;
    done = r.count == rank || shift == 0;
    // A list read from memory: after its first pass only the threshold bin is
    // undecided.  One more read puts the keys above it into the selection and
    // stages the bin's keys in LDS, so the remaining passes read LDS.
    if (BOUND && !staged && !done && pass == first_pass && r.count <= static_cast<uint32_t>(kFinishLdsKeys)) {
      if (t == 0) {
        s_n = 0;
        s_nst = 0;
      }
      __syncthreads();
      for_each_key([&](unsigned long long key) {
        const unsigned long long d = (key - kmin) >> pshift;
        if (d > prefix) {
          const uint32_t w = atomicAdd(&s_n, 1u);
          if (w < static_cast<uint32_t>(p.top_k)) s_sel[w] = key_pos(key);
        } else if (d == prefix) {
          s_keys[atomicAdd(&s_nst, 1u)] = key;
        }
      });
      __syncthreads();
      nwin = min(s_n, static_cast<uint32_t>(p.top_k));
      ncand = s_nst;
      staged = true;
    }
  }

  // Winners from collect (spill mode; bound mode put its own in s_sel when it
  // staged the threshold bin), then the keys at or above the threshold.
  if (!BOUND)
    for (uint32_t i = t; i < nwin; i += blockDim.x) s_sel[i] = p.selbuf[static_cast<size_t>(b) * p.top_k + i];
  if (t == 0) s_n = 0;
  __syncthreads();
  for_each_key([&](unsigned long long key) {
    if (((key - kmin) >> pshift) >= prefix) {
      const uint32_t slot = nwin + atomicAdd(&s_n, 1u);
      if (slot < static_cast<uint32_t>(p.top_k)) s_sel[slot] = key_pos(key);
    }
  });
  __syncthreads();
  // Ascending order.  For out-of-window ranges up to 4096 bitmap words (131072
  // positions), mark the selected positions in a bitmap (in the candidate
  // room, free by now) and read them back in order: each thread counts the
  // bits of its run of at most four words, a block scan gives its first
  // output slot, and it emits its positions.  (Longer runs per thread cost
  // more in LDS bank conflicts than the ranking below.)
  const uint32_t nwords = (static_cast<uint32_t>(dom) + 31) >> 5;
  if (nwords <= 4u * 1024u) {
    uint32_t* bm = reinterpret_cast<uint32_t*>(s_keys);
    for (uint32_t i = t; i < nwords; i += blockDim.x) bm[i] = 0u;
    __syncthreads();
    const int32_t pos = s_sel[t];
    if (pos >= 0 && pos < dom) atomicOr(&bm[pos >> 5], 1u << (pos & 31));
    __syncthreads();
    const uint32_t per = (nwords + 1023) >> 10;
    const uint32_t w0 = t * per, w1 = min(w0 + per, nwords);
    uint32_t cnt = 0;
    for (uint32_t w = w0; w < w1; ++w) cnt += __popc(bm[w]);
    uint32_t slot = block_exclusive_scan<1024>(cnt, s_scan);
    for (uint32_t w = w0; w < w1; ++w) {
      uint32_t bits = bm[w];
      while (bits) {
        const int bit = __ffs(bits) - 1;
        bits &= bits - 1;
        out[slot++] = static_cast<int32_t>(w * 32 + bit);
      }
    }
    if (t < p.window) out[p.top_k + t] = dom + t;
    if (t == 0) p.sel_count[b] = p.budget;
    return;
  }
  // Otherwise each wave sorts its 64 positions by a bitonic network of lane
  // shuffles, and a position's output slot is the number of positions below
  // it over the 16 sorted runs (a binary search in each, through LDS).
  int32_t x = s_sel[t];
  const int lane = t & 63;
#pragma unroll
  for (int size = 2; size <= 64; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      const int32_t y = __shfl_xor(x, stride);
      const bool up = (lane & size) == 0;
      const bool lower = (lane & stride) == 0;
      x = (lower == up) ? min(x, y) : max(x, y);
    }
  }
  int32_t* runs = reinterpret_cast<int32_t*>(s_hist);  // [16][64]
  runs[t] = x;
  __syncthreads();
  int slot_out = 0;
#pragma unroll
  for (int w2 = 0; w2 < 16; ++w2) {
    const int32_t* run = runs + 64 * w2;
    int lo = 0;
#pragma unroll
    for (int step = 32; step > 0; step >>= 1)
      if (run[lo + step - 1] < x) lo += step;
    slot_out += lo + ((lo == 63 && run[63] < x) ? 1 : 0);
  }
  out[slot_out] = x;
  if (t < p.window) out[p.top_k + t] = dom + t;
  if (t == 0) p.sel_count[b] = p.budget;
}

hipError_t launch_collect_finish(const SelectParams& p, int batch, int64_t max_context, hipStream_t s) {
  if (batch == 0) return hipSuccess;
  if (max_context > 0) {
    const dim3 grid(static_cast<unsigned>((max_context + kCollectBlockTokens - 1) / kCollectBlockTokens), batch);
    hipLaunchKernelGGL(collect_kernel, grid, dim3(256), 0, s, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(finish_kernel<false>, dim3(batch), dim3(kTopK), 0, s, p);
  return hipGetLastError();
}

// ---- bound mode ------------------------------------------------------------

// Slack on the pruning threshold and on the upper bounds: 2^-7, four times
// the 2^-9 relative rounding of shat to bf16, and far above fp32 rounding, the
// approximate exp2 / log2, and the rounding-order difference between the
// first pass's own copy of (M_h, Z_h) and the merge's.
constexpr float kLowSlack = 1.f - 1.f / 128.f;
constexpr float kHighSlack = 1.f + 1.f / 128.f;

// Min and max over heads of a tile's bound factors F_h = exp2(u_h - M_h) / Z_h.
__device__ __forceinline__ void tile_factors(const float (&u)[kHeads], const float* s_mx, const float* s_iz,
                                             float& fmin, float& fmax) {
  fmin = INFINITY;
  fmax = 0.f;
#pragma unroll
  for (int h = 0; h < kHeads; ++h) {
    const float f = exp2f(u[h] - s_mx[h]) * s_iz[h];
    fmin = fminf(fmin, f);
    fmax = fmaxf(fmax, f);
  }
}

// A tile's 16 shat values (nv of them real), stored as bf16.
__device__ __forceinline__ void load_tile_shat(const SelectParams& p, int64_t base, int tile, int nv, float (&v)[16]) {
  if ((base & 7) == 0) {  // 16-byte aligned rows
    const uint4* sh = reinterpret_cast<const uint4*>(p.shat + base + 16 * tile);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const uint4 x = sh[q];
      const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        v[8 * q + 2 * k] = __uint_as_float(w[k] << 16);
        v[8 * q + 2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = __uint_as_float(static_cast<uint32_t>(p.shat[base + 16 * tile + min(i, nv - 1)]) << 16);
  }
}

// ... and its 16 per-head u values.
__device__ __forceinline__ void load_tile_bounds(const SelectParams& p, int64_t base, int b, int tile, int nv,
                                                 float (&v)[16], float (&u)[kHeads]) {
  const float4* us = reinterpret_cast<const float4*>(p.tile_stats + tile_slot(base, b, tile) * kHeads);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float4 x = us[q];
    u[4 * q] = x.x; u[4 * q + 1] = x.y; u[4 * q + 2] = x.z; u[4 * q + 3] = x.w;
  }
  load_tile_shat(p, base, tile, nv, v);
}

// The full layer's merge and the bound selection's first pass in one launch.
// Workgroups x < 16 merge head x of sequence y and write its (M, Z).  The
// others histogram the first digit of the lower bounds lb_j = shat_j min_h F_h
// over a block of 4096 * TILES out-of-window positions (TILES 16-token tiles
// per thread: two for very long sequences, whose many workgroups otherwise
// queue on the global atomics of the sequence's one histogram), with (M_h, Z_h) recomputed from the partials' (m, z), read
// from the full pass's packed copy: the merge's result is not written yet,
// and the two differ by rounding order only, which the slack covers.
template <int TILES, bool COMPACT>
__global__ __launch_bounds__(256) void merge_bound_hist_kernel(MergeParams mp, SelectParams p) {
  constexpr int kBlockTokens = 16 * 256 * TILES;
  __shared__ MergeShared msh;
  __shared__ uint32_t s_hist[kRadixBins];
  __shared__ float s_mx[kHeads], s_iz[kHeads];
  // Item j of sequence b: j < 16 merges head j, j >= 16 is histogram block
  // j - 16.  COMPACT: a 1-D grid over the batch's items (ragged batches);
  // otherwise (blockIdx.x, blockIdx.y).
  int b, j;
  if constexpr (COMPACT) {
    auto items = [&](int l) {
      return kHeads + (l > p.budget ? (l - p.window + kBlockTokens - 1) / kBlockTokens : 0);
    };
    if (!find_item(p.seq_offsets, p.batch, p.total_tokens, p.max_context, blockIdx.x, items, b, j)) return;
    b = __builtin_amdgcn_readfirstlane(b);
    j = __builtin_amdgcn_readfirstlane(j);
  } else {
    b = blockIdx.y;
    j = blockIdx.x;
  }
  if (j < kHeads) {
    merge_one(mp, j, b, 0, 0, 0, msh);
    return;
  }
  int64_t base;
  int len;
  seq_bounds(p.seq_offsets, b, p.total_tokens, p.max_context, base, len);
  if (len <= p.budget) return;
  const int dom = len - p.window;
  const int j0 = (j - kHeads) * kBlockTokens;
  if (j0 >= dom) return;
  const int t = threadIdx.x;
  // TILES tiles per thread, 256 tiles apart, all loads issued up front.
  float v[TILES][16], u[TILES][kHeads];
#pragma unroll
  for (int k = 0; k < TILES; ++k) {
    const int tile = (j0 >> 4) + t + 256 * k;
    if (16 * tile < dom) load_tile_bounds(p, base, b, tile, min(16, dom - 16 * tile), v[k], u[k]);
  }
  for (int i = t; i < kRadixBins; i += 256) s_hist[i] = 0;
  head_stats_packed(p.pstats, b, p.chunks_per_seq, (len + mp.chunk - 1) / mp.chunk, s_mx, s_iz);
  __syncthreads();
#pragma unroll
  for (int k = 0; k < TILES; ++k) {
    const int tile = (j0 >> 4) + t + 256 * k;
    if (16 * tile >= dom) continue;
    const int nv = min(16, dom - 16 * tile);
    float fmin, fmax;
    tile_factors(u[k], s_mx, s_iz, fmin, fmax);
    float tmax = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (i < nv) {
        atomicAdd(&s_hist[digit0(v[k][i] * fmin)], 1u);
        tmax = fmaxf(tmax, v[k][i] * fmax);
      }
    }
    // the tile's largest upper bound, so the collection can skip whole tiles
    *reinterpret_cast<float2*>(p.tile_ub + tile_slot(base, b, tile) * 2) = make_float2(tmax, fmax);
  }
  __syncthreads();
  uint32_t* gh = p.hist0 + static_cast<size_t>(b) * kRadixBins;
  for (int i = t; i < kRadixBins; i += 256) {
    const uint32_t c = s_hist[i];
    if (c) atomicAdd(gh + i, c);
  }
}

// A batch whose 2-D grid (longest sequence x batch) would be mostly holes
// runs the selection's per-block kernels on a compact 1-D grid instead.
static bool ragged_batch(const SelectParams& p, int batch, int64_t max_context) {
  return static_cast<double>(batch) * static_cast<double>(max_context) > 2.0 * static_cast<double>(p.total_tokens);
}

hipError_t launch_merge_bound_hist(const MergeParams& mp, const SelectParams& p, int batch, int64_t max_context,
                                   hipStream_t s) {
  if (batch == 0) return hipSuccess;
  // Two tiles per thread only past kHistLongContext tokens: elsewhere the
  // extra parallelism of one tile per thread wins.
  const int tiles = max_context > kHistLongContext ? 2 : 1;
  const int64_t block_tokens = 16 * 256 * tiles;
  if (ragged_batch(p, batch, max_context)) {
    // at most sum_b (16 + ceil(L_b / block)) < 17 B + N / block items
    const int64_t items = static_cast<int64_t>(kHeads + 1) * batch + p.total_tokens / block_tokens;
    const dim3 grid(static_cast<unsigned>(items));
    if (tiles == 2)
      hipLaunchKernelGGL((merge_bound_hist_kernel<2, true>), grid, dim3(256), 0, s, mp, p);
    else
      hipLaunchKernelGGL((merge_bound_hist_kernel<1, true>), grid, dim3(256), 0, s, mp, p);
  } else {
    const dim3 grid(static_cast<unsigned>(kHeads + (max_context + block_tokens - 1) / block_tokens), batch);
    if (tiles == 2)
      hipLaunchKernelGGL((merge_bound_hist_kernel<2, false>), grid, dim3(256), 0, s, mp, p);
    else
      hipLaunchKernelGGL((merge_bound_hist_kernel<1, false>), grid, dim3(256), 0, s, mp, p);
  }
  return hipGetLastError();
}

// Workgroups of the candidate pass for a sequence of len tokens: one per
// 4096 out-of-window positions, and at least one per 256 tokens up to
// kMinCollectBlocks.  Short sequences have many candidates for their length
// (the bounds are loosest on each wave's first tiles: ~40% of a 4K-token
// sequence), and near-uniform scores make most positions candidates, so the
// rescoring needs more waves than the collection; but every workgroup also
// pays for resolving the threshold and building the query, so a batch of
// many short sequences is better served by fewer.
__device__ __forceinline__ int collect_blocks(const SelectParams& p, int len) {
  return len > p.budget ? max((len - p.window + kBoundBlockTokens - 1) / kBoundBlockTokens,
                              min(kMinCollectBlocks, (len + 255) / 256))
                        : 0;
}


// Candidates and their exact keys.  Workgroup j of a sequence (nb of them)
// takes the 16-token tiles j, j + nb, j + 2 nb, ... of its out-of-window
// positions, one tile per thread.  The tiles each wave of the full pass
// visited first have the loosest bounds and sit together at the start of the
// sequence; striding spreads them.  Each workgroup resolves the pruning
// threshold from the finished lower-bound histogram (every workgroup of the
// sequence finds the same one): the lower edge of the bin holding the k-th
// largest lower bound, so at least k positions score at or above it.  It
// keeps the positions whose upper bound reaches it, so every position of the
// exact top-k (ties included) is kept; a tile whose largest upper bound (from
// the first pass) misses the threshold is skipped without reading its
// tokens.  The kept positions gather in LDS, and the workgroup's four waves
// then compute their exact keys, 16 per MFMA tile: the split query from LDS
// and the same MFMA sequence as the full pass give the same logits, and the
// same head-ordered sum as the score pass gives the same score, so the keys
// are bitwise those of the spill path.  Each wave has its next tile's loads in
// flight while it scores the current one.  The keys go to the sequence's one
// list (room taken with one atomic per workgroup) or, past
// kSharedListBlocks workgroups (which would queue on that one counter), to
// the workgroup's own segment with its count.
template <bool FP8, bool COMPACT>
__global__ __launch_bounds__(256) void collect_rescore_kernel(SelectParams p) {
  // the histogram, then (once the threshold is resolved) the candidate list
  __shared__ int32_t s_buf[kBoundBlockTokens];
  static_assert(kBoundBlockTokens >= kRadixBins, "the histogram fits in the list's room");
  __shared__ u32x4 s_q[kQLdsVecs];
  __shared__ float s_lg[4][16][17];
  __shared__ float s_mx[kHeads];
  __shared__ float s_iz[kHeads];
  __shared__ uint32_t s_scan[4];
  __shared__ Resolved s_res;
  __shared__ uint32_t s_cnt, s_base;
  uint32_t* s_hist = reinterpret_cast<uint32_t*>(s_buf);
  int32_t* s_list = s_buf;
  // Workgroup j of sequence b: a compact 1-D grid for ragged batches,
  // (blockIdx.x, blockIdx.y) otherwise.
  int b, j;
  if constexpr (COMPACT) {
    auto blocks = [&](int l) { return collect_blocks(p, l); };
    if (!find_item(p.seq_offsets, p.batch, p.total_tokens, p.max_context, blockIdx.x, blocks, b, j)) return;
    b = __builtin_amdgcn_readfirstlane(b);
    j = __builtin_amdgcn_readfirstlane(j);
  } else {
    b = blockIdx.y;
    j = blockIdx.x;
  }
  int64_t base;
  int len;
  seq_bounds(p.seq_offsets, b, p.total_tokens, p.max_context, base, len);
  if (len <= p.budget) return;
  const int dom = len - p.window;
  const int nb = collect_blocks(p, len);
  if (j >= nb) return;
  const int t = threadIdx.x;
  const int tile = j + t * nb;
  const bool valid = 16 * tile < dom;
  const int nv = min(16, dom - 16 * tile);
  // Every load of the prologue is issued before any is used, so their
  // latencies overlap (one round trip, not one per load): the tile's
  // (largest upper bound, max_h F_h) (a clamped tile when past the end), the
  // histogram, the rescoring's query and the heads' (M, Z).
  const float2 ubf_raw =
      *reinterpret_cast<const float2*>(p.tile_ub + tile_slot(base, b, valid ? tile : (dom - 1) >> 4) * 2);
  const uint32_t* gh = p.hist0 + static_cast<size_t>(b) * kRadixBins;
  uint32_t hv[kRadixBins / 256];
#pragma unroll
  for (int i = 0; i < kRadixBins / 256; ++i) hv[i] = gh[t + 256 * i];
  float4 qa, qc;
  load_q_lds_raw<FP8>(p.q + static_cast<size_t>(b) * kHeads * kDim, qa, qc);
  const float2 mz = *reinterpret_cast<const float2*>(p.stats + (static_cast<int64_t>(b) * kHeads + (t & 15)) * 2);
#pragma unroll
  for (int i = 0; i < kRadixBins / 256; ++i) s_hist[t + 256 * i] = hv[i];
  if (t == 0) s_cnt = 0;
  store_q_lds(qa, qc, p.qscale, s_q);
  if (t < kHeads) {
    s_mx[t] = mz.x;
    s_iz[t] = 1.f / mz.y;
  }
  const float2 ubf = valid ? ubf_raw : make_float2(0.f, 0.f);  // (tile's largest upper bound, its max_h F_h)
  __syncthreads();
  const Resolved r0 = block_resolve<256>(s_hist, kRadixBins, static_cast<uint32_t>(p.top_k), s_scan, &s_res);
  const float thr = __uint_as_float(static_cast<uint32_t>(r0.digit) << 20) * kLowSlack;
  uint32_t mine = 0;  // bit i: token 16 tile + i is a candidate
  if (valid && ubf.x * kHighSlack >= thr) {
    float v[16];
    load_tile_shat(p, base, tile, nv, v);
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (i < nv && v[i] * ubf.y * kHighSlack >= thr) mine |= 1u << i;
  }
  // Room in the LDS list (the histogram is no longer read: block_resolve
  // ended on a barrier): one atomic per wave, lane offsets by a wave prefix
  // sum (per-candidate atomics on one counter serialise).
  {
    const int lane = t & 63;
    const uint32_t cnt = __popc(mine);
    uint32_t incl = cnt;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const uint32_t o = __shfl_up(incl, d);
      if (lane >= d) incl += o;
    }
    uint32_t wbase = 0;
    if (lane == 63 && incl) wbase = atomicAdd(&s_cnt, incl);
    uint32_t slot = __shfl(wbase, 63) + incl - cnt;
    while (mine) {
      const int i = __ffs(mine) - 1;
      mine &= mine - 1;
      s_list[slot++] = 16 * tile + i;
    }
  }
  __syncthreads();
  const int ncand = static_cast<int>(s_cnt);
  const bool shared = nb <= kSharedListBlocks;  // uniform
  if (t == 0) {
    if (shared)
      s_base = ncand ? atomicAdd(p.counters + b * 4 + 1, static_cast<uint32_t>(ncand)) : 0u;
    else
      p.cand_cnt[static_cast<size_t>(b) * p.cand_blocks + j] = static_cast<uint32_t>(ncand);
  }
  const int ntiles = (ncand + 15) >> 4;

  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);  // wave-uniform: scalar loop control
  const int lane = t & 63;
  const int n = lane & 15;
  const int g = lane >> 4;
  constexpr int kRowBytes = FP8 ? kDim : 2 * kDim;
  const int64_t kvb = p.kv_start ? p.kv_start[b] : base;  // the sequence's first K/V row
  const uint8_t* __restrict__ kbase = p.k + kvb * kRowBytes;
  struct Raw {
    u32x4 k[FP8 ? 2 : 4];
    float ks[4];
    int pos;
  };
  // lane (n, g): candidate n of the tile (clamped to the last one), row bytes
  // kload_offset(j, g); ks[r]: the K scale of candidate 4g + r
  auto load = [&](int ct, Raw& r) {
    const int i0 = min(ct, ntiles - 1) * 16;
    r.pos = min(max(s_list[i0 + min(n, ncand - 1 - i0)], 0), dom - 1);
    const uint32_t krow = static_cast<uint32_t>(r.pos) * kRowBytes;
#pragma unroll
    for (int jj = 0; jj < (FP8 ? 2 : 4); ++jj)
      r.k[jj] = *reinterpret_cast<const u32x4*>(kbase + (krow + kload_offset(jj, g)));
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) r.ks[q4] = FP8 ? p.k_scale[kvb + __shfl(r.pos, 4 * g + q4)] : 1.f;
  };
  int ct = wave;
  Raw ra, rb;
  if (ct < ntiles) load(ct, ra);  // uniform over the wave
  __syncthreads();                // s_base
  if (ct >= ntiles) return;       // uniform over the wave; no barrier follows
  const QShared q{s_q, lane};
  unsigned long long* keys = p.cand + (shared ? key_segment(base, b, 0) + s_base : key_segment(base, b, j));
  auto score = [&](int tl, const Raw& r) {
    const int i0 = tl * 16;
    const int nvc = min(16, ncand - i0);
    bf16x8 kf[4];
    if constexpr (FP8) {
      e4m3x16_to_bf16(r.k[0], kf[0], kf[1]);
      e4m3x16_to_bf16(r.k[1], kf[2], kf[3]);
    } else {
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2) kf[s2] = as_bf16x8(r.k[s2]);
    }
    f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int part = 0; part < 3; ++part) {
#pragma unroll
      for (int kq = 0; kq < 4; ++kq) sacc = mfma_bf16_16x16x32(kf[kq], q.get(part, kq), sacc);
    }
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) s_lg[wave][4 * g + q4][n] = sacc[q4] * r.ks[q4];
    asm volatile("" ::: "memory");  // the reads below must follow the writes above
    if (lane < 16) {
      float acc = 0.f;
#pragma unroll
      for (int h = 0; h < kHeads; ++h) acc = __builtin_fmaf(exp2f(s_lg[wave][lane][h] - s_mx[h]), s_iz[h], acc);
      if (lane < nvc) keys[i0 + lane] = select_key(acc, r.pos);
    }
    asm volatile("" ::: "memory");  // the next tile's writes must follow these reads
  };
  // two-slot ring over the wave's tiles ct, ct + 4, ...; a load past the last
  // tile re-reads the last one (unused)
  for (;;) {
    load(ct + 4, rb);
    __builtin_amdgcn_sched_barrier(0);
    score(ct, ra);
    __builtin_amdgcn_sched_barrier(0);
    ct += 4;
    if (ct >= ntiles) break;
    load(ct + 4, ra);
    __builtin_amdgcn_sched_barrier(0);
    score(ct, rb);
    __builtin_amdgcn_sched_barrier(0);
    ct += 4;
    if (ct >= ntiles) break;
  }
}

hipError_t launch_bound_select(const SelectParams& p, int batch, int64_t max_context, bool fp8, hipStream_t s) {
  if (batch == 0) return hipSuccess;
  if (max_context > 0) {
    const bool compact = ragged_batch(p, batch, max_context);
    // compact: at most sum_b (ceil(L_b / block) + kMinCollectBlocks) < N / block + (kMinCollectBlocks + 1) B items
    const int64_t per_seq = std::max<int64_t>((max_context + kBoundBlockTokens - 1) / kBoundBlockTokens, kMinCollectBlocks);
    const dim3 grid = compact ? dim3(static_cast<unsigned>(p.total_tokens / kBoundBlockTokens + (kMinCollectBlocks + 1) * batch))
                              : dim3(static_cast<unsigned>(per_seq), batch);
    if (fp8 && compact)
      hipLaunchKernelGGL((collect_rescore_kernel<true, true>), grid, dim3(256), 0, s, p);
    else if (fp8)
      hipLaunchKernelGGL((collect_rescore_kernel<true, false>), grid, dim3(256), 0, s, p);
    else if (compact)
      hipLaunchKernelGGL((collect_rescore_kernel<false, true>), grid, dim3(256), 0, s, p);
    else
      hipLaunchKernelGGL((collect_rescore_kernel<false, false>), grid, dim3(256), 0, s, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(finish_kernel<true>, dim3(batch), dim3(kTopK), 0, s, p);
  return hipGetLastError();
}

}  // namespace hs2
