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
// shat_j = sum_h a_hj and per 16-token tile the wave's running max and
// (approximately) reciprocal running sum per head, which bound score_j within
// shat_j * [min_h F_h, max_h F_h].
//  1. histogram of the lower bounds' first digit;
//  2. collect the positions whose upper bound reaches the lower edge of the bin
//     holding the k-th largest lower bound: at least k positions have a score
//     at or above that edge, so every position of the exact top-k (ties
//     included) is collected;
//  3. rescore the candidates exactly, with the same arithmetic as the spill
//     path (every position if the list overflowed);
//  4. finish as above over the exact candidate keys.
#include "hs2_device.h"
#include "hs2_internal.h"

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

struct Resolved {
  int digit;        // the bin holding the rank-th largest key
  uint32_t above;   // keys in higher bins
  uint32_t count;   // keys in that bin
};

// Block-wide: find the bin where the count from the top reaches `rank`.
template <int NT>
__device__ Resolved block_resolve(const uint32_t* hist, int nbins, uint32_t rank, uint32_t* s_scan, Resolved* s_out) {
  const int t = threadIdx.x;
  const int per = nbins >= NT ? nbins / NT : 1;
  const int lo = t * per;
  uint32_t sum = 0;
  for (int i = 0; i < per; ++i)
    if (lo + i < nbins) sum += hist[lo + i];
  s_scan[t] = sum;
  __syncthreads();
  for (int off = 1; off < NT; off <<= 1) {
    const uint32_t add = t + off < NT ? s_scan[t + off] : 0u;
    __syncthreads();
    s_scan[t] += add;
    __syncthreads();
  }
  const uint32_t above = s_scan[t] - sum;  // keys in bins above this thread's range
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
        sc[u] = p.score[base + j];
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
      for (int u = 0; u < kBatch; ++u) sc[u] = p.score[base + min(i0 + u * 256 + static_cast<int>(threadIdx.x), c1 - 1)];
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
template <bool BOUND>
__global__ __launch_bounds__(1024) void finish_kernel(SelectParams p) {
  __shared__ uint32_t s_hist[kRadixBins];
  __shared__ uint32_t s_scan[1024];
  __shared__ Resolved s_res;
  __shared__ int32_t s_sel[kTopK];
  __shared__ uint32_t s_n;
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
  const uint32_t ncand = p.counters[b * 4 + 1];
  const bool overflow = ncand > static_cast<uint32_t>(kCandCap);
  const unsigned long long* cand = p.cand + static_cast<size_t>(b) * kCandCap;
  const float* score = p.score + base;
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
    if (!overflow) {
      for (uint32_t i = t; i < ncand; i += blockDim.x) fn(cand[i]);
    } else {
      for (int j = t; j < dom; j += blockDim.x) {
        const float sc = score[j];
        if (BOUND || digit0(sc) == d0) fn(select_key(sc, j));
      }
    }
  };

  // digits of the 63 key bits below the sign: 11, 11, 11, 11, 11, 8
  for (int pass = first_pass; pass < 6 && !done; ++pass) {
    const int bits = pass < 5 ? 11 : 8;
    const int shift = pass < 5 ? 52 - 11 * pass : 0;
    const uint32_t mask = (1u << bits) - 1u;
    for (int i = t; i < kRadixBins; i += blockDim.x) s_hist[i] = 0;
    __syncthreads();
    for_each_key([&](unsigned long long key) {
      if ((key >> pshift) == prefix) atomicAdd(&s_hist[static_cast<uint32_t>(key >> shift) & mask], 1u);
    });
    __syncthreads();
    const Resolved r = block_resolve<1024>(s_hist, 1 << bits, rank, s_scan, &s_res);
    rank -= r.above;
    prefix = (prefix << bits) | static_cast<unsigned long long>(r.digit);
    pshift = shift;
    done = r.count == rank || pass == 5;
  }

  // Winners from collect (spill mode), then the keys at or above the threshold.
  for (uint32_t i = t; i < nwin; i += blockDim.x) s_sel[i] = p.selbuf[static_cast<size_t>(b) * p.top_k + i];
  if (t == 0) s_n = 0;
  __syncthreads();
  for_each_key([&](unsigned long long key) {
    if ((key >> pshift) >= prefix) {
      const uint32_t slot = nwin + atomicAdd(&s_n, 1u);
      if (slot < static_cast<uint32_t>(p.top_k)) s_sel[slot] = key_pos(key);
    }
  });
  __syncthreads();
  for (int size = 2; size <= kTopK; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      const int partner = t ^ stride;
      if (partner > t) {
        const bool up = (t & size) == 0;
        const int32_t a = s_sel[t], c = s_sel[partner];
        if ((a > c) == up) {
          s_sel[t] = c;
          s_sel[partner] = a;
        }
      }
      __syncthreads();
    }
  }
  out[t] = s_sel[t];
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

// Per-tile bound factors F_h = exp2(u_h^t - M_h) / Z_h: their min and max.
__device__ __forceinline__ void tile_factors(const float* __restrict__ ts, const float (&mx)[kHeads],
                                             const float (&iz)[kHeads], float& fmin, float& fmax) {
  fmin = INFINITY;
  fmax = 0.f;
#pragma unroll
  for (int h = 0; h < kHeads; ++h) {
    const float f = exp2f(ts[h] - mx[h]) * iz[h];
    fmin = fminf(fmin, f);
    fmax = fmaxf(fmax, f);
  }
}

__device__ __forceinline__ void load_global_stats(const SelectParams& p, int b, float (&mx)[kHeads], float (&iz)[kHeads]) {
  const float* st = p.stats + static_cast<int64_t>(b) * kHeads * 2;
#pragma unroll
  for (int h = 0; h < kHeads; ++h) {
    mx[h] = st[2 * h];
    iz[h] = 1.f / st[2 * h + 1];
  }
}

// Slack on the pruning threshold and upper bounds: far above fp32 rounding.
constexpr float kLowSlack = 1.f - 1.f / 1024.f;
constexpr float kHighSlack = 1.f + 1.f / 1024.f;

// Histogram of the lower bounds lb_j = shat_j * min_h F_h (first 11-bit digit).
// One thread per 16-token tile.
__global__ __launch_bounds__(256) void bound_hist_kernel(SelectParams p) {
  __shared__ uint32_t s_hist[kRadixBins];
  const int b = blockIdx.y;
  int64_t base;
  int len;
  seq_bounds(p.seq_offsets, b, p.total_tokens, p.max_context, base, len);
  if (len <= p.budget) return;
  const int dom = len - p.window;
  const int j0 = blockIdx.x * kBoundBlockTokens;
  if (j0 >= dom) return;
  float mx[kHeads], iz[kHeads];
  load_global_stats(p, b, mx, iz);
  for (int i = threadIdx.x; i < kRadixBins; i += blockDim.x) s_hist[i] = 0;
  __syncthreads();
  const int tile = (j0 >> 4) + threadIdx.x;
  if (16 * tile < dom) {
    float fmin, fmax;
    tile_factors(p.tile_stats + tile_slot(base, b, tile) * kHeads, mx, iz, fmin, fmax);
    const float4* sh = reinterpret_cast<const float4*>(p.shat + base + 16 * tile);
    const int nv = min(16, dom - 16 * tile);
    // shat rows are 64-byte aligned only when base is a multiple of 16: load scalars otherwise
    float v[16];
    if ((base & 3) == 0) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 x = sh[q];
        v[4 * q] = x.x; v[4 * q + 1] = x.y; v[4 * q + 2] = x.z; v[4 * q + 3] = x.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = p.shat[base + 16 * tile + min(i, nv - 1)];
    }
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (i < nv) atomicAdd(&s_hist[digit0(v[i] * fmin)], 1u);
  }
  __syncthreads();
  uint32_t* gh = p.hist0 + static_cast<size_t>(b) * kRadixBins;
  for (int i = threadIdx.x; i < kRadixBins; i += blockDim.x) {
    const uint32_t c = s_hist[i];
    if (c) atomicAdd(gh + i, c);
  }
}

// Candidates: every out-of-window position whose upper bound reaches the lower
// edge of the bin holding the k-th largest lower bound.  The workgroup builds
// its list in LDS and reserves room in the sequence's list with one atomic.
__global__ __launch_bounds__(256) void collect_bound_kernel(SelectParams p) {
  __shared__ uint32_t s_hist[kRadixBins];
  __shared__ uint32_t s_scan[256];
  __shared__ Resolved s_res;
  __shared__ int32_t s_list[kBoundBlockTokens];
  __shared__ uint32_t s_cnt;
  __shared__ uint32_t s_base;
  const int b = blockIdx.y;
  int64_t base;
  int len;
  seq_bounds(p.seq_offsets, b, p.total_tokens, p.max_context, base, len);
  if (len <= p.budget) return;
  const int dom = len - p.window;
  const int j0 = blockIdx.x * kBoundBlockTokens;
  if (j0 >= dom) return;
  float mx[kHeads], iz[kHeads];
  load_global_stats(p, b, mx, iz);
  const uint32_t* gh = p.hist0 + static_cast<size_t>(b) * kRadixBins;
  for (int i = threadIdx.x; i < kRadixBins; i += blockDim.x) s_hist[i] = gh[i];
  if (threadIdx.x == 0) s_cnt = 0;
  __syncthreads();
  const Resolved r0 = block_resolve<256>(s_hist, kRadixBins, static_cast<uint32_t>(p.top_k), s_scan, &s_res);
  const float thr = __uint_as_float(static_cast<uint32_t>(r0.digit) << 20) * kLowSlack;
  const int tile = (j0 >> 4) + threadIdx.x;
  if (16 * tile < dom) {
    float fmin, fmax;
    tile_factors(p.tile_stats + tile_slot(base, b, tile) * kHeads, mx, iz, fmin, fmax);
    const int nv = min(16, dom - 16 * tile);
    for (int i = 0; i < nv; ++i) {
      const int j = 16 * tile + i;
      if (p.shat[base + j] * fmax * kHighSlack >= thr) s_list[atomicAdd(&s_cnt, 1u)] = j;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) s_base = s_cnt ? atomicAdd(p.counters + b * 4 + 1, s_cnt) : 0u;
  __syncthreads();
  int32_t* cidx = p.cand_idx + static_cast<size_t>(b) * kCandCap;
  for (uint32_t i = threadIdx.x; i < s_cnt; i += blockDim.x) {
    const uint32_t slot = s_base + i;
    if (slot < static_cast<uint32_t>(kCandCap)) cidx[slot] = s_list[i];
  }
}

// Exact scores of the candidates (every out-of-window position when the list
// overflowed): the same split-query MFMA sequence as the full pass gives the
// same logits, and the same head-ordered sum gives the same score as the
// spill path.  Keys go to the candidate key list (or scores to p.score).
template <bool FP8>
__global__ __launch_bounds__(256) void refine_kernel(SelectParams p) {
  __shared__ u32x4 s_q[kQLdsVecs];
  __shared__ float s_lg[4][16][17];
  __shared__ float s_mx[kHeads];
  __shared__ float s_iz[kHeads];
  const int b = blockIdx.y;
  int64_t base;
  int len;
  seq_bounds(p.seq_offsets, b, p.total_tokens, p.max_context, base, len);
  if (len <= p.budget) return;
  const int dom = len - p.window;
  const uint32_t ncand = p.counters[b * 4 + 1];
  const bool overflow = ncand > static_cast<uint32_t>(kCandCap);
  const int items = overflow ? dom : static_cast<int>(ncand);
  const int ntiles = (items + 15) >> 4;
  if (static_cast<int>(blockIdx.x) * 4 >= ntiles) return;  // uniform
  build_q_lds<FP8>(p.q + static_cast<size_t>(b) * kHeads * kDim, p.qscale, s_q);
  if (threadIdx.x < kHeads) {
    s_mx[threadIdx.x] = p.stats[(static_cast<int64_t>(b) * kHeads + threadIdx.x) * 2];
    s_iz[threadIdx.x] = 1.f / p.stats[(static_cast<int64_t>(b) * kHeads + threadIdx.x) * 2 + 1];
  }
  __syncthreads();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform: scalar loop control
  const int lane = threadIdx.x & 63;
  const int n = lane & 15;
  const int g = lane >> 4;
  const QShared q{s_q, lane};
  constexpr int kRowBytes = FP8 ? kDim : 2 * kDim;
  const uint8_t* __restrict__ kbase = p.k + base * kRowBytes;
  const int32_t* cidx = p.cand_idx + static_cast<size_t>(b) * kCandCap;
  for (int tile = blockIdx.x * 4 + wave; tile < ntiles; tile += gridDim.x * 4) {
    const int i0 = tile * 16;
    const int nv = min(16, items - i0);
    const int pos = overflow ? i0 + min(n, nv - 1) : cidx[i0 + min(n, nv - 1)];
    const uint32_t krow = static_cast<uint32_t>(pos) * kRowBytes;
    bf16x8 kf[4];
    if constexpr (FP8) {
      e4m3x16_to_bf16(*reinterpret_cast<const u32x4*>(kbase + (krow + kload_offset(0, g))), kf[0], kf[1]);
      e4m3x16_to_bf16(*reinterpret_cast<const u32x4*>(kbase + (krow + kload_offset(1, g))), kf[2], kf[3]);
    } else {
#pragma unroll
      for (int s = 0; s < 4; ++s) kf[s] = as_bf16x8(*reinterpret_cast<const u32x4*>(kbase + (krow + kload_offset(s, g))));
    }
    f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int part = 0; part < 3; ++part) {
#pragma unroll
      for (int k = 0; k < 4; ++k) sacc = mfma_bf16_16x16x32(kf[k], q.get(part, k), sacc);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int slot = 4 * g + r;
      const int spos = __shfl(pos, slot);  // lane `slot` (group 0) holds that token's position
      const float ks = FP8 ? p.k_scale[base + spos] : 1.f;
      s_lg[wave][slot][n] = sacc[r] * ks;
    }
    asm volatile("" ::: "memory");  // the reads below must follow the writes above
    if (lane < 16) {
      float acc = 0.f;
#pragma unroll
      for (int h = 0; h < kHeads; ++h) acc = __builtin_fmaf(exp2f(s_lg[wave][lane][h] - s_mx[h]), s_iz[h], acc);
      if (lane < nv) {
        if (overflow)
          p.score[base + pos] = acc;
        else
          p.cand[static_cast<size_t>(b) * kCandCap + i0 + lane] = select_key(acc, pos);
      }
    }
    asm volatile("" ::: "memory");  // the next tile's writes must follow these reads
  }
}

hipError_t launch_bound_select(const SelectParams& p, int batch, int64_t max_context, bool fp8, hipStream_t s) {
  if (batch == 0) return hipSuccess;
  if (max_context > 0) {
    const dim3 grid(static_cast<unsigned>((max_context + kBoundBlockTokens - 1) / kBoundBlockTokens), batch);
    hipLaunchKernelGGL(bound_hist_kernel, grid, dim3(256), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(collect_bound_kernel, grid, dim3(256), 0, s, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 rgrid(kRefineBlocks, batch);
    if (fp8)
      hipLaunchKernelGGL(refine_kernel<true>, rgrid, dim3(256), 0, s, p);
    else
      hipLaunchKernelGGL(refine_kernel<false>, rgrid, dim3(256), 0, s, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(finish_kernel<true>, dim3(batch), dim3(kTopK), 0, s, p);
  return hipGetLastError();
}

}  // namespace hs2
