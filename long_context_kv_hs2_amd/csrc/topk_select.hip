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
// Three launches after the scores exist, and no cross-workgroup fence (on a
// multi-XCD part an agent-scope fence writes back the XCD's L2):
//  1. histogram of the first 11-bit digit (score bits 30..20), per-workgroup in
//     LDS, merged by global atomics (fused into the score pass when the scores
//     are computed here);
//  2. collect: every workgroup resolves the first digit D0 from the finished
//     histogram (the same result in all of them), emits the positions whose
//     digit is above D0 (all selected) with one atomic per wave (ballot +
//     popcount), and appends the keys of the D0 bin to a candidate list;
//  3. finish, one workgroup per sequence: radix passes over the candidates in
//     LDS until the threshold key is fixed (over the sequence's scores if the
//     list overflowed), emit the rest, sort the positions ascending (bitonic)
//     and append the window.
#include "hs2_device.h"
#include "hs2_internal.h"

namespace hs2 {

namespace {

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

// Wave-aggregated append: one atomic per wave for all lanes with `take`.
__device__ __forceinline__ uint32_t wave_slot(bool take, uint32_t* counter) {
  const unsigned long long m = __ballot(take);
  if (m == 0) return 0xFFFFFFFFu;
  const int lane = threadIdx.x & 63;
  const int leader = __ffsll(static_cast<long long>(m)) - 1;
  uint32_t first = 0;
  if (lane == leader) first = atomicAdd(counter, static_cast<uint32_t>(__popcll(m)));
  first = __shfl(first, leader);
  return take ? first + static_cast<uint32_t>(__popcll(m & __lanemask_lt())) : 0xFFFFFFFFu;
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
        for (int h = 0; h < kHeads; ++h) acc += exp2f(x[h] - mx[h]) * iz[h];
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
// into the candidate list.
__global__ __launch_bounds__(256) void collect_kernel(SelectParams p) {
  __shared__ uint32_t s_hist[kRadixBins];
  __shared__ uint32_t s_scan[256];
  __shared__ Resolved s_res;
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
  __syncthreads();
  const Resolved r0 = block_resolve<256>(s_hist, kRadixBins, static_cast<uint32_t>(p.top_k), s_scan, &s_res);
  const uint32_t d0 = static_cast<uint32_t>(r0.digit);
  uint32_t* wins = p.counters + b * 4;
  uint32_t* cands = p.counters + b * 4 + 1;
  int32_t* selbuf = p.selbuf + static_cast<size_t>(b) * p.top_k;
  unsigned long long* cand = p.cand + static_cast<size_t>(b) * kCandCap;
  constexpr int kBatch = 16;
  for (int i0 = 0; i0 < kCollectBlockTokens; i0 += kBatch * 256) {
    float sc[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int j = min(j0 + i0 + u * 256 + static_cast<int>(threadIdx.x), j1 - 1);
      sc[u] = p.score[base + j];
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int j = j0 + i0 + u * 256 + static_cast<int>(threadIdx.x);
      const bool valid = j < j1;
      const uint32_t dg = digit0(sc[u]);
      const uint32_t ws = wave_slot(valid && dg > d0, wins);
      if (ws < static_cast<uint32_t>(p.top_k)) selbuf[ws] = j;
      const uint32_t cs = wave_slot(valid && dg == d0, cands);
      if (cs < static_cast<uint32_t>(kCandCap)) cand[cs] = select_key(sc[u], j);
    }
  }
}

// Finish one sequence: resolve the threshold inside the D0 bin, emit, sort.
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
  const uint32_t* gh = p.hist0 + static_cast<size_t>(b) * kRadixBins;
  for (int i = t; i < kRadixBins; i += blockDim.x) s_hist[i] = gh[i];
  __syncthreads();
  const Resolved r0 = block_resolve<1024>(s_hist, kRadixBins, static_cast<uint32_t>(p.top_k), s_scan, &s_res);
  const uint32_t d0 = static_cast<uint32_t>(r0.digit);
  const uint32_t nwin = r0.above;  // positions already in selbuf
  uint32_t rank = static_cast<uint32_t>(p.top_k) - nwin;
  const uint32_t ncand = p.counters[b * 4 + 1];
  const bool overflow = ncand > static_cast<uint32_t>(kCandCap);
  const unsigned long long* cand = p.cand + static_cast<size_t>(b) * kCandCap;
  const float* score = p.score + base;

  // Visit every key of the D0 bin (from the list, or by rescanning the scores).
  auto for_each_key = [&](auto&& fn) {
    if (!overflow) {
      for (uint32_t i = t; i < ncand; i += blockDim.x) fn(cand[i]);
    } else {
      for (int j = t; j < dom; j += blockDim.x) {
        const float sc = score[j];
        if (digit0(sc) == d0) fn(select_key(sc, j));
      }
    }
  };

  unsigned long long prefix = d0;
  int pshift = 52;
  bool done = r0.count == rank;
  // digits of the remaining 52 key bits: 11, 11, 11, 11, 8
  for (int pass = 0; pass < 5 && !done; ++pass) {
    const int bits = pass < 4 ? 11 : 8;
    const int shift = pass < 4 ? 41 - 11 * pass : 0;
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
    done = r.count == rank || pass == 4;
  }

  // Winners from collect, then the D0-bin keys at or above the threshold.
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
  hipLaunchKernelGGL(finish_kernel, dim3(batch), dim3(kTopK), 0, s, p);
  return hipGetLastError();
}

}  // namespace hs2
