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
// Exact radix select on a 64-bit key per token: the fp32 score bits (scores
// are >= 0, so their bit patterns order like the values) above the bitwise
// complement of the position, so larger keys win and equal scores go to the
// lower position; every key is distinct and "the top_k largest keys" is the
// selection exactly.  Up to six passes of 11/11/11/11/11/8 digits; each pass is
// one launch over the sequence's scores with per-workgroup LDS histograms merged
// by global atomics, and the last workgroup of a sequence to finish (counted by
// an atomic ticket after a fence) resolves that pass's digit.  Passes after the
// set is fixed return at once.  Emission uses wave ballots and popcounts for one
// atomic per wave, then one workgroup per sequence sorts the indices ascending
// and appends the window.
#include <limits.h>

#include "hs2_device.h"
#include "hs2_internal.h"

namespace hs2 {

__constant__ int kPassShift[kRadixPasses] = {52, 41, 30, 19, 8, 0};
__constant__ int kPassBits[kRadixPasses] = {11, 11, 11, 11, 11, 8};

__device__ __forceinline__ unsigned long long select_key(float score, int pos) {
  return (static_cast<unsigned long long>(__float_as_uint(score)) << 32) |
         static_cast<unsigned long long>(0xFFFFFFFFu - static_cast<uint32_t>(pos));
}

__global__ __launch_bounds__(256) void select_init_kernel(SelectParams p) {
  const int b = blockIdx.x;
  int64_t base;
  int len;
  seq_bounds(p.seq_offsets, b, p.total_tokens, p.max_context, base, len);
  uint32_t* h = p.hist + static_cast<size_t>(b) * kRadixPasses * kRadixBins;
  for (int i = threadIdx.x; i < kRadixPasses * kRadixBins; i += blockDim.x) h[i] = 0;
  if (threadIdx.x < 8) p.counters[b * 8 + threadIdx.x] = 0;
  if (threadIdx.x == 0) {
    SelectState st;
    st.prefix = 0;
    st.rank = static_cast<uint32_t>(p.top_k);
    st.shift = 63;
    st.done = len <= p.budget ? 1 : 0;
    st.pad[0] = st.pad[1] = st.pad[2] = 0;
    p.state[b] = st;
  }
}

hipError_t launch_select_init(const SelectParams& p, int batch, hipStream_t s) {
  if (batch == 0) return hipSuccess;
  hipLaunchKernelGGL(select_init_kernel, dim3(batch), dim3(256), 0, s, p);
  return hipGetLastError();
}

// Resolve one radix pass of sequence b from its global histogram (run by the
// whole workgroup that finished last).  s_cnt: LDS scratch of kRadixBins.
__device__ void resolve_pass(const SelectParams& p, int b, int pass, uint32_t* s_cnt, uint32_t* s_sum) {
  const int bits = kPassBits[pass];
  const int nbins = 1 << bits;
  const uint32_t* gh = p.hist + (static_cast<size_t>(b) * kRadixPasses + pass) * kRadixBins;
  for (int i = threadIdx.x; i < nbins; i += blockDim.x)
    s_cnt[i] = __hip_atomic_load(gh + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const int per = nbins / 256;
  const int lo = threadIdx.x * per;
  uint32_t sum = 0;
  for (int i = 0; i < per; ++i) sum += s_cnt[lo + i];
  // inclusive suffix sums over threads: s_sum[t] = sum of threads t..255
  s_sum[threadIdx.x] = sum;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    const uint32_t add = threadIdx.x + off < 256 ? s_sum[threadIdx.x + off] : 0;
    __syncthreads();
    s_sum[threadIdx.x] += add;
    __syncthreads();
  }
  const SelectState st = p.state[b];
  const uint32_t above = s_sum[threadIdx.x] - sum;  // keys in bins above this thread's range
  const uint32_t r = st.rank;
  if (above < r && r <= above + sum) {
    uint32_t acc = above;
    for (int i = lo + per - 1; i >= lo; --i) {
      const uint32_t cnt = s_cnt[i];
      if (acc + cnt >= r) {
        SelectState ns;
        ns.rank = r - acc;
        ns.prefix = (st.prefix << bits) | static_cast<unsigned long long>(i);
        ns.shift = kPassShift[pass];
        ns.done = (cnt == ns.rank || pass == kRadixPasses - 1) ? 1 : 0;
        ns.pad[0] = ns.pad[1] = ns.pad[2] = 0;
        p.state[b] = ns;
        break;
      }
      acc += cnt;
    }
  }
}

// Flush the LDS histogram, take a ticket, and resolve if this workgroup is
// the last of its sequence for this pass.
__device__ void finish_pass(const SelectParams& p, int b, int pass, int blocks, uint32_t* s_hist, uint32_t* s_sum) {
  uint32_t* gh = p.hist + (static_cast<size_t>(b) * kRadixPasses + pass) * kRadixBins;
  const int nbins = 1 << kPassBits[pass];
  for (int i = threadIdx.x; i < nbins; i += blockDim.x) {
    const uint32_t c = s_hist[i];
    if (c) atomicAdd(gh + i, c);
  }
  __threadfence();
  __syncthreads();
  __shared__ int s_last;
  if (threadIdx.x == 0) s_last = (atomicAdd(p.counters + b * 8 + pass, 1u) == static_cast<uint32_t>(blocks - 1));
  __syncthreads();
  if (s_last) {
    __threadfence();
    resolve_pass(p, b, pass, s_hist, s_sum);
  }
}

// Score pass: score_j from the spilled log2-domain logits and each head's
// global (max, sum); with `hist`, also the first radix histogram.
template <bool HIST>
__global__ __launch_bounds__(256) void score_pass_kernel(SelectParams p) {
  __shared__ uint32_t s_hist[kRadixBins];
  __shared__ uint32_t s_sum[256];
  __shared__ float s_mx[kHeads];
  __shared__ float s_z[kHeads];
  const int b = blockIdx.y;
  int64_t base;
  int len;
  seq_bounds(p.seq_offsets, b, p.total_tokens, p.max_context, base, len);
  const int j0 = blockIdx.x * kScoreBlockTokens;
  if (j0 >= len) return;
  const int j1 = min(len, j0 + kScoreBlockTokens);
  const bool selecting = HIST && len > p.budget;
  const int dom = len - p.window;
  if (threadIdx.x < kHeads) {
    s_mx[threadIdx.x] = p.stats[(static_cast<int64_t>(b) * kHeads + threadIdx.x) * 2];
    s_z[threadIdx.x] = p.stats[(static_cast<int64_t>(b) * kHeads + threadIdx.x) * 2 + 1];
  }
  if (selecting)
    for (int i = threadIdx.x; i < kRadixBins; i += blockDim.x) s_hist[i] = 0;
  __syncthreads();
  for (int j = j0 + threadIdx.x; j < j1; j += blockDim.x) {
    const float4* lp = reinterpret_cast<const float4*>(p.spill + (base + j) * kHeads);
    float l[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 v = lp[q];
      l[4 * q] = v.x;
      l[4 * q + 1] = v.y;
      l[4 * q + 2] = v.z;
      l[4 * q + 3] = v.w;
    }
    float sc = 0.f;
#pragma unroll
    for (int h = 0; h < kHeads; ++h) sc += exp2f(l[h] - s_mx[h]) / s_z[h];
    p.score[base + j] = sc;
    if (selecting && j < dom) atomicAdd(&s_hist[(__float_as_uint(sc) >> 20) & (kRadixBins - 1)], 1u);
  }
  if (!selecting) return;
  __syncthreads();
  finish_pass(p, b, 0, (len + kScoreBlockTokens - 1) / kScoreBlockTokens, s_hist, s_sum);
}

hipError_t launch_score_pass(const SelectParams& p, int batch, int64_t max_context, bool histogram,
                             hipStream_t s) {
  if (batch == 0 || max_context == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((max_context + kScoreBlockTokens - 1) / kScoreBlockTokens), batch);
  if (histogram)
    hipLaunchKernelGGL(score_pass_kernel<true>, grid, dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(score_pass_kernel<false>, grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

// One radix pass over stored scores (pass 0 when selecting from given scores).
__global__ __launch_bounds__(256) void radix_pass_kernel(SelectParams p, int pass) {
  __shared__ uint32_t s_hist[kRadixBins];
  __shared__ uint32_t s_sum[256];
  __shared__ SelectState s_st;
  const int b = blockIdx.y;
  int64_t base;
  int len;
  seq_bounds(p.seq_offsets, b, p.total_tokens, p.max_context, base, len);
  if (len <= p.budget) return;
  const int dom = len - p.window;
  const int j0 = blockIdx.x * kScoreBlockTokens;
  if (j0 >= dom) return;
  const int j1 = min(dom, j0 + kScoreBlockTokens);
  if (threadIdx.x == 0) s_st = p.state[b];
  for (int i = threadIdx.x; i < kRadixBins; i += blockDim.x) s_hist[i] = 0;
  __syncthreads();
  if (s_st.done) return;  // uniform
  const int shift = kPassShift[pass];
  const uint32_t mask = (1u << kPassBits[pass]) - 1u;
  const int pshift = s_st.shift;
  const unsigned long long prefix = s_st.prefix;
  for (int j = j0 + threadIdx.x; j < j1; j += blockDim.x) {
    const unsigned long long key = select_key(p.score[base + j], j);
    if ((key >> pshift) == prefix) atomicAdd(&s_hist[static_cast<uint32_t>(key >> shift) & mask], 1u);
  }
  __syncthreads();
  finish_pass(p, b, pass, (dom + kScoreBlockTokens - 1) / kScoreBlockTokens, s_hist, s_sum);
}

hipError_t launch_radix_passes(const SelectParams& p, int batch, int64_t max_context, int first_pass,
                               hipStream_t s) {
  if (batch == 0 || max_context == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((max_context + kScoreBlockTokens - 1) / kScoreBlockTokens), batch);
  for (int pass = first_pass; pass < kRadixPasses; ++pass) {
    hipLaunchKernelGGL(radix_pass_kernel, grid, dim3(256), 0, s, p, pass);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Emit every out-of-window position whose key is at or above the threshold:
// exactly top_k of them, in no particular order.
__global__ __launch_bounds__(256) void emit_kernel(SelectParams p) {
  const int b = blockIdx.y;
  int64_t base;
  int len;
  seq_bounds(p.seq_offsets, b, p.total_tokens, p.max_context, base, len);
  if (len <= p.budget) return;
  const int dom = len - p.window;
  const int j0 = blockIdx.x * kScoreBlockTokens;
  if (j0 >= dom) return;
  const int j1 = min(dom, j0 + kScoreBlockTokens);
  const SelectState st = p.state[b];
  const int lane = threadIdx.x & 63;
  for (int i = 0; i < kScoreBlockTokens; i += blockDim.x) {
    const int j = j0 + i + threadIdx.x;
    const bool take = j < j1 && (select_key(p.score[base + j], j) >> st.shift) >= st.prefix;
    const unsigned long long m = __ballot(take);
    if (m == 0) continue;
    const int leader = __ffsll(static_cast<long long>(m)) - 1;
    uint32_t first = 0;
    if (lane == leader) first = atomicAdd(p.counters + b * 8 + 7, static_cast<uint32_t>(__popcll(m)));
    first = __shfl(first, leader);
    if (take) {
      const uint32_t slot = first + static_cast<uint32_t>(__popcll(m & __lanemask_lt()));
      if (slot < static_cast<uint32_t>(p.top_k)) p.selbuf[static_cast<size_t>(b) * p.top_k + slot] = j;
    }
  }
}

// Sort the emitted positions ascending (bitonic, in LDS), append the window,
// or list every position of a short context; pad with -1.
__global__ __launch_bounds__(1024) void finalize_kernel(SelectParams p) {
  __shared__ int32_t s[kTopK];
  const int b = blockIdx.x;
  int64_t base;
  int len;
  seq_bounds(p.seq_offsets, b, p.total_tokens, p.max_context, base, len);
  int32_t* out = p.sel_idx + static_cast<size_t>(b) * p.budget;
  const int t = threadIdx.x;
  if (len <= p.budget) {
    for (int i = t; i < p.budget; i += blockDim.x) out[i] = i < len ? i : -1;
    if (t == 0) p.sel_count[b] = len;
    return;
  }
  const int dom = len - p.window;
  s[t] = p.selbuf[static_cast<size_t>(b) * p.top_k + t];
  __syncthreads();
  for (int size = 2; size <= kTopK; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      const int partner = t ^ stride;
      if (partner > t) {
        const bool up = (t & size) == 0;
        const int32_t a = s[t], c = s[partner];
        if ((a > c) == up) {
          s[t] = c;
          s[partner] = a;
        }
      }
      __syncthreads();
    }
  }
  out[t] = s[t];
  if (t < p.window) out[p.top_k + t] = dom + t;
  if (t == 0) p.sel_count[b] = p.budget;
}

hipError_t launch_emit_finalize(const SelectParams& p, int batch, int64_t max_context, hipStream_t s) {
  if (batch == 0) return hipSuccess;
  if (max_context > 0) {
    const dim3 grid(static_cast<unsigned>((max_context + kScoreBlockTokens - 1) / kScoreBlockTokens), batch);
    hipLaunchKernelGGL(emit_kernel, grid, dim3(256), 0, s, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(finalize_kernel, dim3(batch), dim3(kTopK), 0, s, p);
  return hipGetLastError();
}

}  // namespace hs2
