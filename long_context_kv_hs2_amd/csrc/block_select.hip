// Gen-1 (block-level) selection: the comparator that the pages' ablation sets
// against the token-level selection under the same attention budget.
//
// The previous HySparse picked whole 64-token blocks, so a single relevant
// token spent its block's share of the budget ("Luo Fuli Teases Xiaomi
// MiMo-V3 Architecture", paragraphs on how the sparse layers select and on
// the block-versus-token ablation; readaitime.com news of 2026-09-24,
// paragraph on block versus token selection).  The pages leave the pooling
// and the block grid open; taken here:
//   * blocks [64 i, 64 i + 64) aligned to position 0; the candidates are the
//     complete blocks that end before the 128-token window;
//   * a block's score is the sum of its positions' scores;
//   * the window, plus the top_k / 64 = 16 blocks by (block score descending,
//     block index ascending); a context of at most window + top_k tokens
//     selects every position, as the token-level rule does.
//
// Two launches:
//   block_pool_kernel    one 16-lane group per candidate block sums its 64
//                        scores in a fixed order (coalesced loads, then a
//                        butterfly over the 16 lanes), over a compact 1-D grid
//                        of the non-empty (sequence, 16-block group) items.
//   block_select_kernel  one 1024-thread workgroup per sequence: exact top-16
//                        of the 64-bit keys (block-sum bits above the
//                        complement of the block index, so keys are distinct,
//                        larger is better and equal sums go to the lower
//                        block).  Each thread keeps the best key of the blocks
//                        it owns (strided); t0 = the 16th largest of those
//                        maxima is a lower bound on the 16th largest key (the
//                        16 maxima at or above it are distinct keys), and only
//                        the 16 threads whose maximum reaches t0 can hold keys
//                        >= t0.  Those keys (at most 16 per thread's share)
//                        are sorted and the first 16 taken.
#include "hs2_device.h"
#include "hs2_internal.h"

namespace hs2 {

namespace {

constexpr int kPoolBlocks = 16;  // candidate blocks per pool workgroup (16 lanes each)
constexpr int kSelThreads = 1024;
constexpr int kSortCap = 4096;   // candidate keys: <= 16 * ceil(blocks / 1024) <= 4096 for 2^24 tokens

__device__ __forceinline__ int64_t block_slot(int64_t base, int b, int i) { return (base >> 6) + b + i; }

__device__ __forceinline__ int candidate_blocks(int len) {
  return len > kBudget ? (len - kWindow) / kSelectBlock : 0;
}

__global__ __launch_bounds__(256) void block_pool_kernel(BlockParams p) {
  int b, j;
  if (!find_item(p.seq_offsets, p.batch, p.total_tokens, p.max_context, blockIdx.x,
                 [](int len) { return (candidate_blocks(len) + kPoolBlocks - 1) / kPoolBlocks; }, b, j))
    return;
  int64_t base;
  int len;
  seq_bounds(p.seq_offsets, b, p.total_tokens, p.max_context, base, len);
  const int nb = candidate_blocks(len);
  const int i = j * kPoolBlocks + (threadIdx.x >> 4);
  const int l = threadIdx.x & 15;
  float s = 0.f;
  if (i < nb) {
    const float* src = p.score + base + static_cast<int64_t>(i) * kSelectBlock + l;
    s = ((src[0] + src[16]) + src[32]) + src[48];
  }
#pragma unroll
  for (int off = 8; off > 0; off >>= 1) s += __shfl_xor(s, off);  // every lane ends with the same sum
  if (i < nb && l == 0) p.block_scores[block_slot(base, b, i)] = s;
}

// Sorts s[0, m) descending; m a power of two <= kSortCap; every thread calls it.
__device__ void bitonic_sort_desc(unsigned long long* s, int m) {
  for (int k = 2; k <= m; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < m; i += kSelThreads) {
        const int o = i ^ j;
        if (o > i) {
          const unsigned long long a = s[i], c = s[o];
          const bool down = (i & k) == 0;  // this run ends up descending
          if (down ? a < c : a > c) {
            s[i] = c;
            s[o] = a;
          }
        }
      }
      __syncthreads();
    }
  }
}

__global__ __launch_bounds__(kSelThreads) void block_select_kernel(BlockParams p) {
  __shared__ unsigned long long s_keys[kSortCap];
  __shared__ int s_n;
  __shared__ int s_blk[kTopBlocks];
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  int64_t base;
  int len;
  seq_bounds(p.seq_offsets, b, p.total_tokens, p.max_context, base, len);
  int32_t* out = p.sel_idx + static_cast<int64_t>(b) * kBudget;
  if (len <= kBudget) {
    for (int e = tid; e < kBudget; e += kSelThreads) out[e] = e < len ? e : -1;
    if (tid == 0) p.sel_count[b] = len;
    return;
  }
  const int nb = candidate_blocks(len);  // >= 16
  const float* bs = p.block_scores + block_slot(base, b, 0);
  auto key_of = [&](int i) {
    return (static_cast<unsigned long long>(__float_as_uint(bs[i])) << 32) | (0xFFFFFFFFu - static_cast<uint32_t>(i));
  };
  unsigned long long best = 0;  // 0 is below every key (the low word is never 0)
  for (int i = tid; i < nb; i += kSelThreads) {
    const unsigned long long k = key_of(i);
    best = k > best ? k : best;
  }
  s_keys[tid] = best;
  if (tid == 0) s_n = 0;
  __syncthreads();
  bitonic_sort_desc(s_keys, kSelThreads);
  const unsigned long long t0 = s_keys[kTopBlocks - 1];
  __syncthreads();
  if (best >= t0) {
    for (int i = tid; i < nb; i += kSelThreads) {
      const unsigned long long k = key_of(i);
      if (k >= t0) s_keys[atomicAdd(&s_n, 1)] = k;
    }
  }
  __syncthreads();
  const int n = s_n;
  int m = kTopBlocks;
  while (m < n) m <<= 1;
  for (int e = n + tid; e < m; e += kSelThreads) s_keys[e] = 0;
  __syncthreads();
  bitonic_sort_desc(s_keys, m);
  if (tid < kTopBlocks) {  // the 16 chosen blocks, placed in index order
    const int blk = static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(s_keys[tid]));
    int r = 0;
    for (int q = 0; q < kTopBlocks; ++q) r += static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(s_keys[q])) < blk;
    s_blk[r] = blk;
  }
  __syncthreads();
  for (int e = tid; e < kBudget; e += kSelThreads)
    out[e] = e < kTopK ? s_blk[e / kSelectBlock] * kSelectBlock + (e % kSelectBlock) : len - kBudget + e;
  if (tid == 0) p.sel_count[b] = kBudget;
}

}  // namespace

hipError_t launch_block_select(const BlockParams& p, hipStream_t s) {
  if (p.batch <= 0) return hipSuccess;
  const int64_t pool_grid = p.total_tokens / (kPoolBlocks * kSelectBlock) + p.batch;
  if (p.total_tokens > kBudget) {
    hipLaunchKernelGGL(block_pool_kernel, dim3(static_cast<unsigned>(pool_grid)), dim3(256), 0, s, p);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(block_select_kernel, dim3(p.batch), dim3(kSelThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace hs2
