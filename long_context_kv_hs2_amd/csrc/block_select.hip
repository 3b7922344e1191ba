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
// Block sums come from per-token scores (hs2_block_select) or, without
// per-token scores, from the full pass's per-tile, per-head weight sums
// (the tile-sum pass): a block is four whole 16-token tiles, and its score is
// sum over its tiles and the heads of exp2(m_h - M_h) r_h / Z_h.
//
// Two launches:
//   block_pool_kernel    one workgroup per (sequence, 4 groups of 16 candidate
//                        blocks), over a compact 1-D grid of the non-empty
//                        items: each 16-lane group sums one block's 64 scores
//                        in a fixed order (coalesced loads, then a butterfly
//                        over the 16 lanes), and each 256-thread quarter also
//                        writes its group's largest key.
//   (or merge_block_pool_kernel, from tile sums: one workgroup per head of a
//                        sequence for the full layer's merge, and one per
//                        four groups of 16 candidate blocks, each 16-lane
//                        team taking one block of each group, lane h its
//                        head)
//   block_select_kernel  one 1024-thread workgroup per sequence: the exact
//                        top 16 of the 64-bit keys (block-sum bits above the
//                        complement of the block index, so keys are distinct,
//                        larger is better and equal sums go to the lower
//                        block).  t0 = the 16th largest of the per-thread
//                        maxima of the group keys bounds the 16th largest key
//                        from below (those 16 maxima are distinct keys), so
//                        only blocks of groups whose key reaches t0 can be
//                        chosen: at most 16 groups per thread stride.  The
//                        thread maxima and the candidates are ranked with
//                        in-wave bitonic sorts (shuffles, no barriers); more
//                        than 256 candidates (contexts past 1M tokens) take a
//                        workgroup-wide LDS sort.
#include "hs2_device.h"
#include "hs2_internal.h"
#include "merge.h"

namespace hs2 {

namespace {

constexpr int kPoolBlocks = 16;  // candidate blocks per group (16 lanes each)
constexpr int kPoolGroups = 4;   // groups per pool workgroup (256 threads each)
constexpr int kSelThreads = 1024;
constexpr int kSortCap = 4096;   // candidates: <= 16 * 16 * ceil(groups / 1024) <= 4096 for 2^24 tokens
typedef unsigned long long u64;

__device__ __forceinline__ int64_t block_slot(int64_t base, int b, int i) { return (base >> 6) + b + i; }
__device__ __forceinline__ int64_t group_slot(int64_t base, int b, int g) { return (base >> 10) + b + g; }

__device__ __forceinline__ int candidate_blocks(int len) {
  return len > kBudget ? (len - kWindow) / kSelectBlock : 0;
}

__device__ __forceinline__ u64 block_key(float sum, int i) {
  return (static_cast<u64>(__float_as_uint(sum)) << 32) | (0xFFFFFFFFu - static_cast<uint32_t>(i));
}

__device__ __forceinline__ u64 shfl64(u64 v, int src) {
  const uint32_t lo = __shfl(static_cast<uint32_t>(v), src);
  const uint32_t hi = __shfl(static_cast<uint32_t>(v >> 32), src);
  return (static_cast<u64>(hi) << 32) | lo;
}

// Bitonic sort across the 64 lanes: afterwards lane i holds the i-th largest.
__device__ __forceinline__ u64 wave_sort_desc(u64 v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int k = 2; k <= 64; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      const u64 o = shfl_xor_u64(v, j);
      const bool keep_max = ((lane & j) == 0) == ((lane & k) == 0);
      v = keep_max ? (v > o ? v : o) : (v < o ? v : o);
    }
  }
  return v;
}

// a, b sorted descending across lanes -> the 64 largest of both, sorted
// descending (a max with b reversed is bitonic; one merge network sorts it).
__device__ __forceinline__ u64 wave_merge_desc(u64 a, u64 b) {
  const int lane = threadIdx.x & 63;
  const u64 r = shfl64(b, 63 - lane);
  u64 v = a > r ? a : r;
#pragma unroll
  for (int j = 32; j > 0; j >>= 1) {
    const u64 o = shfl_xor_u64(v, j);
    v = (lane & j) == 0 ? (v > o ? v : o) : (v < o ? v : o);
  }
  return v;
}

// Merge tree over the sorted lists of waves [0, waves) (a power of two): wave
// 0 ends with the 64 largest of them, sorted descending.  Every thread of the
// workgroup calls it (one barrier per level); slots: waves x 64 LDS keys.
__device__ u64 tree_top64(u64 v, int waves, u64* slots) {
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  for (int step = 1; step < waves; step <<= 1) {
    if (wave < waves && wave % (2 * step) == step) slots[wave * 64 + lane] = v;  // each slot written once
    __syncthreads();
    if (wave < waves && wave % (2 * step) == 0) v = wave_merge_desc(v, slots[(wave + step) * 64 + lane]);
  }
  return v;
}

__global__ __launch_bounds__(256 * kPoolGroups) void block_pool_kernel(BlockParams p) {
  __shared__ u64 s_wave_max[4 * kPoolGroups];
  int b, item;
  if (!find_item(p.seq_offsets, p.batch, p.total_tokens, p.max_context, blockIdx.x,
                 [](int len) { return (candidate_blocks(len) + kPoolBlocks * kPoolGroups - 1) / (kPoolBlocks * kPoolGroups); },
                 b, item))
    return;
  int64_t base;
  int len;
  seq_bounds(p.seq_offsets, b, p.total_tokens, p.max_context, base, len);
  const int nb = candidate_blocks(len);
  const int quarter = threadIdx.x >> 8;
  const int g = item * kPoolGroups + quarter;
  const int i = g * kPoolBlocks + ((threadIdx.x & 255) >> 4);
  const int l = threadIdx.x & 15;
  float s = 0.f;
  if (i < nb) {
    const float* src = p.score + base + static_cast<int64_t>(i) * kSelectBlock + l;
    s = ((src[0] + src[16]) + src[32]) + src[48];
  }
#pragma unroll
  for (int off = 8; off > 0; off >>= 1) s += __shfl_xor(s, off);  // every lane ends with the same sum
  if (i < nb && l == 0) p.block_scores[block_slot(base, b, i)] = s;
  u64 key = i < nb ? block_key(s, i) : 0ull;
  key = max(key, shfl_xor_u64(key, 16));
  key = max(key, shfl_xor_u64(key, 32));
  if ((threadIdx.x & 63) == 0) s_wave_max[threadIdx.x >> 6] = key;
  __syncthreads();
  const u64* w = s_wave_max + 4 * quarter;
  if ((threadIdx.x & 255) == 0 && g * kPoolBlocks < nb)
    p.group_keys[group_slot(base, b, g)] = max(max(w[0], w[1]), max(w[2], w[3]));
}

// The full layer's merge and the block sums from the tile-sum pass, one
// launch: workgroups w < 16 B merge head w % 16 of sequence w / 16 (first,
// so the merges, the longest items, start first); the others take four
// groups of 16 candidate blocks each, over a compact grid.  A block's sum:
// per head (lane h of its team) the four tiles' exp2(m_h - M_h) r_h added in
// tile order and multiplied by 1 / Z_h, then summed over the 16 heads by a
// butterfly, which leaves every lane with the same bits.  Every tile of a
// candidate block holds 16 real tokens, so the pass wrote all four.
// (M_h, Z_h) are folded from the partials' packed (m, z), the same values in
// every workgroup of the sequence (the merge's result is not written yet).
// m_h <= M_h, so the factors are at most 1 and r_h at most 16 * 2^8.
constexpr int kTilePoolThreads = kMergeThreads;  // 16 teams of 16 lanes
constexpr int kTilePoolGroups = 4;               // groups of 16 blocks per workgroup: a team takes one block of each
static_assert(kTilePoolThreads == kPoolBlocks * kHeads, "one team per block of a group, one lane per head");

__global__ __launch_bounds__(kTilePoolThreads) void merge_block_pool_kernel(MergeParams mp, BlockParams p) {
  __shared__ MergeShared msh;
  __shared__ float s_mx[kHeads], s_iz[kHeads];
  __shared__ u64 s_team[kTilePoolGroups][kPoolBlocks];
  const int merges = kHeads * p.batch;
  if (static_cast<int>(blockIdx.x) < merges) {
    merge_one(mp, blockIdx.x % kHeads, blockIdx.x / kHeads, 0, 0, 0, msh);
    return;
  }
  auto items = [](int len) {
    const int groups = (candidate_blocks(len) + kPoolBlocks - 1) / kPoolBlocks;
    return (groups + kTilePoolGroups - 1) / kTilePoolGroups;
  };
  int b, item;
  if (!find_item(p.seq_offsets, p.batch, p.total_tokens, p.max_context, blockIdx.x - merges, items, b, item))
    return;
  b = __builtin_amdgcn_readfirstlane(b);
  item = __builtin_amdgcn_readfirstlane(item);
  int64_t base;
  int len;
  seq_bounds(p.seq_offsets, b, p.total_tokens, p.max_context, base, len);
  const int nb = candidate_blocks(len);
  const int team = threadIdx.x >> 4, h = threadIdx.x & 15;
  float m[kTilePoolGroups][4], r[kTilePoolGroups][4];
#pragma unroll
  for (int k = 0; k < kTilePoolGroups; ++k) {  // loads first: they fly while (M, Z) are folded
    const int i = min((item * kTilePoolGroups + k) * kPoolBlocks + team, nb - 1);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t slot = tile_slot(base, b, 4 * i + q) * kHeads + h;
      m[k][q] = p.tile_stats[slot];
      r[k][q] = p.tile_sums[slot];
    }
  }
  head_stats_packed(p.pstats, b, p.chunks_per_seq, (len + p.chunk - 1) / p.chunk, s_mx, s_iz);
  __syncthreads();
  const float mh = s_mx[h], izh = s_iz[h];
#pragma unroll
  for (int k = 0; k < kTilePoolGroups; ++k) {
    const int i = (item * kTilePoolGroups + k) * kPoolBlocks + team;
    float s = ((exp2f(m[k][0] - mh) * r[k][0] + exp2f(m[k][1] - mh) * r[k][1]) + exp2f(m[k][2] - mh) * r[k][2]) +
              exp2f(m[k][3] - mh) * r[k][3];
    s *= izh;
#pragma unroll
    for (int off = 8; off > 0; off >>= 1) s += __shfl_xor(s, off);
    if (h == 0) {
      if (i < nb) p.block_scores[block_slot(base, b, i)] = s;
      s_team[k][team] = i < nb ? block_key(s, i) : 0ull;
    }
  }
  __syncthreads();
  if (threadIdx.x < kTilePoolGroups) {
    const int k = threadIdx.x;
    const int g = item * kTilePoolGroups + k;
    if (g * kPoolBlocks < nb) {
      u64 best = s_team[k][0];
#pragma unroll
      for (int q = 1; q < kPoolBlocks; ++q) best = max(best, s_team[k][q]);
      p.group_keys[group_slot(base, b, g)] = best;
    }
  }
}

// Sorts s[0, m) descending; m a power of two <= kSortCap; every thread calls it.
__device__ void bitonic_sort_desc(u64* s, int m) {
  for (int k = 2; k <= m; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < m; i += kSelThreads) {
        const int o = i ^ j;
        if (o > i) {
          const u64 a = s[i], c = s[o];
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
  __shared__ u64 s_keys[kSortCap];
  __shared__ u64 s_t0;
  __shared__ int s_n;
  __shared__ int s_blk[kTopBlocks];
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
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
  const int ng = (nb + kPoolBlocks - 1) / kPoolBlocks;
  const float* bs = p.block_scores + block_slot(base, b, 0);
  const u64* gk = p.group_keys + group_slot(base, b, 0);
  u64 best = 0;  // 0 is below every key (the low word of a key is never 0)
  for (int g = tid; g < ng; g += kSelThreads) best = max(best, gk[g]);
  // t0: the 16th largest thread maximum (each wave sorts its 64, then a merge tree)
  if (tid == 0) s_n = 0;
  const u64 top = tree_top64(wave_sort_desc(best), kSelThreads / 64, s_keys);
  if (tid == kTopBlocks - 1) s_t0 = top;
  __syncthreads();
  const u64 t0 = s_t0;
  if (best >= t0) {  // the blocks of groups reaching t0: the candidates
    for (int g = tid; g < ng; g += kSelThreads) {
      if (gk[g] < t0) continue;
      float v[kPoolBlocks];
#pragma unroll
      for (int q = 0; q < kPoolBlocks; ++q) {
        const int i = g * kPoolBlocks + q;
        v[q] = i < nb ? bs[i] : 0.f;
      }
#pragma unroll
      for (int q = 0; q < kPoolBlocks; ++q) {
        const int i = g * kPoolBlocks + q;
        if (i < nb) {
          const u64 k = block_key(v[q], i);
          if (k >= t0) s_keys[atomicAdd(&s_n, 1)] = k;
        }
      }
    }
  }
  __syncthreads();
  const int n = s_n;  // 16 <= n <= kSortCap
  if (n <= 256) {  // four waves sort 64 candidates each, then merge
    const u64 v = wave < 4 && tid < n ? s_keys[tid] : 0ull;
    const u64 top = tree_top64(wave_sort_desc(v), 4, s_keys + 256);
    if (tid < kTopBlocks) s_keys[tid] = top;  // wave 0 alone reads LDS from here on until the barrier
    __syncthreads();
  } else {
    int m = 512;
    while (m < n) m <<= 1;
    for (int e = n + tid; e < m; e += kSelThreads) s_keys[e] = 0;
    __syncthreads();
    bitonic_sort_desc(s_keys, m);
  }
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
  const int64_t pool_grid = p.total_tokens / (kPoolGroups * kPoolBlocks * kSelectBlock) + p.batch;
  if (p.total_tokens > kBudget) {
    hipLaunchKernelGGL(block_pool_kernel, dim3(static_cast<unsigned>(pool_grid)), dim3(256 * kPoolGroups), 0, s, p);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(block_select_kernel, dim3(p.batch), dim3(kSelThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_merge_block_pool(const MergeParams& mp, const BlockParams& p, hipStream_t s) {
  if (p.batch <= 0) return hipSuccess;
  // 16 merges per sequence, then sum_b ceil(ceil(nb_b / 16) / 4) <= N / 4096 + B pool items
  const int64_t grid =
      static_cast<int64_t>(kHeads + 1) * p.batch + p.total_tokens / (kTilePoolGroups * kPoolBlocks * kSelectBlock);
  hipLaunchKernelGGL(merge_block_pool_kernel, dim3(static_cast<unsigned>(grid)), dim3(kTilePoolThreads), 0, s, mp, p);
  return hipGetLastError();
}

hipError_t launch_block_rank(const BlockParams& p, hipStream_t s) {
  if (p.batch <= 0) return hipSuccess;
  hipLaunchKernelGGL(block_select_kernel, dim3(p.batch), dim3(kSelThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace hs2
