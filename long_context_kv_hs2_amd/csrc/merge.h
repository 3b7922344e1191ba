// Split-K merge of one (head, sequence) problem of the full layer, shared by
// the plain merge kernel (score path) and the merge fused with the
// selection's first pass (bound path), so both give bitwise the same (M, Z).
//
// A partial holds a reference max m, the sum z of exp2(l - m) and the
// unnormalised output O[16][128] of its tokens (log2 domain).  With
// M = max_c m_c and w_c = exp2(m_c - M): O = sum_c w_c O_c / sum_c w_c z_c.
// The max and the sum are block reductions over a fixed tree; the output
// accumulates the partials in index order, 128 at a time with their weights
// staged in LDS, so every rounding order is fixed and the merge is
// deterministic.
#pragma once

#include "hs2_device.h"
#include "hs2_internal.h"

namespace hs2 {

constexpr int kMergeThreads = 256;  // threads >= kDim only join the reductions

struct MergeShared {
  float red[kMergeThreads / 64];
  float f[kDim];
};

__device__ __forceinline__ float merge_reduce(float v, float* s_red, bool is_max) {
  const int t = threadIdx.x;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const float o = __shfl_xor(v, off);
    v = is_max ? fmaxf(v, o) : v + o;
  }
  if ((t & 63) == 0) s_red[t >> 6] = v;
  __syncthreads();
  const float r = is_max ? fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]))
                         : (s_red[0] + s_red[1]) + (s_red[2] + s_red[3]);
  __syncthreads();
  return r;
}

// Every thread of the workgroup (kMergeThreads) must call this.
__device__ __forceinline__ void merge_one(const MergeParams& p, int h, int b, int layer, int64_t stride_layer,
                                          int64_t out_stride_layer, MergeShared& sh) {
  const int d = threadIdx.x;
  const bool dim = d < kDim;
  int64_t base;
  int len;
  seq_bounds(p.seq_offsets, b, p.total_tokens, p.max_context, base, len);
  const int items = p.count_from_sel ? clamp_count(p.sel_count[b], len, p.budget) : len;
  const int count = (items + p.chunk - 1) / p.chunk;
  const float* pb = p.partials + layer * stride_layer + static_cast<int64_t>(b) * p.stride_seq;
  float mx = -INFINITY;
  if (dim)
    for (int c = d; c < count; c += kDim) mx = fmaxf(mx, pb[static_cast<int64_t>(c) * p.stride_chunk + h]);
  mx = merge_reduce(mx, sh.red, true);
  float zpart = 0.f;
  float acc = 0.f;
  for (int c0 = 0; c0 < count; c0 += kDim) {
    const int c = c0 + d;
    if (dim) {
      float f = 0.f;
      if (c < count) {
        const float* pc = pb + static_cast<int64_t>(c) * p.stride_chunk;
        const float m = pc[h];
        f = m == -INFINITY ? 0.f : exp2f(m - mx);
        zpart += pc[kHeads + h] * f;
      }
      sh.f[d] = f;
    }
    __syncthreads();
    if (dim) {
      const int nc = min(kDim, count - c0);
      const float* po = pb + static_cast<int64_t>(c0) * p.stride_chunk + 2 * kHeads + h * kDim + d;
#pragma unroll 8
      for (int j = 0; j < nc; ++j) acc += po[static_cast<int64_t>(j) * p.stride_chunk] * sh.f[j];
    }
    __syncthreads();
  }
  const float z = merge_reduce(zpart, sh.red, false);
  if (dim) {
    float* out = p.out + layer * out_stride_layer + b * p.out_stride_seq + h * kDim;
    out[d] = count ? acc / z : 0.f;
  }
  if (p.stats && layer == 0 && d == 0) {
    p.stats[(static_cast<int64_t>(b) * kHeads + h) * 2] = mx;
    p.stats[(static_cast<int64_t>(b) * kHeads + h) * 2 + 1] = z;
  }
}

// Each head's (M, Z) over a sequence's `count` partials, from the full pass's
// packed copy of their (m, z) (pstats: [B][chunks_per_seq][m[16], z[16]]):
// 16 lanes per head fold partials l, l + 16, ... online (eight loads in
// flight per lane), then across the 16 lanes.  Threads 0 .. 255 call it;
// s_mx[h] = M_h and s_iz[h] = 1 / Z_h are written (the caller syncs).  The
// order is fixed, so every workgroup that calls it gets the same values;
// they differ from merge_one's by rounding order only.
__device__ __forceinline__ void head_stats_packed(const float* pstats, int b, int chunks_per_seq, int count,
                                                  float* s_mx, float* s_iz) {
  const int t = threadIdx.x;
  const int h = t >> 4, l = t & 15;
  const float* pb = pstats + static_cast<int64_t>(b) * chunks_per_seq * (2 * kHeads);
  float m = -INFINITY, z = 0.f;
  auto fold = [](float& m, float& z, float mc, float zc) {  // (m, z) += (mc, zc)
    if (mc == -INFINITY) return;
    if (mc > m) {
      z = z * exp2f(m - mc) + zc;
      m = mc;
    } else {
      z += zc * exp2f(mc - m);
    }
  };
  constexpr int kBatch = 8;
  for (int c0 = l; c0 < count; c0 += 16 * kBatch) {
    float mv[kBatch], zv[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int c = c0 + 16 * u;
      const float* pc = pb + static_cast<int64_t>(min(c, count - 1)) * (2 * kHeads);
      mv[u] = c < count ? pc[h] : -INFINITY;
      zv[u] = pc[kHeads + h];
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) fold(m, z, mv[u], zv[u]);
  }
#pragma unroll
  for (int off = 8; off > 0; off >>= 1) {
    const float mo = __shfl_xor(m, off), zo = __shfl_xor(z, off);
    fold(m, z, mo, zo);
  }
  if (l == 0) {
    s_mx[h] = m;
    s_iz[h] = 1.f / z;
  }
}

}  // namespace hs2
