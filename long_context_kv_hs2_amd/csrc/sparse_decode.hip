// Sparse-attention layers of a hybrid block at decode (KV Reuse).
//
// The sparse layers own no KV: they read the full layer's shared cache at the
// positions the full layer selected, and every sparse layer of the block reuses
// the same list (toolnavs.com article 2080, section "Ce que fait HySparse2";
// "Luo Fuli Teases Xiaomi MiMo-V3 Architecture", paragraphs on KV Reuse and on
// token selection).  Each layer takes its softmax over the selected positions.
//
// Workgroups of eight waves over (sequence, sparse layer, slice).  A workgroup
// stages its slice of the selected positions in LDS; each wave takes 16 * TILES
// consecutive selected rows and gathers their K and V rows straight into
// registers (16-byte loads, a two-tile ring), with the full layer's tile step
// for all 16 heads.  The eight waves' (m, z, O) are merged through LDS.  With
// one slice per (layer, sequence) the output is written directly; when the
// grid would be too small to fill the chip, the selected rows are cut into
// 2, 4 or 8 slices whose partials a second launch merges.  The layers of a
// sequence read the same rows at about the same time, so HBM serves each row
// about once and the other layers hit in cache.
//
// Window mode serves the Self-Decoder's sliding-window layers, which the
// model's front half mixes with full attention ("Luo Fuli Teases Xiaomi
// MiMo-V3 Architecture", paragraph on the self-decoder / cross-decoder split;
// toolnavs.com article 2080, section "Ce que fait HySparse2"): a layer's cache
// is a ring of `window` rows per sequence (position p in slot p mod window),
// and the rows attended are the window's slots, so no list is read.  The
// current token's rows come from the caller's input (its slot's old row is
// never read) and are stored into the ring by the same workgroup, one
// workgroup per sequence, unsliced.
#include "hs2_device.h"
#include "hs2_internal.h"
#include "merge.h"

namespace hs2 {

namespace {
constexpr int kSparseWaves = 8;
constexpr int kSparseThreads = 64 * kSparseWaves;
// Slices of the selection when each wave takes `tiles` tiles of 16 rows.
constexpr int sparse_slices_for(int tiles) {
  return (kBudget + 16 * kSparseWaves * tiles - 1) / (16 * kSparseWaves * tiles);
}
}  // namespace

template <bool FP8, int TILES, int SLICES = sparse_slices_for(TILES), bool WINDOW = false>
__global__ __launch_bounds__(kSparseThreads) void sparse_attend_kernel(SparseParams p) {
  constexpr int kWaveRows = 16 * TILES;
  constexpr int kSliceRows = kSparseWaves * kWaveRows;
  __shared__ int32_t s_pos[kSliceRows];
  __shared__ float s_m[kSparseWaves][kHeads];
  __shared__ float s_z[kSparseWaves][kHeads];
  __shared__ __attribute__((aligned(16))) float s_o[kSparseWaves][kHeads][kDim];
  constexpr int kRowBytes = FP8 ? kDim : 2 * kDim;

  // Work item j = (b * n_layers + layer) * slices + slice.  Consecutive items
  // go to one XCD (workgroup id i runs on XCD i % 8), so the layers and slices
  // of a sequence share that XCD's L2 when they gather the same rows.
  constexpr int kSlices = SLICES;
  const int items = p.batch * p.n_layers * kSlices;
  const int per_xcd = (items + 7) / 8;
  const int j = static_cast<int>(blockIdx.x & 7) * per_xcd + static_cast<int>(blockIdx.x >> 3);
  if (j >= items) return;  // uniform
  const int slice = j % kSlices;
  const int layer = (j / kSlices) % p.n_layers;
  const int b = j / (kSlices * p.n_layers);
  const int t = threadIdx.x;
  int64_t base;
  int len;
  int count;
  int new_slot = -1;  // window mode: the ring slot of the current token, read from the caller's rows
  if constexpr (WINDOW) {
    const int64_t positions = max<int64_t>(p.lengths[b], 0);
    base = static_cast<int64_t>(b) * p.budget;
    len = p.budget;
    count = static_cast<int>(min<int64_t>(positions, p.budget));
    if (p.k_new && positions > 0) new_slot = static_cast<int>((positions - 1) % p.budget);
  } else {
    seq_bounds(p.seq_offsets, b, p.total_tokens, p.max_context, base, len);
    count = clamp_count(p.sel_count[b], len, p.budget);
  }
  const int s0 = slice * kSliceRows;  // first selected row of the slice
  constexpr bool direct = kSlices == 1;
  if (count == 0) {  // uniform: an empty sequence has a zero output
    if constexpr (direct) {
      float* out = p.out + (static_cast<size_t>(layer) * p.batch + b) * kHeads * kDim;
      for (int i = t; i < kHeads * kDim; i += kSparseThreads) out[i] = 0.f;
    }
    return;
  }
  if (s0 >= count) return;  // uniform: the merge counts only slices with rows
  // Positions, clamped into the sequence (rows past `count` repeat the last one
  // and are masked out in the tile step), so every gather stays in the cache.
  if constexpr (WINDOW) {
    for (int i = t; i < kSliceRows; i += kSparseThreads) s_pos[i] = min(s0 + i, count - 1);
    if (new_slot >= 0 && t < kRowBytes / 4) {  // store the current rows into the ring (nothing here reads that slot)
      const size_t at = (static_cast<size_t>(base) + new_slot) * kRowBytes / 4 + t;
      reinterpret_cast<uint32_t*>(p.ring_k)[at] = reinterpret_cast<const uint32_t*>(p.k_new)[b * kRowBytes / 4 + t];
      reinterpret_cast<uint32_t*>(p.ring_v)[at] = reinterpret_cast<const uint32_t*>(p.v_new)[b * kRowBytes / 4 + t];
      if (FP8 && t == 0) {
        p.ring_ks[base + new_slot] = p.k_new_scale[b];
        p.ring_vs[base + new_slot] = p.v_new_scale[b];
      }
    }
  } else {
    const int32_t* sel = p.sel_idx + static_cast<size_t>(b) * p.budget;
    for (int i = t; i < kSliceRows; i += kSparseThreads) s_pos[i] = min(max(sel[min(s0 + i, count - 1)], 0), len - 1);
  }
  __syncthreads();

  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);  // wave-uniform
  const int lane = t & 63;
  const int n = lane & 15;
  const int g = lane >> 4;
  const int r0 = wave * kWaveRows;                         // within the slice
  const int rows = min(max(count - s0 - r0, 0), kWaveRows);
  const int last = count - 1 - s0;                         // last valid slot of s_pos
  const int64_t kvb = !WINDOW && p.kv_start ? p.kv_start[b] : base;  // the sequence's first K/V row
  const uint8_t* __restrict__ kbase = p.k + kvb * kRowBytes;
  const uint8_t* __restrict__ vbase = p.v + kvb * kRowBytes;
  const float* __restrict__ ksb = FP8 ? p.k_scale + kvb : nullptr;
  const float* __restrict__ vsb = FP8 ? p.v_scale + kvb : nullptr;

  struct Raw {
    u32x4 k[FP8 ? 2 : 4];
    u32x4 v[4];
    float ks[4], vs[4];
  };
  // Tile t: K lane (n, g) holds selected row r0 + 16t + n at row bytes
  // kload_offset(j, g); V lane (n, g) holds row r0 + 16t + 4g + r, dims 8n .. 8n + 7.
  auto load_tile = [&](int tile, Raw& raw) {
    const int i0 = r0 + 16 * tile;
    if constexpr (WINDOW) {  // the current token's slot reads the caller's rows
      const int kp = s_pos[min(i0 + n, last)];
      const uint8_t* ksrc = kp == new_slot ? p.k_new + static_cast<size_t>(b) * kRowBytes : kbase + kp * kRowBytes;
#pragma unroll
      for (int j = 0; j < (FP8 ? 2 : 4); ++j) raw.k[j] = *reinterpret_cast<const u32x4*>(ksrc + kload_offset(j, g));
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tv = s_pos[min(i0 + 4 * g + r, last)];
        const bool cur = tv == new_slot;
        const uint8_t* vsrc = cur ? p.v_new + static_cast<size_t>(b) * kRowBytes : vbase + tv * kRowBytes;
        if constexpr (FP8) {
          const u32x2 w = *reinterpret_cast<const u32x2*>(vsrc + 8 * n);
          raw.v[r] = u32x4{w[0], w[1], 0u, 0u};
          raw.ks[r] = cur ? p.k_new_scale[b] : ksb[tv];
          raw.vs[r] = cur ? p.v_new_scale[b] : vsb[tv];
        } else {
          raw.v[r] = *reinterpret_cast<const u32x4*>(vsrc + 16 * n);
          raw.ks[r] = 1.f;
          raw.vs[r] = 1.f;
        }
      }
    } else {
      const uint32_t krow = static_cast<uint32_t>(s_pos[min(i0 + n, last)]) * kRowBytes;
#pragma unroll
      for (int j = 0; j < (FP8 ? 2 : 4); ++j)
        raw.k[j] = *reinterpret_cast<const u32x4*>(kbase + (krow + kload_offset(j, g)));
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint32_t tv = static_cast<uint32_t>(s_pos[min(i0 + 4 * g + r, last)]);
        if constexpr (FP8) {
          const u32x2 w = *reinterpret_cast<const u32x2*>(vbase + (tv * kRowBytes + 8 * n));
          raw.v[r] = u32x4{w[0], w[1], 0u, 0u};
          raw.ks[r] = ksb[tv];
          raw.vs[r] = vsb[tv];
        } else {
          raw.v[r] = *reinterpret_cast<const u32x4*>(vbase + (tv * kRowBytes + 16 * n));
          raw.ks[r] = 1.f;
          raw.vs[r] = 1.f;
        }
      }
    }
  };

  SoftmaxState st;
  softmax_init(st);
  if (rows > 0) {  // uniform over the wave
    // The query's loads go first: a wait for data counts loads in issue
    // order, so a query loaded after the first two tiles would hold the
    // first step until the second tile had arrived too.
    QRaw qr;
    load_qraw<FP8>(p.q_sparse + ((static_cast<size_t>(layer) * p.batch + b) * kHeads + n) * kDim, g, qr);
    Raw ra, rb;
    load_tile(0, ra);
    if (TILES > 1) load_tile(1, rb);
    QRegs q;
    qregs_from(qr, p.qscale, q);
    auto step = [&](int tile, const Raw& cur) {
      bf16x8 kf[4];
      if constexpr (FP8) {
        e4m3x16_to_bf16(cur.k[0], kf[0], kf[1]);
        e4m3x16_to_bf16(cur.k[1], kf[2], kf[3]);
      } else {
#pragma unroll
        for (int s = 0; s < 4; ++s) kf[s] = as_bf16x8(cur.k[s]);
      }
      float lg[4], pr[4];
      attend_tile<FP8>(q, kf, cur.v, cur.ks, cur.vs, rows - 16 * tile, g, st, lg, pr);
    };
    // Two-slot ring over the wave's tiles, fully unrolled so each slot keeps
    // its registers; tiles wholly past the wave's rows are skipped.
#pragma unroll
    for (int tile = 0; tile < TILES; ++tile) {
      if (tile & 1) {
        if (16 * tile < rows) step(tile, rb);
        if (tile + 2 < TILES) load_tile(tile + 2, rb);
      } else {
        if (16 * tile < rows) step(tile, ra);
        if (tile + 2 < TILES) load_tile(tile + 2, ra);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // Merge the waves through LDS (a wave with no rows has m = -inf).
  const float z = reduce_z(st.z);
  if (g == 0) {
    s_m[wave][n] = st.m;
    s_z[wave][n] = z;
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
#pragma unroll
    for (int i = 0; i < 4; ++i) s_o[wave][n][32 * g + 8 * i + j] = st.o[j][i];
  }
  __syncthreads();
  const int h = t >> 5;         // 16 heads x 32 threads
  const int d0 = (t & 31) * 4;  // four dims each
  float mx = -INFINITY;
#pragma unroll
  for (int w = 0; w < kSparseWaves; ++w) mx = fmaxf(mx, s_m[w][h]);
  float zz = 0.f;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int w = 0; w < kSparseWaves; ++w) {
    const float mw = s_m[w][h];
    if (mw == -INFINITY) continue;
    const float f = exp2f(mw - mx);
    zz += s_z[w][h] * f;
    const float4 o4 = *reinterpret_cast<const float4*>(&s_o[w][h][d0]);
    acc[0] += o4.x * f;
    acc[1] += o4.y * f;
    acc[2] += o4.z * f;
    acc[3] += o4.w * f;
  }
  if constexpr (direct) {
    float* out = p.out + (static_cast<size_t>(layer) * p.batch + b) * kHeads * kDim;
    *reinterpret_cast<float4*>(out + h * kDim + d0) = make_float4(acc[0] / zz, acc[1] / zz, acc[2] / zz, acc[3] / zz);
  } else {
    // Partial of the slice: (m[16], z[16], O[16][128]) unnormalised.
    float* part = p.partials + ((static_cast<size_t>(layer) * p.batch + b) * kSlices + slice) * kPartialFloats;
    if ((t & 31) == 0) {
      part[h] = mx;
      part[kHeads + h] = zz;
    }
    *reinterpret_cast<float4*>(part + 2 * kHeads + h * kDim + d0) = make_float4(acc[0], acc[1], acc[2], acc[3]);
  }
}

__global__ __launch_bounds__(kMergeThreads) void sparse_merge_kernel(MergeParams p, int64_t stride_layer,
                                                                     int64_t out_stride_layer) {
  __shared__ MergeShared sh;
  merge_one(p, blockIdx.x, blockIdx.y, blockIdx.z, stride_layer, out_stride_layer, sh);
}

// Tiles per wave: 9 (one slice per layer and sequence, output written
// directly), else 5, 3, 2 or 1 (2, 3, 5 or 9 slices), the most tiles that
// still give the grid at least kSparseFillWorkgroups workgroups.
int sparse_wave_tiles(int batch, int n_layers) {
  const int64_t wgs = static_cast<int64_t>(batch) * n_layers;
  for (const int tiles : {9, 5, 3, 2})
    if (wgs * sparse_slices_for(tiles) >= kSparseFillWorkgroups) return tiles;
  return 1;
}

template <bool FP8, int TILES>
static void launch_tiles(const SparseParams& p, hipStream_t s) {
  const int items = p.batch * p.n_layers * sparse_slices_for(TILES);
  const dim3 grid(static_cast<unsigned>(8 * ((items + 7) / 8)));
  hipLaunchKernelGGL((sparse_attend_kernel<FP8, TILES>), grid, dim3(kSparseThreads), 0, s, p);
}

template <bool FP8>
static void launch_fp(const SparseParams& p, int tiles, hipStream_t s) {
  switch (tiles) {
    case 9: launch_tiles<FP8, 9>(p, s); break;
    case 5: launch_tiles<FP8, 5>(p, s); break;
    case 3: launch_tiles<FP8, 3>(p, s); break;
    case 2: launch_tiles<FP8, 2>(p, s); break;
    default: launch_tiles<FP8, 1>(p, s); break;
  }
}

int sparse_slices(int batch, int n_layers) { return sparse_slices_for(sparse_wave_tiles(batch, n_layers)); }

template <bool FP8, int TILES>
static void launch_window_tiles(const SparseParams& p, hipStream_t s) {
  const int items = p.batch * p.n_layers;
  const dim3 grid(static_cast<unsigned>(8 * ((items + 7) / 8)));
  hipLaunchKernelGGL((sparse_attend_kernel<FP8, TILES, 1, true>), grid, dim3(kSparseThreads), 0, s, p);
}

template <bool FP8>
static void launch_window_fp(const SparseParams& p, hipStream_t s) {
  const int rows = 16 * kSparseWaves;  // rows per tile step of the eight waves
  if (p.budget <= rows)
    launch_window_tiles<FP8, 1>(p, s);
  else if (p.budget <= 2 * rows)
    launch_window_tiles<FP8, 2>(p, s);
  else if (p.budget <= 3 * rows)
    launch_window_tiles<FP8, 3>(p, s);
  else if (p.budget <= 5 * rows)
    launch_window_tiles<FP8, 5>(p, s);
  else
    launch_window_tiles<FP8, 9>(p, s);
}

hipError_t launch_sparse_window(const SparseParams& p, bool fp8, hipStream_t s) {
  if (p.batch == 0 || p.n_layers == 0) return hipSuccess;
  if (p.budget < 1 || p.budget > kBudget || p.lengths == nullptr || p.n_layers != 1) return hipErrorInvalidValue;
  if (fp8)
    launch_window_fp<true>(p, s);
  else
    launch_window_fp<false>(p, s);
  return hipGetLastError();
}

hipError_t launch_sparse_attend(const SparseParams& p, bool fp8, hipStream_t s) {
  if (p.batch == 0 || p.n_layers == 0) return hipSuccess;
  static_assert(sparse_slices_for(9) == 1, "nine tiles per wave cover the whole selection");
  const int tiles = sparse_wave_tiles(p.batch, p.n_layers);
  const int slices = sparse_slices_for(tiles);
  if (slices > 1 && p.partials == nullptr) return hipErrorInvalidValue;
  if (fp8)
    launch_fp<true>(p, tiles, s);
  else
    launch_fp<false>(p, tiles, s);
  const hipError_t e = hipGetLastError();
  if (slices == 1 || e != hipSuccess) return e;
  MergeParams mp{};
  mp.seq_offsets = p.seq_offsets;
  mp.total_tokens = p.total_tokens;
  mp.max_context = p.max_context;
  mp.budget = p.budget;
  mp.partials = p.partials;
  mp.chunk = 16 * kSparseWaves * tiles;  // selected rows per slice
  mp.chunks_per_seq = slices;
  mp.stride_seq = slices * kPartialFloats;
  mp.stride_chunk = kPartialFloats;
  mp.count_from_sel = 1;
  mp.sel_count = p.sel_count;
  mp.out = p.out;
  mp.out_stride_seq = kHeads * kDim;
  mp.stats = nullptr;
  hipLaunchKernelGGL(sparse_merge_kernel, dim3(kHeads, p.batch, p.n_layers), dim3(kMergeThreads), 0, s, mp,
                     static_cast<int64_t>(p.batch) * slices * kPartialFloats,
                     static_cast<int64_t>(p.batch) * kHeads * kDim);
  return hipGetLastError();
}

}  // namespace hs2
