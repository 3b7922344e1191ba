// Full-attention pass of multi-token decode with the T query tokens of a
// sequence sharing its K/V stream: each K/V row is read once per group of up
// to kMultiQ tokens, instead of once per token.
//
// The reading of multi-token decode is the one the virtual-sequence path
// takes (the pages give no multi-token rule for HySparse2): token t of
// sequence b, at position L_b - T + t, is a decode step of its own over the
// causal prefix [0, L_b - T + t + 1) with its own selection; the selection
// ranks positions by the full layer's attention scores (toolnavs.com article
// 2080, section "Ce que fait HySparse2").  The outputs are exactly those the
// ordinary bound-mode pass leaves for the virtual sequence v = b T + t (its
// split-K partials and their packed statistics, its per-token score bounds
// and per-tile head statistics, its cleared histogram and counters), so the
// merge, the selection and the sparse layers run on the virtual batch
// unchanged.
//
// Work item (b, c): chunk c of real sequence b for the launch's tokens
// [t_first, t_first + nq).  The chunk geometry is the ordinary pass's (tiles
// of 16 tokens dealt round-robin over 4 streams per chunk, one per SIMD) with
// nblk = ceil(L_lo / chunk) chunks, L_lo the prefix length of the group's
// shortest token, over the tokens of the group's longest prefix.  A token
// whose prefix reaches into one more chunk (ceil(L_v / chunk) = nblk + 1: a
// token differs from the shortest by at most 15 positions) gets an empty
// partial there, written by chunk 0, so its merge sees exactly its tokens.
//
// Per tile, the K operand and the V rows are formed once, then every token of
// the wave runs the ordinary tile step (fp32-accurate logits from the
// three-part query, online softmax, P.V) with its own causal mask and state.
// Groups of four tokens run as two waves per SIMD with two tokens each (both
// walk the same tiles; the second wave's loads hit the L2), which measured
// faster than one wave carrying all four (a wave's states then fill the
// register file and nothing covers its latencies).
// The per-tile bound outputs wait in LDS and go out every kFlushTiles tiles of
// a wave: a store shares the load counter (the next wait for loads would
// include its latency), so they are batched rather than issued per tile.
#include "hs2_device.h"
#include "hs2_internal.h"

namespace hs2 {

namespace {

constexpr int kMultiStreams = 4;   // tile streams per workgroup, one per SIMD
constexpr int kFlushTiles = 16;    // staged tiles per wave between flushes
constexpr int kTileOut = 2 * kHeads;  // per tile and token: shat[16], u[16]

// Items of real sequence b (len tokens) for the group's tokens: 0 when every
// token of the group has an empty prefix.
__device__ __forceinline__ int multi_items(const MultiFullParams& mp, int len) {
  const int lo = len - mp.n_query + mp.t_first + 1;         // the group's shortest prefix
  const int hi = lo + mp.nq - 1;                            // and its longest
  if (hi <= 0) return 0;
  return (max(lo, 1) + mp.f.chunk - 1) / mp.f.chunk;
}

// GROUPS token groups of NQ tokens each share the workgroup's streams: wave w
// takes stream w % 4 and tokens NQ (w / 4) .. NQ (w / 4) + NQ - 1 of the
// launch's group, so with two groups two waves on a SIMD walk the same tiles
// (the second's loads hit the L2) and hide each other's latency.
template <bool FP8, int NQ, int GROUPS>
__global__ __launch_bounds__(256 * GROUPS) void full_multi_kernel(MultiFullParams mp) {
  const FullParams& p = mp.f;
  constexpr int kMultiWaves = 4 * GROUPS;
  constexpr int kThreads = 64 * kMultiWaves;
  constexpr int kTok = NQ * GROUPS;  // tokens of the launch's group
  __shared__ u32x4 s_q[kTok][kQLdsVecs];
  // staged bound outputs [wave][tile][token][32]; at the end the merge buffer O[wave][16][128]
  constexpr int kStageFloats = kMultiWaves * kFlushTiles * NQ * kTileOut;
  constexpr int kMergeFloats = kMultiWaves * kHeads * kDim;
  __shared__ __attribute__((aligned(16))) float s_raw[kStageFloats > kMergeFloats ? kStageFloats : kMergeFloats];
  __shared__ float s_m[kMultiWaves][kHeads];
  __shared__ float s_z[kMultiWaves][kHeads];
  __shared__ int s_t0[kMultiWaves][kFlushTiles];  // staged tiles' first tokens

  int b, c;
  if (!find_item(p.seq_offsets, p.batch, p.total_tokens, p.max_context, blockIdx.x,
                 [&](int len) { return multi_items(mp, len); }, b, c))
    return;  // uniform over the workgroup
  b = __builtin_amdgcn_readfirstlane(b);
  c = __builtin_amdgcn_readfirstlane(c);
  int64_t base;
  int len;
  seq_bounds(p.seq_offsets, b, p.total_tokens, p.max_context, base, len);
  constexpr int nq = NQ;  // this wave's tokens
  const int lo = len - mp.n_query + mp.t_first + 1;  // prefix length of the group's first token
  const int hi = lo + kTok - 1;                      // of its last: the tokens this pass reads
  const int nblk = multi_items(mp, len);

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int n = lane & 15;
  const int g = lane >> 4;
  const int tg = wave >> 2;          // this wave's token group
  const int lo_w = lo + NQ * tg;     // prefix length of this wave's first token
  // The ordinary pass's dealing over the group's tokens [0, hi): whole rounds
  // over all nblk chunks, and with one token (the ordinary pass's case: one
  // wave per SIMD, bound by its loads), bf16, a batch of equal lengths and
  // nblk even, the last ~1/kEvenXcdDen of the tiles over the even-XCD
  // workgroups only (they stream faster).  With more tokens a wave's
  // arithmetic hides the XCDs' difference and the split measured slower
  // (two tokens a wave: 495 -> 531 us at 32 x 128K).  So with one token the
  // tiles of every wave are the ordinary pass's, and the outputs its bit for
  // bit.
  const int stream_stride = 16 * kMultiStreams * nblk;
  const int s_a = 16 * (kMultiStreams * c + (wave & 3));  // this wave's first tile
  int nt_a, nt, s_b = 0, stride_b = 0;
  {
    const int tiles = (hi + 15) >> 4;
    const int round = kMultiStreams * nblk;
    const bool split = !FP8 && NQ == 1 && GROUPS == 1 && p.xcd_split && nblk >= 2 && (nblk & 1) == 0 &&
                       tiles >= 4 * kEvenXcdDen * round;
    const int tiles_a = split ? (tiles - tiles / kEvenXcdDen) / round * round : tiles;
    const int len_a = min(hi, 16 * tiles_a);
    nt_a = s_a < len_a ? (len_a - 1 - s_a) / stream_stride + 1 : 0;
    nt = nt_a;
    if (split && (blockIdx.x & 1) == 0) {
      stride_b = 16 * kMultiStreams * (nblk >> 1);
      s_b = 16 * (tiles_a + kMultiStreams * (c >> 1) + (wave & 3));
      nt += s_b < hi ? (hi - 1 - s_b) / stride_b + 1 : 0;
    }
  }
  auto tok0 = [&](int i) { return i < nt_a ? s_a + i * stream_stride : (i < nt ? s_b + (i - nt_a) * stride_b : hi); };

  constexpr int kRowBytes = FP8 ? kDim : 2 * kDim;
  const uint8_t* __restrict__ kbase = p.k + base * kRowBytes;
  const uint8_t* __restrict__ vbase = p.v + base * kRowBytes;
  const float* __restrict__ ksb = FP8 ? p.k_scale + base : nullptr;
  const float* __restrict__ vsb = FP8 ? p.v_scale + base : nullptr;
  const int v_first = b * mp.n_query + mp.t_first;  // virtual sequence of the group's first token
  const int v_wave = v_first + NQ * tg;             // and of this wave's first token

  SoftmaxState st[NQ];
  float cfac[NQ], lcf[NQ];
#pragma unroll
  for (int t = 0; t < NQ; ++t) {
    softmax_init(st[t]);
    cfac[t] = 1.f;
    lcf[t] = 0.f;
  }

  struct Raw {
    u32x4 k[FP8 ? 2 : 4];
    u32x4 v[4];
    float ks[4], vs[4];
  };
  auto load_tile = [&](int t0, Raw& raw) {  // rows clamped to the group's last row
    const uint32_t krow = static_cast<uint32_t>(min(t0 + n, hi - 1)) * kRowBytes;
#pragma unroll
    for (int j = 0; j < (FP8 ? 2 : 4); ++j)
      raw.k[j] = *reinterpret_cast<const u32x4*>(kbase + (krow + kload_offset(j, g)));
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint32_t tv = static_cast<uint32_t>(min(t0 + 4 * g + r, hi - 1));
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
  };

  float* const stage = s_raw + wave * (kFlushTiles * NQ * kTileOut);
  int staged = 0;  // tiles staged by this wave (wave-uniform)
  // Writes the staged tiles' outputs: for every token of the group the shat
  // of its tokens that exist and the tile's u, if the tile holds any of them.
  auto flush = [&]() {
    for (int e = lane; e < staged * nq * 8; e += 64) {
      const int ti = e / (8 * nq), t = (e / 8) % nq, part = e % 8;
      const int t0 = s_t0[wave][ti];
      const int lv = lo_w + t;  // token t's prefix length
      if (t0 >= lv) continue;
      const int v = v_wave + t;
      const int64_t vbase_tok = mp.voffs[v];
      const float* src = stage + (ti * NQ + t) * kTileOut;
      if (part < 4) {
        const float4 x = *reinterpret_cast<const float4*>(src + 4 * part);
        const int tok = t0 + 4 * part;
        const uint16_t vv[4] = {static_cast<uint16_t>(bf16_rne(x.x)), static_cast<uint16_t>(bf16_rne(x.y)),
                                static_cast<uint16_t>(bf16_rne(x.z)), static_cast<uint16_t>(bf16_rne(x.w))};
        uint16_t* dst = p.shat + vbase_tok + tok;
        if (tok + 3 < lv && ((vbase_tok + tok) & 3) == 0) {
          *reinterpret_cast<uint2*>(dst) = make_uint2(vv[0] | (static_cast<uint32_t>(vv[1]) << 16),
                                                      vv[2] | (static_cast<uint32_t>(vv[3]) << 16));
        } else {
          for (int u = 0; u < 4 && tok + u < lv; ++u) dst[u] = vv[u];
        }
      } else {
        *reinterpret_cast<float4*>(p.tile_stats + tile_slot(vbase_tok, v, t0 >> 4) * kHeads + 4 * (part - 4)) =
            *reinterpret_cast<const float4*>(src + kHeads + 4 * (part - 4));
      }
    }
    staged = 0;
  };

  // One tile: the K operand once, the group's product chains interleaved (so
  // the matrix core is not left waiting on one chain's latency), then each
  // token's update with its own causal mask.
  auto step = [&](int t0, bool refresh, const Raw& cur) {
    bf16x8 kf[4];
    if constexpr (FP8) {
      e4m3x16_to_bf16(cur.k[0], kf[0], kf[1]);
      e4m3x16_to_bf16(cur.k[1], kf[2], kf[3]);
    } else {
#pragma unroll
      for (int s = 0; s < 4; ++s) kf[s] = as_bf16x8(cur.k[s]);
    }
    if (t0 >= hi) return;  // the masked tile past the end
    f32x4 sc[NQ];
#pragma unroll
    for (int t = 0; t < NQ; ++t) sc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int part = 0; part < 3; ++part) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
#pragma unroll
        for (int t = 0; t < NQ; ++t)
          sc[t] = mfma_bf16_16x16x32(kf[k], QShared{s_q[NQ * tg + t], lane}.get(part, k), sc[t]);
      }
    }
    // The update of attend_tile, phase by phase over the group's tokens so
    // that their latencies overlap (no token waits on another's chain), with
    // the same arithmetic: a token's head maximum is exchanged across the
    // lane groups only when some lane's own maximum exceeds its reference by
    // the slack (exactly when the exchanged one would), and a token with no
    // position in this tile (or none yet) gets zero weights.
    constexpr float kRescaleSlack = 8.f;
    float lg[NQ][4], pr[NQ][4];
    float lmx[NQ];
#pragma unroll
    for (int t = 0; t < NQ; ++t) {
      const int nv = lo_w + t - t0;  // > 0: positions of this tile in token t's prefix (capped at 16 by the mask)
#pragma unroll
      for (int r = 0; r < 4; ++r) lg[t][r] = (4 * g + r < nv) ? sc[t][r] * cur.ks[r] : -INFINITY;
      lmx[t] = fmaxf(fmaxf(lg[t][0], lg[t][1]), fmaxf(lg[t][2], lg[t][3]));
    }
#pragma unroll
    for (int t = 0; t < NQ; ++t) {
      if (__any(lmx[t] > st[t].m + kRescaleSlack)) {
        float mx = fmaxf(lmx[t], __shfl_xor(lmx[t], 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const bool raise = mx > st[t].m + kRescaleSlack;
        const float mn = raise ? mx : st[t].m;
        const float alpha = __builtin_amdgcn_exp2f(st[t].m - mn);
        st[t].z *= alpha;
#pragma unroll
        for (int j = 0; j < 8; ++j) st[t].o[j] *= alpha;
        st[t].m = mn;
      }
    }
    u32x2 va[8], ph[NQ], pl[NQ];
    pv_v_operand<FP8>(cur.v, va);
#pragma unroll
    for (int t = 0; t < NQ; ++t) {
      const bool live = st[t].m != -INFINITY;
#pragma unroll
      for (int r = 0; r < 4; ++r) pr[t][r] = live ? __builtin_amdgcn_exp2f(lg[t][r] - st[t].m) : 0.f;
      st[t].z += (pr[t][0] + pr[t][1]) + (pr[t][2] + pr[t][3]);
      pv_p_operand<FP8>(pr[t], cur.vs, ph[t], pl[t]);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
#pragma unroll
      for (int t = 0; t < NQ; ++t) st[t].o[j] = mfma_bf16_16x16x16(va[j], ph[t], st[t].o[j]);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
#pragma unroll
      for (int t = 0; t < NQ; ++t) st[t].o[j] = mfma_bf16_16x16x16(va[j], pl[t], st[t].o[j]);
    }
    // Bound outputs (kept only for tiles that hold positions of the token).
    const int slot = staged;
    if (refresh) {
#pragma unroll
      for (int t = 0; t < NQ; ++t) {
        const float z = reduce_z(st[t].z);
        if (z > 0.f) {
          cfac[t] = __builtin_amdgcn_rcpf(z);
          lcf[t] = __builtin_amdgcn_logf(cfac[t]);
        }
      }
    }
#pragma unroll
    for (int t = 0; t < NQ; ++t) {
      float x[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) x[r] = pr[t][r] * cfac[t];
      const float sh = row_sums4(x, n);
      float* out = stage + (slot * NQ + t) * kTileOut;
      if ((n & 3) == 0) out[4 * g + (n >> 2)] = sh;
      if (g == 0) out[kHeads + n] = st[t].m - lcf[t];
    }
    if (lane == 0) s_t0[wave][slot] = t0;
    staged = slot + 1;
    if (staged == kFlushTiles) flush();
  };

  // The queries' loads, then the first tile's, then the split into LDS.
  // (each group's four waves split its tokens' queries as load_q_lds_raw
  // and store_q_lds do with a workgroup of four: wave w % 4 takes k-step w % 4)
  float4 qa[NQ], qc[NQ];
#pragma unroll
  for (int t = 0; t < NQ; ++t)
    load_q8<FP8>(p.q + (static_cast<size_t>(v_wave + t) * kHeads + (lane & 15)) * kDim, wave & 3, lane >> 4, qa[t],
                 qc[t]);
  Raw ra, rb;
  load_tile(tok0(0), ra);
#pragma unroll
  for (int t = 0; t < NQ; ++t) {
    u32x4 ph, pm, pl;
    split_q8(qa[t], qc[t], p.qscale, ph, pm, pl);
    u32x4* dst = s_q[NQ * tg + t];
    dst[(0 * 4 + (wave & 3)) * 64 + lane] = ph;
    dst[(1 * 4 + (wave & 3)) * 64 + lane] = pm;
    dst[(2 * 4 + (wave & 3)) * 64 + lane] = pl;
  }
  __syncthreads();
  // Two-slot ring as in the ordinary pass: the next tile's loads fly while
  // this one is computed; the loop leaves only at its bottom.
  if (nt > 0) {
    for (int k = 0;; k += 2) {
      load_tile(tok0(k + 1), rb);
      __builtin_amdgcn_sched_barrier(0);
      step(tok0(k), true, ra);
      __builtin_amdgcn_sched_barrier(0);
      load_tile(tok0(k + 2), ra);
      __builtin_amdgcn_sched_barrier(0);
      step(tok0(k + 1), false, rb);
      __builtin_amdgcn_sched_barrier(0);
      if (k + 2 >= nt) break;
    }
  }
  if (staged > 0) flush();
  __syncthreads();  // the merge below reuses the staging LDS

  // Each token's partial: merge the four waves through LDS, one token at a time.
  float(*s_o)[kHeads][kDim] = reinterpret_cast<float(*)[kHeads][kDim]>(s_raw);
  // Thread group mg (256 threads) merges the four waves of token group mg.
  constexpr int kDims = kDim * kHeads / 256;  // 8
  const int mg = threadIdx.x >> 8;
  const int h = (threadIdx.x & 255) / (kDim / kDims);
  const int d0 = (threadIdx.x % (kDim / kDims)) * kDims;
#pragma unroll
  for (int t = 0; t < NQ; ++t) {
    const int v = v_first + NQ * mg + t;
    const float z = reduce_z(st[t].z);
    if (g == 0) {
      s_m[wave][n] = st[t].m;
      s_z[wave][n] = z;
    }
#pragma unroll
    for (int q8 = 0; q8 < 8; ++q8) {
#pragma unroll
      for (int i = 0; i < 4; ++i) s_o[wave][n][32 * g + 8 * i + q8] = st[t].o[q8][i];
    }
    __syncthreads();
    float mx = -INFINITY;
#pragma unroll
    for (int w = 4 * mg; w < 4 * mg + 4; ++w) mx = fmaxf(mx, s_m[w][h]);
    float zz = 0.f;
    float acc[kDims];
#pragma unroll
    for (int j = 0; j < kDims; ++j) acc[j] = 0.f;
#pragma unroll
    for (int w = 4 * mg; w < 4 * mg + 4; ++w) {
      const float mw = s_m[w][h];
      if (mw == -INFINITY) continue;  // a wave with no tokens of this prefix
      const float f = exp2f(mw - mx);
      zz += s_z[w][h] * f;
#pragma unroll
      for (int j = 0; j < kDims; ++j) acc[j] += s_o[w][h][d0 + j] * f;
    }
    const size_t item = static_cast<size_t>(v) * p.chunks_per_seq + c;
    float* out = p.partials + item * kPartialFloats;
    if (d0 == 0) {
      out[h] = mx;
      out[kHeads + h] = zz;
      p.pstats[item * 2 * kHeads + h] = mx;
      p.pstats[item * 2 * kHeads + kHeads + h] = zz;
    }
    float4* o4 = reinterpret_cast<float4*>(out + 2 * kHeads + h * kDim + d0);
#pragma unroll
    for (int j = 0; j < kDims / 4; ++j)
      o4[j] = make_float4(acc[4 * j], acc[4 * j + 1], acc[4 * j + 2], acc[4 * j + 3]);
    __syncthreads();  // before the next token's values overwrite the buffer
  }
  if (c == 0) {
    // Per token: the selection's histogram and counters cleared, and the empty
    // partial of the one chunk its prefix may reach beyond the group's nblk.
    for (int t = 0; t < kTok; ++t) {
      const int v = v_first + t;
      uint4* hz = reinterpret_cast<uint4*>(p.hist0 + static_cast<size_t>(v) * kRadixBins);
      for (int i = threadIdx.x; i < kRadixBins / 4; i += kThreads) hz[i] = make_uint4(0u, 0u, 0u, 0u);
      if (threadIdx.x < 4) p.counters[v * 4 + threadIdx.x] = 0u;
      const int lv = lo + t;
      if (lv > 0 && (lv + p.chunk - 1) / p.chunk > nblk) {
        const size_t item = static_cast<size_t>(v) * p.chunks_per_seq + nblk;
        float* out = p.partials + item * kPartialFloats;
        for (int i = threadIdx.x; i < kPartialFloats; i += kThreads) out[i] = i < kHeads ? -INFINITY : 0.f;
        if (threadIdx.x < 2 * kHeads) p.pstats[item * 2 * kHeads + threadIdx.x] = threadIdx.x < kHeads ? -INFINITY : 0.f;
      }
    }
  }
}

}  // namespace

hipError_t launch_full_multi(const MultiFullParams& mp, hipStream_t s) {
  const FullParams& p = mp.f;
  if (p.batch == 0) return hipSuccess;
  if (mp.nq < 1 || mp.nq > kMultiQ) return hipErrorInvalidValue;
  // at most sum_b ceil(L_b / chunk) < N / chunk + B work items
  const int64_t items = std::min<int64_t>(static_cast<int64_t>(p.batch) * ((p.max_context + p.chunk - 1) / p.chunk),
                                          (p.total_tokens + p.chunk - 1) / p.chunk + p.batch);
  if (items <= 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(items));
  const dim3 b4(256), b8(512);
  switch ((mp.nq - 1) * 2 + (mp.fp8 ? 1 : 0)) {
    case 0: hipLaunchKernelGGL((full_multi_kernel<false, 1, 1>), grid, b4, 0, s, mp); break;
    case 1: hipLaunchKernelGGL((full_multi_kernel<true, 1, 1>), grid, b4, 0, s, mp); break;
    case 2: hipLaunchKernelGGL((full_multi_kernel<false, 2, 1>), grid, b4, 0, s, mp); break;
    case 3: hipLaunchKernelGGL((full_multi_kernel<true, 2, 1>), grid, b4, 0, s, mp); break;
    case 4: hipLaunchKernelGGL((full_multi_kernel<false, 3, 1>), grid, b4, 0, s, mp); break;
    case 5: hipLaunchKernelGGL((full_multi_kernel<true, 3, 1>), grid, b4, 0, s, mp); break;
    case 6: hipLaunchKernelGGL((full_multi_kernel<false, 2, 2>), grid, b8, 0, s, mp); break;
    case 7: hipLaunchKernelGGL((full_multi_kernel<true, 2, 2>), grid, b8, 0, s, mp); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace hs2
