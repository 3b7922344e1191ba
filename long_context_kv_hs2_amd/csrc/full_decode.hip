// Full-attention layer of a hybrid block at decode: split-K flash decoding
// over the shared MQA cache, keeping each token's logits for the score pass.
//
// The full-attention layer attends over the whole context and its attention
// scores pick the positions the sparse layers reuse (toolnavs.com article 2080,
// section "Ce que fait HySparse2"; "Luo Fuli Teases Xiaomi MiMo-V3
// Architecture", paragraph on keeping a few full-attention layers).
//
// Work split: one workgroup per (sequence, chunk of `chunk` tokens), four
// waves, each wave streaming a quarter of the chunk in tiles of 16 tokens
// straight from HBM into registers (16-byte loads), so every K/V byte is read
// exactly once.  Per tile: S^T = K Q^T on bf16 MFMA with the query split into
// three exact bf16 parts (fp32-accurate logits), an online softmax per head in
// registers, and O^T += V^T P^T on bf16 MFMA with each weight split into a
// bf16 head and tail (16 significant bits).  The four waves' (m, z, O) are
// merged through LDS into one partial per workgroup.  Four modes: BOUND keeps
// per-token score bounds for the selection, SPILL keeps every logit for the
// score pass, PLAIN keeps nothing (full attention alone), TILE_SUMS keeps per
// tile and head the sum of the weights (gen-1 block selection).  In the first
// two the first workgroup of each sequence also clears the sequence's
// selection histogram and counters for the kernels that follow.
#include <algorithm>

#include "hs2_device.h"
#include "hs2_internal.h"

namespace hs2 {

// BOUND: instead of spilling the 16 logits of each token, keep per token
// shat_j = sum_h exp2(l_hj - m_h^t) c_h^t (written as bf16) with the wave's running max m^t after
// the token's tile and c^t ~ 1 / (running sum z^t), and per tile and head
// u_h^t = m_h^t - log2 c_h^t.  Then score_j = sum_h a_hj F_h^t with
// F_h^t = exp2(m_h^t - M_h) / (c_h^t Z_h) = exp2(u_h^t - M_h) / Z_h, so score_j
// lies in shat_j * [min_h F_h^t, max_h F_h^t]; the selection prunes with these
// bounds and rescores the survivors exactly.
// Bound-mode outputs of one wave's tiles wait in LDS until the loop ends: on
// CDNA loads and stores share one in-order completion counter, so stores in
// the streaming loop would put their write latency into every load wait.
constexpr int kTileOut = 2 * kHeads;  // shat[16], u[16] (TILE_SUMS: r[16], m[16])
// TILE_SUMS: per tile and head, r_h = sum over the tile's tokens of
// p_hj = exp2(l_hj - m_h), m_h being the wave's reference max the weights are
// taken against; the score mass of the tile for head h is then
// exp2(m_h - M_h) r_h / Z_h once the merge knows (M_h, Z_h), and a 64-token
// block's score (four whole tiles) is the sum of that over its tiles and the
// heads.  The same LDS staging and end-of-loop flush as BOUND.

// Work item wg of the 1-D grid: the non-empty (sequence, chunk) pairs of the
// batch, numbered in order.  A 1-D grid of just these deals the workgroups
// evenly over the XCDs; a 2-D grid over the longest sequence has holes, and
// an XCD that is dealt more non-empty workgroups than it holds at once runs
// a second round while the others idle.  Every lane of the wave computes the
// same answer; false past the last item.
__device__ bool find_work(const FullParams& p, int wg, int& b, int& c) {
  const int lane = threadIdx.x & 63;
  int carry = 0;  // items of the sequences before this pass
  for (int s0 = 0; s0 < p.batch; s0 += 64) {
    const int sb = s0 + lane;
    int64_t sbase = 0;
    int slen = 0;
    if (sb < p.batch) seq_bounds(p.seq_offsets, sb, p.total_tokens, p.max_context, sbase, slen);
    const int nb = (slen + p.chunk - 1) / p.chunk;
    int incl = nb;  // inclusive prefix sum over the wave
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int o = __shfl_up(incl, d);
      if (lane >= d) incl += o;
    }
    const int total = __shfl(incl, 63);
    if (wg < carry + total) {
      const uint64_t hit = __ballot(carry + incl > wg);
      const int src = __ffsll(static_cast<unsigned long long>(hit)) - 1;
      b = s0 + src;
      c = wg - carry - __shfl(incl - nb, src);
      return true;
    }
    carry += total;
  }
  return false;
}

// Waves per workgroup and tile streams per workgroup (see the kernel).
template <bool FP8> constexpr int full_waves() { return FP8 ? 8 : 4; }
template <bool FP8> constexpr int full_streams() { return FP8 ? 28 : 4; }

template <bool FP8, int MODE>
__global__ __launch_bounds__(64 * full_waves<FP8>()) void full_partial_kernel(FullParams p) {
  constexpr bool BOUND = MODE == kFullBound;
  constexpr bool SPILL = MODE == kFullSpill;
  constexpr bool TSUM = MODE == kFullTileSums;
  constexpr bool STAGED = BOUND || TSUM;  // per-tile outputs staged in LDS
  constexpr int kWaves = full_waves<FP8>();
  constexpr int kStreams = full_streams<FP8>();
  constexpr int kThreads = 64 * kWaves;
  // Tiles of one wave (a bound for the flush loop) and of one workgroup
  // (bound-mode LDS slots).  E4M3: a wave holds at most 4 (chunk / 448 + 1)
  // and a workgroup chunk / 16 + kStreams.  bf16: a wave holds at most
  // chunk / 64 + 1, or with the even-XCD split below at most
  // (chunk / 64) (1 + 1 / D) + 4 (D = kEvenXcdDen), and a workgroup four waves'.
  constexpr int kBf16WaveTiles = (max_chunk(false) / 64 * (kEvenXcdDen + 1) / kEvenXcdDen + 4 + 15) / 16 * 16;
  constexpr int kMaxWaveTiles = FP8 ? (4 * (max_chunk(true) / (16 * kStreams) + 1) + 15) / 16 * 16 : kBf16WaveTiles;
  constexpr int kLocalTiles = FP8 ? max_chunk(FP8) / 16 + kStreams : kStreams * kMaxWaveTiles;
  __shared__ float s_m[kWaves][kHeads];
  __shared__ float s_z[kWaves][kHeads];
  // the merge buffer O[kWaves][16][128] and, before it, the bound-mode tile outputs
  __shared__ __attribute__((aligned(16))) float s_raw[STAGED ? kLocalTiles * kTileOut : kWaves * kHeads * kDim];
  __shared__ u32x4 s_q[kQLdsVecs];
  float(*s_o)[kHeads][kDim] = reinterpret_cast<float(*)[kHeads][kDim]>(s_raw);

  int b, c;
  if (!find_work(p, blockIdx.x, b, c)) return;  // uniform over the workgroup
  b = __builtin_amdgcn_readfirstlane(b);
  c = __builtin_amdgcn_readfirstlane(c);
  int64_t base;
  int len;
  seq_bounds(p.seq_offsets, b, p.total_tokens, p.max_context, base, len);

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform: scalar loop control
  const int lane = threadIdx.x & 63;
  const int n = lane & 15;
  const int g = lane >> 4;
  // Tiles of 16 tokens are dealt round-robin over the tile streams of all the
  // sequence's workgroups (tile kStreams * (k * nblk + c) + v is the k-th of
  // stream v of workgroup c), so at any moment they stream one compact region
  // of the cache (better DRAM locality than a contiguous range per wave).
  // With a bf16 cache each of the four waves (one per SIMD) takes one stream.
  // With E4M3 two waves share each SIMD, and the older one's loads are served
  // about 4/3 as fast, so on each SIMD the older wave takes four streams and
  // the younger three of seven: the two finish together.  A wave visits its
  // streams' k-th tiles in stream order, then the (k + 1)-th.  The split-K
  // merge does not depend on which tokens a partial holds.
  //
  // bf16, a batch of equal lengths and an even number of chunks: workgroup w
  // runs on XCD w mod 8 (the dispatcher deals workgroups round-robin over the
  // XCDs), and with one wave per SIMD the workgroups on odd XCDs stream about
  // 6.5% slower than those on even ones (per-workgroup end times, the same on
  // every part measured; a ragged batch is set by its longest sequences).  So
  // the sequence's tiles are dealt in two regions: whole rounds over all its
  // workgroups up to ~(1 - 1/D) of its tiles, then the rest over its even-XCD
  // workgroups only (every other chunk, nblk / 2 of them), which thus take
  // D + 1 tiles for every D - 1 of the others (D = kEvenXcdDen).  The split
  // depends only on the batch, so every partial holds the same tokens on
  // every call.
  const int nblk = (len + p.chunk - 1) / p.chunk;
  const int simd = FP8 ? (wave & 3) : wave;
  const int per = FP8 ? (wave < 4 ? 4 : 3) : 1;                 // streams of this wave
  const int v0 = FP8 ? 7 * simd + (wave < 4 ? 0 : 4) : wave;    // its first stream
  const int stream_stride = 16 * kStreams * nblk;               // tokens between a stream's tiles
  int nt = 0;                                                   // this wave's tiles
  int nt_a = 0, s_a = 0, s_b = 0, stride_b = 0;                 // bf16: the two regions
  if constexpr (FP8) {
    for (int j = 0; j < per; ++j) {
      const int s0 = 16 * (kStreams * c + v0 + j);
      nt += s0 < len ? (len - 1 - s0) / stream_stride + 1 : 0;
    }
  } else {
    const int tiles = (len + 15) >> 4;
    const int round = kStreams * nblk;  // tiles of one round over all the sequence's workgroups
    // (region A ends on a whole round, so the even-XCD share is 1/D to 1/D +
    // round / tiles: split only with at least 4 D rounds, within a quarter of 1/D)
    const bool split = p.xcd_split && nblk >= 2 && (nblk & 1) == 0 && tiles >= 4 * kEvenXcdDen * round;
    const int tiles_a = split ? (tiles - tiles / kEvenXcdDen) / round * round : tiles;
    const int len_a = min(len, 16 * tiles_a);
    s_a = 16 * (kStreams * c + wave);
    nt_a = s_a < len_a ? (len_a - 1 - s_a) / stream_stride + 1 : 0;
    nt = nt_a;
    if (split && (blockIdx.x & 1) == 0) {
      // the sequence's even-XCD workgroups are every other chunk, starting
      // at chunk 0 or 1: this one is the (c / 2)-th of them
      stride_b = 16 * kStreams * (nblk >> 1);
      s_b = 16 * (tiles_a + kStreams * (c >> 1) + wave);
      nt += s_b < len ? (len - 1 - s_b) / stride_b + 1 : 0;
    }
  }
  // The i-th tile of the wave; a wave's tiles are in increasing token order,
  // so the valid ones are i < nt.  len: past the end.
  auto tok0 = [&](int i) {
    if constexpr (FP8) {
      return i < nt ? 16 * (kStreams * c + v0 + i % per) + (i / per) * stream_stride : len;
    } else {
      return i < nt_a ? s_a + i * stream_stride : (i < nt ? s_b + (i - nt_a) * stride_b : len);
    }
  };
  auto local = [&](int i) { return (i / per) * kStreams + v0 + i % per; };  // LDS slot of the i-th tile

  const QShared q{s_q, lane};  // filled below, after the first tile's loads are issued

  constexpr int kRowBytes = FP8 ? kDim : 2 * kDim;
  // Uniform per-sequence bases; lanes address rows with 32-bit offsets
  // (a sequence spans at most 2^24 rows, so its bytes fit in 32 bits).
  const int64_t kvb = p.kv_start ? p.kv_start[b] : base;  // the sequence's first K/V row
  const uint8_t* __restrict__ kbase = p.k + kvb * kRowBytes;
  const uint8_t* __restrict__ vbase = p.v + kvb * kRowBytes;
  const float* __restrict__ ksb = FP8 ? p.k_scale + kvb : nullptr;
  const float* __restrict__ vsb = FP8 ? p.v_scale + kvb : nullptr;
  float* __restrict__ spill = SPILL ? p.spill + base * kHeads : nullptr;
  uint16_t* __restrict__ shat = BOUND ? p.shat + base : nullptr;

  SoftmaxState st;
  softmax_init(st);

  // Raw tile registers: K lane (n, g) holds token t0 + n at row bytes
  // kload_offset(j, g); V lane (n, g) holds token t0 + 4g + r, dims 8n .. 8n + 7.
  // Rows past the end are clamped to a valid row and masked out in the tile step.
  struct Raw {
    u32x4 k[FP8 ? 2 : 4];
    u32x4 v[4];
    float ks[4], vs[4];
  };
  // Loads are issued unconditionally (rows clamped to the sequence's last
  // row), so the compiler can count exactly which loads are still in flight
  // when a tile is consumed; a prefetch past the end re-reads one cached row.
  auto load_tile = [&](int t0, Raw& raw) {
    const uint32_t krow = static_cast<uint32_t>(min(t0 + n, len - 1)) * kRowBytes;
#pragma unroll
    for (int j = 0; j < (FP8 ? 2 : 4); ++j)
      raw.k[j] = *reinterpret_cast<const u32x4*>(kbase + (krow + kload_offset(j, g)));
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint32_t tv = static_cast<uint32_t>(min(t0 + 4 * g + r, len - 1));
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
  // Bound mode: c_h ~ 1 / (head h's running sum), refreshed every other tile,
  // and its log2.  Any c_h > 0 gives valid bounds as long as the stored u
  // uses the same c_h: the bounds divide by exactly what shat multiplied by.
  float cfac = 1.f, lcf = 0.f;
  auto step = [&](int t0, int ti, bool refresh, const Raw& cur) {
    const int nv = min(16, len - t0);  // <= 0: a masked tile past the end
    bf16x8 kf[4];
    if constexpr (FP8) {
      e4m3x16_to_bf16(cur.k[0], kf[0], kf[1]);
      e4m3x16_to_bf16(cur.k[1], kf[2], kf[3]);
    } else {
#pragma unroll
      for (int s = 0; s < 4; ++s) kf[s] = as_bf16x8(cur.k[s]);
    }
    float lg[4], pr[4];
    attend_tile<FP8>(q, kf, cur.v, cur.ks, cur.vs, nv, g, st, lg, pr);
    if constexpr (BOUND) {
      if (refresh) {
        cfac = __builtin_amdgcn_rcpf(reduce_z(st.z));
        lcf = __builtin_amdgcn_logf(cfac);  // error ~1e-7: far inside the selection's 2^-10 slack
      }
      // a_hj = p_hj * c_h summed over the heads: lane n of row g ends with
      // token 4g + (n >> 2)
      float x[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) x[r] = pr[r] * cfac;
      const float sh = row_sums4(x, n);
      if (nv <= 0) return;  // the masked tile past the end has no slot
      float* out = s_raw + local(ti) * kTileOut;
      if ((n & 3) == 0) out[4 * g + (n >> 2)] = sh;
      if (g == 0) out[kHeads + n] = st.m - lcf;  // u_h = m_h - log2 c_h
    } else if constexpr (SPILL) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (4 * g + r < nv) spill[static_cast<uint32_t>(t0 + 4 * g + r) * kHeads + n] = lg[r];
      }
    } else if constexpr (TSUM) {
      // head n's weights over the tile: four tokens in the lane, then over
      // the four lane groups (masked tokens weigh 0); every lane of the
      // head ends with the same sum
      float x = (pr[0] + pr[1]) + (pr[2] + pr[3]);
      x += __shfl_xor(x, 16);
      x += __shfl_xor(x, 32);
      if (nv <= 0) return;  // the masked tile past the end has no slot
      float* out = s_raw + local(ti) * kTileOut;
      if (g == 0) {
        out[n] = x;
        out[kHeads + n] = st.m;
      }
    }
  };

  // Two-slot ring, unrolled so each slot keeps its own registers: while one
  // tile is computed the next tile's loads are in flight.  (Rotating slots by
  // copying would wait for the in-flight loads at every copy.)  The scheduling
  // barriers pin each batch of loads ahead of the math of the tile before it;
  // left free, the scheduler sinks them past that math and the prefetch is lost.
  // The loop leaves only at its bottom: an exit between the two halves gives
  // the compiler a path on which the second slot's loads reach the loop top
  // still in flight, and it then waits for them before the next loads are
  // issued, every iteration.  So the second half always runs; when a wave has
  // an odd number of tiles its last step sees a tile past the end, fully
  // masked (zero weights, no outputs).
  // The query's loads go first, then the first tile's, which stay in flight
  // while the query operand is built: a wait for data counts loads in issue
  // order, so the other order would hold the build until the tile arrived.
  float4 qa, qc;
  if (threadIdx.x < 256) load_q_lds_raw<FP8>(p.q + static_cast<size_t>(b) * kHeads * kDim, qa, qc);
  Raw ra, rb;
  load_tile(tok0(0), ra);
  if (threadIdx.x < 256) store_q_lds(qa, qc, p.qscale, s_q);
  __syncthreads();
  if (nt > 0) {
    for (int k = 0;; k += 2) {
      load_tile(tok0(k + 1), rb);
      __builtin_amdgcn_sched_barrier(0);
      step(tok0(k), k, true, ra);
      __builtin_amdgcn_sched_barrier(0);
      load_tile(tok0(k + 2), ra);
      __builtin_amdgcn_sched_barrier(0);
      step(tok0(k + 1), k + 1, false, rb);
      __builtin_amdgcn_sched_barrier(0);
      if (k + 2 >= nt) break;
    }
  }

  if constexpr (STAGED) {
    // Write this wave's tile outputs: shat of the tokens that exist (TILE_SUMS:
    // the sums r of every tile), and the per-tile u (m) of every tile.
    // 16-byte stores, all issued before any completes: the flush is on the
    // critical path of the workgroup's end.
    const int ntiles = nt;
    if constexpr (TSUM) {
#pragma unroll
      for (int it = 0; it < kMaxWaveTiles * 4 / 64; ++it) {
        const int i = lane + 64 * it;  // float4 i: tile i / 4, heads 4 (i % 4) ..
        const int ti = i >> 2, e = 4 * (i & 3);
        if (ti < ntiles) {
          const int tile = tok0(ti) >> 4;
          *reinterpret_cast<float4*>(p.tile_sums + tile_slot(base, b, tile) * kHeads + e) =
              *reinterpret_cast<const float4*>(s_raw + local(ti) * kTileOut + e);
        }
      }
    }
#pragma unroll
    for (int it = 0; it < (BOUND ? kMaxWaveTiles * 4 / 64 : 0); ++it) {
      const int i = lane + 64 * it;  // float4 i: tile i / 4, tokens 4 (i % 4) ..
      const int ti = i >> 2, e = 4 * (i & 3);
      if (ti < ntiles) {
        const float4 v = *reinterpret_cast<const float4*>(s_raw + local(ti) * kTileOut + e);
        const int tok = tok0(ti) + e;
        // bf16, round to nearest even: the selection's slack covers the 2^-9
        // relative rounding
        const uint32_t b01 = bf16_rne(v.x) | (bf16_rne(v.y) << 16), b23 = bf16_rne(v.z) | (bf16_rne(v.w) << 16);
        if (tok + 3 < len && (base & 3) == 0) {  // 8-byte aligned: tok is a multiple of 4
          *reinterpret_cast<uint2*>(shat + tok) = make_uint2(b01, b23);
        } else {
          const uint16_t vv[4] = {static_cast<uint16_t>(b01), static_cast<uint16_t>(b01 >> 16),
                                  static_cast<uint16_t>(b23), static_cast<uint16_t>(b23 >> 16)};
          for (int u = 0; u < 4 && tok + u < len; ++u) shat[tok + u] = vv[u];
        }
      }
    }
#pragma unroll
    for (int it = 0; it < kMaxWaveTiles * 4 / 64; ++it) {
      const int i = lane + 64 * it;  // float4 i: tile i / 4, heads 4 (i % 4) ..
      const int ti = i >> 2, e = 4 * (i & 3);
      if (ti < ntiles) {
        const int tile = tok0(ti) >> 4;
        *reinterpret_cast<float4*>(p.tile_stats + tile_slot(base, b, tile) * kHeads + e) =
            *reinterpret_cast<const float4*>(s_raw + local(ti) * kTileOut + kHeads + e);
      }
    }
    __syncthreads();  // the merge below reuses this LDS
  }

  // Merge the waves through LDS.
  const float z = reduce_z(st.z);
  if (g == 0) {
    s_m[wave][n] = st.m;
    s_z[wave][n] = z;
  }
#pragma unroll
  for (int t = 0; t < 8; ++t) {
#pragma unroll
    for (int i = 0; i < 4; ++i) s_o[wave][n][32 * g + 8 * i + t] = st.o[t][i];
  }
  __syncthreads();

  // thread -> (head h, dims d0 .. d0 + kDims - 1)
  constexpr int kDims = kDim * kHeads / kThreads;  // 8 (bf16) or 4 (E4M3)
  const int h = threadIdx.x / (kDim / kDims);
  const int d0 = (threadIdx.x % (kDim / kDims)) * kDims;
  float mx = -INFINITY;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) mx = fmaxf(mx, s_m[w][h]);
  float zz = 0.f;
  float acc[kDims];
#pragma unroll
  for (int j = 0; j < kDims; ++j) acc[j] = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const float mw = s_m[w][h];
    if (mw == -INFINITY) continue;  // a wave with no tokens
    const float f = exp2f(mw - mx);
    zz += s_z[w][h] * f;
#pragma unroll
    for (int j = 0; j < kDims; ++j) acc[j] += s_o[w][h][d0 + j] * f;
  }
  const size_t item = static_cast<size_t>(b) * p.chunks_per_seq + c;
  float* out = p.partials + item * kPartialFloats;
  if (d0 == 0) {
    out[h] = mx;
    out[kHeads + h] = zz;
    if constexpr (MODE != kFullPlain) {
      p.pstats[item * 2 * kHeads + h] = mx;  // compact copy for the selection's first pass
      p.pstats[item * 2 * kHeads + kHeads + h] = zz;
    }
  }
  float4* o4 = reinterpret_cast<float4*>(out + 2 * kHeads + h * kDim + d0);
#pragma unroll
  for (int j = 0; j < kDims / 4; ++j) o4[j] = make_float4(acc[4 * j], acc[4 * j + 1], acc[4 * j + 2], acc[4 * j + 3]);
  if ((BOUND || SPILL) && c == 0) {
    uint4* hz = reinterpret_cast<uint4*>(p.hist0 + static_cast<size_t>(b) * kRadixBins);
    for (int i = threadIdx.x; i < kRadixBins / 4; i += kThreads) hz[i] = make_uint4(0u, 0u, 0u, 0u);
    if (threadIdx.x < 4) p.counters[b * 4 + threadIdx.x] = 0u;
  }
}

template <bool FP8, int MODE>
static void launch_mode(const FullParams& p, dim3 grid, hipStream_t s) {
  hipLaunchKernelGGL((full_partial_kernel<FP8, MODE>), grid, dim3(64 * full_waves<FP8>()), 0, s, p);
}

hipError_t launch_full_partial(const FullParams& p, int batch, bool fp8, int mode, hipStream_t s) {
  if (batch == 0) return hipSuccess;
  // at most sum_b ceil(L_b / chunk) < N / chunk + B work items
  const int64_t items = std::min<int64_t>(static_cast<int64_t>(batch) * p.chunks_per_seq,
                                          (p.total_tokens + p.chunk - 1) / p.chunk + batch);
  const dim3 grid(static_cast<unsigned>(items));
  switch (mode) {
    case kFullBound: fp8 ? launch_mode<true, kFullBound>(p, grid, s) : launch_mode<false, kFullBound>(p, grid, s); break;
    case kFullSpill: fp8 ? launch_mode<true, kFullSpill>(p, grid, s) : launch_mode<false, kFullSpill>(p, grid, s); break;
    case kFullPlain: fp8 ? launch_mode<true, kFullPlain>(p, grid, s) : launch_mode<false, kFullPlain>(p, grid, s); break;
    case kFullTileSums:
      fp8 ? launch_mode<true, kFullTileSums>(p, grid, s) : launch_mode<false, kFullTileSums>(p, grid, s);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace hs2
