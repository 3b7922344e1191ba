// Sparse-attention layers of a hybrid block at decode (KV Reuse), and the
// Self-Decoder's sliding-window layers.
//
// The sparse layers own no KV: they read the full layer's shared cache at the
// positions the full layer selected, and every sparse layer of the block reuses
// the same list (toolnavs.com article 2080, section "Ce que fait HySparse2";
// "Luo Fuli Teases Xiaomi MiMo-V3 Architecture", paragraphs on KV Reuse and on
// token selection).  Each layer takes its softmax over the selected positions.
//
// Sparse layers (sparse_reuse_kernel): one workgroup of eight waves per
// (sequence, slice of the selection).  The workgroup gathers its slice's K
// and V rows from HBM into LDS once, 144 rows a round (all of a round's
// 16-byte loads in flight together; with several rounds the next round's
// loads fly while the current round is computed), and every sparse layer
// attends over them there: each row crosses HBM once for all layers, and
// the layers' 16 x n_s query rows share it.  Each layer is two virtual waves
// (even and odd 16-row tiles of the slice), each with its own query in
// registers and its own online-softmax state, running the full layer's tile
// step; eight waves hold the virtual waves of four layers (from five layers
// on, a second workgroup of the same slice serves layers 4..7, gathering the
// slice again).  The odd virtual wave hands its state to the
// even one through LDS, which writes the layer's output (one slice per
// sequence) or the slice's partial, merged by a second launch in slice order.
// The slice count depends on the batch size alone, so a layer's result is
// the same bit for bit whether it runs alone or with the others.
//
// Window mode (sparse_window_kernel) serves the Self-Decoder's sliding-window
// layers, which the model's front half mixes with full attention ("Luo Fuli
// Teases Xiaomi MiMo-V3 Architecture", paragraph on the self-decoder /
// cross-decoder split; toolnavs.com article 2080, section "Ce que fait
// HySparse2"): a layer's cache is a ring of `window` rows per sequence
// (position p in slot p mod window), and the rows attended are the window's
// slots, so no list is read.  The current token's rows come from the
// caller's input (its slot's old row is never read) and are stored into the
// ring by the same workgroup, one workgroup per sequence.
#include <type_traits>

#include "hs2_device.h"
#include "hs2_internal.h"

namespace hs2 {

namespace {
constexpr int kSparseWaves = 8;
constexpr int kSparseThreads = 64 * kSparseWaves;
constexpr int kRoundRows = kBudget / 8;            // rows gathered per round: 144, 9 tiles of 16
constexpr int kRoundTiles = kRoundRows / 16;
constexpr int kLdsPad = 16;                        // bytes after each LDS row: spreads rows over the banks
constexpr int kMergeLaneFloats = 2 + 32;           // a virtual wave's state per lane: m, z, O^T tile
constexpr int kGroupLayers = kSparseWaves / 2;     // layers a workgroup serves (two virtual waves each)
constexpr int kSparseQParts = 2;                   // query parts in the sparse layers' logits
}  // namespace

// Slices of each sequence's selection: the most of 8, 4, 2, 1 that keeps the
// grid within one workgroup per CU of a 256-CU part (a second round of
// workgroups would wait for the first); a slice is 8 / slices rounds of 144
// rows.  Depends on the batch size only (see the file comment).
int sparse_slices(int batch) {
  for (const int s : {8, 4, 2})
    if (static_cast<int64_t>(batch) * s <= 256) return s;
  return 1;
}

// The slices' partials of one (sequence, layer), for head h and dims
// d0 .. d0 + 7: every partial needed is loaded at once, then combined in
// slice order (O = sum_c w_c O_c / sum_c w_c z_c, w_c = exp2(m_c - max_c
// m_c)).  `used` = the slices with rows.
template <int SLICES>
__device__ __forceinline__ void merge_slices(const SparseParams& p, int b, int layer, int used, int h, int d0) {
  const float* part = p.partials + (static_cast<size_t>(layer) * p.batch + b) * SLICES * kPartialFloats;
  float m[SLICES], z[SLICES];
  float4 o[SLICES][2];
#pragma unroll
  for (int c = 0; c < SLICES; ++c) {
    if (c < used) {
      const float* pc = part + c * kPartialFloats;
      m[c] = pc[h];
      z[c] = pc[kHeads + h];
      o[c][0] = *reinterpret_cast<const float4*>(pc + 2 * kHeads + h * kDim + d0);
      o[c][1] = *reinterpret_cast<const float4*>(pc + 2 * kHeads + h * kDim + d0 + 4);
    }
  }
  float mx = -INFINITY;
#pragma unroll
  for (int c = 0; c < SLICES; ++c)
    if (c < used) mx = fmaxf(mx, m[c]);
  float zz = 0.f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < SLICES; ++c) {
    if (c >= used) continue;
    const float w = exp2f(m[c] - mx);
    zz += z[c] * w;
    acc[0] += o[c][0].x * w;
    acc[1] += o[c][0].y * w;
    acc[2] += o[c][0].z * w;
    acc[3] += o[c][0].w * w;
    acc[4] += o[c][1].x * w;
    acc[5] += o[c][1].y * w;
    acc[6] += o[c][1].z * w;
    acc[7] += o[c][1].w * w;
  }
  float* out = p.out + ((static_cast<size_t>(layer) * p.batch + b) * kHeads + h) * kDim + d0;
  const float iz = used ? 1.f / zz : 0.f;
  *reinterpret_cast<float4*>(out) = make_float4(acc[0] * iz, acc[1] * iz, acc[2] * iz, acc[3] * iz);
  *reinterpret_cast<float4*>(out + 4) = make_float4(acc[4] * iz, acc[5] * iz, acc[6] * iz, acc[7] * iz);
}

// Slices with rows of sequence b (the merge reads only those).
template <int SLICES>
__device__ __forceinline__ int used_slices(const SparseParams& p, int b) {
  int64_t base;
  int len;
  seq_bounds(p.seq_offsets, b, p.total_tokens, p.max_context, base, len);
  const int count = clamp_count(p.sel_count[b], len, p.budget);
  return (count + kBudget / SLICES - 1) / (kBudget / SLICES);
}

template <bool FP8, int SLICES>
__global__ __launch_bounds__(kSparseThreads) void sparse_reuse_kernel(SparseParams p, int groups) {
  constexpr int kRowBytes = FP8 ? kDim : 2 * kDim;
  constexpr int kLdsRow = kRowBytes + kLdsPad;
  constexpr int kSliceRows = kBudget / SLICES;                 // 144, 288, 576 or 1152
  constexpr int kRounds = kSliceRows / kRoundRows;             // 1, 2, 4 or 8
  constexpr bool kTwoBuffers = kRounds > 1;
  constexpr int kBufBytes = 2 * kRoundRows * kLdsRow;          // K rows then V rows
  constexpr int kQBytes = kGroupLayers * kHeads * kDim * 4;    // the group's queries, fp32
  // LDS: round buffers, then the queries (with two buffers they use the second
  // one's room: they are read into registers before that buffer is filled);
  // the merge of the virtual waves reuses the first buffer at the end.
  constexpr int kRawBytes = kTwoBuffers ? 2 * kBufBytes : kBufBytes + kQBytes;
  static_assert(kGroupLayers * kMergeLaneFloats * 64 * 4 <= kBufBytes, "merge room");
  static_assert(kQBytes <= kBufBytes, "query room");
  __shared__ __attribute__((aligned(16))) uint8_t s_raw[kRawBytes];
  __shared__ float s_ks[kTwoBuffers ? 2 : 1][kRoundRows], s_vs[kTwoBuffers ? 2 : 1][kRoundRows];
  float* const s_q = reinterpret_cast<float*>(s_raw + kBufBytes);

  const int grp = static_cast<int>(blockIdx.x) % groups;  // layers [4 grp, 4 grp + 4)
  const int b = static_cast<int>(blockIdx.x) / (groups * SLICES);
  const int slice = static_cast<int>(blockIdx.x) / groups % SLICES;
  const int layer0 = kGroupLayers * grp;
  const int t = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int lane = t & 63;
  const int n = lane & 15;
  const int g = lane >> 4;
  const int s0 = slice * kSliceRows;  // first selected row of the slice
  const int nlay = min(kGroupLayers, p.n_layers - layer0);
  const int vw = wave;                // virtual wave: layer layer0 + vw / 2, tiles of parity vw % 2
  const bool active = vw < 2 * nlay;

  // The sequence's bounds and selection count (uniform: scalar loads), then
  // the slice's positions; a thread's gather pieces cover kRowsPer rows, the
  // same rows for K and V, and E4M3 threads below 256 also take a row's scale.
  int64_t base;
  int len;
  seq_bounds(p.seq_offsets, b, p.total_tokens, p.max_context, base, len);
  const int count = clamp_count(p.sel_count[b], len, p.budget);
  const int64_t kvb = p.kv_start ? p.kv_start[b] : base;  // the sequence's first K/V row
  constexpr int kRowPieces = kRowBytes / 16;
  constexpr int kRowStep = kSparseThreads / kRowPieces;                  // 32 or 64
  constexpr int kRowsPer = (kRoundRows + kRowStep - 1) / kRowStep;       // 5 or 3 (the last partial)
  const int row0 = t / kRowPieces;  // this thread's rows: row0 + kRowStep * i (< kRoundRows)
  const int piece = t % kRowPieces;
  const int srow = t % kRoundRows;  // the row whose scale this thread takes (E4M3, t < 2 * kRoundRows)
  // One round: the positions go straight to registers; several: through LDS
  // (registers for all of them would crowd out the tile step's).
  const int32_t* sel = p.sel_idx + static_cast<size_t>(b) * p.budget + s0;
  __shared__ int32_t s_pos[kTwoBuffers ? kSliceRows : 1];
  int32_t praw[kRowsPer];
  int32_t sraw = 0;
  if constexpr (kTwoBuffers) {
    constexpr int kPer = (kSliceRows + kSparseThreads - 1) / kSparseThreads;
    int32_t v[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) v[i] = sel[min(t + kSparseThreads * i, kSliceRows - 1)];  // all issued first
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      if (t + kSparseThreads * i < kSliceRows) s_pos[t + kSparseThreads * i] = v[i];
  } else {
    // unconditional loads (a row past the round reads the round's last
    // entry, unused): a load under a branch costs a round trip of its own
#pragma unroll
    for (int i = 0; i < kRowsPer; ++i) praw[i] = sel[min(row0 + kRowStep * i, kRoundRows - 1)];
    if (FP8) sraw = sel[srow];
  }
  if (count == 0) {  // uniform: an empty sequence has zero outputs
    if (SLICES == 1)
      for (int layer = layer0; layer < layer0 + nlay; ++layer) {
        float* out = p.out + (static_cast<size_t>(layer) * p.batch + b) * kHeads * kDim;
        for (int i = t; i < kHeads * kDim; i += kSparseThreads) out[i] = 0.f;
      }
    return;
  }
  if (s0 >= count) return;  // uniform: the merge reads only slices with rows
  const int rows_valid = min(count - s0, kSliceRows);
  const int rounds = (rows_valid + kRoundRows - 1) / kRoundRows;

  const uint8_t* __restrict__ kbase = p.k + kvb * kRowBytes;
  const uint8_t* __restrict__ vbase = p.v + kvb * kRowBytes;
  const float* __restrict__ ksb = FP8 ? p.k_scale + kvb : nullptr;
  const float* __restrict__ vsb = FP8 ? p.v_scale + kvb : nullptr;
  if constexpr (kTwoBuffers) __syncthreads();  // s_pos

  // Positions are clamped into the sequence: rows past `count` read a valid
  // row and are masked out in the tile step.  A thread's loads go in row
  // order (K and V of a row together), so the rows of the round's first half
  // (tiles 0..4) land first.
  struct Gather {
    u32x4 k[kRowsPer], v[kRowsPer];
    float sc;
  };
  auto position = [&](int r, int row, int i) {  // selected position of row `row` of round r
    return kTwoBuffers ? s_pos[r * kRoundRows + row] : (i < 0 ? sraw : praw[i]);
  };
  auto gather_issue = [&](int r, Gather& gr) {
    if constexpr (FP8) {
      if (t < 2 * kRoundRows) {
        const uint32_t pos = static_cast<uint32_t>(min(max(position(r, srow, -1), 0), len - 1));
        gr.sc = t < kRoundRows ? ksb[pos] : vsb[pos];
      }
    }
#pragma unroll
    for (int i = 0; i < kRowsPer; ++i) {
      // One round: every load issued (a row past the round repeats the last
      // and is not stored), so the waits for the first half are exact.
      if (kTwoBuffers && row0 + kRowStep * i >= kRoundRows) continue;
      const int row = min(row0 + kRowStep * i, kRoundRows - 1);
      const uint32_t pos = static_cast<uint32_t>(min(max(position(r, row, i), 0), len - 1)) * kRowBytes + piece * 16;
      gr.k[i] = *reinterpret_cast<const u32x4*>(kbase + pos);
      gr.v[i] = *reinterpret_cast<const u32x4*>(vbase + pos);
    }
  };
  // Stores the thread's pieces of rows [lo, hi) (and, with lo == 0, the scales).
  auto gather_store = [&](int buf, const Gather& gr, int lo, int hi) {
    uint8_t* dst = s_raw + buf * kBufBytes + piece * 16;
    if constexpr (FP8) {
      if (lo == 0) {
        if (t < kRoundRows) s_ks[buf][t] = gr.sc;
        else if (t < 2 * kRoundRows) s_vs[buf][t - kRoundRows] = gr.sc;
      }
    }
#pragma unroll
    for (int i = 0; i < kRowsPer; ++i) {
      const int row = row0 + kRowStep * i;
      if (row >= lo && row < hi) {
        *reinterpret_cast<u32x4*>(dst + row * kLdsRow) = gr.k[i];
        *reinterpret_cast<u32x4*>(dst + (kRoundRows + row) * kLdsRow) = gr.v[i];
      }
    }
  };

  // The group's queries, fp32 [layer][16][128], loaded once for all its
  // virtual waves and issued ahead of the rows.
  constexpr int kQVecs = kQBytes / 16 / kSparseThreads;  // 4 float4 per thread
  float4 qv[kQVecs];
  {
    const float* qsrc = p.q_sparse + (static_cast<size_t>(layer0) * p.batch + b) * kHeads * kDim;
#pragma unroll
    for (int i = 0; i < kQVecs; ++i) {
      const int e = 4 * (t + kSparseThreads * i);  // element of [layer][head][dim]
      const int layer = min(e / (kHeads * kDim), nlay - 1);  // a layer past the group repeats the last (unused)
      qv[i] = *reinterpret_cast<const float4*>(qsrc + static_cast<size_t>(layer) * p.batch * kHeads * kDim +
                                               e % (kHeads * kDim));
    }
  }
  Gather gr;
  gather_issue(0, gr);
#pragma unroll
  for (int i = 0; i < kQVecs; ++i) reinterpret_cast<float4*>(s_q)[t + kSparseThreads * i] = qv[i];
  // One round: the first half's rows are computed while the second half's
  // are still arriving.  Several rounds: whole rounds, the next one's loads
  // in flight while the current one is computed.
  constexpr int kHalfRows = 5 * 16;
  gather_store(0, gr, 0, kTwoBuffers ? kRoundRows : kHalfRows);
  __syncthreads();
  QRegs q;
  SoftmaxState st;
  softmax_init(st);
  if (active) {
    QRaw qr;
    load_qraw<FP8>(s_q + ((vw >> 1) * kHeads + n) * kDim, g, qr);  // LDS reads
    qregs_from(qr, p.qscale, q);
  }
  if (kTwoBuffers) __syncthreads();  // the queries' room is the second buffer

  // A virtual wave's NT tiles (parity + 2 * (i0 + i)) of round r from LDS
  // buffer `buf`, in one multi-tile step.
  auto steps = [&](auto nt_tag, int buf, int r, int i0) {
    constexpr int NT = decltype(nt_tag)::value;
    const int parity = vw & 1;
    const uint8_t* bb = s_raw + buf * kBufBytes;
    bf16x8 kf[NT][4];
    float ks[NT][4];
    int nvalid[NT];
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const int tile = parity + 2 * (i0 + i);
      nvalid[i] = rows_valid - r * kRoundRows - 16 * tile;
      const uint8_t* kt = bb + (16 * tile + n) * kLdsRow;
      if constexpr (FP8) {
        const u32x4 k0 = *reinterpret_cast<const u32x4*>(kt + kload_offset(0, g));
        const u32x4 k1 = *reinterpret_cast<const u32x4*>(kt + kload_offset(1, g));
        e4m3x16_to_bf16(k0, kf[i][0], kf[i][1]);
        e4m3x16_to_bf16(k1, kf[i][2], kf[i][3]);
      } else {
#pragma unroll
        for (int s = 0; s < 4; ++s) kf[i][s] = as_bf16x8(*reinterpret_cast<const u32x4*>(kt + kload_offset(s, g)));
      }
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) ks[i][rr] = FP8 ? s_ks[buf][16 * tile + 4 * g + rr] : 1.f;
    }
    attend_tiles<FP8, NT, kSparseQParts>(q, kf, ks, nvalid, g, st, [&](int i, u32x4(&vraw)[4], float(&vs)[4]) {
      const int tile = parity + 2 * (i0 + i);
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int row = 16 * tile + 4 * g + rr;
        const uint8_t* vt = bb + (kRoundRows + row) * kLdsRow;
        if constexpr (FP8) {
          const u32x2 w = *reinterpret_cast<const u32x2*>(vt + 8 * n);
          vraw[rr] = u32x4{w[0], w[1], 0u, 0u};
          vs[rr] = s_vs[buf][row];
        } else {
          vraw[rr] = *reinterpret_cast<const u32x4*>(vt + 16 * n);
          vs[rr] = 1.f;
        }
      }
    });
  };
  // Of a round's nine tiles the even virtual wave takes 0, 2, 4 | 6, 8 and
  // the odd one 1, 3 | 5, 7: the first group lies in the first half (rows
  // 0..79), the second in the second; a group whose first tile has no row is
  // skipped (nor then have its others).
  auto first_group = [&](int buf, int r) {
    if (active && rows_valid - r * kRoundRows - 16 * (vw & 1) > 0) {
      if ((vw & 1) == 0) steps(std::integral_constant<int, 3>{}, buf, r, 0);
      else steps(std::integral_constant<int, 2>{}, buf, r, 0);
    }
  };
  auto second_group = [&](int buf, int r) {
    const int left = rows_valid - r * kRoundRows - 16 * (vw & 1);
    if (active) {
      if ((vw & 1) == 0) {
        if (left > 16 * 6) steps(std::integral_constant<int, 2>{}, buf, r, 3);
      } else {
        if (left > 16 * 4) steps(std::integral_constant<int, 2>{}, buf, r, 2);
      }
    }
  };

  if constexpr (!kTwoBuffers) {
    first_group(0, 0);
    gather_store(0, gr, kHalfRows, kRoundRows);
    __syncthreads();
    second_group(0, 0);
    __syncthreads();
  } else {
    for (int r = 0; r < rounds; ++r) {  // uniform
      const int buf = r & 1;
      if (r + 1 < rounds) gather_issue(r + 1, gr);  // in flight while this round is computed
      first_group(buf, r);
      second_group(buf, r);
      if (r + 1 < rounds) gather_store(buf ^ 1, gr, 0, kRoundRows);
      __syncthreads();
    }
  }

  // The odd virtual wave of each layer hands its state to the even one.
  float* s_merge = reinterpret_cast<float*>(s_raw);  // [layer of the group][kMergeLaneFloats][64]
  if (active && (vw & 1)) {
    float* dst = s_merge + (vw >> 1) * kMergeLaneFloats * 64 + lane;
    dst[0] = st.m;
    dst[64] = st.z;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[(2 + 4 * j + i) * 64] = st.o[j][i];
    }
  }
  // The even virtual wave of each layer: the layer's state of the slice,
  // merged with the odd one's, written as the output (one slice) or as the
  // slice's partial.
  auto write_layer = [&]() {
    const int layer = layer0 + (vw >> 1);
    const float* src = s_merge + (vw >> 1) * kMergeLaneFloats * 64 + lane;
    const float m0 = st.m, m1 = src[0];
    const float mx = fmaxf(m0, m1);
    const float f0 = m0 == -INFINITY ? 0.f : exp2f(m0 - mx);
    const float f1 = m1 == -INFINITY ? 0.f : exp2f(m1 - mx);
    const float z = reduce_z(st.z * f0 + src[64] * f1);
    f32x4 o[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
#pragma unroll
      for (int i = 0; i < 4; ++i) o[j][i] = st.o[j][i] * f0 + src[(2 + 4 * j + i) * 64] * f1;
    }
    // lane (n, g) holds O[head n][dim 32 g + 8 i + j] in o[j][i]
    if (SLICES == 1) {
      float* out = p.out + ((static_cast<size_t>(layer) * p.batch + b) * kHeads + n) * kDim + 32 * g;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        *reinterpret_cast<float4*>(out + 8 * i) = make_float4(o[0][i] / z, o[1][i] / z, o[2][i] / z, o[3][i] / z);
        *reinterpret_cast<float4*>(out + 8 * i + 4) = make_float4(o[4][i] / z, o[5][i] / z, o[6][i] / z, o[7][i] / z);
      }
    } else {
      float* part = p.partials + ((static_cast<size_t>(layer) * p.batch + b) * SLICES + slice) * kPartialFloats;
      if (g == 0) {
        part[n] = mx;
        part[kHeads + n] = z;
      }
      float* po = part + 2 * kHeads + n * kDim + 32 * g;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        *reinterpret_cast<float4*>(po + 8 * i) = make_float4(o[0][i], o[1][i], o[2][i], o[3][i]);
        *reinterpret_cast<float4*>(po + 8 * i + 4) = make_float4(o[4][i], o[5][i], o[6][i], o[7][i]);
      }
    }
  };
  __syncthreads();
  if (active && !(vw & 1)) write_layer();
}


// One workgroup per (sequence, layer): thread t takes head t / 16, dims 8 (t % 16) ..
template <int SLICES>
__global__ __launch_bounds__(256) void sparse_slice_merge_kernel(SparseParams p) {
  merge_slices<SLICES>(p, blockIdx.x, blockIdx.y, used_slices<SLICES>(p, blockIdx.x), threadIdx.x >> 4,
                       (threadIdx.x & 15) * 8);
}

template <bool FP8, int SLICES>
static void launch_reuse(const SparseParams& p, hipStream_t s) {
  const int groups = (p.n_layers + kGroupLayers - 1) / kGroupLayers;
  const dim3 grid(static_cast<unsigned>(p.batch * SLICES * groups));
  hipLaunchKernelGGL((sparse_reuse_kernel<FP8, SLICES>), grid, dim3(kSparseThreads), 0, s, p, groups);
  if constexpr (SLICES > 1)
    hipLaunchKernelGGL((sparse_slice_merge_kernel<SLICES>), dim3(p.batch, p.n_layers), dim3(256), 0, s, p);
}

template <bool FP8>
static void launch_reuse_fp(const SparseParams& p, int slices, hipStream_t s) {
  switch (slices) {
    case 8: launch_reuse<FP8, 8>(p, s); break;
    case 4: launch_reuse<FP8, 4>(p, s); break;
    case 2: launch_reuse<FP8, 2>(p, s); break;
    default: launch_reuse<FP8, 1>(p, s); break;
  }
}

hipError_t launch_sparse_attend(const SparseParams& p, bool fp8, hipStream_t s) {
  if (p.batch == 0 || p.n_layers == 0) return hipSuccess;
  if (p.n_layers > kSparseWaves || p.budget != kBudget) return hipErrorInvalidValue;
  const int slices = sparse_slices(p.batch);
  if (slices > 1 && p.partials == nullptr) return hipErrorInvalidValue;
  if (fp8)
    launch_reuse_fp<true>(p, slices, s);
  else
    launch_reuse_fp<false>(p, slices, s);
  return hipGetLastError();
}

// ---- window mode ---------------------------------------------------------------
// Eight waves, each taking 16 * TILES consecutive window slots straight into
// registers (16-byte loads, a two-tile ring) with the full layer's tile step;
// the waves' (m, z, O) merged through LDS.
template <bool FP8, int TILES>
__global__ __launch_bounds__(kSparseThreads) void sparse_window_kernel(SparseParams p) {
  constexpr int kWaveRows = 16 * TILES;
  constexpr int kSliceRows = kSparseWaves * kWaveRows;
  __shared__ int32_t s_pos[kSliceRows];
  __shared__ float s_m[kSparseWaves][kHeads];
  __shared__ float s_z[kSparseWaves][kHeads];
  __shared__ __attribute__((aligned(16))) float s_o[kSparseWaves][kHeads][kDim];
  constexpr int kRowBytes = FP8 ? kDim : 2 * kDim;

  // Consecutive workgroups go to one XCD (workgroup id i runs on XCD i % 8).
  const int items = p.batch;
  const int per_xcd = (items + 7) / 8;
  const int b = static_cast<int>(blockIdx.x & 7) * per_xcd + static_cast<int>(blockIdx.x >> 3);
  if (b >= items) return;  // uniform
  const int t = threadIdx.x;
  const int64_t positions = max<int64_t>(p.lengths[b], 0);
  const int64_t base = static_cast<int64_t>(b) * p.budget;
  const int count = static_cast<int>(min<int64_t>(positions, p.budget));
  // the ring slot of the current token, read from the caller's rows
  const int new_slot = p.k_new && positions > 0 ? static_cast<int>((positions - 1) % p.budget) : -1;
  if (count == 0) {  // uniform: an empty sequence has a zero output
    float* out = p.out + static_cast<size_t>(b) * kHeads * kDim;
    for (int i = t; i < kHeads * kDim; i += kSparseThreads) out[i] = 0.f;
    return;
  }
  // Slots past `count` repeat the last one and are masked out in the tile step.
  for (int i = t; i < kSliceRows; i += kSparseThreads) s_pos[i] = min(i, count - 1);
  if (new_slot >= 0 && t < kRowBytes / 4) {  // store the current rows into the ring (nothing here reads that slot)
    const size_t at = (static_cast<size_t>(base) + new_slot) * kRowBytes / 4 + t;
    reinterpret_cast<uint32_t*>(p.ring_k)[at] = reinterpret_cast<const uint32_t*>(p.k_new)[b * kRowBytes / 4 + t];
    reinterpret_cast<uint32_t*>(p.ring_v)[at] = reinterpret_cast<const uint32_t*>(p.v_new)[b * kRowBytes / 4 + t];
    if (FP8 && t == 0) {
      p.ring_ks[base + new_slot] = p.k_new_scale[b];
      p.ring_vs[base + new_slot] = p.v_new_scale[b];
    }
  }
  __syncthreads();

  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);  // wave-uniform
  const int lane = t & 63;
  const int n = lane & 15;
  const int g = lane >> 4;
  const int r0 = wave * kWaveRows;
  const int rows = min(max(count - r0, 0), kWaveRows);
  const int last = count - 1;
  const uint8_t* __restrict__ kbase = p.k + base * kRowBytes;
  const uint8_t* __restrict__ vbase = p.v + base * kRowBytes;
  const float* __restrict__ ksb = FP8 ? p.k_scale + base : nullptr;
  const float* __restrict__ vsb = FP8 ? p.v_scale + base : nullptr;

  struct Raw {
    u32x4 k[FP8 ? 2 : 4];
    u32x4 v[4];
    float ks[4], vs[4];
  };
  // Tile t: K lane (n, g) holds slot r0 + 16t + n at row bytes kload_offset(j, g);
  // V lane (n, g) holds slot r0 + 16t + 4g + r, dims 8n .. 8n + 7.
  auto load_tile = [&](int tile, Raw& raw) {
    const int i0 = r0 + 16 * tile;
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
  };

  SoftmaxState st;
  softmax_init(st);
  if (rows > 0) {  // uniform over the wave
    // The query's loads go first: a wait for data counts loads in issue
    // order, so a query loaded after the first two tiles would hold the
    // first step until the second tile had arrived too.
    QRaw qr;
    load_qraw<FP8>(p.q_sparse + (static_cast<size_t>(b) * kHeads + n) * kDim, g, qr);
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
  float* out = p.out + static_cast<size_t>(b) * kHeads * kDim;
  *reinterpret_cast<float4*>(out + h * kDim + d0) = make_float4(acc[0] / zz, acc[1] / zz, acc[2] / zz, acc[3] / zz);
}

template <bool FP8, int TILES>
static void launch_window_tiles(const SparseParams& p, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(8 * ((p.batch + 7) / 8)));
  hipLaunchKernelGGL((sparse_window_kernel<FP8, TILES>), grid, dim3(kSparseThreads), 0, s, p);
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

}  // namespace hs2
