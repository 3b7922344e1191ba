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
// registers, and O^T += V^T P^T on fp32 MFMA (fp32 probabilities).  The four
// waves' (m, z, O) are merged through LDS into one partial per workgroup.
#include "hs2_device.h"
#include "hs2_internal.h"

namespace hs2 {

template <bool FP8>
__global__ __launch_bounds__(256) void full_partial_kernel(FullParams p) {
  __shared__ float s_m[4][kHeads];
  __shared__ float s_z[4][kHeads];
  __shared__ float s_o[4][kHeads][kDim];

  const int b = blockIdx.y;
  const int c = blockIdx.x;
  int64_t base;
  int len;
  seq_bounds(p.seq_offsets, b, p.total_tokens, p.max_context, base, len);
  const int c0 = c * p.chunk;
  if (c0 >= len) return;  // uniform over the workgroup
  const int c1 = min(len, c0 + p.chunk);

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int n = lane & 15;
  const int g = lane >> 4;
  const int sub = p.chunk >> 2;
  const int w0 = c0 + wave * sub;
  const int w1 = min(c1, w0 + sub);

  QFrag q;
  load_qfrag(p.q + (static_cast<size_t>(b) * kHeads + n) * kDim, p.qscale, g, q);

  constexpr int kRowBytes = FP8 ? kDim : 2 * kDim;
  const uint8_t* kbase = p.k + base * kRowBytes;
  const uint8_t* vbase = p.v + base * kRowBytes;
  float* spill = p.spill + base * kHeads;

  SoftmaxState st;
  softmax_init(st);

  // Raw tile registers: K lane (n, g) holds token t0 + n, bytes of dims
  // 32g .. 32g + 31; V lane (n, g) holds token t0 + 4g + r, dims 8n .. 8n + 7.
  // Rows past the end are clamped to a valid row and masked out in the tile step.
  struct Raw {
    u32x4 k[4];
    u32x4 v[4];
    float ks[4], vs[4];
  };
  auto load_tile = [&](int t0, Raw& raw) {
    const int nv = min(16, w1 - t0);
    const int tk = t0 + min(n, nv - 1);
    if constexpr (FP8) {
      const u32x4* src = reinterpret_cast<const u32x4*>(kbase + static_cast<size_t>(tk) * kRowBytes + 32 * g);
      raw.k[0] = src[0];
      raw.k[1] = src[1];
    } else {
      const u32x4* src = reinterpret_cast<const u32x4*>(kbase + static_cast<size_t>(tk) * kRowBytes + 64 * g);
#pragma unroll
      for (int s = 0; s < 4; ++s) raw.k[s] = src[s];
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tv = t0 + min(4 * g + r, nv - 1);
      if constexpr (FP8) {
        const u32x2 w = *reinterpret_cast<const u32x2*>(vbase + static_cast<size_t>(tv) * kRowBytes + 8 * n);
        raw.v[r] = u32x4{w[0], w[1], 0u, 0u};
        raw.ks[r] = p.k_scale[base + tv];
        raw.vs[r] = p.v_scale[base + tv];
      } else {
        raw.v[r] = *reinterpret_cast<const u32x4*>(vbase + static_cast<size_t>(tv) * kRowBytes + 16 * n);
        raw.ks[r] = 1.f;
        raw.vs[r] = 1.f;
      }
    }
  };

  Raw cur, nxt;
  if (w0 < w1) load_tile(w0, cur);
  for (int t0 = w0; t0 < w1; t0 += 16) {
    const int nv = min(16, w1 - t0);
    if (t0 + 16 < w1) load_tile(t0 + 16, nxt);  // in flight during this tile's math
    bf16x8 kf[4];
    if constexpr (FP8) {
      e4m3x16_to_bf16(cur.k[0], kf[0], kf[1]);
      e4m3x16_to_bf16(cur.k[1], kf[2], kf[3]);
    } else {
#pragma unroll
      for (int s = 0; s < 4; ++s) kf[s] = as_bf16x8(cur.k[s]);
    }
    float vf[4][8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if constexpr (FP8)
        e4m3x8_to_f32(u32x2{cur.v[r][0], cur.v[r][1]}, vf[r]);
      else
        bf16x8_to_f32(cur.v[r], vf[r]);
    }
    float lg[4];
    attend_tile(q, kf, vf, cur.ks, cur.vs, nv, g, st, lg);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (4 * g + r < nv) spill[static_cast<size_t>(t0 + 4 * g + r) * kHeads + n] = lg[r];
    }
    cur = nxt;
  }

  // Merge the four waves through LDS.
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

  const int h = threadIdx.x >> 4;
  const int d0 = (threadIdx.x & 15) * 8;
  float mx = -INFINITY;
#pragma unroll
  for (int w = 0; w < 4; ++w) mx = fmaxf(mx, s_m[w][h]);
  float zz = 0.f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float mw = s_m[w][h];
    if (mw == -INFINITY) continue;  // a wave with no tokens
    const float f = exp2f(mw - mx);
    zz += s_z[w][h] * f;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] += s_o[w][h][d0 + j] * f;
  }
  float* out = p.partials + (static_cast<size_t>(b) * p.chunks_per_seq + c) * kPartialFloats;
  if ((threadIdx.x & 15) == 0) {
    out[h] = mx;
    out[kHeads + h] = zz;
  }
  float4* o4 = reinterpret_cast<float4*>(out + 2 * kHeads + h * kDim + d0);
  o4[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
  o4[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
}

hipError_t launch_full_partial(const FullParams& p, int batch, bool fp8, hipStream_t s) {
  if (batch == 0) return hipSuccess;
  const dim3 grid(p.chunks_per_seq, batch);
  if (fp8)
    hipLaunchKernelGGL(full_partial_kernel<true>, grid, dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(full_partial_kernel<false>, grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

// Merge split-K partials: per (head, sequence, layer) one workgroup of 128
// threads (one per output dim) combines the partials in a fixed order.
__global__ __launch_bounds__(128) void merge_kernel(MergeParams p, int64_t stride_layer, int64_t out_stride_layer) {
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int layer = blockIdx.z;
  const int d = threadIdx.x;
  int64_t base;
  int len;
  seq_bounds(p.seq_offsets, b, p.total_tokens, p.max_context, base, len);
  const int items = p.count_from_sel ? clamp_count(p.sel_count[b], len, p.budget) : len;
  const int count = (items + p.chunk - 1) / p.chunk;
  const float* pb = p.partials + layer * stride_layer + static_cast<int64_t>(b) * p.stride_seq;
  float mx = -INFINITY;
  for (int c = 0; c < count; ++c) mx = fmaxf(mx, pb[static_cast<int64_t>(c) * p.stride_chunk + h]);
  float z = 0.f;
  float acc = 0.f;
  for (int c = 0; c < count; ++c) {
    const float* pc = pb + static_cast<int64_t>(c) * p.stride_chunk;
    const float f = exp2f(pc[h] - mx);
    z += pc[kHeads + h] * f;
    acc += pc[2 * kHeads + h * kDim + d] * f;
  }
  float* out = p.out + layer * out_stride_layer + b * p.out_stride_seq + h * kDim;
  out[d] = count ? acc / z : 0.f;
  if (p.stats && layer == 0 && d == 0) {
    p.stats[(static_cast<int64_t>(b) * kHeads + h) * 2] = mx;
    p.stats[(static_cast<int64_t>(b) * kHeads + h) * 2 + 1] = z;
  }
}

hipError_t launch_merge(const MergeParams& p, int batch, hipStream_t s) {
  if (batch == 0) return hipSuccess;
  hipLaunchKernelGGL(merge_kernel, dim3(kHeads, batch, 1), dim3(kDim), 0, s, p, int64_t(0), int64_t(0));
  return hipGetLastError();
}

hipError_t launch_merge_layers(const MergeParams& p, int batch, int layers, int64_t stride_layer,
                               int64_t out_stride_layer, hipStream_t s) {
  if (batch == 0 || layers == 0) return hipSuccess;
  hipLaunchKernelGGL(merge_kernel, dim3(kHeads, batch, layers), dim3(kDim), 0, s, p, stride_layer,
                     out_stride_layer);
  return hipGetLastError();
}

}  // namespace hs2
