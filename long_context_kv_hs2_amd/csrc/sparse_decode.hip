// Sparse-attention layers of a hybrid block at decode (KV Reuse).
//
// The sparse layers own no KV: they read the full layer's shared cache at the
// positions the full layer selected, and every sparse layer of the block reuses
// the same list (toolnavs.com article 2080, section "Ce que fait HySparse2";
// "Luo Fuli Teases Xiaomi MiMo-V3 Architecture", paragraphs on KV Reuse and on
// token selection).  Each layer takes its softmax over the selected positions.
//
// One workgroup per (sequence, slice of 128 selected positions) gathers those
// K and V rows from HBM into LDS once; its four waves then serve the sparse
// layers (wave w takes layers w, w+4, ...), all 16 heads at a time, with the
// same MFMA tile step as the full layer.  Split partials are merged after.
#include "hs2_device.h"
#include "hs2_internal.h"

namespace hs2 {

template <bool FP8>
__global__ __launch_bounds__(256) void sparse_partial_kernel(SparseParams p) {
  constexpr int kRowBytes = FP8 ? kDim : 2 * kDim;
  constexpr int kPitch = kRowBytes + 16;  // pad rows so the 16 row reads of a K fragment spread over banks
  __shared__ __attribute__((aligned(16))) uint8_t s_k[kSparseRows * kPitch];
  __shared__ __attribute__((aligned(16))) uint8_t s_v[kSparseRows * kPitch];
  __shared__ float s_ks[kSparseRows];
  __shared__ float s_vs[kSparseRows];

  const int split = blockIdx.x;
  const int b = blockIdx.y;
  int64_t base;
  int len;
  seq_bounds(p.seq_offsets, b, p.total_tokens, p.max_context, base, len);
  const int count = clamp_count(p.sel_count[b], len, p.budget);
  const int r0 = split * kSparseRows;
  if (r0 >= count) return;  // uniform
  const int rows = min(kSparseRows, count - r0);
  const int32_t* sel = p.sel_idx + static_cast<size_t>(b) * p.budget + r0;

  // Gather: rows past `rows` copy the last valid row (masked out later).  All
  // of a thread's loads are issued before any is stored to LDS.
  constexpr int kChunks = kRowBytes / 16;
  constexpr int kPer = kSparseRows * kChunks / 256;
  u32x4 kv[kPer], vv[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int c = threadIdx.x + 256 * i;
    const int row = c / kChunks;
    const int part = c % kChunks;
    const int64_t pos = base + min(max(sel[min(row, rows - 1)], 0), len - 1);
    kv[i] = *reinterpret_cast<const u32x4*>(p.k + pos * kRowBytes + 16 * part);
    vv[i] = *reinterpret_cast<const u32x4*>(p.v + pos * kRowBytes + 16 * part);
  }
  float ksc = 1.f, vsc = 1.f;
  if constexpr (FP8) {
    if (threadIdx.x < kSparseRows) {
      const int64_t pos = base + min(max(sel[min(static_cast<int>(threadIdx.x), rows - 1)], 0), len - 1);
      ksc = p.k_scale[pos];
      vsc = p.v_scale[pos];
    }
  }
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int c = threadIdx.x + 256 * i;
    const int row = c / kChunks;
    const int part = c % kChunks;
    *reinterpret_cast<u32x4*>(s_k + row * kPitch + 16 * part) = kv[i];
    *reinterpret_cast<u32x4*>(s_v + row * kPitch + 16 * part) = vv[i];
  }
  if constexpr (FP8) {
    if (threadIdx.x < kSparseRows) {
      s_ks[threadIdx.x] = ksc;
      s_vs[threadIdx.x] = vsc;
    }
  }
  __syncthreads();

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform: scalar loop control
  const int lane = threadIdx.x & 63;
  const int n = lane & 15;
  const int g = lane >> 4;
  for (int layer = wave; layer < p.n_layers; layer += 4) {
    QRegs q;
    load_qregs<FP8>(p.q_sparse + ((static_cast<size_t>(layer) * p.batch + b) * kHeads + n) * kDim, p.qscale, g, q);
    SoftmaxState st;
    softmax_init(st);
    for (int t0 = 0; t0 < rows; t0 += 16) {
      const int nv = min(16, rows - t0);
      bf16x8 kf[4];
      const uint8_t* krow = s_k + (t0 + n) * kPitch;
      if constexpr (FP8) {
        e4m3x16_to_bf16(*reinterpret_cast<const u32x4*>(krow + kload_offset(0, g)), kf[0], kf[1]);
        e4m3x16_to_bf16(*reinterpret_cast<const u32x4*>(krow + kload_offset(1, g)), kf[2], kf[3]);
      } else {
#pragma unroll
        for (int s = 0; s < 4; ++s) kf[s] = as_bf16x8(*reinterpret_cast<const u32x4*>(krow + kload_offset(s, g)));
      }
      u32x4 vraw[4];
      float ks[4], vs[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = t0 + 4 * g + r;
        if constexpr (FP8) {
          const u32x2 w = *reinterpret_cast<const u32x2*>(s_v + row * kPitch + 8 * n);
          vraw[r] = u32x4{w[0], w[1], 0u, 0u};
          ks[r] = s_ks[row];
          vs[r] = s_vs[row];
        } else {
          vraw[r] = *reinterpret_cast<const u32x4*>(s_v + row * kPitch + 16 * n);
          ks[r] = 1.f;
          vs[r] = 1.f;
        }
      }
      float lg[4], pr[4];
      attend_tile<FP8>(q, kf, vraw, ks, vs, nv, g, st, lg, pr);
    }
    const float z = reduce_z(st.z);
    float* out = p.partials + ((static_cast<size_t>(b) * p.n_layers + layer) * p.splits + split) * kPartialFloats;
    if (g == 0) {
      out[n] = st.m;
      out[kHeads + n] = z;
    }
    // lane (n, g) holds O[head n][dims 32g .. 32g + 31] as o[t][i] -> dim 32g + 8i + t
    float* orow = out + 2 * kHeads + n * kDim + 32 * g;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float4* o4 = reinterpret_cast<float4*>(orow + 8 * i);
      o4[0] = make_float4(st.o[0][i], st.o[1][i], st.o[2][i], st.o[3][i]);
      o4[1] = make_float4(st.o[4][i], st.o[5][i], st.o[6][i], st.o[7][i]);
    }
  }
}

hipError_t launch_sparse_partial(const SparseParams& p, bool fp8, hipStream_t s) {
  if (p.batch == 0 || p.n_layers == 0) return hipSuccess;
  const dim3 grid(p.splits, p.batch);
  if (fp8)
    hipLaunchKernelGGL(sparse_partial_kernel<true>, grid, dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(sparse_partial_kernel<false>, grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace hs2
