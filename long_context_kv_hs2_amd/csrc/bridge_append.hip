// Decode-time KV Bridging: each decode step, the current token's shared
// hidden state is projected by every bridged layer's own W_k and W_v, and the
// results are written into those layers' caches at the token's row (the same
// projection as the prefill bridge, one row per sequence: toolnavs.com
// article 2080 (ko), section "HySparse2가 한 일"; "Luo Fuli Teases Xiaomi
// MiMo-V3 Architecture", paragraph on KV Bridging).
//
// A [B x d_model] . [d_model x 128] product per output matrix is too small for
// the prefill GEMM's tiles, and what it must move is the weights (2 * n_bridged
// x d_model x 128 bf16, 6.3 MB at d_model 4096 and 3 layers): split-K.
//   bridge_append_partial_kernel  one workgroup per (row group of 64
//     sequences, output matrix, 128-deep slice of d_model): the weight slice
//     (32 KB) is staged in LDS with 16-byte loads, all in flight at once; four waves each take 32 of
//     the 128 columns over the whole slice on v_mfma_f32_16x16x32_bf16, so no
//     wave-to-wave reduction is needed; the fp32 partial sums go to the
//     workspace.
//   bridge_append_finish_kernel  one workgroup per (sequence, matrix): sums
//     the slices' partials in slice order (the same bits every run), rounds to
//     bf16 or quantises the row to E4M3 with its per-token scale (row max / 448,
//     the prefill bridge's rule), and writes row seq_offsets[b + 1] - 1.
#include "hs2_device.h"
#include "hs2_internal.h"

namespace hs2 {

namespace {

constexpr int kRowGroup = 64;  // sequences per partial workgroup (4 row tiles of 16)
constexpr int kWPitch = kDim + 8;  // LDS row pitch of the weight slice, in bf16 elements

template <int RT>
__global__ __launch_bounds__(256) void bridge_append_partial_kernel(AppendParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t s_w[kAppendSliceK * kWPitch];
  const int k_slices = p.d_model / kAppendSliceK;
  const int ks = blockIdx.x % k_slices;
  const int mat = (blockIdx.x / k_slices) % p.n_out;
  const int r0 = (blockIdx.x / (k_slices * p.n_out)) * kRowGroup;
  const int k0 = ks * kAppendSliceK;
  const uint16_t* w = p.w[mat];
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int n = lane & 15;
  const int g = lane >> 4;
  // The hidden rows' fragments for the whole slice, loaded before the weights
  // so both are in flight together.
  constexpr int kSteps = kAppendSliceK / 32;
  u32x4 ha[kSteps][RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int row = min(r0 + 16 * rt + n, p.batch - 1);  // rows past the batch compute, and are not written
    const uint16_t* hrow = p.hidden + static_cast<size_t>(row) * p.d_model + k0 + 8 * g;
#pragma unroll
    for (int st = 0; st < kSteps; ++st) ha[st][rt] = *reinterpret_cast<const u32x4*>(hrow + 32 * st);
  }
  constexpr int kLoads = kAppendSliceK * (kDim / 8) / 256;  // 16-byte loads per thread, all in flight at once
  u32x4 staged[kLoads];
#pragma unroll
  for (int j = 0; j < kLoads; ++j) {
    const int c = threadIdx.x + 256 * j;
    staged[j] = *reinterpret_cast<const u32x4*>(w + static_cast<size_t>(k0 + (c >> 4)) * kDim + (c & 15) * 8);
  }
#pragma unroll
  for (int j = 0; j < kLoads; ++j) {
    const int c = threadIdx.x + 256 * j;
    *reinterpret_cast<u32x4*>(&s_w[(c >> 4) * kWPitch + (c & 15) * 8]) = staged[j];
  }
  __syncthreads();
  f32x4 acc[RT][2];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) acc[rt][0] = acc[rt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int st = 0; st < kSteps; ++st) {
    const int kk = 32 * st;
    bf16x8 a[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) a[rt] = as_bf16x8(ha[st][rt]);
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      const int col = wave * 32 + ct * 16 + n;
      uint32_t v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        v[j] = static_cast<uint32_t>(s_w[(kk + 8 * g + 2 * j) * kWPitch + col]) |
               (static_cast<uint32_t>(s_w[(kk + 8 * g + 2 * j + 1) * kWPitch + col]) << 16);
      const bf16x8 bfrag = as_bf16x8(u32x4{v[0], v[1], v[2], v[3]});
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) acc[rt][ct] = mfma_bf16_16x16x32(a[rt], bfrag, acc[rt][ct]);
    }
  }
  // Fragment (rt, ct): lane (n, g) holds D[row 4g + e][column n].
  const int width = p.n_out * kDim;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = r0 + 16 * rt + 4 * g + e;
        if (row < p.batch)
          p.partials[(static_cast<size_t>(ks) * p.batch + row) * width + mat * kDim + wave * 32 + ct * 16 + n] =
              acc[rt][ct][e];
      }
}

template <bool FP8>
__global__ __launch_bounds__(kDim) void bridge_append_finish_kernel(AppendParams p) {
  __shared__ float s_max[2];
  const int mat = blockIdx.x % p.n_out;
  const int b = blockIdx.x / p.n_out;
  const int c = threadIdx.x;
  int64_t base;
  int len;
  seq_bounds(p.seq_offsets, b, p.total_tokens, p.total_tokens, base, len);
  if (len == 0) return;  // an empty sequence has no current token
  const int64_t row = base + len - 1;
  const int k_slices = p.d_model / kAppendSliceK;
  const int width = p.n_out * kDim;
  const float* src = p.partials + static_cast<size_t>(b) * width + mat * kDim + c;
  const size_t stride = static_cast<size_t>(p.batch) * width;
  // slices in order, loaded 32 at a time (all of them for d_model 4096)
  float v = 0.f;
  for (int k0 = 0; k0 < k_slices; k0 += 32) {
    float part[32];
#pragma unroll
    for (int j = 0; j < 32; ++j) part[j] = k0 + j < k_slices ? src[(k0 + j) * stride] : 0.f;
#pragma unroll
    for (int j = 0; j < 32; ++j) v += part[j];
  }
  if constexpr (FP8) {
    float a = fabsf(v);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) a = fmaxf(a, __shfl_xor(a, off));
    if ((c & 63) == 0) s_max[c >> 6] = a;
    __syncthreads();
    a = fmaxf(s_max[0], s_max[1]);
    const float scale = a > 0.f ? a / 448.f : 1.f;
    static_cast<uint8_t*>(p.out[mat])[row * kDim + c] = static_cast<uint8_t>(f32_to_e4m3_rne_sat(v / scale));
    if (c == 0) p.scale[mat][row] = scale;
  } else {
    static_cast<uint16_t*>(p.out[mat])[row * kDim + c] = static_cast<uint16_t>(bf16_rne(v));
  }
}

}  // namespace

hipError_t launch_bridge_append(const AppendParams& p, hipStream_t s) {
  if (p.batch <= 0) return hipSuccess;
  const int k_slices = p.d_model / kAppendSliceK;
  const int row_groups = (p.batch + kRowGroup - 1) / kRowGroup;
  const dim3 grid(static_cast<unsigned>(row_groups * p.n_out * k_slices));
  if (p.batch <= 16)
    hipLaunchKernelGGL(bridge_append_partial_kernel<1>, grid, dim3(256), 0, s, p);
  else if (p.batch <= 32)
    hipLaunchKernelGGL(bridge_append_partial_kernel<2>, grid, dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(bridge_append_partial_kernel<4>, grid, dim3(256), 0, s, p);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  const dim3 fgrid(static_cast<unsigned>(p.batch * p.n_out));
  if (p.fp8)
    hipLaunchKernelGGL(bridge_append_finish_kernel<true>, fgrid, dim3(kDim), 0, s, p);
  else
    hipLaunchKernelGGL(bridge_append_finish_kernel<false>, fgrid, dim3(kDim), 0, s, p);
  return hipGetLastError();
}

}  // namespace hs2
