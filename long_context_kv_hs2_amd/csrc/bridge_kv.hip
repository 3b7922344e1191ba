// KV-Bridging projection: every bridged full-attention layer builds its own K
// and V from one shared self-decoder hidden state with its own projections
// (toolnavs.com article 2080 (ko), section "HySparse2가 한 일"; (fr), section
// "Ce que fait HySparse2"; "Luo Fuli Teases Xiaomi MiMo-V3 Architecture",
// paragraph on KV Bridging).  All 2 * n_bridged projections form one GEMM
//   C[T x (n_out*128)] = H[T x d_model] . [W_k0 | W_v0 | W_k1 | ...]
// on bf16 MFMA with fp32 accumulation, so H is streamed once for all of them.
//
// The weights (a few MB) are first transposed into the workspace so that both
// operands are contiguous along the reduction dim, the layout the MFMA
// fragments read.  GEMM tiles: 256 rows x 256 columns (two output matrices)
// per workgroup of eight waves, each wave 128 x 64; k-step 64; LDS double
// buffering, with the next two k-steps' global loads in flight in registers.
// A tile this large keeps each CU's operand traffic (about 30 bytes per clock
// at the MFMA peak) within what its load path delivers; 128 x 128 tiles need
// twice that.  Workgroups are ordered so the column tiles of one row block
// run back to back on the same XCD and share its L2.
#include "hs2_device.h"
#include "hs2_internal.h"

namespace hs2 {

namespace {
constexpr int kBM = 256;  // workgroup tile: 256 rows x 256 output columns
constexpr int kBN = 256;
constexpr int kBK = 64;   // k-step: two 16x16x32 MFMAs deep
constexpr int kWM = 128;  // wave tile (8 waves, 2 x 4)
constexpr int kWN = 64;
constexpr int kPitch = kBK * 2 + 16;  // bytes per LDS row (padded: 8 rows of a fragment read hit all banks)
}  // namespace

struct WeightPtrs {
  const uint16_t* w[8];
};

// W [d_model][128] (row = reduction index) -> W_t [128][d_model], 64 x 128 tiles.
__global__ __launch_bounds__(256) void transpose_w_kernel(WeightPtrs src_w, int d_model, uint16_t* w_t) {
  __shared__ uint16_t tile[64][kDim + 2];
  const int o = blockIdx.y;
  const int k0 = blockIdx.x * 64;
  const uint16_t* src = src_w.w[o];
  for (int i = threadIdx.x; i < 64 * kDim; i += blockDim.x) {
    const int r = i / kDim, c = i % kDim;
    tile[r][c] = src[static_cast<size_t>(k0 + r) * kDim + c];
  }
  __syncthreads();
  uint16_t* dst = w_t + static_cast<size_t>(o) * kDim * d_model;
  for (int i = threadIdx.x; i < 64 * kDim; i += blockDim.x) {
    const int c = i / 64, r = i % 64;
    dst[static_cast<size_t>(c) * d_model + k0 + r] = tile[r][c];
  }
}

hipError_t launch_bridge_transpose_w(const uint16_t* const* w, int n_out, int d_model, uint16_t* w_t,
                                     hipStream_t s) {
  WeightPtrs p{};
  for (int i = 0; i < n_out && i < 8; ++i) p.w[i] = w[i];
  hipLaunchKernelGGL(transpose_w_kernel, dim3(d_model / 64, n_out), dim3(256), 0, s, p, d_model, w_t);
  return hipGetLastError();
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

template <bool FP8OUT>
__global__ __launch_bounds__(512) void bridge_gemm_kernel(BridgeParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t s_a[2][kBM * kPitch];
  __shared__ __attribute__((aligned(16))) uint8_t s_b[2][kBN * kPitch];
  __shared__ float s_amax[2][2][kBM];  // E4M3 output: [matrix][half of its columns][row] partial row maxima

  // XCD-aware order: workgroup id i runs on XCD i % 8; give the column tiles
  // of one row block consecutive slots on one XCD, so they share its L2.
  const int n_ct = p.n_out * kDim / kBN;
  const int id = blockIdx.x;
  const int xcd = id & 7;
  const int slot = id >> 3;
  const int m_tiles = static_cast<int>((p.n_tokens + kBM - 1) / kBM);
  const int mt = (slot / n_ct) * 8 + xcd;
  const int ct = slot % n_ct;
  if (mt >= m_tiles) return;
  const int64_t m0 = static_cast<int64_t>(mt) * kBM;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int n = lane & 15;
  const int g = lane >> 4;
  const int wm = (wave & 1) * kWM;
  const int wn = (wave >> 1) * kWN;

  // Global -> register staging: each thread moves 4 x 16 B of A and of B per
  // k-step.  Chunk c = tid + 512 * j: row c / 8, 16-byte column c % 8.
  const uint16_t* a_src[4];
  const uint16_t* b_src[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = tid + 512 * j;
    const int row = c >> 3, col = (c & 7) * 8;
    const int64_t arow = min<int64_t>(m0 + row, p.n_tokens - 1);  // clamp the ragged last block
    a_src[j] = p.hidden + arow * p.d_model + col;
    b_src[j] = p.w_t + (static_cast<int64_t>(ct) * kBN + row) * p.d_model + col;
  }
  // Register slots for the k-steps in flight.  (k-steps past the end re-read
  // the last one: unconditional loads keep the compiler's count of loads in
  // flight exact.)
  struct Slot {
    u32x4 a[4], b[4];
  };
  const int k_steps = p.d_model / kBK;
  auto load_tile = [&](int ks, Slot& r) {
    const int k0 = min(ks, k_steps - 1) * kBK;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      r.a[j] = *reinterpret_cast<const u32x4*>(a_src[j] + k0);
      r.b[j] = *reinterpret_cast<const u32x4*>(b_src[j] + k0);
    }
  };
  auto store_tile = [&](int buf, const Slot& r) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = tid + 512 * j;
      const int row = c >> 3, colb = (c & 7) * 16;
      *reinterpret_cast<u32x4*>(&s_a[buf][row * kPitch + colb]) = r.a[j];
      *reinterpret_cast<u32x4*>(&s_b[buf][row * kPitch + colb]) = r.b[j];
    }
  };

  constexpr int kFM = kWM / 16, kFN = kWN / 16;  // 16 x 16 fragments per wave
  f32x4 acc[kFM][kFN];
#pragma unroll
  for (int i = 0; i < kFM; ++i)
#pragma unroll
    for (int j = 0; j < kFN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // One k-step of 64, as two MFMA steps of 32: lane (n, g) of fragment i holds
  // row 16i + n, k = 32 kk + 8g .. + 7.
  auto compute = [&](int buf) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      bf16x8 af[kFM], bfr[kFN];
#pragma unroll
      for (int i = 0; i < kFM; ++i)
        af[i] = as_bf16x8(*reinterpret_cast<const u32x4*>(&s_a[buf][(wm + 16 * i + n) * kPitch + kk * 64 + 16 * g]));
#pragma unroll
      for (int j = 0; j < kFN; ++j)
        bfr[j] = as_bf16x8(*reinterpret_cast<const u32x4*>(&s_b[buf][(wn + 16 * j + n) * kPitch + kk * 64 + 16 * g]));
#pragma unroll
      for (int i = 0; i < kFM; ++i)
#pragma unroll
        for (int j = 0; j < kFN; ++j) acc[i][j] = mfma_bf16_16x16x32(af[i], bfr[j], acc[i][j]);
    }
  };
  // At the top of k-step ks: LDS buffer ks & 1 holds tile ks and the two
  // register slots hold tiles ks + 1 and ks + 2 in flight.  After computing
  // tile ks, tile ks + 1 goes to the other buffer (whose readers finished at
  // the last barrier) and its slot takes tile ks + 3.  Unrolled by two so
  // each slot keeps its registers.
  Slot sa, sb;
  load_tile(0, sa);
  load_tile(1, sb);
  store_tile(0, sa);
  load_tile(2, sa);
  __syncthreads();
  for (int ks = 0;; ks += 2) {
    compute(0);
    store_tile(1, sb);
    __syncthreads();
    if (ks + 1 >= k_steps) break;
    load_tile(ks + 3, sb);
    compute(1);
    store_tile(0, sa);
    __syncthreads();
    if (ks + 2 >= k_steps) break;
    load_tile(ks + 4, sa);
  }

  // Epilogue.  Fragment (i, j) holds D[row 4g + e][col n] in lane (n, g);
  // tile column c belongs to output matrix c / 128 (two per workgroup).  The
  // rounded values are staged in LDS (the operand buffers are free: the loop
  // ended on a barrier), matrix 0 in s_a and matrix 1 in s_b, as [row][128]
  // elements, and then written out row by row with 16-byte stores.
  //   bf16: round to nearest even.
  //   E4M3: per row and matrix, scale = (largest |value|) / 448 in fp32 (1 for
  //   an all-zero row), code = E4M3(value / scale); the row maxima are reduced
  //   over the 16 lanes of a fragment row and then over the two waves that
  //   share the matrix, through LDS.
  constexpr int kElemBytes = FP8OUT ? 1 : 2;
  constexpr int kRowBytes = kDim * kElemBytes;  // staged bytes per row and matrix
  static_assert(kBM * kRowBytes <= 2 * kBM * kPitch, "one matrix of the tile fits in one operand buffer");
  const int mat = wn >> 7;         // output matrix of this wave (local: 0 or 1)
  const int half = (wn >> 6) & 1;  // which 64 of its 128 columns
  uint8_t* stage = mat == 0 ? &s_a[0][0] : &s_b[0][0];
  float scale[kFM][4];
  if constexpr (FP8OUT) {
#pragma unroll
    for (int i = 0; i < kFM; ++i) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float a = 0.f;
#pragma unroll
        for (int j = 0; j < kFN; ++j) a = fmaxf(a, fabsf(acc[i][j][e]));
#pragma unroll
        for (int off = 8; off > 0; off >>= 1) a = fmaxf(a, __shfl_xor(a, off));  // over the 16 lanes n
        if (n == 0) s_amax[mat][half][wm + 16 * i + 4 * g + e] = a;
      }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kFM; ++i) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = wm + 16 * i + 4 * g + e;
        const float a = fmaxf(s_amax[mat][0][r], s_amax[mat][1][r]);
        scale[i][e] = a > 0.f ? a / 448.f : 1.f;
        const int64_t row = m0 + r;
        if (half == 0 && n == 0 && row < p.n_tokens) p.scale[ct * (kBN / kDim) + mat][row] = scale[i][e];
      }
    }
  }
#pragma unroll
  for (int j = 0; j < kFN; ++j) {
    const int c = (wn & (kDim - 1)) + 16 * j + n;  // column within the matrix
#pragma unroll
    for (int i = 0; i < kFM; ++i) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = wm + 16 * i + 4 * g + e;
        if constexpr (FP8OUT) {
          stage[r * kRowBytes + c] = static_cast<uint8_t>(f32_to_e4m3_rne_sat(acc[i][j][e] / scale[i][e]));
        } else {
          *reinterpret_cast<uint16_t*>(stage + r * kRowBytes + 2 * c) = f32_to_bf16_rne(acc[i][j][e]);
        }
      }
    }
  }
  __syncthreads();
  constexpr int kChunks = kRowBytes / 16;  // 16-byte pieces per row
#pragma unroll
  for (int k = 0; k < 2 * kBM * kChunks / 512; ++k) {
    const int idx = tid + 512 * k;
    const int mm = idx / (kBM * kChunks);
    const int r = (idx / kChunks) % kBM;
    const int q = idx % kChunks;
    const int64_t row = m0 + r;
    if (row < p.n_tokens) {
      const uint8_t* src = (mm == 0 ? &s_a[0][0] : &s_b[0][0]) + r * kRowBytes + 16 * q;
      uint8_t* dst = reinterpret_cast<uint8_t*>(p.out[ct * (kBN / kDim) + mm]) + row * kRowBytes + 16 * q;
      *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(src);
    }
  }
}

hipError_t launch_bridge_gemm(const BridgeParams& p, hipStream_t s) {
  if (p.n_tokens == 0) return hipSuccess;
  const int64_t m_tiles = (p.n_tokens + kBM - 1) / kBM;
  const int64_t groups = (m_tiles + 7) / 8;  // row blocks per XCD, rounded up
  const int64_t blocks = groups * 8 * (p.n_out * kDim / kBN);
  if (p.fp8)
    hipLaunchKernelGGL(bridge_gemm_kernel<true>, dim3(static_cast<unsigned>(blocks)), dim3(512), 0, s, p);
  else
    hipLaunchKernelGGL(bridge_gemm_kernel<false>, dim3(static_cast<unsigned>(blocks)), dim3(512), 0, s, p);
  return hipGetLastError();
}

}  // namespace hs2
