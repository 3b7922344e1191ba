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
// per workgroup of eight waves, each wave 128 x 64; k-steps of 64 (one
// 128-byte line of every operand row).  Operands go from global memory
// straight into LDS (no register staging), two k-step buffers: one computed
// while the next is in flight, with the fragments of the next half step read
// into registers under the MFMAs of the current one.  A tile this
// large keeps each CU's operand traffic (about 30 bytes per clock at the MFMA
// peak) within what its load path delivers; 128 x 128 tiles need twice that.
// Workgroups are ordered so the column tiles of one row block run back to
// back on the same XCD and share its L2.
#include "hs2_device.h"
#include "hs2_internal.h"

namespace hs2 {

namespace {
constexpr int kBM = 256;  // workgroup tile: 256 rows x 256 output columns
constexpr int kBN = 256;
constexpr int kBK = 64;   // k-step: 128 bytes of each row, two 16x16x32 MFMAs deep
constexpr int kWM = 128;  // wave tile (8 waves, 2 x 4)
constexpr int kWN = 64;
constexpr int kRow = kBK * 2;          // bytes per LDS row of a k-step (one 128-byte line)
constexpr int kBufBytes = kBM * kRow;  // one k-step of A rows (or of B rows): 32 KB
static_assert(kBM == kBN, "A and B k-step buffers have one size");
constexpr int kBuffersA = 3;  // A k-steps in LDS: one computed, two in flight
constexpr int kBuffersB = 2;  // B k-steps in LDS: one computed, one in flight
constexpr int kLdsBytes = (kBuffersA + kBuffersB) * kBufBytes;  // 160 KB, the whole LDS of a CU
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

// LDS position of 16-byte chunk c (0..7) of an operand row r is
// c ^ swizzle(r).  A fragment read has lanes n = 0..15 on rows r0 + n (r0 a
// multiple of 16), all at one chunk; unswizzled 128-byte rows put those 16
// lanes on two bank groups.  Rotating the chunk by (r >> 1) & 7 spreads them
// over all 16 and measures as fast as a linear read on gfx950 (a
// ds_read_b128 pattern probe timed against the linear pattern).
__device__ __forceinline__ int swizzle(int r) { return (r >> 1) & 7; }

typedef __attribute__((address_space(1))) void global_void;
typedef __attribute__((address_space(3))) void lds_void;

template <bool FP8OUT>
__global__ __launch_bounds__(512) void bridge_gemm_kernel(BridgeParams p) {
  // Three A and two B k-step buffers of 32 KB (rows of 128 bytes, no padding:
  // the 16-byte chunks of row r sit at position chunk ^ swizzle(r)); the
  // epilogue stages the outputs and the E4M3 row maxima in the same room.
  __shared__ __attribute__((aligned(16))) uint8_t s_raw[kLdsBytes];
  uint8_t* const s_a = s_raw;
  uint8_t* const s_b = s_raw + kBuffersA * kBufBytes;

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
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int n = lane & 15;
  const int g = lane >> 4;
  const int wm = (wave & 1) * kWM;
  const int wn = (wave >> 1) * kWN;

  // Direct global -> LDS loads: a wave instruction moves 8 rows x 128 bytes
  // (whole cache lines: a k-step of 64 never leaves half a line for the next
  // one to fetch again), lane L taking row (L >> 3) of the 8 and LDS position
  // L & 7, which holds the row's chunk (L & 7) ^ swizzle.  Wave w moves A rows
  // [32 w, 32 w + 32) and B rows [32 w, 32 w + 32) of each k-step (four
  // instructions each).
  const uint16_t* a_src[4];
  const uint16_t* b_src[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = 32 * wave + 8 * j + (lane >> 3);
    const int chunk = (lane & 7) ^ swizzle(row);
    const int64_t arow = min<int64_t>(m0 + row, p.n_tokens - 1);  // clamp the ragged last block
    a_src[j] = p.hidden + arow * p.d_model + chunk * 8;
    b_src[j] = p.w_t + (static_cast<int64_t>(ct) * kBN + row) * p.d_model + chunk * 8;
  }
  const int k_steps = p.d_model / kBK;
  // Loads of k-step ks (clamped: steps past the end re-read the last, unused).
  auto issue_a = [&](int ks) {
    const int k0 = min(ks, k_steps - 1) * kBK;
    uint8_t* buf = s_a + (ks % kBuffersA) * kBufBytes;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      __builtin_amdgcn_global_load_lds((global_void*)(a_src[j] + k0), (lds_void*)(buf + (32 * wave + 8 * j) * kRow),
                                       16, 0, 0);
  };
  auto issue_b = [&](int ks) {
    const int k0 = min(ks, k_steps - 1) * kBK;
    uint8_t* buf = s_b + (ks % kBuffersB) * kBufBytes;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      __builtin_amdgcn_global_load_lds((global_void*)(b_src[j] + k0), (lds_void*)(buf + (32 * wave + 8 * j) * kRow),
                                       16, 0, 0);
  };

  constexpr int kFM = kWM / 16, kFN = kWN / 16;  // 16 x 16 fragments per wave
  f32x4 acc[kFM][kFN];
#pragma unroll
  for (int i = 0; i < kFM; ++i)
#pragma unroll
    for (int j = 0; j < kFN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Half k-step h of step ks (k = 64 ks + 32 h .. + 31) on 16x16x32 MFMAs:
  // lane (n, g) of fragment i holds row 16 i + n, chunk 4 h + g.
  struct Frags {
    bf16x8 a[kFM], b[kFN];
  };
  auto read = [&](int ks, int h, Frags& f) {
    const uint8_t* abuf = s_a + (ks % kBuffersA) * kBufBytes;
    const uint8_t* bbuf = s_b + (ks % kBuffersB) * kBufBytes;
    const int c = 4 * h + g;
#pragma unroll
    for (int i = 0; i < kFM; ++i) {
      const int row = wm + 16 * i + n;
      f.a[i] = as_bf16x8(*reinterpret_cast<const u32x4*>(abuf + row * kRow + 16 * (c ^ swizzle(row))));
    }
#pragma unroll
    for (int j = 0; j < kFN; ++j) {
      const int row = wn + 16 * j + n;
      f.b[j] = as_bf16x8(*reinterpret_cast<const u32x4*>(bbuf + row * kRow + 16 * (c ^ swizzle(row))));
    }
  };
  auto mma = [&](const Frags& f) {
#pragma unroll
    for (int i = 0; i < kFM; ++i)
#pragma unroll
      for (int j = 0; j < kFN; ++j) acc[i][j] = mfma_bf16_16x16x32(f.a[i], f.b[j], acc[i][j]);
  };
  // Pipeline, one barrier per k-step, in its middle.  The first half of step
  // ks runs the MFMAs of half 0 (fragments already in registers) while the
  // reads of half 1 fly.  Then the middle barrier M(ks): this thread's loads
  // of step ks + 1 have landed and its reads of step ks have returned; after
  // the barrier every thread's loads of ks + 1 are visible and no wave reads
  // the buffers of step ks any more, so they take the B loads of step ks + 2
  // and the A loads of step ks + 3, while half 0 of step ks + 1 is read under
  // the MFMAs of half 1.  The A rows (the hidden states, mostly from HBM) are
  // thus asked for two k-steps ahead, the B rows (the weights, L2-resident)
  // one.  Loads complete in issue order (four per thread per operand and
  // step) and at M(ks) the last four issued are A(ks + 2), so vmcnt(4) leaves
  // exactly those in flight.  The wait and the barrier share one asm block (a
  // fenced barrier would also wait for the loads in flight); sched_barrier(0)
  // keeps the compiler from sinking the reads back next to their MFMAs.
  // Steps past the end re-read the last k-step and are never used.
  static_assert(kBuffersA == 3 && kBuffersB == 2, "the waits below count this pipeline's loads in flight");
  issue_b(0);
  issue_a(0);
  issue_a(1);
  issue_b(1);
  issue_a(2);
  asm volatile("s_waitcnt vmcnt(12)\n\ts_barrier" ::: "memory");  // B(0) and A(0) landed
  Frags f0, f1;
  read(0, 0, f0);
  // The compiler does not see that an asm wait has completed earlier reads
  // and would hold the first MFMA until the reads issued after it return; an
  // empty asm that takes the fragments as operands moves its wait there.
  auto settle = [&](Frags& f) {
#pragma unroll
    for (int i = 0; i < kFM; ++i) asm volatile("" : "+v"(f.a[i]));
#pragma unroll
    for (int j = 0; j < kFN; ++j) asm volatile("" : "+v"(f.b[j]));
  };
  // Within each half the loads and reads are threaded between the MFMAs
  // (sched_group_barrier: one MFMA, then one load or read), so the MFMA pipe
  // restarts right after the barrier instead of after their issue.
  constexpr int kMfma = kFM * kFN, kReads = kFM + kFN;
  for (int ks = 0; ks < k_steps; ++ks) {
    settle(f0);
    __builtin_amdgcn_sched_barrier(0);
    read(ks, 1, f1);
    mma(f0);
#pragma unroll
    for (int i = 0; i < kReads; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
    }
    __builtin_amdgcn_sched_group_barrier(0x008, kMfma - kReads, 0);
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt vmcnt(4) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    settle(f1);
    __builtin_amdgcn_sched_barrier(0);
    issue_b(ks + 2);
    issue_a(ks + 3);
    read(ks + 1, 0, f0);
    mma(f1);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // global -> LDS load
    }
#pragma unroll
    for (int i = 0; i < kReads; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, kMfma - kReads - 8, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");  // the unused loads, before the LDS is reused
  __syncthreads();

  // Epilogue.  Fragment (i, j) holds D[row 4g + e][col n] in lane (n, g);
  // tile column c belongs to output matrix c / 128 (two per workgroup).  The
  // rounded values are staged in LDS (the operand buffers are free: the loop
  // ended on a barrier), matrix 0 then matrix 1, each as [row][128] elements,
  // and then written out row by row with 16-byte stores.
  //   bf16: round to nearest even.
  //   E4M3: per row and matrix, scale = (largest |value|) / 448 in fp32 (1 for
  //   an all-zero row), code = E4M3(value / scale); the row maxima are reduced
  //   over the 16 lanes of a fragment row and then over the two waves that
  //   share the matrix, through LDS.
  constexpr int kElemBytes = FP8OUT ? 1 : 2;
  constexpr int kRowBytes = kDim * kElemBytes;  // staged bytes per row and matrix
  constexpr int kStageBytes = kBM * kRowBytes;  // one matrix of the tile
  static_assert(2 * kStageBytes + sizeof(float) * 2 * 2 * kBM <= kLdsBytes, "staging and row maxima fit in the LDS");
  float (*s_amax)[2][kBM] = reinterpret_cast<float (*)[2][kBM]>(s_raw + 2 * kStageBytes);  // [matrix][half][row]
  const int mat = wn >> 7;         // output matrix of this wave (local: 0 or 1)
  const int half = (wn >> 6) & 1;  // which 64 of its 128 columns
  uint8_t* stage = s_raw + mat * kStageBytes;
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
      const uint8_t* src = s_raw + mm * kStageBytes + r * kRowBytes + 16 * q;
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
