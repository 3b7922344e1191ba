// Self-Decoder sliding-window layers at decode.
//
// The model's front half (the Self-Decoder) mixes full-attention and
// sliding-window layers ("Luo Fuli Teases Xiaomi MiMo-V3 Architecture",
// paragraph on the self-decoder / cross-decoder split; toolnavs.com article
// 2080, section "Ce que fait HySparse2").  A window layer at decode attends to
// its `window` most recent positions, the current token included; its cache is
// a ring of `window` rows per sequence, position p in slot p mod window (the
// pages give no window size; 128, the local window they do give, is the
// default the workloads use).
//
// swa_prep_kernel writes the current token's K and V rows into their slot
// (when the caller passes them) and the ring slots the window covers (all of
// them once the ring is full, else slots 0 .. L-1) as a selection list; the
// attention itself is the sparse layers' gather kernel over those rows, in
// one unsliced launch.
#include "hs2_device.h"
#include "hs2_internal.h"

namespace hs2 {

namespace {

constexpr int kPrepThreads = 128;

__global__ __launch_bounds__(kPrepThreads) void swa_prep_kernel(SwaParams p) {
  const int b = blockIdx.x;
  const int t = threadIdx.x;
  const int64_t len = max<int64_t>(p.lengths[b], 0);
  const int count = static_cast<int>(min<int64_t>(len, p.window));
  for (int i = t; i < p.window; i += kPrepThreads) p.sel_idx[static_cast<size_t>(b) * p.window + i] = i < count ? i : -1;
  if (t == 0) {
    p.sel_count[b] = count;
    p.offs[b] = static_cast<int64_t>(b) * p.window;
    if (b == p.batch - 1) p.offs[p.batch] = static_cast<int64_t>(p.batch) * p.window;
  }
  if (p.k_new && len > 0) {
    const int64_t slot = static_cast<int64_t>(b) * p.window + (len - 1) % p.window;
    const int words = p.fp8 ? kDim / 4 : kDim / 2;  // 32-bit words per row
    if (t < words) {
      reinterpret_cast<uint32_t*>(p.ring_k + slot * words * 4)[t] =
          reinterpret_cast<const uint32_t*>(p.k_new + static_cast<size_t>(b) * words * 4)[t];
      reinterpret_cast<uint32_t*>(p.ring_v + slot * words * 4)[t] =
          reinterpret_cast<const uint32_t*>(p.v_new + static_cast<size_t>(b) * words * 4)[t];
    }
    if (p.fp8 && t == 0) {
      p.ring_ks[slot] = p.k_new_scale[b];
      p.ring_vs[slot] = p.v_new_scale[b];
    }
  }
}

}  // namespace

hipError_t launch_swa_prep(const SwaParams& p, hipStream_t s) {
  if (p.batch <= 0) return hipSuccess;
  hipLaunchKernelGGL(swa_prep_kernel, dim3(p.batch), dim3(kPrepThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace hs2
