// Multi-token decode (speculative verification): T query tokens of a sequence
// in one step.  The pages describe no multi-token rule for HySparse2; the
// reading taken: the T tokens occupy the sequence's last T cache rows and
// token t, at position L - T + t, is a decode step of its own over the causal
// prefix [0, L - T + t], with its own selection.
//
// The B * T tokens run as a batch of virtual sequences through the ordinary
// kernels: virtual sequence b * T + t has length max(0, L_b - T + t + 1), its
// workspace range (scores, bounds, candidate keys) is its own, packed by
// these lengths, and its K/V rows start at the real sequence's first row
// (kv_start).  multi_prep_kernel writes both arrays.
#include "hs2_device.h"
#include "hs2_internal.h"

namespace hs2 {

namespace {

constexpr int kPrepThreads = 1024;

__global__ __launch_bounds__(kPrepThreads) void multi_prep_kernel(MultiParams p) {
  __shared__ int64_t s_sum[kPrepThreads];
  const int n = p.batch * p.n_query;
  const int per = (n + kPrepThreads - 1) / kPrepThreads;
  const int t = threadIdx.x;
  const int i0 = t * per;
  const int i1 = min(i0 + per, n);
  auto length_of = [&](int i, int64_t& base) {
    const int b = i / p.n_query;
    const int tok = i % p.n_query;
    int len;
    seq_bounds(p.seq_offsets, b, p.total_tokens, p.max_context, base, len);
    return max(0, len - p.n_query + tok + 1);
  };
  int64_t sum = 0;
  for (int i = i0; i < i1; ++i) {
    int64_t base;
    sum += length_of(i, base);
    p.kv_start[i] = base;
  }
  s_sum[t] = sum;
  __syncthreads();
  for (int d = 1; d < kPrepThreads; d <<= 1) {  // inclusive scan of the per-thread sums
    const int64_t add = t >= d ? s_sum[t - d] : 0;
    __syncthreads();
    s_sum[t] += add;
    __syncthreads();
  }
  int64_t run = s_sum[t] - sum;  // exclusive
  for (int i = i0; i < i1; ++i) {
    int64_t base;
    p.voffs[i] = run;
    run += length_of(i, base);
  }
  if (t == kPrepThreads - 1) p.voffs[n] = s_sum[t];
}

}  // namespace

hipError_t launch_multi_prep(const MultiParams& p, hipStream_t s) {
  if (p.batch <= 0) return hipSuccess;
  hipLaunchKernelGGL(multi_prep_kernel, dim3(1), dim3(kPrepThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace hs2
