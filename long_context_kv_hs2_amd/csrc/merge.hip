// Split-K merge of the full layer's partials, one problem per head and
// sequence (the score path; the bound path fuses it with its first pass).
#include "merge.h"

namespace hs2 {

__global__ __launch_bounds__(kMergeThreads) void merge_kernel(MergeParams p, int64_t stride_layer,
                                                              int64_t out_stride_layer) {
  __shared__ MergeShared sh;
  merge_one(p, blockIdx.x, blockIdx.y, blockIdx.z, stride_layer, out_stride_layer, sh);
}

hipError_t launch_merge(const MergeParams& p, int batch, hipStream_t s) {
  if (batch == 0) return hipSuccess;
  hipLaunchKernelGGL(merge_kernel, dim3(kHeads, batch, 1), dim3(kMergeThreads), 0, s, p, int64_t(0), int64_t(0));
  return hipGetLastError();
}

}  // namespace hs2
