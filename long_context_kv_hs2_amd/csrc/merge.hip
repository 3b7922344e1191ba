// Split-K merges: the full layer's partials (one problem per head and
// sequence) and the sparse layers' (per head, sequence and layer).
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

hipError_t launch_merge_layers(const MergeParams& p, int batch, int layers, int64_t stride_layer,
                               int64_t out_stride_layer, hipStream_t s) {
  if (batch == 0 || layers == 0) return hipSuccess;
  hipLaunchKernelGGL(merge_kernel, dim3(kHeads, batch, layers), dim3(kMergeThreads), 0, s, p, stride_layer,
                     out_stride_layer);
  return hipGetLastError();
}

}  // namespace hs2
