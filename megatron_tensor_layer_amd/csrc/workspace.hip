// Workspace preparation: the arrival-counter area that every kernel splitting
// a sum over workgroups keeps at the start of its workspace.
//
// A completed call leaves its counters zero (the last arrival wraps each one
// back), so a workspace serves any sequence of calls once it has been zeroed.
// The zeroing is a small fill kernel rather than hipMemsetAsync, so a caller
// may record it into a HIP graph.
#include "common.h"
#include "kernels.h"

namespace tpk {

namespace {

__global__ void __launch_bounds__(256) zero_words_kernel(unsigned* __restrict__ p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

}  // namespace

hipError_t counters_reset_launch(void* workspace, size_t bytes, hipStream_t stream) {
  const int n = (int)(std::min(bytes, kWsCounterBytes) / 4);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(zero_words_kernel, dim3((n + 255) / 256), dim3(256), 0, stream,
                     static_cast<unsigned*>(workspace), n);
  return hipGetLastError();
}

}  // namespace tpk
