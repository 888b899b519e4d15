// Workspace preparation: the arrival-counter area that every kernel splitting
// a sum over workgroups keeps at the start of its workspace.
//
// A completed call leaves its counters zero (the last arrival wraps each one
// back), so a workspace serves any sequence of calls once it has been zeroed.
// The zeroing is a small fill kernel rather than hipMemsetAsync, so a caller
// may record it into a HIP graph.
#include <mutex>

#include "common.h"
#include "kernels.h"

// Library-owned scratch for callers that cannot allocate (see
// static_scratch below).  In host code this name is only a stand-in for the
// symbol: its device address comes from hipGetSymbolAddress, per device.
static __device__ __align__(256) unsigned char scratch[tpk::kStaticScratchBytes];

namespace tpk {

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t static_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    // once per device, with that device current: the array's address there
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

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
