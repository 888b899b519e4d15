// Read-only HBM stream: the achievable read rate of this chip for the access
// pattern of the decode kernels, against which their streams are judged.
//
// Decode time is the time to read the rank's weights once (lecture
// "Distributed Serving", §1.1 and §3.4), so the useful ceiling is what a pure
// read of a large buffer reaches, not the data-sheet peak.  The kernel reads
// each byte once: one workgroup of 16 waves per CU, each wave a contiguous
// span of the buffer, 1 KB (64 lanes x 16 bytes) per load instruction and
// three loads in flight per wave -- on MI355X the depth that streams fastest
// (48 KB per CU; deeper queues measured slower).  Each lane folds what it
// read into one word (x ^ w of each 16-byte chunk) and stores it, so the
// loads cannot be dropped and the result checks that every byte was read.
#include "common.h"
#include "kernels.h"

namespace tpk {

namespace {

constexpr int kWaves = 16;
constexpr uint32_t kOob = 0x80000000u;

__global__ void __launch_bounds__(64 * kWaves)
stream_read_kernel(const void* __restrict__ buf, uint32_t bytes, uint32_t per_wave,
                   unsigned* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const uint32_t gw = blockIdx.x * kWaves + (threadIdx.x >> 6);  // global wave
  const __amdgpu_buffer_rsrc_t r = make_rsrc(buf, bytes);
  const uint32_t first = gw * per_wave;                           // this wave's 1 KB blocks
  auto off = [&](uint32_t i) -> uint32_t {
    return i < per_wave ? (first + i) * 1024u + lane * 16u : kOob;
  };
  unsigned acc = 0;
  u32x4_t v0 = buf_load16<kAuxNT>(r, off(0));
  u32x4_t v1 = buf_load16<kAuxNT>(r, off(1));
  u32x4_t v2 = buf_load16<kAuxNT>(r, off(2));
  for (uint32_t i = 0; i < per_wave; i += 3) {
    acc ^= v0.x ^ v0.w;
    v0 = buf_load16<kAuxNT>(r, off(i + 3));
    acc ^= v1.x ^ v1.w;
    v1 = buf_load16<kAuxNT>(r, off(i + 4));
    acc ^= v2.x ^ v2.w;
    v2 = buf_load16<kAuxNT>(r, off(i + 5));
  }
  sink[blockIdx.x * (64 * kWaves) + threadIdx.x] = acc;
}

int cus_of_current_device() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return n;
}

}  // namespace

size_t stream_read_sink_words() { return (size_t)cus_of_current_device() * 64 * kWaves; }

hipError_t stream_read_launch(const void* buf, size_t bytes, unsigned* sink, hipStream_t stream) {
  const int cus = cus_of_current_device();
  if (cus < 1 || bytes == 0 || (bytes % 1024) || bytes > (size_t(1) << 31))
    return hipErrorInvalidValue;
  const uint32_t blocks = (uint32_t)(bytes / 1024);
  const uint32_t waves = (uint32_t)cus * kWaves;
  const uint32_t per_wave = (blocks + waves - 1) / waves;
  hipLaunchKernelGGL(stream_read_kernel, dim3(cus), dim3(64 * kWaves), 0, stream, buf,
                     (uint32_t)bytes, per_wave, sink);
  return hipGetLastError();
}

}  // namespace tpk
