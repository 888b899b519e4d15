// Sum of t rank partials, Y = sum_{r=0}^{t-1} P_r, in fp32 and rank order.
//
// This is the value the all-reduce after a row-parallel block delivers
// (lecture "Distributed Serving", §3.3 and §4.3); on one device it is an
// HBM-bound streaming sum of t*n fp32 values.  Each thread owns 4
// consecutive elements.  It issues the 16-byte loads of up to kBatch ranks
// of its column together, then adds them in rank order, batch after batch, so
// the result is bitwise deterministic and a batch costs one memory round
// trip instead of one per rank.
#include "common.h"
#include "kernels.h"

namespace tpk {

constexpr int kBatch = 8;  // rank loads in flight per thread

template <int OUT_BF16>
__global__ void __launch_bounds__(256)
reduce_kernel(int t, int64_t n4, int64_t n, const f32x4_t* __restrict__ P, void* __restrict__ Y) {
  const int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (v >= n4) return;
  const int64_t stride = n / 4;  // float4 per rank
  f32x4_t s = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int r0 = 0; r0 < t; r0 += kBatch) {
    f32x4_t p[kBatch];
#pragma unroll
    for (int e = 0; e < kBatch; ++e)
      p[e] = r0 + e < t ? __builtin_nontemporal_load(P + (int64_t)(r0 + e) * stride + v)
                        : f32x4_t{0.f, 0.f, 0.f, 0.f};
    // rank order, starting from rank 0's value itself
#pragma unroll
    for (int e = 0; e < kBatch; ++e)
      if (r0 + e < t) s = (r0 + e == 0) ? p[e] : s + p[e];
  }
  if constexpr (OUT_BF16) {
    u32x2_t o;
    o.x = pack_bf16x2(s.x, s.y);
    o.y = pack_bf16x2(s.z, s.w);
    reinterpret_cast<u32x2_t*>(Y)[v] = o;
  } else {
    reinterpret_cast<f32x4_t*>(Y)[v] = s;
  }
}

hipError_t reduce_launch(int t, int64_t n, const float* P, bool out_bf16, void* Y,
                         hipStream_t stream) {
  const int64_t n4 = n / 4;
  const int64_t blocks = (n4 + 255) / 256;
  if (out_bf16)
    hipLaunchKernelGGL(reduce_kernel<1>, dim3((unsigned)blocks), dim3(256), 0, stream, t, n4, n,
                       reinterpret_cast<const f32x4_t*>(P), Y);
  else
    hipLaunchKernelGGL(reduce_kernel<0>, dim3((unsigned)blocks), dim3(256), 0, stream, t, n4, n,
                       reinterpret_cast<const f32x4_t*>(P), Y);
  return hipGetLastError();
}

}  // namespace tpk
