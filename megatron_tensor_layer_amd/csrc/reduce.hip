// Sum of t rank partials, Y = sum_{r=0}^{t-1} P_r, in fp32 and rank order.
//
// This is the value the all-reduce after a row-parallel block delivers
// (lecture "Distributed Serving", §3.3 and §4.3); on one device it is an
// HBM-bound streaming sum of t*n fp32 values.  Each thread owns 4
// consecutive elements and adds its t values in rank order, so the result is
// bitwise deterministic.  A thread waits for each load before the next add;
// the bytes in flight come from the many resident waves instead (a few
// thousand workgroups at prefill sizes, about 32 KB per CU).  Issuing 4 or 8
// of a thread's rank loads before adding them was slower on MI355X: 29 and
// 31 us against 26 us for 8 partials of [512, 8192] (too many bytes in flight
// per CU), and no faster at [32, 8192], where the launch dominates.
#include "common.h"
#include "kernels.h"

namespace tpk {

template <int OUT_BF16>
__global__ void __launch_bounds__(256)
reduce_kernel(int t, int64_t n4, int64_t n, const f32x4_t* __restrict__ P, void* __restrict__ Y) {
  const int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (v >= n4) return;
  const int64_t stride = n / 4;  // float4 per rank
  f32x4_t s = __builtin_nontemporal_load(P + v);
  for (int r = 1; r < t; ++r) {
    const f32x4_t p = __builtin_nontemporal_load(P + (int64_t)r * stride + v);
    s += p;
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
