// The step after a row-parallel block's all-reduce, fused into one pass over
// each hidden row: the residual stream h = residual + sum_r P_r (fp32, rank
// order), stored in its dtype, then RMSNorm of the stored h scaled by the
// replicated gamma -- the input of the next column-parallel projection, which
// every rank computes for itself (lecture "Distributed Serving", §4.2).
//
// One workgroup of 16 waves per row: each thread owns CPT 4-element chunks
// of the row and keeps them in registers between the two halves (sum of
// squares, then scale), so the row is read once.  The t partial loads of a
// chunk are issued four at a time before they are added in rank order.
#include "common.h"
#include "kernels.h"

namespace tpk {

namespace {

constexpr int kThreads = 1024;

__device__ __forceinline__ f32x4_t load4(const void* p, int64_t idx4, bool bf16) {
  if (bf16) {
    const u32x2_t v = reinterpret_cast<const u32x2_t*>(p)[idx4];
    return f32x4_t{bf16_bits_to_f32(v.x & 0xffffu), bf16_bits_to_f32(v.x >> 16),
                   bf16_bits_to_f32(v.y & 0xffffu), bf16_bits_to_f32(v.y >> 16)};
  }
  return reinterpret_cast<const f32x4_t*>(p)[idx4];
}

// Store 4 values in the dtype; returns the values as stored.
__device__ __forceinline__ f32x4_t store4(void* p, int64_t idx4, f32x4_t v, bool bf16) {
  if (bf16) {
    u32x2_t o;
    o.x = pack_bf16x2(v.x, v.y);
    o.y = pack_bf16x2(v.z, v.w);
    reinterpret_cast<u32x2_t*>(p)[idx4] = o;
    return f32x4_t{bf16_bits_to_f32(o.x & 0xffffu), bf16_bits_to_f32(o.x >> 16),
                   bf16_bits_to_f32(o.y & 0xffffu), bf16_bits_to_f32(o.y >> 16)};
  }
  reinterpret_cast<f32x4_t*>(p)[idx4] = v;
  return v;
}

template <int CPT>
__global__ void __launch_bounds__(kThreads)
residual_rmsnorm_kernel(int t, int D, const float* __restrict__ P, const void* residual,
                        bool h_bf16, void* h, const void* __restrict__ gamma, bool x_bf16,
                        void* __restrict__ x, float eps, int64_t plane4) {
  __shared__ float red[kThreads / 64];
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x;
  const int c4 = D / 4;
  const int64_t base4 = row * c4;

  f32x4_t hv[CPT];
  float ss = 0.0f;
#pragma unroll
  for (int k = 0; k < CPT; ++k) {
    const int c = tid + k * kThreads;
    if (c >= c4) continue;
    const int64_t e4 = base4 + c;
    f32x4_t v = residual ? load4(residual, e4, h_bf16) : f32x4_t{0.f, 0.f, 0.f, 0.f};
    const f32x4_t* pp = reinterpret_cast<const f32x4_t*>(P) + e4;
    int r = 0;
    for (; r + 4 <= t; r += 4) {
      const f32x4_t a = __builtin_nontemporal_load(pp + (int64_t)r * plane4);
      const f32x4_t b = __builtin_nontemporal_load(pp + (int64_t)(r + 1) * plane4);
      const f32x4_t cc = __builtin_nontemporal_load(pp + (int64_t)(r + 2) * plane4);
      const f32x4_t d = __builtin_nontemporal_load(pp + (int64_t)(r + 3) * plane4);
      v += a;
      v += b;
      v += cc;
      v += d;
    }
    for (; r < t; ++r) v += __builtin_nontemporal_load(pp + (int64_t)r * plane4);
    hv[k] = store4(h, e4, v, h_bf16);
    ss += hv[k].x * hv[k].x + hv[k].y * hv[k].y + hv[k].z * hv[k].z + hv[k].w * hv[k].w;
  }
  if (!x) return;

  // row sum of squares: wave butterfly, then the 16 wave sums in fixed order
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, 64);
  if ((tid & 63) == 0) red[tid >> 6] = ss;
  __syncthreads();
  float tot = 0.0f;
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) tot += red[w];
  const float inv = 1.0f / sqrtf(tot / (float)D + eps);

#pragma unroll
  for (int k = 0; k < CPT; ++k) {
    const int c = tid + k * kThreads;
    if (c >= c4) continue;
    const f32x4_t g = load4(gamma, c, x_bf16);
    store4(x, base4 + c, hv[k] * inv * g, x_bf16);
  }
}

}  // namespace

hipError_t residual_rmsnorm_launch(int t, int I, int D, const float* P, int64_t p_rows,
                                   const void* residual, bool h_bf16, void* h, const void* gamma,
                                   bool x_bf16, void* x, float eps, hipStream_t stream) {
  const int c4 = D / 4;
  const int64_t plane4 = p_rows * c4;  // one rank's partial, in float4
  const int cpt = (c4 + kThreads - 1) / kThreads;
#define TPK_LAUNCH(N)                                                                            \
  hipLaunchKernelGGL(residual_rmsnorm_kernel<N>, dim3(I), dim3(kThreads), 0, stream, t, D, P,    \
                     residual, h_bf16, h, gamma, x_bf16, x, eps, plane4)
  if (cpt <= 1)
    TPK_LAUNCH(1);
  else if (cpt <= 2)
    TPK_LAUNCH(2);
  else if (cpt <= 4)
    TPK_LAUNCH(4);
  else if (cpt <= 8)
    TPK_LAUNCH(8);
  else
    return hipErrorInvalidValue;
#undef TPK_LAUNCH
  return hipGetLastError();
}

}  // namespace tpk
