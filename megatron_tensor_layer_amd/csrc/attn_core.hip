// Attention core of one rank (test support: it joins the QKV projection to
// o_proj; it is not a projection).  Each rank computes its own heads
// completely (lecture "Distributed Serving", §4.2).  One wavefront per
// (token, local head): scores q.k/sqrt(hd) over the causal window of the
// token's sequence, online softmax in fp32, probability-weighted sum of the
// values of the head's KV group.  Plain and unoptimised on purpose.
#include "common.h"
#include "kernels.h"

namespace tpk {

__global__ void __launch_bounds__(64)
attn_core_kernel(int I, int S, int nq, int nkv, int hd, const uint16_t* __restrict__ qkv,
                 uint16_t* __restrict__ A) {
  const int i = blockIdx.x;
  const int j = blockIdx.y;
  const int lane = threadIdx.x;
  const int N = (nq + 2 * nkv) * hd;
  const int g = (j * nkv) / nq;
  const int s0 = (i / S) * S;
  const float scale = 1.0f / sqrtf((float)hd);
  constexpr int EPL = 4;  // elements per lane, hd <= 256

  float q[EPL], o[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    const int c = lane + 64 * e;
    q[e] = (c < hd) ? bf16_bits_to_f32(qkv[(int64_t)i * N + j * hd + c]) : 0.0f;
    o[e] = 0.0f;
  }
  float m = -INFINITY, l = 0.0f;
  for (int p = s0; p <= i; ++p) {
    const uint16_t* kp = qkv + (int64_t)p * N + (nq + g) * hd;
    const uint16_t* vp = qkv + (int64_t)p * N + (nq + nkv + g) * hd;
    float d = 0.0f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const int c = lane + 64 * e;
      if (c < hd) d += q[e] * bf16_bits_to_f32(kp[c]);
    }
#pragma unroll
    for (int msk = 32; msk >= 1; msk /= 2) d += __shfl_xor(d, msk, 64);
    const float s = d * scale;
    const float mn = fmaxf(m, s);
    const float corr = expf(m - mn);
    const float pe = expf(s - mn);
    l = l * corr + pe;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const int c = lane + 64 * e;
      const float vv = (c < hd) ? bf16_bits_to_f32(vp[c]) : 0.0f;
      o[e] = o[e] * corr + pe * vv;
    }
    m = mn;
  }
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    const int c = lane + 64 * e;
    if (c < hd) A[(int64_t)i * (nq * hd) + j * hd + c] = f32_to_bf16_bits(o[e] / l);
  }
}

hipError_t attn_core_launch(int I, int S, int nq, int nkv, int hd, const uint16_t* qkv,
                            uint16_t* A, hipStream_t stream) {
  hipLaunchKernelGGL(attn_core_kernel, dim3(I, nq), dim3(64), 0, stream, I, S, nq, nkv, hd, qkv,
                     A);
  return hipGetLastError();
}

}  // namespace tpk
