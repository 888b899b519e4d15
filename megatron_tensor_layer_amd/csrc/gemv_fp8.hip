// Decode projections for few tokens (I <= 8) with weight-only one-byte
// storage: y[i, n] = s[n] * sum_k x[i, k] w(code[n, k]), activations bf16,
// w = e4m3 (FP8) or the signed int8 value, by the launch's format.
//
// Decode streams the rank's weights once per step (lecture "Distributed
// Serving", §1.1 and §3.4); one byte per weight halves that stream.  The
// kernel is the bf16 few-token kernel with a different chunk: a lane's
// 16-byte weight chunk holds 16 K values, so it pairs with two 16-byte chunks
// of each token's activations.  gfx950's v_cvt_scalef32_pk_bf16_fp8 decodes
// two OCP E4M3 codes straight to packed bf16 (every E4M3 value is exact in
// bf16), and the decoded pairs feed v_dot2_f32_bf16 (fp32 sums).  The per-row scale multiplies the
// finished dot product once, in the epilogue.
#include "common.h"
#include "kernels.h"

namespace tpk {

namespace {

__device__ __forceinline__ float dot8(const u32x4_t& w, const u32x4_t& x, float acc) {
  acc = dot2_bf16(w.x, x.x, acc);
  acc = dot2_bf16(w.y, x.y, acc);
  acc = dot2_bf16(w.z, x.z, acc);
  acc = dot2_bf16(w.w, x.w, acc);
  return acc;
}

// X [I, K] bf16 (row stride ldx); W0/W1 [N, K] fp8 codes, S0/S1 [N] fp32 row
// scales (W1/S1: up matrix, SwiGLU only); out [I, N] (row stride ldo).
template <int NI, int J, int R, int EPI, int FMT>
__global__ void __launch_bounds__(512)
gemv_fp8_kernel(int I, int K, int N, const uint16_t* __restrict__ X, int64_t ldx,
                const uint8_t* __restrict__ W0, const float* __restrict__ S0,
                const uint8_t* __restrict__ W1, const float* __restrict__ S1,
                void* __restrict__ out, int64_t ldo) {
  constexpr int RP = (EPI == EPI_SWIGLU) ? R / 2 : R;
  constexpr int V = R * NI;
  static_assert(EPI != EPI_SWIGLU || (R % 2) == 0, "SwiGLU needs gate/up row pairs");

  __shared__ float red[8][64];
  const int tid = threadIdx.x, nthr = blockDim.x, lane = tid & 63, wave = tid >> 6;
  const int nwave = nthr >> 6;

  // chunk c = tid + j * nthr covers K [16c, 16c + 16): 16 weight bytes,
  // 32 activation bytes
  uint32_t woff[J];
#pragma unroll
  for (int j = 0; j < J; ++j) woff[j] = (uint32_t)(tid + j * nthr) * 16u;
  const uint32_t wrow_bytes = (uint32_t)K;

  u32x4_t xr[J][NI][2];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const __amdgpu_buffer_rsrc_t xrow =
        make_rsrc(X + (int64_t)i * ldx, i < I ? (uint32_t)K * 2u : 0u);
#pragma unroll
    for (int j = 0; j < J; ++j) {
      xr[j][i][0] = buf_load16(xrow, 2u * woff[j]);
      xr[j][i][1] = buf_load16(xrow, 2u * woff[j] + 16u);
    }
  }

  const int nblk = (N + RP - 1) / RP;
  for (int blk = blockIdx.x; blk < nblk; blk += gridDim.x) {
    u32x4_t wr[R][J];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int col = blk * RP + (r % RP);
      const uint8_t* Wm = (EPI == EPI_SWIGLU && r >= RP) ? W1 : W0;
      if (col < N) {
        const __amdgpu_buffer_rsrc_t wrow = make_rsrc(Wm + (int64_t)col * K, wrow_bytes);
#pragma unroll
        for (int j = 0; j < J; ++j) wr[r][j] = buf_load16<kAuxNT>(wrow, woff[j]);
      } else {
#pragma unroll
        for (int j = 0; j < J; ++j) wr[r][j] = u32x4_t{0u, 0u, 0u, 0u};
      }
    }
    float acc[V];
#pragma unroll
    for (int q = 0; q < V; ++q) acc[q] = 0.0f;
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int j = 0; j < J; ++j) {
        u32x4_t lo, hi;
        if constexpr (FMT == kFmtInt8)
          decode16_i8(wr[r][j], lo, hi);
        else
          decode16(wr[r][j], lo, hi);
#pragma unroll
        for (int i = 0; i < NI; ++i)
          acc[r * NI + i] = dot8(hi, xr[j][i][1], dot8(lo, xr[j][i][0], acc[r * NI + i]));
      }

    wave_fold<V>(acc, lane);
    if ((lane % (64 / V)) == 0) red[wave][lane / (64 / V)] = acc[0];
    __syncthreads();

    if (tid < RP * NI) {
      const int p = tid % RP, i = tid / RP;
      const int col = blk * RP + p;
      if (col < N && i < I) {
        float s0 = 0.0f;
        for (int w = 0; w < nwave; ++w) s0 += red[w][p * NI + i];
        s0 *= S0[col];
        if constexpr (EPI == EPI_SWIGLU) {
          float s1 = 0.0f;
          for (int w = 0; w < nwave; ++w) s1 += red[w][(RP + p) * NI + i];
          s1 *= S1[col];
          static_cast<uint16_t*>(out)[(int64_t)i * ldo + col] = f32_to_bf16_bits(silu(s0) * s1);
        } else {
          static_cast<float*>(out)[(int64_t)i * ldo + col] = s0;
        }
      }
    }
    __syncthreads();
  }
}

// Rows per block: in-flight weight registers R*J*4 <= 32 (each chunk also
// expands to 8 bf16 registers), per-lane partial sums R*NI <= 32.
template <int NI, int J, int EPI>
constexpr int fp8_rows_per_block() {
  constexpr int r0 = (NI <= 2 ? 8 : (NI == 4 ? 8 : 4)) / J;
  constexpr int r1 = r0 < 1 ? 1 : r0;
  return (EPI == EPI_SWIGLU && r1 < 2) ? 2 : r1;
}

template <int NI, int J, int EPI>
hipError_t launch_fp8(int I, int K, int N, const uint16_t* X, int64_t ldx, const uint8_t* W0,
                      const float* S0, const uint8_t* W1, const float* S1, void* out, int64_t ldo,
                      int nthreads, int fmt, hipStream_t stream) {
  constexpr int R = fp8_rows_per_block<NI, J, EPI>();
  constexpr int RP = (EPI == EPI_SWIGLU) ? R / 2 : R;
  const int nblk = (N + RP - 1) / RP;
  if (fmt == kFmtInt8)
    hipLaunchKernelGGL((gemv_fp8_kernel<NI, J, R, EPI, kFmtInt8>), dim3(nblk), dim3(nthreads), 0,
                       stream, I, K, N, X, ldx, W0, S0, W1, S1, out, ldo);
  else
    hipLaunchKernelGGL((gemv_fp8_kernel<NI, J, R, EPI, kFmtE4M3>), dim3(nblk), dim3(nthreads), 0,
                       stream, I, K, N, X, ldx, W0, S0, W1, S1, out, ldo);
  return hipGetLastError();
}

template <int NI, int EPI>
hipError_t launch_fp8_j(int I, int K, int N, const uint16_t* X, int64_t ldx, const uint8_t* W0,
                        const float* S0, const uint8_t* W1, const float* S1, void* out,
                        int64_t ldo, int fmt, hipStream_t stream) {
  const int chunks = K / 16;
  int J = 1;
  while (chunks > J * 512) J *= 2;
  const int nthreads = std::min(512, ((chunks + J - 1) / J + 63) / 64 * 64);
  switch (J) {  // K <= kFp8MaxK = 16 * 512 * 2
    case 1: return launch_fp8<NI, 1, EPI>(I, K, N, X, ldx, W0, S0, W1, S1, out, ldo, nthreads, fmt, stream);
    case 2: return launch_fp8<NI, 2, EPI>(I, K, N, X, ldx, W0, S0, W1, S1, out, ldo, nthreads, fmt, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

template <int EPI>
hipError_t gemv_fp8_launch(int I, int K, int N, const uint16_t* X, const uint8_t* W0,
                           const float* S0, const uint8_t* W1, const float* S1, void* out,
                           int64_t ldo, int fmt, hipStream_t stream) {
  if (I <= 1) return launch_fp8_j<1, EPI>(I, K, N, X, K, W0, S0, W1, S1, out, ldo, fmt, stream);
  if (I <= 2) return launch_fp8_j<2, EPI>(I, K, N, X, K, W0, S0, W1, S1, out, ldo, fmt, stream);
  if (I <= 4) return launch_fp8_j<4, EPI>(I, K, N, X, K, W0, S0, W1, S1, out, ldo, fmt, stream);
  return launch_fp8_j<8, EPI>(I, K, N, X, K, W0, S0, W1, S1, out, ldo, fmt, stream);
}

template hipError_t gemv_fp8_launch<EPI_F32>(int, int, int, const uint16_t*, const uint8_t*,
                                             const float*, const uint8_t*, const float*, void*,
                                             int64_t, int, hipStream_t);
template hipError_t gemv_fp8_launch<EPI_SWIGLU>(int, int, int, const uint16_t*, const uint8_t*,
                                                const float*, const uint8_t*, const float*, void*,
                                                int64_t, int, hipStream_t);

}  // namespace tpk
