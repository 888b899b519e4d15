// Decode projections for few tokens (I <= 8): y[i, n] = sum_k x[i, k] w[n, k].
//
// Decode is bound by reading the rank's weight shard once per step (lecture
// "Distributed Serving", §1.1 and §3.4), so this kernel is built around
// streaming W from HBM at full rate:
//   * every lane owns J fixed 16-byte chunks of the K axis (chunk
//     c = tid + j * blockDim); the activations of those chunks for all NI
//     tokens are loaded once into registers, so the inner loop touches no LDS;
//   * a workgroup walks blocks of R weight rows; for each row it reads
//     blockDim * 16 contiguous bytes per chunk step, i.e. perfectly coalesced
//     128-bit loads, all R*J of them issued before any arithmetic;
//   * bf16 products use v_dot2_f32_bf16 (two MACs per lane-op, fp32 sums);
//   * the R*NI per-lane partial sums are folded across the wavefront by a
//     halving butterfly (each step ships half the live values to the partner
//     lane), then across waves through 4 KB of LDS in fixed wave order, so the
//     result is deterministic.
// The SwiGLU variant reads gate row f and up row f in the same block and
// applies silu(g) * u before the single store of H (lecture §4.1: the
// elementwise op stays local to the rank).
#include "common.h"
#include "kernels.h"

namespace tpk {

template <typename T>
struct Elem;
template <>
struct Elem<uint16_t> {
  static constexpr int per16 = 8;
};
template <>
struct Elem<float> {
  static constexpr int per16 = 4;
};

// acc += <w, x> over one 16-byte chunk.
__device__ __forceinline__ float chunk_dot(const u32x4_t& w, const u32x4_t& x, float acc,
                                           uint16_t) {
  acc = dot2_bf16(w.x, x.x, acc);
  acc = dot2_bf16(w.y, x.y, acc);
  acc = dot2_bf16(w.z, x.z, acc);
  acc = dot2_bf16(w.w, x.w, acc);
  return acc;
}
__device__ __forceinline__ float chunk_dot(const u32x4_t& w, const u32x4_t& x, float acc, float) {
  acc = fmaf(__uint_as_float(w.x), __uint_as_float(x.x), acc);
  acc = fmaf(__uint_as_float(w.y), __uint_as_float(x.y), acc);
  acc = fmaf(__uint_as_float(w.z), __uint_as_float(x.z), acc);
  acc = fmaf(__uint_as_float(w.w), __uint_as_float(x.w), acc);
  return acc;
}

template <typename T>
__device__ __forceinline__ void store_dt(void* out, int64_t idx, float v);
template <>
__device__ __forceinline__ void store_dt<uint16_t>(void* out, int64_t idx, float v) {
  static_cast<uint16_t*>(out)[idx] = f32_to_bf16_bits(v);
}
template <>
__device__ __forceinline__ void store_dt<float>(void* out, int64_t idx, float v) {
  static_cast<float*>(out)[idx] = v;
}

// X  [I, K] (row stride ldx elements), W0/W1 [N, K] (W1: up matrix, SwiGLU only)
// out [I, N] (row stride ldo elements): fp32 (EPI_F32) or T.
template <typename T, int NI, int J, int R, int EPI>
__global__ void __launch_bounds__(512)
gemv_kernel(int I, int K, int N, const T* __restrict__ X, int64_t ldx,
            const T* __restrict__ W0, const T* __restrict__ W1, void* __restrict__ out,
            int64_t ldo) {
  constexpr int RP = (EPI == EPI_SWIGLU) ? R / 2 : R;  // output columns per block
  constexpr int V = R * NI;
  static_assert(EPI != EPI_SWIGLU || (R % 2) == 0, "SwiGLU needs gate/up row pairs");

  __shared__ float red[8][64];

  const int tid = threadIdx.x;
  const int nthr = blockDim.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int nwave = nthr >> 6;

  // byte offset of each of this lane's chunks inside a row
  uint32_t loff[J];
#pragma unroll
  for (int j = 0; j < J; ++j) loff[j] = (uint32_t)(tid + j * nthr) * 16u;
  const uint32_t row_bytes = (uint32_t)K * (uint32_t)sizeof(T);

  // activations of this lane's chunks, all tokens (chunks past K read zero)
  u32x4_t xr[J][NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const __amdgpu_buffer_rsrc_t xrow = make_rsrc(X + (int64_t)i * ldx, i < I ? row_bytes : 0u);
#pragma unroll
    for (int j = 0; j < J; ++j) xr[j][i] = buf_load16(xrow, loff[j]);
  }

  const int nblk = (N + RP - 1) / RP;
  for (int blk = blockIdx.x; blk < nblk; blk += gridDim.x) {
    // issue every weight load of the block first; one buffer resource per
    // row (scalar registers), the lane offset selects the chunk
    u32x4_t wr[R][J];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int col = blk * RP + (r % RP);
      const T* Wm = (EPI == EPI_SWIGLU && r >= RP) ? W1 : W0;
      if (col < N) {
        const __amdgpu_buffer_rsrc_t wrow = make_rsrc(Wm + (int64_t)col * K, row_bytes);
#pragma unroll
        for (int j = 0; j < J; ++j) wr[r][j] = buf_load16<kAuxNT>(wrow, loff[j]);
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
      for (int j = 0; j < J; ++j)
#pragma unroll
        for (int i = 0; i < NI; ++i)
          acc[r * NI + i] = chunk_dot(wr[r][j], xr[j][i], acc[r * NI + i], T{});

    wave_fold<V>(acc, lane);
    if ((lane % (64 / V)) == 0) red[wave][lane / (64 / V)] = acc[0];
    __syncthreads();

    if (tid < RP * NI) {
      const int p = tid % RP;   // output column within the block
      const int i = tid / RP;   // token
      const int col = blk * RP + p;
      if (col < N && i < I) {
        float s0 = 0.0f;
        for (int w = 0; w < nwave; ++w) s0 += red[w][p * NI + i];
        if constexpr (EPI == EPI_SWIGLU) {
          float s1 = 0.0f;
          for (int w = 0; w < nwave; ++w) s1 += red[w][(RP + p) * NI + i];
          store_dt<T>(out, (int64_t)i * ldo + col, silu(s0) * s1);
        } else if constexpr (EPI == EPI_F32) {
          static_cast<float*>(out)[(int64_t)i * ldo + col] = s0;
        } else {
          store_dt<T>(out, (int64_t)i * ldo + col, s0);
        }
      }
    }
    __syncthreads();
  }
}

// Rows per block: keeps the in-flight weight registers (R*J*4 VGPRs) at
// <= 64 and the per-lane partial sums R*NI at <= 32.
template <int NI, int J, int EPI>
constexpr int rows_per_block() {
  constexpr int r0 = (NI <= 2 ? 16 : (NI == 4 ? 8 : 4)) / J;
  constexpr int r1 = r0 < 1 ? 1 : r0;
  return (EPI == EPI_SWIGLU && r1 < 2) ? 2 : r1;
}

template <typename T, int NI, int J, int EPI>
static hipError_t launch_nij(int I, int K, int N, const T* X, int64_t ldx, const T* W0,
                             const T* W1, void* out, int64_t ldo, int nthreads,
                             hipStream_t stream) {
  constexpr int R = rows_per_block<NI, J, EPI>();
  constexpr int RP = (EPI == EPI_SWIGLU) ? R / 2 : R;
  const int nblk = (N + RP - 1) / RP;
  hipLaunchKernelGGL((gemv_kernel<T, NI, J, R, EPI>), dim3(nblk), dim3(nthreads), 0, stream,
                     I, K, N, X, ldx, W0, W1, out, ldo);
  return hipGetLastError();
}

template <typename T, int EPI, int J>
static hipError_t launch_j(int I, int K, int N, const T* X, int64_t ldx, const T* W0,
                           const T* W1, void* out, int64_t ldo, int nthreads,
                           hipStream_t stream) {
  if (I <= 1) return launch_nij<T, 1, J, EPI>(I, K, N, X, ldx, W0, W1, out, ldo, nthreads, stream);
  if (I <= 2) return launch_nij<T, 2, J, EPI>(I, K, N, X, ldx, W0, W1, out, ldo, nthreads, stream);
  if (I <= 4) return launch_nij<T, 4, J, EPI>(I, K, N, X, ldx, W0, W1, out, ldo, nthreads, stream);
  return launch_nij<T, 8, J, EPI>(I, K, N, X, ldx, W0, W1, out, ldo, nthreads, stream);
}

// Host entry: I <= 8 tokens per launch (the caller splits larger I).
// Workgroups of up to 8 waves; each lane owns J = 1..8 chunks per row.
template <typename T, int EPI>
hipError_t gemv_launch(int I, int K, int N, const T* X, int64_t ldx, const T* W0,
                       const T* W1, void* out, int64_t ldo, hipStream_t stream) {
  constexpr int E = Elem<T>::per16;
  const int KC = K / E;
  int J = 1;
  while (KC > J * 512 && J < 8) J *= 2;
  const int nwave = (KC + 64 * J - 1) / (64 * J);
  if (nwave > 8) return hipErrorInvalidValue;
  const int nthreads = 64 * nwave;
  if (J == 1) return launch_j<T, EPI, 1>(I, K, N, X, ldx, W0, W1, out, ldo, nthreads, stream);
  if (J == 2) return launch_j<T, EPI, 2>(I, K, N, X, ldx, W0, W1, out, ldo, nthreads, stream);
  if (J == 4) return launch_j<T, EPI, 4>(I, K, N, X, ldx, W0, W1, out, ldo, nthreads, stream);
  return launch_j<T, EPI, 8>(I, K, N, X, ldx, W0, W1, out, ldo, nthreads, stream);
}


template hipError_t gemv_launch<uint16_t, EPI_F32>(int, int, int, const uint16_t*, int64_t,
                                                   const uint16_t*, const uint16_t*, void*,
                                                   int64_t, hipStream_t);
template hipError_t gemv_launch<uint16_t, EPI_DT>(int, int, int, const uint16_t*, int64_t,
                                                  const uint16_t*, const uint16_t*, void*,
                                                  int64_t, hipStream_t);
template hipError_t gemv_launch<uint16_t, EPI_SWIGLU>(int, int, int, const uint16_t*, int64_t,
                                                      const uint16_t*, const uint16_t*, void*,
                                                      int64_t, hipStream_t);
template hipError_t gemv_launch<float, EPI_F32>(int, int, int, const float*, int64_t,
                                                const float*, const float*, void*, int64_t,
                                                hipStream_t);
template hipError_t gemv_launch<float, EPI_DT>(int, int, int, const float*, int64_t,
                                               const float*, const float*, void*, int64_t,
                                               hipStream_t);
template hipError_t gemv_launch<float, EPI_SWIGLU>(int, int, int, const float*, int64_t,
                                                   const float*, const float*, void*, int64_t,
                                                   hipStream_t);

}  // namespace tpk
