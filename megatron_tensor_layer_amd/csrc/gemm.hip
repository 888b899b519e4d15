// Projections for many tokens: C[M, N] = A[M, K] . W[N, K]^T on bf16 MFMA.
//
// Both operands are K-contiguous (activations row-major, weights
// output-major), so each lane's MFMA operand -- 8 consecutive K elements of
// one row -- is a single 16-byte load from either matrix.
//   * workgroup tile BM x BN, K step BK, 4 waves in a WM x WN grid, each wave
//     computing (BM/WM) x (BN/WN) with v_mfma_f32_32x32x16_bf16;
//   * A and W tiles staged in LDS, double-buffered: the next K step's global
//     loads are in flight while MFMA consumes the current buffer; rows are
//     padded by 16 bytes so the 32 rows a 128-bit LDS read touches fall in
//     distinct banks;
//   * the SwiGLU variant stages gate rows f0.. and up rows f0.. of the same
//     F block in one W tile, so a wave holds g and u of the same (m, f) in
//     identical accumulator lanes and writes silu(g) * u once (lecture
//     "Distributed Serving", §4.1: the elementwise op is local to the rank);
//   * workgroups are dispatched round-robin over the 8 XCDs; the linear
//     block id is remapped so that tiles sharing a W block run on the same
//     XCD and its L2 serves the re-reads.
#include "common.h"
#include "kernels.h"

namespace tpk {

namespace {

constexpr int kPad = 8;  // bf16 elements of padding per LDS row

// Row m of the 32x32 accumulator element r (0..15) held by lane `lane` of
// v_mfma_f32_32x32x16_bf16; the column is lane % 32.
__device__ __forceinline__ int acc_row32(int r, int lane) {
  return (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
}

template <int BM, int BN, int BK, int WM, int WN, int EPI>
__global__ void __launch_bounds__(256)
gemm_kernel(int M, int N, int K, const uint16_t* __restrict__ A, int64_t lda,
            const uint16_t* __restrict__ W0, const uint16_t* __restrict__ W1,
            void* __restrict__ out, int64_t ldo) {
  static_assert(WM * WN == 4, "4 waves");
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int MS = TM / 32, NS = TN / 32;
  static_assert(MS >= 1 && NS >= 1 && TM % 32 == 0 && TN % 32 == 0, "wave tile");
  static_assert(EPI != EPI_SWIGLU || NS % 2 == 0, "SwiGLU pairs gate/up subtiles");
  constexpr int LDK = BK + kPad;
  constexpr int KCH = BK / 8;                 // 16-byte chunks per tile row
  constexpr int A_CH = BM * KCH / 256;        // chunks per thread
  constexpr int B_CH = BN * KCH / 256;
  static_assert(A_CH * 256 == BM * KCH && B_CH * 256 == BN * KCH, "tile / thread split");

  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM][LDK];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN][LDK];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  // ---- tile of this workgroup, XCD-aware
  const int mt_n = (M + BM - 1) / BM;
  const int cols_per_tile = (EPI == EPI_SWIGLU) ? BN / 2 : BN;
  const int nt_n = (N + cols_per_tile - 1) / cols_per_tile;
  const int ntiles = mt_n * nt_n;
  int b = blockIdx.x;
  if ((ntiles & 7) == 0) b = (b & 7) * (ntiles >> 3) + (b >> 3);
  const int tm = b % mt_n, tn = b / mt_n;
  const int m0 = tm * BM;
  const int c0 = tn * cols_per_tile;  // first output column

  // ---- global -> register staging
  const int KT = (K + BK - 1) / BK;
  const int KC = K / 8;
  u32x4_t ra[A_CH], rb[B_CH];

  auto load_tiles = [&](int kt) {
#pragma unroll
    for (int s = 0; s < A_CH; ++s) {
      const int q = tid + s * 256;
      const int row = q / KCH, kc = kt * KCH + q % KCH;
      const int m = m0 + row;
      ra[s] = (m < M && kc < KC)
                  ? *reinterpret_cast<const u32x4_t*>(A + (int64_t)m * lda + (int64_t)kc * 8)
                  : u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int s = 0; s < B_CH; ++s) {
      const int q = tid + s * 256;
      const int row = q / KCH, kc = kt * KCH + q % KCH;
      const uint16_t* Wm;
      int n;
      if (EPI == EPI_SWIGLU) {
        Wm = row < BN / 2 ? W0 : W1;
        n = c0 + (row < BN / 2 ? row : row - BN / 2);
      } else {
        Wm = W0;
        n = c0 + row;
      }
      rb[s] = (n < N && kc < KC)
                  ? __builtin_nontemporal_load(
                        reinterpret_cast<const u32x4_t*>(Wm + (int64_t)n * K + (int64_t)kc * 8))
                  : u32x4_t{0u, 0u, 0u, 0u};
    }
  };
  auto store_tiles = [&](int buf) {
#pragma unroll
    for (int s = 0; s < A_CH; ++s) {
      const int q = tid + s * 256;
      *reinterpret_cast<u32x4_t*>(&As[buf][q / KCH][(q % KCH) * 8]) = ra[s];
    }
#pragma unroll
    for (int s = 0; s < B_CH; ++s) {
      const int q = tid + s * 256;
      *reinterpret_cast<u32x4_t*>(&Bs[buf][q / KCH][(q % KCH) * 8]) = rb[s];
    }
  };

  // tile row of W feeding subtile ns of this wave
  auto b_row0 = [&](int ns) {
    if (EPI == EPI_SWIGLU) {
      const int half = NS / 2;
      return (ns < half) ? wn * (TN / 2) + ns * 32 : BN / 2 + wn * (TN / 2) + (ns - half) * 32;
    }
    return wn * TN + ns * 32;
  };

  f32x16_t acc[MS][NS];
#pragma unroll
  for (int i = 0; i < MS; ++i)
#pragma unroll
    for (int j = 0; j < NS; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  load_tiles(0);
  store_tiles(0);
  __syncthreads();

  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < KT) load_tiles(kt + 1);
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int kof = kk * 16 + (lane >> 5) * 8;
      bf16x8_t af[MS], bfr[NS];
#pragma unroll
      for (int i = 0; i < MS; ++i)
        af[i] = *reinterpret_cast<const bf16x8_t*>(&As[buf][wm * TM + i * 32 + (lane & 31)][kof]);
#pragma unroll
      for (int j = 0; j < NS; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8_t*>(&Bs[buf][b_row0(j) + (lane & 31)][kof]);
#pragma unroll
      for (int i = 0; i < MS; ++i)
#pragma unroll
        for (int j = 0; j < NS; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < KT) store_tiles(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue
#pragma unroll
  for (int i = 0; i < MS; ++i) {
#pragma unroll
    for (int j = 0; j < ((EPI == EPI_SWIGLU) ? NS / 2 : NS); ++j) {
      int col;
      if (EPI == EPI_SWIGLU)
        col = c0 + wn * (TN / 2) + j * 32 + (lane & 31);
      else
        col = c0 + wn * TN + j * 32 + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm * TM + i * 32 + acc_row32(r, lane);
        if (m < M && col < N) {
          if constexpr (EPI == EPI_SWIGLU) {
            const float g = acc[i][j][r], u = acc[i][j + NS / 2][r];
            static_cast<uint16_t*>(out)[(int64_t)m * ldo + col] = f32_to_bf16_bits(silu(g) * u);
          } else if constexpr (EPI == EPI_F32) {
            static_cast<float*>(out)[(int64_t)m * ldo + col] = acc[i][j][r];
          } else {
            static_cast<uint16_t*>(out)[(int64_t)m * ldo + col] = f32_to_bf16_bits(acc[i][j][r]);
          }
        }
      }
    }
  }
}

template <int BM, int BN, int BK, int WM, int WN, int EPI>
hipError_t launch_cfg(int M, int N, int K, const uint16_t* A, int64_t lda, const uint16_t* W0,
                      const uint16_t* W1, void* out, int64_t ldo, hipStream_t stream) {
  const int cols = (EPI == EPI_SWIGLU) ? BN / 2 : BN;
  const int ntiles = ((M + BM - 1) / BM) * ((N + cols - 1) / cols);
  hipLaunchKernelGGL((gemm_kernel<BM, BN, BK, WM, WN, EPI>), dim3(ntiles), dim3(256), 0, stream,
                     M, N, K, A, lda, W0, W1, out, ldo);
  return hipGetLastError();
}

}  // namespace

template <int EPI>
hipError_t gemm_launch(int M, int N, int K, const uint16_t* A, int64_t lda, const uint16_t* W0,
                       const uint16_t* W1, void* out, int64_t ldo, hipStream_t stream) {
  if (M <= 64)
    return launch_cfg<64, 128, 64, 2, 2, EPI>(M, N, K, A, lda, W0, W1, out, ldo, stream);
  return launch_cfg<128, 128, 64, 2, 2, EPI>(M, N, K, A, lda, W0, W1, out, ldo, stream);
}

template hipError_t gemm_launch<EPI_F32>(int, int, int, const uint16_t*, int64_t,
                                         const uint16_t*, const uint16_t*, void*, int64_t,
                                         hipStream_t);
template hipError_t gemm_launch<EPI_DT>(int, int, int, const uint16_t*, int64_t,
                                        const uint16_t*, const uint16_t*, void*, int64_t,
                                        hipStream_t);
template hipError_t gemm_launch<EPI_SWIGLU>(int, int, int, const uint16_t*, int64_t,
                                            const uint16_t*, const uint16_t*, void*, int64_t,
                                            hipStream_t);

}  // namespace tpk
