// Internal launchers of the gfx950 kernels (C++ linkage; not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <cmath>

namespace tpk {

// Raise a kernel's dynamic-LDS limit to `bytes` on the current device, once
// per device: the attribute belongs to the kernel on each device.  `done`
// keeps one bit per device already raised (a device index past 63 is raised
// on every call).
inline hipError_t dyn_lds_once(const void* kern, int bytes, std::atomic<uint64_t>& done) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = (dev >= 0 && dev < 64) ? (uint64_t(1) << dev) : 0;
  if (bit && (done.load(std::memory_order_relaxed) & bit)) return hipSuccess;
  e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_relaxed);
  return e;
}

// Split-K workspace layout shared by every kernel that splits K: a fixed
// area of 32-bit arrival counters (zero before the first use; each completed
// call leaves it zero), then the fp32 partial sums.  The fixed size lets
// calls of any shape share one workspace.
constexpr size_t kWsCounterBytes = 8192;
constexpr int kWsMaxCounters = int(kWsCounterBytes / 4);
// Zero the counter area (the first min(bytes, kWsCounterBytes) bytes) of a
// workspace with a fill kernel on `stream`.
hipError_t counters_reset_launch(void* workspace, size_t bytes, hipStream_t stream);

// Size of the library's static scratch array (one per device, held until
// the process ends), and its device address on the current device, looked
// up once per device.  Used only by the entry point for callers that cannot
// allocate.
constexpr size_t kStaticScratchBytes = size_t(32) << 20;
hipError_t static_scratch(void** ptr);

// Largest contraction length (elements) the few-token kernel handles:
// 8 chunks of 16 bytes per lane, 512 lanes.
constexpr int64_t kGemvMaxK16 = 8 * 512 * 8;   // bf16
constexpr int64_t kGemvMaxK32 = 8 * 512 * 4;   // fp32
constexpr int kGemvMaxTokens = 8;

// y[i, n] = sum_k X[i, k] W0[n, k] for I <= 8 tokens (EPI_SWIGLU: W0 gate,
// W1 up, y = silu(.) * (.)).  T = uint16_t (bf16 bits) or float.
template <typename T, int EPI>
hipError_t gemv_launch(int I, int K, int N, const T* X, int64_t ldx, const T* W0,
                       const T* W1, void* out, int64_t ldo, hipStream_t stream);

// Weight-only FP8 few-token product: y[i, n] = S[n] * sum_k X[i, k] e4m3(W[n, k]),
// X bf16, W one OCP E4M3 byte per weight, S fp32 per row (EPI_F32 or
// EPI_SWIGLU with W1/S1 the up matrix); I <= 8, K a multiple of 16 and at
// most kFp8MaxK.
constexpr int kFp8MaxTokens = 8;
constexpr int64_t kFp8MaxK = 16384;
// fmt: kFmtE4M3 or kFmtInt8 (common.h), the code format of W0 and W1.
template <int EPI>
hipError_t gemv_fp8_launch(int I, int K, int N, const uint16_t* X, const uint8_t* W0,
                           const float* S0, const uint8_t* W1, const float* S1, void* out,
                           int64_t ldo, int fmt, hipStream_t stream);

// Same product on bf16 MFMA for 9..64 tokens, weights streamed once from HBM,
// K split over workgroups; `workspace` (splitk_workspace_bytes) holds the
// arrival counters and the fp32 partial sums (layout above).
constexpr int kSplitKMaxTokens = 64;
constexpr int64_t kSplitKMaxK = int64_t(1) << 23;
size_t splitk_workspace_bytes(int I, int K, int N, bool swiglu);
// Whether the split-K kernel is the better choice for this projection: it is
// unless the activations of a full K range do not fit LDS (many tokens, long K).
bool splitk_suits(int I, int K, int N, bool swiglu);
// Whether the split-K kernel can run this projection at all (a K range of
// activations fits LDS); the FP8 path has no tiled alternative.
bool splitk_plannable(int I, int K, int N, bool swiglu);
template <int EPI>
hipError_t splitk_launch(int I, int K, int N, const uint16_t* X, const uint16_t* W0,
                         const uint16_t* W1, void* out, int64_t ldo, void* workspace,
                         hipStream_t stream);
// The weight-only FP8 form of the same kernel (weights as in gemv_fp8_launch:
// E4M3 codes, one fp32 scale per row); same plan and workspace as bf16.
template <int EPI>
hipError_t splitk_fp8_launch(int I, int K, int N, const uint16_t* X, const uint8_t* W0,
                             const float* S0, const uint8_t* W1, const float* S1, void* out,
                             int64_t ldo, void* workspace, int fmt, hipStream_t stream);

// Same product for 9..32 tokens with each workgroup covering the whole K
// axis of two 16-row weight tiles (no workspace); rowstream_suits says when
// it beats the split-K kernel.
constexpr int kRowStreamMaxTokens = 32;
constexpr int kRowStreamMaxK = 1 << 20;
int rowstream_slice(int K);
int rowstream_rows(int N, bool swiglu);
int rowstream_grid(int N, bool swiglu);
bool rowstream_suits(int I, int K, int N, bool swiglu);
template <int EPI>
hipError_t rowstream_launch(int I, int K, int N, const uint16_t* X, const uint16_t* W0,
                            const uint16_t* W1, void* out, int64_t ldo, hipStream_t stream);
// The weight-only FP8 form (weights as in gemv_fp8_launch; EPI_F32 or
// EPI_SWIGLU; K a multiple of 16).
template <int EPI>
hipError_t rowstream_fp8_launch(int I, int K, int N, const uint16_t* X, const uint8_t* W0,
                                const float* S0, const uint8_t* W1, const float* S1, void* out,
                                int64_t ldo, int fmt, hipStream_t stream);

// Same product on bf16 MFMA for any M (128 x 128 or 256 x 128 tiles, by a
// cost model).  When the tiles cannot fill the chip, K is split over
// workgroups and `workspace` (gemm_workspace_bytes, 0 when not split) holds
// the arrival counters and the fp32 partial tiles (layout above).
size_t gemm_workspace_bytes(int M, int N, int K, bool swiglu);
// Largest K of the GEMM kernels: a tile's operand rows (up to 256 x K bf16)
// are addressed with 32-bit byte offsets.
constexpr int64_t kGemmMaxK = int64_t(1) << 22;
template <int EPI>
hipError_t gemm_launch(int M, int N, int K, const uint16_t* A, int64_t lda, const uint16_t* W0,
                       const uint16_t* W1, void* out, int64_t ldo, void* workspace,
                       hipStream_t stream);

// The same GEMM with one-byte weight codes of format fmt (kFmtE4M3 or
// kFmtInt8) and one fp32 scale per weight row (S0; S1 for the up rows of
// EPI_SWIGLU), bf16 activations, 128 x 128 tiles; K a multiple of 16.
// Workspace as gemm_launch (gemm_q8_workspace_bytes).
size_t gemm_q8_workspace_bytes(int M, int N, int K, bool swiglu);
template <int EPI>
hipError_t gemm_q8_launch(int M, int N, int K, const uint16_t* A, int64_t lda, const uint8_t* W0,
                          const float* S0, const uint8_t* W1, const float* S1, void* out,
                          int64_t ldo, void* workspace, int fmt, hipStream_t stream);

// Read-only stream of `bytes` (a multiple of 1 KB, at most 2 GiB) with the
// decode kernels' access pattern; one word per thread of the grid
// (stream_read_sink_words) to `sink`.
size_t stream_read_sink_words();
hipError_t stream_read_launch(const void* buf, size_t bytes, unsigned* sink, hipStream_t stream);

hipError_t reduce_launch(int t, int64_t n, const float* P, bool out_bf16, void* Y,
                         hipStream_t stream);

// h = residual + sum_r P_r (rank order), then x = RMSNorm(h as stored) * gamma
// (x == nullptr: h only) for I rows; one workgroup per row, D <= kNormMaxD.
// P points at the first of the I rows in rank 0's partial; each rank's
// partial holds p_rows rows (I for full rows, more for a sequence shard).
constexpr int kNormMaxD = 32768;
hipError_t residual_rmsnorm_launch(int t, int I, int D, const float* P, int64_t p_rows,
                                   const void* residual, bool h_bf16, void* h, const void* gamma,
                                   bool x_bf16, void* x, float eps, hipStream_t stream);

// Decode attention over the rank's KV cache (head_dim <= 128, at most 32
// query heads per KV group); `workspace` (attn_decode_workspace_bytes, 0
// when the positions are not split) holds counters and chunk states.
size_t attn_decode_workspace_bytes(int B, int nkv, int hd, int Lmax);
hipError_t attn_decode_launch(int B, int nq, int nkv, int hd, int Lmax, const int* lens,
                              const uint16_t* qkv, uint16_t* Kc, uint16_t* Vc, uint16_t* A,
                              void* workspace, hipStream_t stream);

hipError_t attn_core_launch(int I, int S, int nq, int nkv, int hd, const uint16_t* qkv,
                            uint16_t* A, hipStream_t stream);

}  // namespace tpk
