// C ABI of the TP-shard library (declared in include/tpshard.h).
//
// Host side only: validates arguments without touching the GPU, picks a
// kernel family by the token count and enqueues it on the caller's stream.
//   bf16, I <= 8   few-token streaming kernel (VALU dot2), weights read once
//                  (from 5 tokens only for small weight matrices)
//   bf16, I <= 64  split-K or whole-K weight streaming on MFMA (workspace
//                  for split-K partials)
//   bf16, I > 64   MFMA tiled kernel (4-stage LDS pipeline, K split when
//                  the tiles cannot fill the chip)
//   fp32           few-token streaming kernel, 8 tokens per launch
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstring>

#include "../../include/tpshard.h"
#include "common.h"
#include "kernels.h"

namespace {

constexpr int64_t kMaxDim = int64_t(1) << 26;  // per-dimension limit (int indexing)

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Range {
  const char* lo;
  const char* hi;
};
Range rng(const void* p, int64_t bytes) {
  const char* c = static_cast<const char*>(p);
  return Range{c, c + bytes};
}
bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

bool dims_ok(int64_t v) { return v >= 1 && v <= kMaxDim; }

tp_status_t launched(hipError_t e) { return e == hipSuccess ? TP_OK : TP_ERR_LAUNCH; }

// Kernel family for a bf16 projection of I tokens with contraction length K.
enum class Path { Gemv, RowStream, SplitK, Gemm };
Path bf16_path(int64_t I, int64_t K, int64_t N, bool swiglu) {
  // few tokens: weight streaming on VALU; past K = kGemvMaxK16 / 2 the
  // 8-token variant runs out of registers, so 5..8 tokens go to MFMA there
  const int64_t kmax = (I <= 4) ? tpk::kGemvMaxK16 : tpk::kGemvMaxK16 / 2;
  const bool gemv_ok = I <= tpk::kGemvMaxTokens && K <= kmax;
  if (gemv_ok && I <= 4) return Path::Gemv;
  // At 5..8 tokens the VALU kernel's cross-lane sums of 8 token rows limit
  // it on large matrices, where the MFMA kernels win: measured kernel time
  // per call on the Llama TP=8 MLP, 33.1 + 17.0 us against 23.9 + 11.6.  On
  // small ones their fixed costs lose (Qwen2.5-1.5B TP=2 QKV 6.1 us against
  // 4.4).  Crossovers: about 16 MB of weights for the whole-K kernel
  // (o_proj, 16.8 MB: 6.0 against 7.2), 32 MB for split K (QKV, 21 MB:
  // 10.3 against 9.3).
  const double wbytes = 2.0 * (double)K * (double)N * (swiglu ? 2.0 : 1.0);
  if (I <= tpk::kRowStreamMaxTokens && K <= tpk::kRowStreamMaxK && N <= INT32_MAX &&
      (!gemv_ok || wbytes >= 16e6) &&
      tpk::rowstream_suits((int)std::max<int64_t>(I, 9), (int)K, (int)N, swiglu))
    return Path::RowStream;
  if (I <= tpk::kSplitKMaxTokens && K <= tpk::kSplitKMaxK && (!gemv_ok || wbytes >= 32e6) &&
      tpk::splitk_suits((int)I, (int)K, (int)N, swiglu))
    return Path::SplitK;
  return gemv_ok ? Path::Gemv : Path::Gemm;
}

// A projection the GEMM would take with a K beyond its 32-bit operand offsets.
bool gemm_k_too_long(int64_t I, int64_t K, int64_t N, bool swiglu, tp_dtype_t dt) {
  return dt == TP_BF16 && K > tpk::kGemmMaxK && bf16_path(I, K, N, swiglu) == Path::Gemm;
}

// Workspace of one projection (split-K partial sums; 0 when not split).
size_t proj_workspace(int64_t I, int64_t K, int64_t N, bool swiglu, tp_dtype_t dt) {
  if (dt != TP_BF16 || I < 1) return 0;
  switch (bf16_path(I, K, N, swiglu)) {
    case Path::Gemv: return 0;
    case Path::RowStream: return 0;
    case Path::SplitK: return tpk::splitk_workspace_bytes((int)I, (int)K, (int)N, swiglu);
    case Path::Gemm: return tpk::gemm_workspace_bytes((int)I, (int)N, (int)K, swiglu);
  }
  return 0;
}

// One projection out[I, N] = in[I, K] . W[N, K]^T with epilogue EPI.
template <int EPI>
hipError_t project(int64_t I, int64_t K, int64_t N, tp_dtype_t dt, const void* in,
                   const void* W0, const void* W1, void* out, void* ws, hipStream_t s) {
  using tpk::gemm_launch;
  using tpk::gemv_launch;
  // element size of the stored output (fp32 partial or dtype)
  const int64_t osz = (EPI == tpk::EPI_F32 || dt == TP_F32) ? 4 : 2;
  if (dt == TP_BF16) {
    auto X = static_cast<const uint16_t*>(in);
    auto A0 = static_cast<const uint16_t*>(W0);
    auto A1 = static_cast<const uint16_t*>(W1);
    switch (bf16_path(I, K, N, EPI == tpk::EPI_SWIGLU)) {
      case Path::Gemv:
        return gemv_launch<uint16_t, EPI>((int)I, (int)K, (int)N, X, K, A0, A1, out, N, s);
      case Path::RowStream:
        return tpk::rowstream_launch<EPI>((int)I, (int)K, (int)N, X, A0, A1, out, N, s);
      case Path::SplitK:
        return tpk::splitk_launch<EPI>((int)I, (int)K, (int)N, X, A0, A1, out, N, ws, s);
      case Path::Gemm:
        return gemm_launch<EPI>((int)I, (int)N, (int)K, X, K, A0, A1, out, N, ws, s);
    }
  }
  auto X = static_cast<const float*>(in);
  auto A0 = static_cast<const float*>(W0);
  auto A1 = static_cast<const float*>(W1);
  // tokens per launch: 8, or 4 where each lane holds 8 chunks (K > 8192)
  const int64_t step = (K > tpk::kGemvMaxK32 / 2) ? 4 : tpk::kGemvMaxTokens;
  for (int64_t i0 = 0; i0 < I; i0 += step) {
    const int64_t n = (I - i0) < step ? (I - i0) : step;
    hipError_t e = gemv_launch<float, EPI>((int)n, (int)K, (int)N, X + i0 * K, K, A0, A1,
                                           static_cast<char*>(out) + i0 * N * osz, N, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

bool dtype_ok(tp_dtype_t dt) { return dt == TP_F32 || dt == TP_BF16; }
int64_t esize(tp_dtype_t dt) { return dt == TP_F32 ? 4 : 2; }

}  // namespace

extern "C" {

int tp_abi_version(void) { return 1; }

const char* tp_status_string(tp_status_t s) {
  switch (s) {
    case TP_OK: return "TP_OK";
    case TP_ERR_INVALID: return "TP_ERR_INVALID";
    case TP_ERR_MISALIGNED: return "TP_ERR_MISALIGNED";
    case TP_ERR_UNSUPPORTED: return "TP_ERR_UNSUPPORTED";
    case TP_ERR_LAUNCH: return "TP_ERR_LAUNCH";
    case TP_ERR_WORKSPACE: return "TP_ERR_WORKSPACE";
  }
  return "TP_ERR_UNKNOWN";
}

size_t tp_shard_mlp_workspace_size(int64_t I, int64_t D, int64_t F_local, tp_dtype_t dt) {
  if (!dtype_ok(dt) || I < 1 || I > kMaxDim || !dims_ok(D) || !dims_ok(F_local)) return 0;
  // gate/up+SwiGLU then down run one after the other and share the workspace
  return std::max(proj_workspace(I, D, F_local, true, dt),
                  proj_workspace(I, F_local, D, false, dt));
}

}  // extern "C"

namespace {
// Every check of tp_shard_mlp except those on the workspace; TP_OK when the
// call may go ahead (I == 0 included).
tp_status_t mlp_args_status(int64_t I, int64_t D, int64_t F_local, tp_dtype_t dt, const void* X,
                            const void* W_gate, const void* W_up, const void* W_down,
                            const void* H, const float* P) {
  if (!dtype_ok(dt) || I < 0 || I > kMaxDim || !dims_ok(D) || !dims_ok(F_local))
    return TP_ERR_INVALID;
  if (I == 0) return TP_OK;
  if (!X || !W_gate || !W_up || !W_down || !H || !P) return TP_ERR_INVALID;
  if ((D % 8) || (F_local % 8)) return TP_ERR_MISALIGNED;
  if (!aligned16(X) || !aligned16(W_gate) || !aligned16(W_up) || !aligned16(W_down) ||
      !aligned16(H) || !aligned16(P))
    return TP_ERR_MISALIGNED;
  const int64_t es = esize(dt);
  const Range rX = rng(X, I * D * es), rG = rng(W_gate, F_local * D * es),
              rU = rng(W_up, F_local * D * es), rD = rng(W_down, D * F_local * es),
              rH = rng(H, I * F_local * es), rP = rng(P, I * D * 4);
  for (Range in : {rX, rG, rU, rD})
    if (overlap(rH, in) || overlap(rP, in)) return TP_ERR_INVALID;
  if (overlap(rH, rP)) return TP_ERR_INVALID;
  if (dt == TP_F32 && (D > tpk::kGemvMaxK32 || F_local > tpk::kGemvMaxK32))
    return TP_ERR_UNSUPPORTED;
  if (gemm_k_too_long(I, D, F_local, true, dt) || gemm_k_too_long(I, F_local, D, false, dt))
    return TP_ERR_UNSUPPORTED;
  return TP_OK;
}
}  // namespace

extern "C" {

tp_status_t tp_shard_mlp(int64_t I, int64_t D, int64_t F_local, tp_dtype_t dt, const void* X,
                         const void* W_gate, const void* W_up, const void* W_down, void* H,
                         float* P, void* workspace, size_t workspace_bytes, void* stream) {
  const tp_status_t st = mlp_args_status(I, D, F_local, dt, X, W_gate, W_up, W_down, H, P);
  if (st != TP_OK || I == 0) return st;
  const size_t need = tp_shard_mlp_workspace_size(I, D, F_local, dt);
  if (need > 0) {
    if (workspace == nullptr || workspace_bytes < need) return TP_ERR_WORKSPACE;
    if (!aligned16(workspace)) return TP_ERR_MISALIGNED;
    const int64_t es = esize(dt);
    const Range rW = rng(workspace, (int64_t)need);
    for (Range o : {rng(X, I * D * es), rng(W_gate, F_local * D * es),
                    rng(W_up, F_local * D * es), rng(W_down, D * F_local * es),
                    rng(H, I * F_local * es), rng(P, I * D * 4)})
      if (overlap(rW, o)) return TP_ERR_INVALID;
  }

  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();  // clear a stale error so the checks below are ours
  hipError_t e = project<tpk::EPI_SWIGLU>(I, D, F_local, dt, X, W_gate, W_up, H, workspace, s);
  if (e != hipSuccess) return TP_ERR_LAUNCH;
  e = project<tpk::EPI_F32>(I, F_local, D, dt, H, W_down, nullptr, P, workspace, s);
  return launched(e);
}

size_t tp_shard_mlp_noalloc_max_workspace(void) { return tpk::kStaticScratchBytes; }

tp_status_t tp_shard_mlp_noalloc(int64_t I, int64_t D, int64_t F_local, tp_dtype_t dt,
                                 const void* X, const void* W_gate, const void* W_up,
                                 const void* W_down, void* H, float* P, void* stream) {
  const tp_status_t st = mlp_args_status(I, D, F_local, dt, X, W_gate, W_up, W_down, H, P);
  if (st != TP_OK || I == 0) return st;
  const size_t need = tp_shard_mlp_workspace_size(I, D, F_local, dt);
  if (need > tpk::kStaticScratchBytes) return TP_ERR_WORKSPACE;
  if (need == 0) return tp_shard_mlp(I, D, F_local, dt, X, W_gate, W_up, W_down, H, P, nullptr,
                                     0, stream);
  void* scratch = nullptr;
  (void)hipGetLastError();
  if (tpk::static_scratch(&scratch) != hipSuccess) return TP_ERR_LAUNCH;
  // the array keeps the last call's contents: clear the counters first
  if (tpk::counters_reset_launch(scratch, need, static_cast<hipStream_t>(stream)) != hipSuccess)
    return TP_ERR_LAUNCH;
  return tp_shard_mlp(I, D, F_local, dt, X, W_gate, W_up, W_down, H, P, scratch,
                      tpk::kStaticScratchBytes, stream);
}

size_t tp_shard_attn_proj_workspace_size(tp_attn_phase_t phase, int64_t I, int64_t D,
                                         int64_t n_q_local, int64_t n_kv_local,
                                         int64_t head_dim, tp_dtype_t dt) {
  if (!dtype_ok(dt) || I < 1 || I > kMaxDim || !dims_ok(D) || !dims_ok(n_q_local) ||
      !dims_ok(head_dim))
    return 0;
  if (phase == TP_ATTN_QKV) {
    if (!dims_ok(n_kv_local)) return 0;
    return proj_workspace(I, D, (n_q_local + 2 * n_kv_local) * head_dim, false, dt);
  }
  if (phase == TP_ATTN_O) return proj_workspace(I, n_q_local * head_dim, D, false, dt);
  return 0;
}

tp_status_t tp_shard_attn_proj(tp_attn_phase_t phase, int64_t I, int64_t D, int64_t n_q_local,
                               int64_t n_kv_local, int64_t head_dim, tp_dtype_t dt,
                               const void* in, const void* W, void* out, void* workspace,
                               size_t workspace_bytes, void* stream) {
  if (phase != TP_ATTN_QKV && phase != TP_ATTN_O) return TP_ERR_INVALID;
  if (!dtype_ok(dt) || I < 0 || I > kMaxDim || !dims_ok(D) || !dims_ok(n_q_local) ||
      !dims_ok(head_dim) || (phase == TP_ATTN_QKV && !dims_ok(n_kv_local)))
    return TP_ERR_INVALID;
  const int64_t K = (phase == TP_ATTN_QKV) ? D : n_q_local * head_dim;
  const int64_t N = (phase == TP_ATTN_QKV) ? (n_q_local + 2 * n_kv_local) * head_dim : D;
  if (K > kMaxDim || N > kMaxDim) return TP_ERR_INVALID;
  if (I == 0) return TP_OK;
  if (!in || !W || !out) return TP_ERR_INVALID;
  if ((D % 8) || (head_dim % 8)) return TP_ERR_MISALIGNED;
  if (!aligned16(in) || !aligned16(W) || !aligned16(out)) return TP_ERR_MISALIGNED;
  const int64_t es = esize(dt);
  const int64_t osz = (phase == TP_ATTN_O) ? 4 : es;
  const Range rIn = rng(in, I * K * es), rW = rng(W, N * K * es), rO = rng(out, I * N * osz);
  if (overlap(rO, rIn) || overlap(rO, rW)) return TP_ERR_INVALID;
  if (dt == TP_F32 && K > tpk::kGemvMaxK32) return TP_ERR_UNSUPPORTED;
  if (gemm_k_too_long(I, K, N, false, dt)) return TP_ERR_UNSUPPORTED;
  const size_t need =
      tp_shard_attn_proj_workspace_size(phase, I, D, n_q_local, n_kv_local, head_dim, dt);
  if (need > 0) {
    if (workspace == nullptr || workspace_bytes < need) return TP_ERR_WORKSPACE;
    if (!aligned16(workspace)) return TP_ERR_MISALIGNED;
    const Range rWs = rng(workspace, (int64_t)need);
    if (overlap(rWs, rIn) || overlap(rWs, rW) || overlap(rWs, rO)) return TP_ERR_INVALID;
  }

  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (phase == TP_ATTN_QKV)
    return launched(project<tpk::EPI_DT>(I, K, N, dt, in, W, nullptr, out, workspace, s));
  return launched(project<tpk::EPI_F32>(I, K, N, dt, in, W, nullptr, out, workspace, s));
}

tp_status_t tp_partial_reduce(int32_t t, int64_t n, const float* partials, tp_dtype_t out_dt,
                              void* Y, void* stream) {
  if (t < 1 || n < 0 || !dtype_ok(out_dt)) return TP_ERR_INVALID;
  if (n == 0) return TP_OK;
  if (!partials || !Y) return TP_ERR_INVALID;
  if (n % 8) return TP_ERR_MISALIGNED;
  if (!aligned16(partials) || !aligned16(Y)) return TP_ERR_MISALIGNED;
  if ((int64_t)t * n / 4 > (int64_t(1) << 40)) return TP_ERR_UNSUPPORTED;
  if ((n / 4 + 255) / 256 > INT32_MAX) return TP_ERR_UNSUPPORTED;
  if (overlap(rng(Y, n * esize(out_dt)), rng(partials, (int64_t)t * n * 4)))
    return TP_ERR_INVALID;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  return launched(tpk::reduce_launch(t, n, partials, out_dt == TP_BF16, Y, s));
}

namespace {
// The one-byte path for I tokens: the few-token VALU kernel up to 4 tokens
// (K within kFp8MaxK), the split-K MFMA kernel from 5 to 64 (measured on the
// Llama-3.1-70B TP=8 share: 27.0 us against about 33 at 4 tokens, 36.8
// against about 33 at 5), and the one-byte GEMM for more tokens or when no
// split-K plan fits (the VALU kernel up to 8 tokens).
enum class Fp8Path { None, Gemv, SplitK, Gemm };
Fp8Path fp8_path(int64_t I, int64_t D, int64_t F_local) {
  if (I < 1) return Fp8Path::None;
  const bool gemv_ok = I <= tpk::kFp8MaxTokens && D <= tpk::kFp8MaxK && F_local <= tpk::kFp8MaxK;
  if (gemv_ok && I <= 4) return Fp8Path::Gemv;
  if (I <= tpk::kSplitKMaxTokens && tpk::splitk_plannable((int)I, (int)D, (int)F_local, true) &&
      tpk::splitk_plannable((int)I, (int)F_local, (int)D, false))
    return Fp8Path::SplitK;
  return gemv_ok ? Fp8Path::Gemv : Fp8Path::Gemm;
}

// On the MFMA path (from 5 tokens), the FP8 down projection streams whole K
// per workgroup when the row-streaming kernel suits its shape, as the bf16
// down does from 9 tokens: at 5..8 tokens it beats split K too (Llama TP=8
// MLP: 31.0 us against 33.1-33.5).
bool fp8_down_rowstream(int64_t I, int64_t D, int64_t F_local) {
  return I <= tpk::kRowStreamMaxTokens && F_local <= tpk::kRowStreamMaxK && D <= INT32_MAX &&
         tpk::rowstream_suits((int)std::max<int64_t>(I, 9), (int)F_local, (int)D, false);
}
}  // namespace

size_t tp_shard_mlp_fp8_workspace_size(int64_t I, int64_t D, int64_t F_local) {
  if (I < 1 || I > kMaxDim || !dims_ok(D) || !dims_ok(F_local) || (D % 16) || (F_local % 16))
    return 0;
  const Fp8Path path = fp8_path(I, D, F_local);
  if (path == Fp8Path::Gemm)
    return std::max(tpk::gemm_q8_workspace_bytes((int)I, (int)F_local, (int)D, true),
                    tpk::gemm_q8_workspace_bytes((int)I, (int)D, (int)F_local, false));
  if (path != Fp8Path::SplitK) return 0;
  const size_t down = fp8_down_rowstream(I, D, F_local)
                          ? 0
                          : tpk::splitk_workspace_bytes((int)I, (int)F_local, (int)D, false);
  return std::max(tpk::splitk_workspace_bytes((int)I, (int)D, (int)F_local, true), down);
}

}  // extern "C"

namespace {
// The weight-only MLP share with one-byte codes of format fmt (kFmtE4M3 or
// kFmtInt8) and one fp32 scale per output row; both formats run the same
// kernels and plans, only the decode of a 16-byte chunk of codes differs.
tp_status_t mlp_bytew(int fmt, int64_t I, int64_t D, int64_t F_local, const void* X,
                      const void* W_gate, const float* s_gate, const void* W_up,
                      const float* s_up, const void* W_down, const float* s_down, void* H,
                      float* P, void* workspace, size_t workspace_bytes, void* stream) {
  if (I < 0 || I > kMaxDim || !dims_ok(D) || !dims_ok(F_local)) return TP_ERR_INVALID;
  if (I == 0) return TP_OK;
  if (!X || !W_gate || !s_gate || !W_up || !s_up || !W_down || !s_down || !H || !P)
    return TP_ERR_INVALID;
  if ((D % 16) || (F_local % 16)) return TP_ERR_MISALIGNED;
  for (const void* p : {X, W_gate, W_up, W_down, static_cast<const void*>(H),
                        static_cast<const void*>(P)})
    if (!aligned16(p)) return TP_ERR_MISALIGNED;
  for (const float* p : {s_gate, s_up, s_down})
    if (reinterpret_cast<uintptr_t>(p) & 3u) return TP_ERR_MISALIGNED;
  const Range rX = rng(X, I * D * 2), rG = rng(W_gate, F_local * D), rU = rng(W_up, F_local * D),
              rD = rng(W_down, D * F_local), rsg = rng(s_gate, F_local * 4),
              rsu = rng(s_up, F_local * 4), rsd = rng(s_down, D * 4),
              rH = rng(H, I * F_local * 2), rP = rng(P, I * D * 4);
  for (Range in : {rX, rG, rU, rD, rsg, rsu, rsd})
    if (overlap(rH, in) || overlap(rP, in)) return TP_ERR_INVALID;
  if (overlap(rH, rP)) return TP_ERR_INVALID;
  const Fp8Path path = fp8_path(I, D, F_local);
  if (path == Fp8Path::None) return TP_ERR_UNSUPPORTED;
  if (path == Fp8Path::Gemm && (D > tpk::kGemmMaxK || F_local > tpk::kGemmMaxK))
    return TP_ERR_UNSUPPORTED;
  const size_t need = tp_shard_mlp_fp8_workspace_size(I, D, F_local);
  if (need > 0) {
    if (workspace == nullptr || workspace_bytes < need) return TP_ERR_WORKSPACE;
    if (!aligned16(workspace)) return TP_ERR_MISALIGNED;
    const Range rW = rng(workspace, (int64_t)need);
    for (Range o : {rX, rG, rU, rD, rsg, rsu, rsd, rH, rP})
      if (overlap(rW, o)) return TP_ERR_INVALID;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  auto Xb = static_cast<const uint16_t*>(X);
  auto Hb = static_cast<const uint16_t*>(H);
  auto g8 = static_cast<const uint8_t*>(W_gate), u8 = static_cast<const uint8_t*>(W_up),
       d8 = static_cast<const uint8_t*>(W_down);
  hipError_t e;
  if (path == Fp8Path::Gemv) {
    e = tpk::gemv_fp8_launch<tpk::EPI_SWIGLU>((int)I, (int)D, (int)F_local, Xb, g8, s_gate, u8,
                                              s_up, H, F_local, fmt, s);
    if (e != hipSuccess) return TP_ERR_LAUNCH;
    return launched(tpk::gemv_fp8_launch<tpk::EPI_F32>((int)I, (int)F_local, (int)D, Hb, d8,
                                                       s_down, nullptr, nullptr, P, D, fmt, s));
  }
  if (path == Fp8Path::Gemm) {
    e = tpk::gemm_q8_launch<tpk::EPI_SWIGLU>((int)I, (int)F_local, (int)D, Xb, D, g8, s_gate, u8,
                                             s_up, H, F_local, workspace, fmt, s);
    if (e != hipSuccess) return TP_ERR_LAUNCH;
    return launched(tpk::gemm_q8_launch<tpk::EPI_F32>((int)I, (int)D, (int)F_local, Hb, F_local,
                                                      d8, s_down, nullptr, nullptr, P, D,
                                                      workspace, fmt, s));
  }
  e = tpk::splitk_fp8_launch<tpk::EPI_SWIGLU>((int)I, (int)D, (int)F_local, Xb, g8, s_gate, u8,
                                              s_up, H, F_local, workspace, fmt, s);
  if (e != hipSuccess) return TP_ERR_LAUNCH;
  if (fp8_down_rowstream(I, D, F_local))
    return launched(tpk::rowstream_fp8_launch<tpk::EPI_F32>((int)I, (int)F_local, (int)D, Hb, d8,
                                                            s_down, nullptr, nullptr, P, D, fmt,
                                                            s));
  return launched(tpk::splitk_fp8_launch<tpk::EPI_F32>((int)I, (int)F_local, (int)D, Hb, d8,
                                                       s_down, nullptr, nullptr, P, D, workspace,
                                                       fmt, s));
}
}  // namespace

extern "C" {

tp_status_t tp_shard_mlp_fp8(int64_t I, int64_t D, int64_t F_local, const void* X,
                             const void* W_gate, const float* s_gate, const void* W_up,
                             const float* s_up, const void* W_down, const float* s_down,
                             void* H, float* P, void* workspace, size_t workspace_bytes,
                             void* stream) {
  return mlp_bytew(tpk::kFmtE4M3, I, D, F_local, X, W_gate, s_gate, W_up, s_up, W_down, s_down,
                   H, P, workspace, workspace_bytes, stream);
}

size_t tp_shard_mlp_int8_workspace_size(int64_t I, int64_t D, int64_t F_local) {
  return tp_shard_mlp_fp8_workspace_size(I, D, F_local);
}

tp_status_t tp_shard_mlp_int8(int64_t I, int64_t D, int64_t F_local, const void* X,
                              const void* W_gate, const float* s_gate, const void* W_up,
                              const float* s_up, const void* W_down, const float* s_down,
                              void* H, float* P, void* workspace, size_t workspace_bytes,
                              void* stream) {
  return mlp_bytew(tpk::kFmtInt8, I, D, F_local, X, W_gate, s_gate, W_up, s_up, W_down, s_down,
                   H, P, workspace, workspace_bytes, stream);
}

tp_status_t tp_residual_rmsnorm(int32_t t, int64_t I, int64_t D, const float* partials,
                                const void* residual, tp_dtype_t h_dt, void* h,
                                const void* gamma, tp_dtype_t x_dt, void* x, float eps,
                                void* stream) {
  if (t < 0 || I < 0 || I > INT32_MAX || !dims_ok(D) || !dtype_ok(h_dt) || !dtype_ok(x_dt))
    return TP_ERR_INVALID;
  if (!(eps >= 0.0f) || eps > 3.0e38f) return TP_ERR_INVALID;  // rejects NaN and inf too
  if (I == 0) return TP_OK;
  if (!h || (t > 0 && !partials) || (t == 0 && !residual) || (!gamma) != (!x))
    return TP_ERR_INVALID;
  if (D % 8) return TP_ERR_MISALIGNED;
  if (D > tpk::kNormMaxD) return TP_ERR_UNSUPPORTED;
  for (const void* p : {static_cast<const void*>(partials), residual, static_cast<const void*>(h),
                        gamma, static_cast<const void*>(x)})
    if (p && !aligned16(p)) return TP_ERR_MISALIGNED;
  const int64_t n = I * D;
  const Range rP = rng(partials, (int64_t)t * n * 4), rR = rng(residual, residual ? n * esize(h_dt) : 0),
              rH = rng(h, n * esize(h_dt)), rG = rng(gamma, gamma ? D * esize(x_dt) : 0),
              rX = rng(x, x ? n * esize(x_dt) : 0);
  if (t > 0 && overlap(rH, rP)) return TP_ERR_INVALID;
  if (residual && residual != h && overlap(rH, rR)) return TP_ERR_INVALID;  // exact alias is in place
  if (x) {
    for (Range o : {rP, rR, rH, rG})
      if (overlap(rX, o)) return TP_ERR_INVALID;
    if (overlap(rH, rG)) return TP_ERR_INVALID;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  return launched(tpk::residual_rmsnorm_launch(t, (int)I, (int)D, partials, I, residual,
                                               h_dt == TP_BF16, h, gamma, x_dt == TP_BF16, x,
                                               eps, s));
}

tp_status_t tp_reduce_scatter_rmsnorm(int32_t t, int32_t rank, int64_t I, int64_t D,
                                      const float* partials, const void* residual,
                                      tp_dtype_t h_dt, void* h, const void* gamma,
                                      tp_dtype_t x_dt, void* x, float eps, void* stream) {
  if (t < 1 || rank < 0 || rank >= t || I < 0 || I > INT32_MAX || !dims_ok(D) ||
      !dtype_ok(h_dt) || !dtype_ok(x_dt))
    return TP_ERR_INVALID;
  if (!(eps >= 0.0f) || eps > 3.0e38f) return TP_ERR_INVALID;
  if (I % t) return TP_ERR_INVALID;  // the sequence splits evenly over the ranks
  if (I == 0) return TP_OK;
  if (!partials || !h || (!gamma) != (!x)) return TP_ERR_INVALID;
  if (D % 8) return TP_ERR_MISALIGNED;
  if (D > tpk::kNormMaxD) return TP_ERR_UNSUPPORTED;
  for (const void* p : {static_cast<const void*>(partials), residual, static_cast<const void*>(h),
                        gamma, static_cast<const void*>(x)})
    if (p && !aligned16(p)) return TP_ERR_MISALIGNED;
  const int64_t Is = I / t, ns = Is * D;
  const Range rP = rng(partials, (int64_t)t * I * D * 4),
              rR = rng(residual, residual ? ns * esize(h_dt) : 0), rH = rng(h, ns * esize(h_dt)),
              rG = rng(gamma, gamma ? D * esize(x_dt) : 0), rX = rng(x, x ? ns * esize(x_dt) : 0);
  if (overlap(rH, rP)) return TP_ERR_INVALID;
  if (residual && residual != h && overlap(rH, rR)) return TP_ERR_INVALID;
  if (x) {
    for (Range o : {rP, rR, rH, rG})
      if (overlap(rX, o)) return TP_ERR_INVALID;
    if (overlap(rH, rG)) return TP_ERR_INVALID;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  return launched(tpk::residual_rmsnorm_launch(t, (int)Is, (int)D, partials + rank * ns, I,
                                               residual, h_dt == TP_BF16, h, gamma,
                                               x_dt == TP_BF16, x, eps, s));
}

namespace {
// Shared checks of the decode-attention sizes; TP_OK if supported.
tp_status_t decode_sizes(int64_t B, int64_t nq, int64_t nkv, int64_t hd, int64_t Lmax) {
  if (B < 0 || B > INT32_MAX || nq < 1 || nq > 65535 || nkv < 1 || nkv > nq || hd < 1 ||
      Lmax < 1 || Lmax > INT32_MAX)
    return TP_ERR_INVALID;
  if (nq % nkv) return TP_ERR_INVALID;  // every KV group serves the same number of heads
  if (hd % 8 || Lmax % 8) return TP_ERR_MISALIGNED;
  if (hd > 128 || nq / nkv > 32) return TP_ERR_UNSUPPORTED;
  if (B * nkv * Lmax * hd * 2 >= (int64_t(1) << 31)) return TP_ERR_UNSUPPORTED;
  if (B * (nq + 2 * nkv) * hd * 2 >= (int64_t(1) << 31)) return TP_ERR_UNSUPPORTED;
  return TP_OK;
}
}  // namespace

size_t tp_attn_decode_workspace_size(int64_t B, int64_t n_q_local, int64_t n_kv_local,
                                     int64_t head_dim, int64_t L_max) {
  if (decode_sizes(B, n_q_local, n_kv_local, head_dim, L_max) != TP_OK || B == 0) return 0;
  return tpk::attn_decode_workspace_bytes((int)B, (int)n_kv_local, (int)head_dim, (int)L_max);
}

tp_status_t tp_attn_decode(int64_t B, int64_t n_q_local, int64_t n_kv_local, int64_t head_dim,
                           int64_t L_max, const int32_t* lens, const void* qkv, void* K_cache,
                           void* V_cache, void* A, void* workspace, size_t workspace_bytes,
                           void* stream) {
  const tp_status_t st = decode_sizes(B, n_q_local, n_kv_local, head_dim, L_max);
  if (st != TP_OK) return st;
  if (B == 0) return TP_OK;
  if (!lens || !qkv || !K_cache || !V_cache || !A) return TP_ERR_INVALID;
  if (!aligned16(qkv) || !aligned16(K_cache) || !aligned16(V_cache) || !aligned16(A) ||
      (reinterpret_cast<uintptr_t>(lens) & 3u))
    return TP_ERR_MISALIGNED;
  const int64_t N = (n_q_local + 2 * n_kv_local) * head_dim;
  const int64_t cache = B * n_kv_local * L_max * head_dim * 2;
  const Range rL = rng(lens, B * 4), rQ = rng(qkv, B * N * 2), rK = rng(K_cache, cache),
              rV = rng(V_cache, cache), rA = rng(A, B * n_q_local * head_dim * 2);
  for (Range in : {rL, rQ, rK, rV})
    if (overlap(rA, in)) return TP_ERR_INVALID;
  for (Range in : {rL, rQ, rV})
    if (overlap(rK, in)) return TP_ERR_INVALID;
  for (Range in : {rL, rQ})
    if (overlap(rV, in)) return TP_ERR_INVALID;
  const size_t need = tp_attn_decode_workspace_size(B, n_q_local, n_kv_local, head_dim, L_max);
  if (need > 0) {
    if (workspace == nullptr || workspace_bytes < need) return TP_ERR_WORKSPACE;
    if (!aligned16(workspace)) return TP_ERR_MISALIGNED;
    const Range rW = rng(workspace, (int64_t)need);
    for (Range o : {rL, rQ, rK, rV, rA})
      if (overlap(rW, o)) return TP_ERR_INVALID;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  return launched(tpk::attn_decode_launch(
      (int)B, (int)n_q_local, (int)n_kv_local, (int)head_dim, (int)L_max, lens,
      static_cast<const uint16_t*>(qkv), static_cast<uint16_t*>(K_cache),
      static_cast<uint16_t*>(V_cache), static_cast<uint16_t*>(A), need ? workspace : nullptr, s));
}

tp_status_t tp_attn_core(int64_t I, int64_t S, int64_t n_q_local, int64_t n_kv_local,
                         int64_t head_dim, const void* qkv, void* A, void* stream) {
  if (I < 0 || I > INT32_MAX || !dims_ok(S) || !dims_ok(n_kv_local) || n_q_local < 1 ||
      n_q_local > 65535 || head_dim < 1 || n_kv_local > n_q_local)
    return TP_ERR_INVALID;
  if (I == 0) return TP_OK;
  if (I % S) return TP_ERR_INVALID;
  if (head_dim > 256) return TP_ERR_UNSUPPORTED;
  if (!qkv || !A) return TP_ERR_INVALID;
  if (head_dim % 8) return TP_ERR_MISALIGNED;
  if (!aligned16(qkv) || !aligned16(A)) return TP_ERR_MISALIGNED;
  const int64_t N = (n_q_local + 2 * n_kv_local) * head_dim;
  if (I * N * 2 >= (int64_t(1) << 31)) return TP_ERR_UNSUPPORTED;  // 32-bit buffer offsets
  if (overlap(rng(A, I * n_q_local * head_dim * 2), rng(qkv, I * N * 2))) return TP_ERR_INVALID;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  return launched(tpk::attn_core_launch((int)I, (int)S, (int)n_q_local, (int)n_kv_local,
                                        (int)head_dim, static_cast<const uint16_t*>(qkv),
                                        static_cast<uint16_t*>(A), s));
}

tp_status_t tp_workspace_reset(void* workspace, size_t workspace_bytes, void* stream) {
  if (!workspace || workspace_bytes == 0) return TP_ERR_INVALID;
  if (!aligned16(workspace)) return TP_ERR_MISALIGNED;
  (void)hipGetLastError();
  return launched(
      tpk::counters_reset_launch(workspace, workspace_bytes, static_cast<hipStream_t>(stream)));
}

size_t tp_stream_read_sink_words(void) { return tpk::stream_read_sink_words(); }

tp_status_t tp_stream_read(const void* buf, size_t bytes, uint32_t* sink, size_t sink_words,
                           void* stream) {
  if (!buf || !sink || bytes == 0 || bytes > (size_t(1) << 31)) return TP_ERR_INVALID;
  if ((bytes % 1024) || !aligned16(buf) || !aligned16(sink)) return TP_ERR_MISALIGNED;
  const size_t need = tpk::stream_read_sink_words();
  if (need == 0 || sink_words < need) return TP_ERR_INVALID;
  if (overlap(rng(buf, (int64_t)bytes), rng(sink, (int64_t)(need * 4)))) return TP_ERR_INVALID;
  (void)hipGetLastError();
  return launched(tpk::stream_read_launch(buf, bytes, sink, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
