// Decode projections for 9..32 tokens whose weight matrix has enough rows to
// give every CU its own: y[m, n] = sum_k X[m, k] W[n, k] on bf16 MFMA, each
// workgroup covering the whole K axis of its rows, so no partial sums leave
// the workgroup.
//
// Decode reads each weight of the rank's shard once per step (lecture
// "Distributed Serving", §1.1 and §3.4).  Splitting K over workgroups lets
// each stage a slice of the activations once, but its cross-workgroup finish
// (partials written, one atomic, the last arrival reading them back) is a
// chain of dependent memory round trips at the end of the kernel.  Here:
//   * a workgroup owns two weight tiles of up to 16 rows (a gate tile and the
//     up tile of the same F rows for SwiGLU), as few rows as give about one
//     workgroup per CU, and eight waves: wave w streams tile
//     w % 2 over K slice w / 2 of four, rows whole cache lines at a time (one
//     load instruction: 4 rows x 256 contiguous bytes), two groups of 128 K
//     in flight, each group transposed through a private 4 KB LDS tile into
//     the B operand of v_mfma_f32_16x16x32_bf16;
//   * the activations stream through LDS in chunks of 256 K per slice,
//     double-buffered, by direct global->LDS copies (16-byte slots
//     XOR-swizzled by token); every CU reads all of X, which at these token
//     counts is no more than its share of the weights;
//   * the four K slices of a tile are summed through LDS in slice order
//     (deterministic) and stored with the epilogue (fp32, bf16, silu(g) * u);
//   * weight-only FP8 (OCP E4M3 codes, one fp32 scale per row): a group of
//     128 K is 128 bytes per row, two load instructions of 8 rows x 128
//     bytes, four groups in flight (the bf16 path's bytes); each 16-byte
//     chunk of codes is decoded exactly into two bf16 chunks on its way into
//     the transpose tile, and the summed rows are scaled in the epilogue.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace tpk {

namespace {

constexpr int kGK = 128;        // K per streamed weight group
constexpr int kKC = 256;        // K per activation chunk (two groups)
constexpr int kKW = 4;          // K slices per workgroup
constexpr int kTiles = 2;       // 16-row weight tiles per workgroup
constexpr int kWaves = kKW * kTiles;
constexpr int kThreads = 64 * kWaves;
constexpr int kTileBytes = 16 * kGK * 2;   // one wave's transpose tile
constexpr uint32_t kOob = 0x80000000u;
constexpr int kCUs = 256;

template <int MT>
constexpr int xslice_bytes() { return 16 * MT * kKC * 2; }          // one slice's chunk
template <int MT>
constexpr int xbuf_bytes() { return kKW * xslice_bytes<MT>(); }      // one chunk of all slices
template <int MT>
constexpr int lds_bytes() { return 2 * xbuf_bytes<MT>() + kWaves * kTileBytes; }
static_assert(lds_bytes<2>() <= 160 * 1024, "two chunks of 32 tokens and the tiles fit LDS");

// X DMA instructions per wave per chunk: each slice's chunk is 16 MT token
// rows of 512 bytes = 8 MT instructions of 1 KB.
template <int MT>
constexpr int xpw() { return kKW * 8 * MT / kWaves; }

template <int MT, int EPI, int P, int WF>
__global__ void __launch_bounds__(kThreads)
rowstream_kernel(int I, int K, int N, const uint16_t* __restrict__ X,
                 const void* __restrict__ W0, const void* __restrict__ W1,
                 const float* __restrict__ S0, const float* __restrict__ S1, int KS,
                 int RPT, void* __restrict__ out, int64_t ldo) {
  constexpr bool F8 = WF != kWBf16;  // one-byte codes with a row scale
  constexpr int XPW = xpw<MT>();
  constexpr int ES = F8 ? 1 : 2;   // bytes per weight
  constexpr int LPG = F8 ? 2 : 4;  // load instructions per 128-K group
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tw = wave & 1, sl = wave >> 1;  // tile, K slice
  unsigned char* tile = lds + 2 * xbuf_bytes<MT>() + wave * kTileBytes;

  // ---- this wave's RPT (<= 16) weight rows, padded to a 16-row MFMA tile;
  //      rows past RPT or past the matrix read zero and fetch nothing
  int wrow0;
  const void* wmat;
  if constexpr (EPI == EPI_SWIGLU) {
    wrow0 = blockIdx.x * RPT;  // the same F rows of gate (tile 0) and up (tile 1)
    wmat = tw == 0 ? W0 : W1;
  } else {
    wrow0 = (blockIdx.x * 2 + tw) * RPT;
    wmat = W0;
  }
  const int rows = max(0, min(RPT, N - wrow0));
  const __amdgpu_buffer_rsrc_t wr =
      make_rsrc_uniform(static_cast<const unsigned char*>(wmat) + (rows ? (int64_t)wrow0 * K * ES : 0),
                (uint32_t)rows * (uint32_t)K * (uint32_t)ES);
  const int kb = sl * KS, ke = min(K, kb + KS);  // this wave's K slice
  const int NC = KS / kKC;                       // chunks per slice (same for all)
  const int NG = 2 * NC;

  // group g of the slice, instruction p: bf16 rows 4p + lane/16, 16-byte
  // chunk lane%16 (8 K); FP8 rows 8p + lane/8, chunk lane%8 (16 K)
  auto issue_w = [&](int g, u32x4_t (&v)[LPG]) {
    constexpr int KPC = 16 / ES;    // K per 16-byte chunk
    constexpr int CPR = kGK / KPC;  // chunks per row of a group: 16 (bf16), 8 (FP8)
    constexpr int RPI = 64 / CPR;   // rows per load instruction: 4, 8
    static_assert(RPI * LPG == 16, "a group is 16 rows");
    const int k = kb + g * kGK + (lane % CPR) * KPC;
    const bool ok = g < NG && k < ke;
#pragma unroll
    for (int p = 0; p < LPG; ++p) {
      const uint32_t r = RPI * p + lane / CPR;
      v[p] = buf_load16<kAuxNT>(wr, opaque(ok ? (r * (uint32_t)K + (uint32_t)k) * (uint32_t)ES : kOob));
    }
  };

  // chunk c of every slice into buffer c & 1: instruction q of the chunk
  // covers slice q / (8 MT), token rows 2 (q % (8 MT)) + lane / 32; lane
  // fills slot lane % 32 of its row with chunk slot ^ (token & 15).  Chunks
  // past the end (and tokens past I) are zero-filled.
  const u32x4_t xr = rsrc_words(X, (uint32_t)I * (uint32_t)K * 2u);
  const uint32_t lx = lds_addr(lds);
  auto issue_x = [&](int c) {
    const uint32_t base = lx + (c & 1) * xbuf_bytes<MT>();
#pragma unroll
    for (int h = 0; h < XPW; ++h) {
      const int q = wave + h * kWaves;
      const int s = q / (8 * MT);
      const int t = 2 * (q % (8 * MT)) + (lane >> 5);
      const int slot = lane & 31;
      const int k = s * KS + c * kKC + ((slot ^ (t & 15)) * 8);
      const bool ok = c < NC && t < I && k < min(K, (s + 1) * KS);
      lds_dma16(xr, ok ? ((uint32_t)t * (uint32_t)K + (uint32_t)k) * 2u : kOob, base + q * 1024);
    }
  };

  f32x4_t acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  u32x4_t wv[P][LPG];

  // P weight groups are in flight per wave (P = 2: one chunk ahead, 4: two).
  // Order of this wave's loads: W(0 .. P-3), X(0), W(P-2), W(P-1), then per
  // chunk step c: X(c + 1) and, as groups 2c and 2c + 1 are consumed,
  // W(2c + P) and W(2c + P + 1).  So X(c) is always followed by exactly two
  // weight groups and W(g) by 4 (P - 1) + 2 XPW (P = 4) or 4 + XPW (P = 2)
  // loads (LPG per group: 4 bf16, 2 FP8).  Past the end the offsets are
  // out of range (zero, nothing fetched), so the counts never change.
  static_assert(P == 2 || P == 4, "two or four groups in flight");
  constexpr int kAfterW = P == 4 ? 3 * LPG + 2 * XPW : LPG + XPW;
#pragma unroll
  for (int g = 0; g < P - 2; ++g) issue_w(g, wv[g]);
  issue_x(0);
  issue_w(P - 2, wv[P - 2]);
  issue_w(P - 1, wv[P - 1]);
  // one chunk step; `par` = c % 2 is a constant in each unrolled copy, so the
  // weight register set of each group is known at compile time
  auto step = [&](int c, auto par) {
    wait_vmcnt<2 * LPG>();  // X(c) has landed: only the two groups after it may not
    __syncthreads();  // everyone's part of X(c); chunk c - 1's buffer is free
    issue_x(c + 1);
    const unsigned char* xs = lds + (c & 1) * xbuf_bytes<MT>() + sl * xslice_bytes<MT>();
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int g = 2 * c + b;
      u32x4_t (&w)[LPG] = wv[(2 * decltype(par)::value + b) % P];
      wait_vmcnt<kAfterW>();  // W(g) has landed
      // transpose through the tile: row r, bf16 chunk c at slot c ^ r; an
      // FP8 chunk of 16 codes decodes exactly into two bf16 chunks
      if constexpr (F8) {
#pragma unroll
        for (int p = 0; p < LPG; ++p) {
          const int r = 8 * p + (lane >> 3), c = 2 * (lane & 7);
          u32x4_t lo, hi;
          if constexpr (WF == kWInt8)
            decode16_i8(w[p], lo, hi);
          else
            decode16(w[p], lo, hi);
          *reinterpret_cast<u32x4_t*>(tile + r * 256 + ((c ^ r) * 16)) = lo;
          *reinterpret_cast<u32x4_t*>(tile + r * 256 + (((c + 1) ^ r) * 16)) = hi;
        }
      } else {
#pragma unroll
        for (int p = 0; p < LPG; ++p) {
          const int r = 4 * p + (lane >> 4);
          *reinterpret_cast<u32x4_t*>(tile + r * 256 + (((lane & 15) ^ r) * 16)) = w[p];
        }
      }
      issue_w(g + P, w);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int n = lane & 15, ch = 4 * j + (lane >> 4);
        const bf16x8_t bw = *reinterpret_cast<const bf16x8_t*>(tile + n * 256 + ((ch ^ n) * 16));
        const int xc = b * 16 + ch;  // 16-byte chunk within the 256-K chunk
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const int t = mt * 16 + (lane & 15);
          const bf16x8_t ax =
              *reinterpret_cast<const bf16x8_t*>(xs + t * (kKC * 2) + ((xc ^ (t & 15)) * 16));
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ax, bw, acc[mt], 0, 0, 0);
        }
      }
    }
  };
  for (int c = 0; c < NC; c += 2) {
    step(c, std::integral_constant<int, 0>{});
    if (c + 1 < NC) step(c + 1, std::integral_constant<int, 1>{});
  }

  // ---- the four slices of each tile, summed in slice order through LDS
  wait_vmcnt<0>();  // the zero-fill copies past the end have landed
  __syncthreads();
  f32x4_t* red = reinterpret_cast<f32x4_t*>(lds);  // [wave][mt][lane]
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) red[(wave * MT + mt) * 64 + lane] = acc[mt];
  __syncthreads();
  if (wave >= kTiles) return;
  // wave tw: tile tw's sums; C[m = 4 (lane / 16) + e][n = lane % 16]
  f32x4_t sum[kTiles][MT];
#pragma unroll
  for (int t2 = 0; t2 < kTiles; ++t2)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      f32x4_t s4 = red[((t2 + 0 * kTiles) * MT + mt) * 64 + lane];
#pragma unroll
      for (int s = 1; s < kKW; ++s) s4 += red[((t2 + s * kTiles) * MT + mt) * 64 + lane];
      sum[t2][mt] = s4;
    }
  const int n = lane & 15;  // tile row of this lane's sums
  if (n >= RPT) return;
  if constexpr (EPI == EPI_SWIGLU) {
    if (wave != 0) return;
    const int col = blockIdx.x * RPT + n;
    // FP8: the row scales of gate and up multiply the summed rows
    const float sg = F8 ? (col < N ? S0[col] : 0.0f) : 1.0f;
    const float su = F8 ? (col < N ? S1[col] : 0.0f) : 1.0f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = mt * 16 + (lane >> 4) * 4 + e;
        if (m < I && col < N)
          static_cast<uint16_t*>(out)[(int64_t)m * ldo + col] =
              f32_to_bf16_bits(silu(sum[0][mt][e] * sg) * (sum[1][mt][e] * su));
      }
  } else {
    const int col = (blockIdx.x * 2 + wave) * RPT + n;
    const float sc = F8 ? (col < N ? S0[col] : 0.0f) : 1.0f;  // FP8 row scale
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = mt * 16 + (lane >> 4) * 4 + e;
        const float v = (wave == 0 ? sum[0][mt][e] : sum[1][mt][e]) * sc;
        if (m < I && col < N) {
          if constexpr (EPI == EPI_F32)
            static_cast<float*>(out)[(int64_t)m * ldo + col] = v;
          else
            static_cast<uint16_t*>(out)[(int64_t)m * ldo + col] = f32_to_bf16_bits(v);
        }
      }
  }
}

template <int MT, int EPI, int WF>
hipError_t launch_mt(int I, int K, int N, const uint16_t* X, const void* W0, const void* W1,
                     const float* S0, const float* S1, void* out, int64_t ldo,
                     hipStream_t stream) {
  constexpr bool F8 = WF != kWBf16;
  // bf16: 2 groups of 128 K in flight per wave (4 measured slower); FP8: 4,
  // the same bytes in flight
  auto kern = rowstream_kernel<MT, EPI, F8 ? 4 : 2, WF>;
  static std::atomic<uint64_t> lds_raised{0};
  {
    const hipError_t e = dyn_lds_once(reinterpret_cast<const void*>(kern), lds_bytes<MT>(),
                                      lds_raised);
    if (e != hipSuccess) return e;
  }
  const int KS = rowstream_slice(K);
  const int rpt = rowstream_rows(N, EPI == EPI_SWIGLU);
  const int grid = rowstream_grid(N, EPI == EPI_SWIGLU);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreads), lds_bytes<MT>(), stream, I, K, N, X, W0,
                     W1, S0, S1, KS, rpt, out, ldo);
  return hipGetLastError();
}

}  // namespace

// Rows per weight tile: the fewest (at most 16) that give about one
// workgroup per CU -- 14 for the Llama-70B TP=8 gate/up (3584 F rows on 256
// workgroups instead of 224 of 16).
int rowstream_rows(int N, bool swiglu) {
  const int per_wg = (N + kCUs - 1) / kCUs;  // rows of each matrix per workgroup
  return std::min(16, swiglu ? per_wg : (per_wg + 1) / 2);
}

int rowstream_grid(int N, bool swiglu) {
  const int rpt = rowstream_rows(N, swiglu);
  return swiglu ? (N + rpt - 1) / rpt : (N + 2 * rpt - 1) / (2 * rpt);
}

int rowstream_slice(int K) {  // K per slice: whole 256-K chunks
  const int per = (K + kKW - 1) / kKW;
  return (per + kKC - 1) / kKC * kKC;
}

// Measured against the split-K kernel on MI355X at 9..32 tokens: faster
// when K is short enough for the split-K finish to dominate (Llama-70B TP=8
// o_proj, K = 1024: 7.0 us against 9.2 at 32 tokens; down, K = 3584: 15.3
// against 16.4), slower for the TP=8 gate/up (K = 8192: 28.6 against 27.3
// on 224 workgroups of 16 rows, 30.0 on 256 of 14), where every CU
// streaming all of X costs more than the finish saves.
bool rowstream_suits(int I, int K, int N, bool swiglu) {
  if (I < 9 || I > kRowStreamMaxTokens || K < 1024 || K > 4096) return false;
  // every CU reads all of X: keep a workgroup's weight rows (2 tiles) at
  // least half its activation rows' worth, i.e. tiles of at least 8 rows
  if (rowstream_rows(N, swiglu) < 8) return false;
  return rowstream_grid(N, swiglu) <= kCUs;  // one round of workgroups
}

template <int EPI>
hipError_t rowstream_launch(int I, int K, int N, const uint16_t* X, const uint16_t* W0,
                            const uint16_t* W1, void* out, int64_t ldo, hipStream_t stream) {
  if (I < 1 || I > kRowStreamMaxTokens || K < 1 || K > kRowStreamMaxK || N < 1)
    return hipErrorInvalidValue;
  if (I <= 16) return launch_mt<1, EPI, kWBf16>(I, K, N, X, W0, W1, nullptr, nullptr, out, ldo, stream);
  return launch_mt<2, EPI, kWBf16>(I, K, N, X, W0, W1, nullptr, nullptr, out, ldo, stream);
}

template <int EPI>
hipError_t rowstream_fp8_launch(int I, int K, int N, const uint16_t* X, const uint8_t* W0,
                                const float* S0, const uint8_t* W1, const float* S1, void* out,
                                int64_t ldo, int fmt, hipStream_t stream) {
  if (I < 1 || I > kRowStreamMaxTokens || K < 1 || K > kRowStreamMaxK || N < 1 || (K % 16))
    return hipErrorInvalidValue;
  if (fmt == kFmtInt8) {
    if (I <= 16) return launch_mt<1, EPI, kWInt8>(I, K, N, X, W0, W1, S0, S1, out, ldo, stream);
    return launch_mt<2, EPI, kWInt8>(I, K, N, X, W0, W1, S0, S1, out, ldo, stream);
  }
  if (I <= 16) return launch_mt<1, EPI, kWE4M3>(I, K, N, X, W0, W1, S0, S1, out, ldo, stream);
  return launch_mt<2, EPI, kWE4M3>(I, K, N, X, W0, W1, S0, S1, out, ldo, stream);
}

template hipError_t rowstream_fp8_launch<EPI_F32>(int, int, int, const uint16_t*, const uint8_t*,
                                                  const float*, const uint8_t*, const float*,
                                                  void*, int64_t, int, hipStream_t);
template hipError_t rowstream_fp8_launch<EPI_SWIGLU>(int, int, int, const uint16_t*,
                                                     const uint8_t*, const float*,
                                                     const uint8_t*, const float*, void*,
                                                     int64_t, int, hipStream_t);

template hipError_t rowstream_launch<EPI_F32>(int, int, int, const uint16_t*, const uint16_t*,
                                              const uint16_t*, void*, int64_t, hipStream_t);
template hipError_t rowstream_launch<EPI_DT>(int, int, int, const uint16_t*, const uint16_t*,
                                             const uint16_t*, void*, int64_t, hipStream_t);
template hipError_t rowstream_launch<EPI_SWIGLU>(int, int, int, const uint16_t*, const uint16_t*,
                                                 const uint16_t*, void*, int64_t, hipStream_t);

}  // namespace tpk
