// Decode projections for 9..64 tokens: y[m, n] = sum_k X[m, k] W[n, k] on bf16
// MFMA, streaming W from HBM once at close to the achievable read rate.
//
// Decode reads each weight of the rank's shard once per step (lecture
// "Distributed Serving", §1.1 and §3.4); the design is about keeping every CU
// streaming until the end:
//   * the weight rows (for SwiGLU: gate rows, then up rows) are cut into
//     16-row tiles and the K axis into NS ranges; a workgroup owns NW tiles
//     times one K range, and the host picks NW and NS so the grid is close to
//     one workgroup per CU (256 on MI355X) -- no second, half-empty wave of
//     workgroups;
//   * each wave streams its own tile: one load instruction reads 4 rows x 256
//     contiguous bytes (whole cache lines) into registers, P groups of 128 K
//     in flight; the group is transposed through a private 4 KB LDS tile
//     (16-byte slots XOR-swizzled by row, conflict-free both ways) into the B
//     operand of v_mfma_f32_16x16x32_bf16;
//   * the activations of the workgroup's K range are staged once in LDS with
//     direct global->LDS loads and shared by all waves (A operand);
//   * no barrier after the start: waves run independently;
//   * each workgroup writes fp32 partial sums part[split][m][row]; the last
//     of a row block's NS workgroups to arrive (an arrival counter in the
//     workspace, one atomic each) adds the NS partials in split order -- deterministic,
//     whichever arrives last -- and applies the epilogue: fp32 store, bf16
//     store, or silu(gate) * up (lecture §4.1: the SwiGLU elementwise op is
//     local to the rank).  A SwiGLU row block holds the gate tiles and the up
//     tiles of the same F block, so the epilogue has both;
//   * one kernel launch per projection: no separate reduction pass;
//   * weight-only FP8 (OCP E4M3 codes, one fp32 scale per output row): a
//     group of 128 K is 128 bytes per row, two load instructions of 8 rows x
//     128 bytes; each 16-byte chunk of codes is decoded exactly to two bf16
//     chunks on its way into the transpose tile, four groups in flight (the
//     bf16 path's bytes in flight), and the finishing workgroup multiplies
//     each summed row by its scale before the epilogue.
#include "common.h"
#include "kernels.h"

namespace tpk {

namespace {

typedef __attribute__((address_space(3))) void lds_void_t;
constexpr uint32_t kOob = 0x80000000u;  // buffer offset past any record: reads zero
constexpr int kAuxSys = 17;             // sc0 sc1: system coherent, bypasses L1 and L2
constexpr int kGK = 128;                // K elements per streamed group
constexpr int kLdsMax = 160 * 1024 - 1024;  // dynamic LDS budget (static LDS sits before it)
constexpr int kCUs = 256;

// Row space of the partial sums: row block rb holds NW 16-row tiles.  Single
// matrix (N rows): block rb covers rows [16 NW rb, 16 NW (rb + 1)).  SwiGLU
// (gate W0 and up W1, N rows each): block rb covers F rows f0 = 8 NW rb ..
// f0 + 8 NW, its first NW/2 tiles from gate, the other NW/2 from up.
template <int MT, int P, int EPI, int WF, int MAXT>
__global__ void __launch_bounds__(MAXT)
splitk_kernel(int I, int K, int N, const uint16_t* __restrict__ X,
              const void* __restrict__ W0, const void* __restrict__ W1,
              const float* __restrict__ S0, const float* __restrict__ S1, int KR,
              unsigned* __restrict__ counters, float* __restrict__ part, int NR,
              void* __restrict__ out, int64_t ldo) {
  constexpr bool F8 = WF != kWBf16;  // one-byte codes with a row scale
  constexpr int TOK = 16 * MT;
  constexpr int ES = F8 ? 1 : 2;    // bytes per weight
  constexpr int LPG = F8 ? 2 : 4;   // load instructions per 128-K group
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  __shared__ int is_last;
  const int NW = blockDim.x >> 6;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int XRB = KR * 2;                                   // LDS bytes per token row
  unsigned char* xs = lds;
  unsigned char* tile = lds + TOK * XRB + wave * 4096;
  const int ns = (K + KR - 1) / KR;
  const int split = blockIdx.x % ns;
  const int rb = blockIdx.x / ns;
  const int k0 = split * KR;
  const int kend = min(K, k0 + KR);

  // ---- activations of this K range -> LDS; slot s of token t holds chunk s ^ (t & 15)
  {
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(X, (uint32_t)I * (uint32_t)K * 2u);
    const int XSL = KR / 8;
    const int XI = TOK * XSL / 64;
    for (int q = wave; q < XI; q += NW) {
      const int slot = q * 64 + lane;
      const int t = slot / XSL, sl = slot % XSL;
      const int k = k0 + (sl ^ (t & 15)) * 8;
      const uint32_t off = (k < kend) ? ((uint32_t)t * (uint32_t)K + (uint32_t)k) * 2u : kOob;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_void_t*)(xs + q * 1024), 16, off, 0, 0, 0);
    }
  }

  // ---- this wave's 16 weight rows: uniform base, rows past the matrix read zero
  int wrow0;
  const void* wmat;
  if constexpr (EPI == EPI_SWIGLU) {
    const int half = NW / 2;
    wrow0 = rb * 16 * half + 16 * (wave % half);
    wmat = wave < half ? W0 : W1;
  } else {
    wrow0 = (rb * NW + wave) * 16;
    wmat = W0;
  }
  const int rows = max(0, min(16, N - wrow0));
  const __amdgpu_buffer_rsrc_t wr =
      make_rsrc_uniform(static_cast<const unsigned char*>(wmat) + (int64_t)wrow0 * K * ES,
                (uint32_t)rows * (uint32_t)K * (uint32_t)ES);
  const int NG = (kend - k0 + kGK - 1) / kGK;

  // group g, instruction p: bf16 rows 4p + lane/16, 16-byte chunk lane%16
  // (8 K) of the group; FP8 rows 8p + lane/8, 16-byte chunk lane%8 (16 K)
  auto issue = [&](int g, u32x4_t (&v)[LPG]) {
    constexpr int KPC = 16 / ES;     // K per 16-byte chunk
    constexpr int CPR = kGK / KPC;   // chunks per row of a group: 16 (bf16), 8 (FP8)
    constexpr int RPI = 64 / CPR;    // rows per load instruction: 4, 8
    static_assert(RPI * LPG == 16, "a group is 16 rows");
    const int k = k0 + g * kGK + (lane % CPR) * KPC;
    const bool ok = g < NG && k < kend;
#pragma unroll
    for (int p = 0; p < LPG; ++p) {
      const uint32_t r = RPI * p + lane / CPR;
      v[p] = buf_load16<kAuxNT>(wr, opaque(ok ? (r * (uint32_t)K + (uint32_t)k) * (uint32_t)ES : kOob));
    }
  };

  u32x4_t wv[P][LPG];
#pragma unroll
  for (int b = 0; b < P; ++b) issue(b, wv[b]);
  f32x4_t acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // the activation loads are older than every weight load: once group 0 has
  // landed, so has this wave's share of X; the barrier publishes all shares
  wait_vmcnt<(P - 1) * LPG>();
  __syncthreads();

  for (int g0 = 0; g0 < NG; g0 += P) {
#pragma unroll
    for (int b = 0; b < P; ++b) {
      const int g = g0 + b;
      wait_vmcnt<(P - 1) * LPG>();
      // transpose through the tile: row r, bf16 chunk c at slot c ^ r
      if constexpr (F8) {
#pragma unroll
        for (int p = 0; p < LPG; ++p) {
          const int r = 8 * p + (lane >> 3), c = 2 * (lane & 7);
          u32x4_t lo, hi;
          if constexpr (WF == kWInt8)
            decode16_i8(wv[b][p], lo, hi);
          else
            decode16(wv[b][p], lo, hi);
          *reinterpret_cast<u32x4_t*>(tile + r * 256 + ((c ^ r) * 16)) = lo;
          *reinterpret_cast<u32x4_t*>(tile + r * 256 + (((c + 1) ^ r) * 16)) = hi;
        }
      } else {
#pragma unroll
        for (int p = 0; p < LPG; ++p) {
          const int r = 4 * p + (lane >> 4);
          *reinterpret_cast<u32x4_t*>(tile + r * 256 + (((lane & 15) ^ r) * 16)) = wv[b][p];
        }
      }
      issue(g + P, wv[b]);  // past the end: out-of-range offsets, nothing fetched
      if (g < NG) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int n = lane & 15, c = 4 * j + (lane >> 4);
          const bf16x8_t bw = *reinterpret_cast<const bf16x8_t*>(tile + n * 256 + ((c ^ n) * 16));
          const int xc = g * 16 + c;
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            const int t = mt * 16 + (lane & 15);
            const bf16x8_t ax =
                *reinterpret_cast<const bf16x8_t*>(xs + t * XRB + ((xc ^ (t & 15)) * 16));
            acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ax, bw, acc[mt], 0, 0, 0);
          }
        }
      }
    }
  }

  // ---- partial tile C[m][n] (m = (lane/16)*4 + j token, n = lane%16 row) ->
  // row-space column 16 (NW rb + wave) + n of split plane `split`.  The
  // partials cross workgroups (and XCDs, whose L2s are not coherent with each
  // other): they are stored system-coherent (sc0 sc1, written through to
  // memory) and read back the same way, so no cache-wide writeback or
  // invalidate is needed; the arrival counter is a device-scope atomic.
  const int64_t plane = (int64_t)I * NR;
  const __amdgpu_buffer_rsrc_t pr = make_rsrc(part, (uint32_t)(ns * plane * 4));
  {
    const int col = (rb * NW + wave) * 16 + (lane & 15);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int m = mt * 16 + (lane >> 4) * 4 + j;
        const float v = acc[mt][j];  // bit_cast of a vector-element lvalue reads element 0
        if (m < I)
          __builtin_amdgcn_raw_buffer_store_b32(
              __builtin_bit_cast(uint32_t, v), pr, (uint32_t)((split * plane + (int64_t)m * NR + col) * 4), 0,
              kAuxSys);
      }
  }

  // ---- the last of the block's ns workgroups reduces and stores the block
  wait_vmcnt<0>();  // this wave's partial stores have reached memory
  __syncthreads();
  if (tid == 0) is_last = arrive_last(counters + rb, (unsigned)ns);
  __syncthreads();
  if (!is_last) return;

  const int cols = (EPI == EPI_SWIGLU) ? 8 * NW : 16 * NW;  // output columns of the block
  const int cbase = rb * cols;
  const int ncols = min(cols, N - cbase);
  const int cq = (ncols + 3) / 4;
  const int rs0 = rb * NW * 16;                             // block's first row-space column
  // Sums of the ns split planes at element offsets q[0 .. NQ) (NQ = 2 for
  // SwiGLU: the gate and the up columns), each in split order.  16 / NQ
  // splits of every offset are in flight per batch -- gate and up together --
  // so up to 16 (one offset) or 8 (two) splits cost one memory round trip;
  // offsets of splits past ns are out of range and read zero (x + 0 == x),
  // so the batch needs no branch.  A workgroup of at most 4 waves (launch
  // bound 256) has the registers for 32 loads in flight: its threads sum two
  // items per batch (a 1024-thread bound leaves 128 registers, too few).
  auto sum_splits = [&](const auto& q, auto& s) {
    constexpr int NQ = sizeof(s) / sizeof(s[0]);
    constexpr int B = (MAXT <= 256 ? 32 : 16) / NQ;
#pragma unroll
    for (int i = 0; i < NQ; ++i) s[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int r = 0; r < ns; r += B) {
      f32x4_t v[NQ][B];
#pragma unroll
      for (int i = 0; i < NQ; ++i)
#pragma unroll
        for (int e = 0; e < B; ++e)
          v[i][e] = __builtin_bit_cast(
              f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                           pr, r + e < ns ? (uint32_t)((q[i] + (r + e) * plane) * 4) : kOob, 0,
                           kAuxSys));
#pragma unroll
      for (int i = 0; i < NQ; ++i)
#pragma unroll
        for (int e = 0; e < B; ++e) s[i] += v[i][e];
    }
  };
  auto store_item = [&](int m, int c, int n, const f32x4_t& v) {
    if constexpr (EPI == EPI_F32) {
      float* o = static_cast<float*>(out) + (int64_t)m * ldo + cbase + c;
      if (n == 4 && ((reinterpret_cast<uintptr_t>(o) & 15) == 0)) {
        *reinterpret_cast<f32x4_t*>(o) = v;
      } else {
        for (int e = 0; e < n; ++e) o[e] = v[e];
      }
    } else {
      // 4 columns as one 8-byte store where aligned (the finish ends the
      // kernel, so its store count is on the critical path)
      uint16_t* o = static_cast<uint16_t*>(out) + (int64_t)m * ldo + cbase + c;
      if (n == 4 && ((reinterpret_cast<uintptr_t>(o) & 7) == 0)) {
        *reinterpret_cast<u32x2_t*>(o) = u32x2_t{pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w)};
      } else {
        for (int e = 0; e < n; ++e) o[e] = f32_to_bf16_bits(v[e]);
      }
    }
  };
  if constexpr (MAXT <= 256 && EPI != EPI_SWIGLU && !F8) {
    // items idx and idx + NW * 64 of a thread summed in one batch
    const int step = NW * 64;
    for (int idx = tid; idx < I * cq; idx += 2 * step) {
      const int idx2 = idx + step;
      const bool has2 = idx2 < I * cq;
      const int m = idx / cq, c = (idx % cq) * 4;
      const int m2 = has2 ? idx2 / cq : m, c2 = has2 ? (idx2 % cq) * 4 : c;
      const int64_t qq[2] = {(int64_t)m * NR + rs0 + c, (int64_t)m2 * NR + rs0 + c2};
      f32x4_t sv[2];
      sum_splits(qq, sv);
      store_item(m, c, min(4, ncols - c), sv[0]);
      if (has2) store_item(m2, c2, min(4, ncols - c2), sv[1]);
    }
    return;
  }
  for (int idx = tid; idx < I * cq; idx += NW * 64) {
    const int m = idx / cq, c = (idx % cq) * 4;
    const int64_t q = (int64_t)m * NR + rs0 + c;
    const int n = min(4, ncols - c);
    f32x4_t v;
    // FP8 row scales, loaded before the partials so both are in flight together
    float sc0[4] = {1.f, 1.f, 1.f, 1.f}, sc1[4] = {1.f, 1.f, 1.f, 1.f};
    if constexpr (F8) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sc0[e] = e < n ? S0[cbase + c + e] : 0.0f;
        if constexpr (EPI == EPI_SWIGLU) sc1[e] = e < n ? S1[cbase + c + e] : 0.0f;
      }
    }
    if constexpr (EPI == EPI_SWIGLU) {
      const int64_t qq[2] = {q, q + cols};
      f32x4_t gu[2];
      sum_splits(qq, gu);
      f32x4_t s4 = gu[0], u = gu[1];
      if constexpr (F8) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          s4[e] *= sc0[e];
          u[e] *= sc1[e];
        }
      }
      v = f32x4_t{silu(s4.x) * u.x, silu(s4.y) * u.y, silu(s4.z) * u.z, silu(s4.w) * u.w};
    } else {
      const int64_t qq[1] = {q};
      f32x4_t sv[1];
      sum_splits(qq, sv);
      f32x4_t s4 = sv[0];
      if constexpr (F8) {
#pragma unroll
        for (int e = 0; e < 4; ++e) s4[e] *= sc0[e];
      }
      v = s4;
    }
    store_item(m, c, n, v);
  }
}

struct Plan {
  int nw = 0;      // waves (16-row tiles) per workgroup
  int kr = 0;      // K elements per split (multiple of kGK)
  int ns = 0;      // number of K splits
  int rbs = 0;     // row blocks
  int nr = 0;      // row-space width = 16 * nw * rbs
  int lds = 0;     // dynamic LDS bytes
  int grid = 0;
};

size_t plan_bytes(const Plan& pl, int I) {
  return kWsCounterBytes + (size_t)pl.ns * (size_t)I * (size_t)pl.nr * sizeof(float);
}

Plan plan_for(int I, int K, int N, bool swiglu, int nw, int ns_req) {
  Plan pl;
  const int mt = (I + 15) / 16;
  const int groups = (K + kGK - 1) / kGK;
  const int gps = (groups + ns_req - 1) / ns_req;
  pl.nw = nw;
  pl.kr = gps * kGK;
  pl.ns = (groups + gps - 1) / gps;
  pl.rbs = swiglu ? (N + 8 * nw - 1) / (8 * nw) : (N + 16 * nw - 1) / (16 * nw);
  pl.nr = 16 * nw * pl.rbs;
  pl.lds = 16 * mt * pl.kr * 2 + nw * 4096;
  pl.grid = pl.rbs * pl.ns;
  return pl;
}

// Choose the K split (ns) and waves per workgroup (nw).  Measured on MI355X
// over the decode projections of the Llama-3.1-70B and Qwen2.5-1.5B rank
// shares (9..64 tokens): with 4 waves per workgroup, split K until the grid
// nears one workgroup per CU, keeping 256..1408 K elements per split (short
// ranges multiply the partial sums, long ones make slow-starting
// workgroups); then use the fewest waves (at least 4) that keep the grid
// within one workgroup per CU.  When the activations of the K range do not
// fit LDS the range shrinks.
int target_groups(int K, int tiles) {  // K groups per split the rule aims for
  const int groups = (K + kGK - 1) / kGK;
  const int rbs4 = (tiles + 3) / 4;  // row blocks at 4 waves
  const int ns = std::max(1, kCUs / rbs4);
  const int gps = (groups + ns - 1) / ns;
  return std::min(std::min(std::max(gps, 2), 11), groups);
}

int weight_tiles(int N, bool swiglu) {  // 16-row weight tiles
  return swiglu ? (N + 7) / 8 : (N + 15) / 16;
}

Plan make_plan(int I, int K, int N, bool swiglu) {
  const int groups = (K + kGK - 1) / kGK;
  const int tiles = weight_tiles(N, swiglu);
  int gps = target_groups(K, tiles);
  for (;;) {
    const int ns = (groups + gps - 1) / gps;
    const int per_split = std::max(1, kCUs / ns);  // row blocks that fit beside the splits
    int nw = std::max(4, (tiles + per_split - 1) / per_split);
    if (swiglu) nw += nw & 1;
    nw = std::min(nw, 16);
    Plan pl = plan_for(I, K, N, swiglu, nw, ns);
    const bool fits = pl.lds <= kLdsMax && (double)pl.ns * I * pl.nr * 4.0 < 2147483648.0;
    if (fits || gps == 1) return fits ? pl : Plan{};
    --gps;
  }
}

template <int MT, int EPI, int WF = kWBf16>
hipError_t launch_plan(const Plan& pl, int I, int K, int N, const uint16_t* X, const void* W0,
                       const void* W1, void* out, int64_t ldo, void* workspace,
                       hipStream_t stream, const float* S0 = nullptr, const float* S1 = nullptr) {
  constexpr bool F8 = WF != kWBf16;
  // plans of at most 4 waves run the variant bounded to 256 threads (more
  // registers per wave: the finish sums two items per batch)
  const bool small = pl.nw <= 4;
  auto kern = small ? splitk_kernel<MT, F8 ? 4 : 2, EPI, WF, 256>
                    : splitk_kernel<MT, F8 ? 4 : 2, EPI, WF, 1024>;
  static std::atomic<uint64_t> lds_raised[2];  // per variant, one bit per device
  {
    const hipError_t e = dyn_lds_once(reinterpret_cast<const void*>(kern), kLdsMax,
                                      lds_raised[small]);
    if (e != hipSuccess) return e;
  }
  if (pl.rbs > kWsMaxCounters) return hipErrorInvalidValue;
  auto* counters = static_cast<unsigned*>(workspace);
  float* part = reinterpret_cast<float*>(static_cast<char*>(workspace) + kWsCounterBytes);
  hipLaunchKernelGGL(kern, dim3(pl.grid), dim3(pl.nw * 64), pl.lds, stream, I, K, N, X, W0, W1,
                     S0, S1, pl.kr, counters, part, pl.nr, out, ldo);
  return hipGetLastError();
}

}  // namespace

bool splitk_suits(int I, int K, int N, bool swiglu) {
  if (I < 1 || I > kSplitKMaxTokens || K > kSplitKMaxK) return false;
  const Plan pl = make_plan(I, K, N, swiglu);
  if (pl.grid == 0) return false;
  // K range cut below half the target by LDS: the tiled kernel does better
  return 2 * (pl.kr / kGK) >= target_groups(K, weight_tiles(N, swiglu));
}

bool splitk_plannable(int I, int K, int N, bool swiglu) {
  return I >= 1 && I <= kSplitKMaxTokens && K <= kSplitKMaxK &&
         make_plan(I, K, N, swiglu).grid > 0;
}

size_t splitk_workspace_bytes(int I, int K, int N, bool swiglu) {
  return plan_bytes(make_plan(I, K, N, swiglu), I);
}

template <int EPI>
hipError_t splitk_launch(int I, int K, int N, const uint16_t* X, const uint16_t* W0,
                         const uint16_t* W1, void* out, int64_t ldo, void* workspace,
                         hipStream_t stream) {
  const Plan pl = make_plan(I, K, N, EPI == EPI_SWIGLU);
  if (pl.grid == 0) return hipErrorInvalidValue;
  if (I <= 16) return launch_plan<1, EPI>(pl, I, K, N, X, W0, W1, out, ldo, workspace, stream);
  if (I <= 32) return launch_plan<2, EPI>(pl, I, K, N, X, W0, W1, out, ldo, workspace, stream);
  if (I <= 48) return launch_plan<3, EPI>(pl, I, K, N, X, W0, W1, out, ldo, workspace, stream);
  return launch_plan<4, EPI>(pl, I, K, N, X, W0, W1, out, ldo, workspace, stream);
}

template hipError_t splitk_launch<EPI_F32>(int, int, int, const uint16_t*, const uint16_t*,
                                           const uint16_t*, void*, int64_t, void*, hipStream_t);
template hipError_t splitk_launch<EPI_DT>(int, int, int, const uint16_t*, const uint16_t*,
                                          const uint16_t*, void*, int64_t, void*, hipStream_t);
template hipError_t splitk_launch<EPI_SWIGLU>(int, int, int, const uint16_t*, const uint16_t*,
                                              const uint16_t*, void*, int64_t, void*,
                                              hipStream_t);

template <int EPI>
hipError_t splitk_fp8_launch(int I, int K, int N, const uint16_t* X, const uint8_t* W0,
                             const float* S0, const uint8_t* W1, const float* S1, void* out,
                             int64_t ldo, void* workspace, int fmt, hipStream_t stream) {
  const Plan pl = make_plan(I, K, N, EPI == EPI_SWIGLU);
  if (pl.grid == 0) return hipErrorInvalidValue;
#define TPK_F8(MTV)                                                                       \
  (fmt == kFmtInt8 ? launch_plan<MTV, EPI, kWInt8>(pl, I, K, N, X, W0, W1, out, ldo, workspace, \
                                                    stream, S0, S1)                           \
                   : launch_plan<MTV, EPI, kWE4M3>(pl, I, K, N, X, W0, W1, out, ldo, workspace, \
                                                    stream, S0, S1))
  if (I <= 16) return TPK_F8(1);
  if (I <= 32) return TPK_F8(2);
  if (I <= 48) return TPK_F8(3);
  return TPK_F8(4);
#undef TPK_F8
}

template hipError_t splitk_fp8_launch<EPI_F32>(int, int, int, const uint16_t*, const uint8_t*,
                                               const float*, const uint8_t*, const float*, void*,
                                               int64_t, void*, int, hipStream_t);
template hipError_t splitk_fp8_launch<EPI_SWIGLU>(int, int, int, const uint16_t*, const uint8_t*,
                                                  const float*, const uint8_t*, const float*,
                                                  void*, int64_t, void*, int, hipStream_t);

}  // namespace tpk
