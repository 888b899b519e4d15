// Projections for many tokens: C[M, N] = A[M, K] . W[N, K]^T on bf16 MFMA
// (v_mfma_f32_32x32x16_bf16, fp32 accumulation).
//
// Prefill and large decode batches are the compute-heavy side of the layer
// (lecture "Distributed Serving", §3.4: 2·B·D·F/n FLOPs per rank); the kernel
// is shaped for gfx950's measured balance -- a 64x64 wave tile keeps MFMA
// busy only with 8 waves per CU to cover LDS latency, and 128x128 workgroup
// tiles keep about one workgroup per CU at the per-rank shapes:
//   * workgroup tile 128 x 128, eight waves: a 2 x 2 grid of 64 x 64 wave
//     tiles, twice -- the two wave groups take alternate 16-wide K steps of
//     every stage and are summed through LDS at the end;
//   * both operands are K-contiguous (activations row-major, weights
//     output-major) and are copied global -> LDS by the buffer unit directly
//     (no register staging), 64 K per stage, 5 stages (all 160 KB of LDS),
//     4 in flight -- at these shapes the copies wait on HBM misses, so the
//     bytes in flight set the speed; in LDS a
//     tile row is 128 bytes and its 16-byte chunk c sits in slot
//     c ^ ((row / 2) % 8), so the 32 rows one MFMA operand read touches
//     cover all 64 banks once;
//   * the SwiGLU variant stages gate rows f0.. and up rows f0.. of the same F
//     block in one W tile and gives each wave 32 gate and the matching 32 up
//     rows, so silu(g) * u is formed in registers (lecture §4.1: the
//     elementwise op is local to the rank);
//   * when the tiles alone cannot fill the chip (decode batches of 65..256
//     tokens) the K axis is split over workgroups: each writes an fp32
//     partial tile, and the last of a tile's workgroups to arrive sums the
//     partials in split order (deterministic) and applies the epilogue.
//     Partials cross XCDs, whose L2s are not coherent, so they are written
//     and read system-coherent; the arrival counter is one device atomic;
//   * workgroups go round-robin to the 8 XCDs; the block id is remapped so
//     that each XCD runs a contiguous range of tiles, and tiles sharing a W
//     block (same N block, other M blocks) are neighbours in that range.
#include "common.h"
#include "kernels.h"

namespace tpk {

namespace {

constexpr int BM = 128, BN = 128, BK = 64, S = 5;
constexpr int kThreads = 512;
constexpr int kRowB = BK * 2;                  // bytes per LDS tile row
constexpr int kStageA = BM * kRowB;            // 16 KB
constexpr int kStage = (BM + BN) * kRowB;      // 32 KB
constexpr int kLds = S * kStage;               // 160 KB: all of a CU's LDS
constexpr uint32_t kOob = 0x80000000u;         // buffer offset past any record: reads zero
constexpr int kAuxSys = 17;                    // sc0 sc1: system coherent
constexpr int kCUs = 256;
static_assert(4 * 16 * 64 * 4 <= kStageA, "a wave pair's K-group reduction fits one stage buffer");
static_assert(2 * BM * BN * 4 + 4 <= kLds, "the arrival flag follows both K groups' tiles");

__device__ __forceinline__ void wait_lgkmcnt0() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt at their maxima
}

// LDS byte offset of (row, logical 16-byte chunk) inside one operand tile.
__device__ __forceinline__ int lds_off(int row, int chunk) {
  return row * kRowB + ((chunk ^ ((row >> 1) & 7)) << 4);
}

// Row m (within the 32x32 tile) of accumulator element r held by `lane`; the
// column is lane % 32.
__device__ __forceinline__ int acc_row32(int r, int lane) {
  return (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
}

template <int EPI>
__device__ __forceinline__ void store_out(void* out, int64_t ldo, int m, int col, float v) {
  if constexpr (EPI == EPI_F32)
    static_cast<float*>(out)[(int64_t)m * ldo + col] = v;
  else
    static_cast<uint16_t*>(out)[(int64_t)m * ldo + col] = f32_to_bf16_bits(v);
}

// Columns col .. col + n - 1 (n <= 4) of output row m: one 16-byte (fp32) or
// 8-byte (bf16) store when all four are in range and aligned.
template <int EPI>
__device__ __forceinline__ void store_out4(void* out, int64_t ldo, int m, int col, int n,
                                           f32x4_t v) {
  if constexpr (EPI == EPI_F32) {
    float* o = static_cast<float*>(out) + (int64_t)m * ldo + col;
    if (n == 4 && (reinterpret_cast<uintptr_t>(o) & 15) == 0) {
      *reinterpret_cast<f32x4_t*>(o) = v;
      return;
    }
    for (int e = 0; e < n; ++e) o[e] = v[e];
  } else {
    uint16_t* o = static_cast<uint16_t*>(out) + (int64_t)m * ldo + col;
    if (n == 4 && (reinterpret_cast<uintptr_t>(o) & 7) == 0) {
      *reinterpret_cast<u32x2_t*>(o) =
          u32x2_t{f32_to_bf16_bits(v[0]) | ((uint32_t)f32_to_bf16_bits(v[1]) << 16),
                  f32_to_bf16_bits(v[2]) | ((uint32_t)f32_to_bf16_bits(v[3]) << 16)};
      return;
    }
    for (int e = 0; e < n; ++e) o[e] = f32_to_bf16_bits(v[e]);
  }
}

// Split-K finish, run by the last of a tile's ns workgroups: the ns fp32
// partial tiles (TM x TN, W-tile row order, plane `plane` apart; for SwiGLU
// the up partial of column c sits at column c + TN / 2) are summed in split
// order and the epilogue writes out[m0 + r][c0 + c].  An item is 4 columns of
// one row.  A thread's items are summed together rather than one after
// another: each round trip loads kB = 4 splits of IQ / kNQ items (and of gate
// and up), 4 IQ loads in flight, so up to 4 splits cost one memory round trip
// per IQ / kNQ items instead of one per item and matrix.  The split's plane
// offset is the same for every lane and travels in the scalar offset, so a
// load needs no address register of its own.  Rows past M read zero through
// an out-of-range lane offset, splits past ns are not loaded.  When the
// finishing workgroup's own partial is still in LDS (own >= 0: the sum of
// the row-major tiles own0 and own1), that split is taken from there.
template <int EPI, int TM, int TN, int THREADS, int IQ>
__device__ __forceinline__ void finish_splits(const __amdgpu_buffer_rsrc_t pr, int64_t tbase,
                                              int64_t plane, int ns, int m0, int c0, int M,
                                              int N, void* out, int64_t ldo, int tid, int own,
                                              const f32x4_t* own0, const f32x4_t* own1) {
  constexpr int kNQ = (EPI == EPI_SWIGLU) ? 2 : 1;  // gate and up
  constexpr int kCols = TN / kNQ;                   // output columns of the tile
  constexpr int kQ = kCols / 4;                     // items per tile row
  constexpr int kNI = TM * kQ / THREADS;            // items per thread
  constexpr int kIP = IQ / kNQ;                     // items per pass
  constexpr int kB = 4;                             // splits per round trip
  static_assert(TM * kQ % THREADS == 0 && kNI % kIP == 0, "whole passes of items");
#pragma unroll 1
  for (int p = 0; p < kNI / kIP; ++p) {
    f32x4_t s[kIP][kNQ];
    uint32_t off[kIP][kNQ];  // byte offset of the item in split 0
    int fi[kIP][kNQ];        // its float4 index within the tile
    int tr[kIP], tc[kIP];
#pragma unroll
    for (int i = 0; i < kIP; ++i) {
      const int idx = tid + (p * kIP + i) * THREADS;
      tr[i] = idx / kQ;
      tc[i] = (idx % kQ) * 4;
#pragma unroll
      for (int q = 0; q < kNQ; ++q) {
        s[i][q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        fi[i][q] = (tr[i] * TN + q * kCols + tc[i]) / 4;
        off[i][q] = m0 + tr[i] < M ? (uint32_t)((tbase + 4 * fi[i][q]) * 4) : kOob;
      }
    }
    for (int s0 = 0; s0 < ns; s0 += kB) {
      f32x4_t v[kIP][kNQ][kB];
#pragma unroll
      for (int e = 0; e < kB; ++e) {
        const int sp = s0 + e;
#pragma unroll
        for (int i = 0; i < kIP; ++i)
#pragma unroll
          for (int q = 0; q < kNQ; ++q) {
            if (sp == own)
              v[i][q][e] = own0[fi[i][q]] + own1[fi[i][q]];
            else if (sp < ns)
              v[i][q][e] = __builtin_bit_cast(
                  f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                               pr, off[i][q], (uint32_t)(sp * plane * 4), kAuxSys));
            else
              v[i][q][e] = f32x4_t{0.f, 0.f, 0.f, 0.f};
          }
      }
#pragma unroll
      for (int i = 0; i < kIP; ++i)
#pragma unroll
        for (int q = 0; q < kNQ; ++q)
#pragma unroll
          for (int e = 0; e < kB; ++e) s[i][q] += v[i][q][e];
    }
#pragma unroll
    for (int i = 0; i < kIP; ++i) {
      const int m = m0 + tr[i];
      if (m >= M) continue;
      f32x4_t v = s[i][0];
      if constexpr (EPI == EPI_SWIGLU) {
        const f32x4_t u = s[i][1];
        v = f32x4_t{silu(v.x) * u.x, silu(v.y) * u.y, silu(v.z) * u.z, silu(v.w) * u.w};
      }
      const int n = min(4, N - (c0 + tc[i]));
      store_out4<EPI == EPI_F32 ? EPI_F32 : EPI_DT>(out, ldo, m, c0 + tc[i], n, v);
    }
  }
}

// One launch: grid = tiles * ns workgroups of 512 threads, 128 KB static LDS.
//   KR: K elements per split (multiple of BK); ns = ceil(K / KR).
//   counters/part: split-K workspace (unused when ns == 1).
template <int EPI>
__global__ void __launch_bounds__(kThreads)
gemm_kernel(int M, int N, int K, const uint16_t* __restrict__ A, int64_t lda,
            const uint16_t* __restrict__ W0, const uint16_t* __restrict__ W1,
            void* __restrict__ out, int64_t ldo, int KR, unsigned* __restrict__ counters,
            float* __restrict__ part) {
  // S stages of (A tile, W tile); after the K loop the same memory holds
  // the K-group reduction and the split-K arrival flag
  __shared__ __attribute__((aligned(16))) unsigned char smem[kLds];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar registers
  const int g = wave >> 2;              // K group
  const int wm = (wave >> 1) & 1, wn = wave & 1;

  // ---- tile and split of this workgroup, XCD-aware
  const int mt_n = (M + BM - 1) / BM;
  constexpr int kCols = (EPI == EPI_SWIGLU) ? BN / 2 : BN;  // output columns per tile
  const int nt_n = (N + kCols - 1) / kCols;
  const int tiles = mt_n * nt_n;
  const int ns = (K + KR - 1) / KR;
  const int G = tiles * ns;
  int b = blockIdx.x;
  const int G8 = G & ~7;
  if (b < G8) b = (b & 7) * (G8 >> 3) + (b >> 3);
  const int split = b / tiles;
  const int tile = b % tiles;
  const int tm = tile % mt_n, tn = tile / mt_n;
  const int m0 = tm * BM, c0 = tn * kCols;
  const int kb = split * KR, ke = min(K, kb + KR);

  // ---- operand sources: X rows m0.., W rows c0.. (SwiGLU: 64 gate + 64 up)
  const u32x4_t ra = rsrc_words(A + (int64_t)m0 * lda, (uint32_t)min(BM, M - m0) * (uint32_t)lda * 2u);
  const int wrows = min(kCols, N - c0);
  const u32x4_t rw0 = rsrc_words(W0 + (int64_t)c0 * K, (uint32_t)wrows * (uint32_t)K * 2u);
  const u32x4_t rw1 = rsrc_words((EPI == EPI_SWIGLU ? W1 : W0) + (int64_t)c0 * K,
                                 (uint32_t)wrows * (uint32_t)K * 2u);

  // Stage st (K from kb + 64 st) into buffer buf.  One instruction writes
  // 1 KB = 8 tile rows; lane l fills slot l % 8 of row 8q + l / 8 with the
  // logical chunk that lds_off places there.  Wave w issues A and W
  // instructions w and w + 8.  Past the K range (or past M / N) the offset
  // is out of range and the slot is zero-filled.
  const int rr = lane >> 3, sl = lane & 7;
  const uint32_t lsm = lds_addr(smem);
  // Stage order.  Weight rows K * 2 bytes apart, with K a multiple of 2048
  // (16 KB rows at D = 8192), put every workgroup of a split on the same low
  // address bits at once while they stream in lockstep, which crowds a few
  // memory channels.  With one M block (no W tile shared through L2 by
  // neighbouring workgroups) each W tile therefore starts its K range at
  // stage tn % NT and wraps around: 64-token gate/up 37.7 -> 30.0 us.  With
  // several M blocks the common order is kept: rotating it there lost the
  // L2 reuse of shared tiles (512-token gate/up 77 -> 89 us).
  const int NT = (ke - kb + BK - 1) / BK;
  const int rot = (mt_n == 1 && K % 2048 == 0) ? tn % NT : 0;
  auto issue = [&](int st, int buf) {
    const uint32_t la = lsm + buf * kStage, lb = la + kStageA;
    int sr = st + rot;  // stages past NT - 1 start at ke: zero-filled
    if (sr >= NT) sr = st < NT ? sr - NT : NT;
    const int k0 = kb + sr * BK;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int q = wave + h * 8;
      const int r = q * 8 + rr;
      const int c = sl ^ ((r >> 1) & 7);
      const int k = k0 + c * 8;
      const bool kin = k < ke;
      const uint32_t oa = (kin && m0 + r < M) ? (uint32_t)r * (uint32_t)lda * 2u + (uint32_t)k * 2u
                                              : kOob;
      lds_dma16(ra, oa, la + q * 1024);
      int wr;  // row within its weight matrix block
      if constexpr (EPI == EPI_SWIGLU)
        wr = r & 63;  // h == 0: gate rows (r < 64), h == 1: up rows
      else
        wr = r;
      const uint32_t ow = (kin && wr < wrows) ? (uint32_t)wr * (uint32_t)K * 2u + (uint32_t)k * 2u
                                              : kOob;
      lds_dma16((EPI == EPI_SWIGLU && h == 1) ? rw1 : rw0, ow, lb + q * 1024);
    }
  };

  // W tile rows feeding this wave's two 32-column fragments
  int brow[2];
  if constexpr (EPI == EPI_SWIGLU) {
    brow[0] = wn * 32;       // gate f = c0 + wn*32 + lane%32
    brow[1] = 64 + wn * 32;  // up, same f
  } else {
    brow[0] = wn * 64;
    brow[1] = wn * 64 + 32;
  }

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

#pragma unroll
  for (int st = 0; st < S - 1; ++st) issue(st, st);

  for (int kt = 0; kt < NT; ++kt) {
    wait_vmcnt<(S - 2) * 4>();  // this wave's part of stage kt has landed
    __syncthreads();            // everyone's has; stage kt - 1 is consumed
    const unsigned char* sa = smem + (kt % S) * kStage;
    const unsigned char* sb = sa + kStageA;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = (2 * g + h) * 2 + (lane >> 5);  // 16-wide K step 2g + h
      bf16x8_t af[2], bw[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        af[i] = *reinterpret_cast<const bf16x8_t*>(sa + lds_off(wm * 64 + i * 32 + (lane & 31), c));
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bw[j] = *reinterpret_cast<const bf16x8_t*>(sb + lds_off(brow[j] + (lane & 31), c));
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bw[j], acc[i][j], 0, 0, 0);
    }
    // refill stage kt - 1 (free since the barrier above) after this stage's
    // MFMAs are issued: a copy issue that stalls on a full memory pipeline
    // then no longer delays them (measured 4-7 % faster at K = 8192)
    issue(kt + S - 1, (kt + S - 1) % S);
  }

  wait_vmcnt<0>();  // zero-fill loads of stages past the end have landed
  __syncthreads();

  // ---- both K groups write their accumulators to LDS as row-major [BM][BN]
  // tiles (W-tile row order; for SwiGLU the up column of gate column c sits
  // at c + 64); every thread then adds the two groups over runs of 4 columns
  // and stores 16-byte (fp32) or 8-byte (bf16) runs -- a few store
  // instructions per thread instead of 32..64 single-element stores in each
  // wave of one group
  float* tg = reinterpret_cast<float*>(smem) + g * (BM * BN);
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        tg[(wm * 64 + i * 32 + acc_row32(r, lane)) * BN + brow[j] + (lane & 31)] = acc[i][j][r];
  __syncthreads();
  const f32x4_t* t0 = reinterpret_cast<const f32x4_t*>(smem);
  const f32x4_t* t1 = t0 + BM * BN / 4;

  if (ns > 1) {
    // ---- split K: partial tile [BM][BN], then arrival
    const int64_t tile_elems = (int64_t)BM * BN;
    const __amdgpu_buffer_rsrc_t pr =
        make_rsrc(part, (uint32_t)((int64_t)ns * tiles * tile_elems * 4));
    const int64_t tbase = (int64_t)tile * tile_elems;  // split 0 of this tile
    const int64_t plane = (int64_t)tiles * tile_elems;
#pragma unroll
    for (int k = 0; k < BM * BN / 4 / kThreads; ++k) {
      const int q = tid + k * kThreads;
      __builtin_amdgcn_raw_buffer_store_b128(
          __builtin_bit_cast(u32x4_t, t0[q] + t1[q]), pr,
          (uint32_t)((split * plane + tbase + 4 * q) * 4), 0, kAuxSys);
    }
    int* is_last = reinterpret_cast<int*>(smem + 2 * BM * BN * 4);  // past both tiles
    wait_vmcnt<0>();  // partial stores have reached memory
    __syncthreads();
    if (tid == 0) *is_last = arrive_last(counters + tile, (unsigned)ns);
    __syncthreads();
    if (!*is_last) return;
    finish_splits<EPI, BM, BN, kThreads, 8>(pr, tbase, plane, ns, m0, c0, M, N, out, ldo, tid,
                                            split, t0, t1);
    return;
  }

  // ---- direct epilogue: item = 4 output columns of one row
  constexpr int kQ = kCols / 4;  // items per tile row
#pragma unroll
  for (int k = 0; k < BM * kQ / kThreads; ++k) {
    const int idx = tid + k * kThreads;
    const int tr = idx / kQ, tc = (idx % kQ) * 4;
    const int m = m0 + tr;
    if (m >= M || c0 + tc >= N) continue;
    const int fi = (tr * BN + tc) / 4;
    f32x4_t v = t0[fi] + t1[fi];
    if constexpr (EPI == EPI_SWIGLU) {
      const f32x4_t u = t0[fi + 16] + t1[fi + 16];  // up: 64 columns on
      v = f32x4_t{silu(v.x) * u.x, silu(v.y) * u.y, silu(v.z) * u.z, silu(v.w) * u.w};
    }
    store_out4<EPI == EPI_F32 ? EPI_F32 : EPI_DT>(out, ldo, m, c0 + tc, min(4, N - (c0 + tc)), v);
  }
}

// ---------------------------------------------------------------- 256 x 256
// The same product with 256 x 256 workgroup tiles for many tokens (M >= 384):
// per K element a CU copies 2 x 256 rows for 2 x 256 x 256 FLOPs, twice the
// FLOPs per copied byte of the 128 x 128 tile.  At these shapes the global
// -> LDS copy stream of a CU runs at about 24-26 B/clk however deep the
// pipeline (the L1's misses in flight over their latency), which caps a
// 128 x 128 tile near 41 % of MFMA peak and a 256 x 256 tile near 75 %.
//   * eight waves in a 2 x 4 grid of 128 x 64 wave tiles (4 x 2 MFMA
//     fragments, 128 fp32 accumulators per lane), no K groups;
//   * K stages of 32 (64-byte tile rows, 32 KB per stage), five stages (all
//     160 KB of LDS), four in flight; 16-byte chunk c of row r sits in slot
//     c ^ ((r / 4) % 4), so each 16-lane phase of an operand read covers all
//     64 banks once;
//   * SwiGLU: the W tile is 128 gate rows then the same 128 up rows, and
//     each wave holds 32 gate and the matching 32 up columns;
//   * split K and the XCD-aware order as in the 128 x 128 kernel.
constexpr int BB = 256;                          // tile rows of A and of W
constexpr int BKB = 32;                          // K per stage
constexpr int kRowBB = BKB * 2;                  // 64-byte tile rows
constexpr int kStageBA = BB * kRowBB;            // 16 KB
constexpr int kStageB = 2 * kStageBA;            // 32 KB
constexpr int SB = 5;
constexpr int kLdsB = SB * kStageB;              // 160 KB

__device__ __forceinline__ int lds_off64(int row, int chunk) {
  return row * kRowBB + ((chunk ^ ((row >> 2) & 3)) << 4);
}

// NWB waves: 8 in a 2 x 4 grid of 128 x 64 wave tiles (used), or 4 in a
// 2 x 2 grid of 128 x 128 -- a third fewer LDS bytes per MFMA at one wave per
// SIMD, but measured 3-4 % slower at 512 tokens (TP=1 gate/up 605 us
// against 582), so only the 8-wave form is launched.
template <int EPI, int NWB>
__global__ void __launch_bounds__(NWB * 64)
gemm_big_kernel(int M, int N, int K, const uint16_t* __restrict__ A, int64_t lda,
                const uint16_t* __restrict__ W0, const uint16_t* __restrict__ W1,
                void* __restrict__ out, int64_t ldo, int KR, unsigned* __restrict__ counters,
                float* __restrict__ part) {
  // S stages of (A tile, W tile); after the K loop the first word holds the
  // split-K arrival flag
  __shared__ __attribute__((aligned(16))) unsigned char smem[kLdsB];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  constexpr int WNW = NWB / 2;              // waves along N
  constexpr int NF = 8 / WNW;               // 32-column fragments per wave: 2 or 4
  constexpr int kInstB = 32 / NWB;          // copy instructions per wave per stage
  constexpr int kThr = NWB * 64;
  const int wm = wave / WNW, wn = wave % WNW;

  const int mt_n = (M + BB - 1) / BB;
  constexpr int kCols = (EPI == EPI_SWIGLU) ? BB / 2 : BB;  // output columns per tile
  const int nt_n = (N + kCols - 1) / kCols;
  const int tiles = mt_n * nt_n;
  const int ns = (K + KR - 1) / KR;
  const int G = tiles * ns;
  int b = blockIdx.x;
  const int G8 = G & ~7;
  if (b < G8) b = (b & 7) * (G8 >> 3) + (b >> 3);
  const int split = b / tiles;
  const int tile = b % tiles;
  const int tm = tile % mt_n, tn = tile / mt_n;
  const int m0 = tm * BB, c0 = tn * kCols;
  const int kb = split * KR, ke = min(K, kb + KR);

  const u32x4_t ra = rsrc_words(A + (int64_t)m0 * lda, (uint32_t)min(BB, M - m0) * (uint32_t)lda * 2u);
  const int wrows = min(kCols, N - c0);
  const u32x4_t rw0 = rsrc_words(W0 + (int64_t)c0 * K, (uint32_t)wrows * (uint32_t)K * 2u);
  const u32x4_t rw1 = rsrc_words((EPI == EPI_SWIGLU ? W1 : W0) + (int64_t)c0 * K,
                                 (uint32_t)wrows * (uint32_t)K * 2u);

  // Stage st into buffer buf: 32 instructions of 1 KB (16 tile rows each),
  // 16 for A then 16 for W; wave w issues instructions w, w + NWB, ...
  // Lane l fills slot l % 4 of row 16 q + l / 4 with the logical chunk that
  // lds_off64 places there.
  const int rr = lane >> 2, sl = lane & 3;
  const uint32_t lsm = lds_addr(smem);
  auto issue = [&](int st, int buf) {
    const uint32_t la = lsm + buf * kStageB;
    const int k0 = kb + st * BKB;
#pragma unroll
    for (int h = 0; h < kInstB; ++h) {
      const int q = wave + h * NWB;           // 0..31; q < 16: A rows, else W rows
      const int r = (q & 15) * 16 + rr;       // row in its 256-row tile
      const int c = sl ^ ((r >> 2) & 3);
      const int k = k0 + c * 8;
      const bool kin = k < ke;
      if (h < kInstB / 2) {
        const uint32_t oa = (kin && m0 + r < M) ? (uint32_t)r * (uint32_t)lda * 2u + (uint32_t)k * 2u
                                                : kOob;
        lds_dma16(ra, oa, la + q * 1024);
      } else {
        const int wr = (EPI == EPI_SWIGLU) ? (r & 127) : r;
        const uint32_t ow = (kin && wr < wrows) ? (uint32_t)wr * (uint32_t)K * 2u + (uint32_t)k * 2u
                                                : kOob;
        lds_dma16((EPI == EPI_SWIGLU && r >= 128) ? rw1 : rw0, ow, la + q * 1024);
      }
    }
  };

  // W tile rows of this wave's fragments.  SwiGLU: the first NF/2 are gate
  // rows of F = c0 + wn (128/WNW) + 32 j + lane%32, the last NF/2 the up
  // rows of the same F.
  int brow[NF];
#pragma unroll
  for (int j = 0; j < NF; ++j) {
    if constexpr (EPI == EPI_SWIGLU)
      brow[j] = (j < NF / 2 ? 0 : 128) + wn * (128 / WNW) + (j % (NF / 2)) * 32;
    else
      brow[j] = wn * (256 / WNW) + j * 32;
  }

  f32x16_t acc[4][NF];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NF; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // Operands of one 16-wide K step (ks) of a stage, read one step ahead of
  // the MFMAs that use them.
  bf16x8_t af[2][4], bw[2][NF];
  auto read_ops = [&](int buf, int ks, bf16x8_t (&a)[4], bf16x8_t (&w)[NF]) {
    const unsigned char* sa = smem + buf * kStageB;
    const unsigned char* sb = sa + kStageBA;
    const int c = ks * 2 + (lane >> 5);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      a[i] = *reinterpret_cast<const bf16x8_t*>(sa + lds_off64(wm * 128 + i * 32 + (lane & 31), c));
#pragma unroll
    for (int j = 0; j < NF; ++j)
      w[j] = *reinterpret_cast<const bf16x8_t*>(sb + lds_off64(brow[j] + (lane & 31), c));
  };
  auto mfmas = [&](const bf16x8_t (&a)[4], const bf16x8_t (&w)[NF]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < NF; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], w[j], acc[i][j], 0, 0, 0);
  };

  // All SB buffers hold stages in flight: stage kt + SB is copied into the
  // buffer of stage kt once every wave has its last operands of stage kt in
  // registers.  The barrier sits between the two K steps' MFMAs of a stage:
  // the pipe drains the first step's MFMAs while the waves meet, and the
  // second step's run while the next stage's first operands are read.
  const int NT = (ke - kb + BKB - 1) / BKB;
#pragma unroll
  for (int st = 0; st < SB; ++st)
    if (st < NT) issue(st, st);
  if (NT >= SB)
    wait_vmcnt<(SB - 1) * kInstB>();  // stage 0 has landed
  else
    wait_vmcnt<0>();
  __syncthreads();
  read_ops(0, 0, af[0], bw[0]);
  int buf = 0;  // kt % SB
  // The two K steps of stage kt: the next step's 4 + NF operand reads are
  // issued ahead of the current step's 4 NF MFMAs (the scheduler is held to
  // that order).
  auto first_half = [&]() {
    read_ops(buf, 1, af[1], bw[1]);
    mfmas(af[0], bw[0]);
    __builtin_amdgcn_sched_group_barrier(0x100, 4 + NF, 0);  // DS reads
    __builtin_amdgcn_sched_group_barrier(0x008, 4 * NF, 0);  // MFMA
    __builtin_amdgcn_sched_barrier(0);                  // nothing moves past here
  };
  auto second_half = [&]() {
    buf = buf == SB - 1 ? 0 : buf + 1;
    read_ops(buf, 0, af[0], bw[0]);
    mfmas(af[1], bw[1]);
    __builtin_amdgcn_sched_group_barrier(0x100, 4 + NF, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 4 * NF, 0);
    __builtin_amdgcn_sched_barrier(0);
  };
  int kt = 0;
  // steady state: stage kt + 1 has landed once the SB - 2 stages after it
  // are the only ones in flight; stage kt + SB refills stage kt's buffer
  for (; kt < NT - SB; ++kt) {
    first_half();
    wait_vmcnt<(SB - 2) * kInstB>();
    wait_lgkmcnt0();  // this wave's reads of stage kt are in registers
    __syncthreads();  // everyone's have; stage kt + 1 is in LDS
    if constexpr (EPI == EPI_SWIGLU) {
      // refill after the second half's MFMAs: TP=1 gate/up 547-551 -> 527-537
      // us on one box; the fp32 down product measured 5 % slower this way
      const int ib = buf;
      second_half();
      issue(kt + SB, ib);
    } else {
      issue(kt + SB, buf);
      second_half();
    }
  }
  // the last stages: nothing more to copy
  for (; kt < NT - 1; ++kt) {
    first_half();
    if (kt + SB - 1 < NT)
      wait_vmcnt<(SB - 2) * kInstB>();
    else
      wait_vmcnt<0>();
    wait_lgkmcnt0();
    __syncthreads();
    second_half();
  }
  read_ops(buf, 1, af[1], bw[1]);
  mfmas(af[0], bw[0]);
  mfmas(af[1], bw[1]);

  if (ns == 1) {
    if constexpr (EPI == EPI_SWIGLU) {
#pragma unroll
      for (int j = 0; j < NF / 2; ++j) {
        const int col = c0 + wn * (128 / WNW) + j * 32 + (lane & 31);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int m = m0 + wm * 128 + i * 32 + acc_row32(r, lane);
            if (m < M && col < N)
              store_out<EPI_DT>(out, ldo, m, col, silu(acc[i][j][r]) * acc[i][j + NF / 2][r]);
          }
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NF; ++j) {
          const int col = c0 + wn * (256 / WNW) + j * 32 + (lane & 31);
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int m = m0 + wm * 128 + i * 32 + acc_row32(r, lane);
            if (m < M && col < N) store_out<EPI>(out, ldo, m, col, acc[i][j][r]);
          }
        }
    }
    return;
  }

  // ---- split K: partial tile [BB][BB] in W-tile row order, then arrival
  const int64_t tile_elems = (int64_t)BB * BB;
  const __amdgpu_buffer_rsrc_t pr =
      make_rsrc(part, (uint32_t)((int64_t)ns * tiles * tile_elems * 4));
  const int64_t tbase = (int64_t)tile * tile_elems;
  const int64_t plane = (int64_t)tiles * tile_elems;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NF; ++j) {
      const int tc = brow[j] + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int tr = wm * 128 + i * 32 + acc_row32(r, lane);
        const float v = acc[i][j][r];
        __builtin_amdgcn_raw_buffer_store_b32(
            __builtin_bit_cast(uint32_t, v), pr,
            (uint32_t)((split * plane + tbase + tr * BB + tc) * 4), 0, kAuxSys);
      }
    }
  int* is_last = reinterpret_cast<int*>(smem);  // the stages are consumed
  wait_vmcnt<0>();  // partial stores have reached memory
  __syncthreads();
  if (tid == 0) *is_last = arrive_last(counters + tile, (unsigned)ns);
  __syncthreads();
  if (!*is_last) return;
  finish_splits<EPI, BB, BB, kThr, 4>(pr, tbase, plane, ns, m0, c0, M, N, out, ldo, tid, -1,
                                      nullptr, nullptr);
}

struct Plan {
  bool big = false;  // 256 x 256 tiles
  int tiles = 0;
  int ns = 0;  // K splits
  int kr = 0;  // K per split
  int grid = 0;
};

// Cost model (CU cycles) for a tile size and split count.  A workgroup's
// main loop runs at the rate its copy stream reaches next to the MFMA work,
// measured on this chip at the prefill shapes with every CU busy: about
// 21 B/clk per CU for 128 x 128 tiles and 12.5 B/clk for 256 x 256 (whose
// copies then interleave less well with the longer MFMA runs), or at the
// MFMA rate if that is lower.  Workgroups run in rounds of one per CU; with
// split K each workgroup also writes its partial tile and the last of a
// tile's workgroups reads all of them, each at the slower of a CU's stream
// (about 24 B/clk) and its share of HBM (about 2 KB/clk for the chip).
double plan_cost(int tiles, int ns, bool big, int K) {
  const int bm = big ? BB : BM, bn = big ? BB : BN;
  const double rate = big ? 12.5 : 21.0;
  const double kspl = std::ceil((double)K / BK / ns) * BK;  // K per split
  const double copy = (double)(bm + bn) * kspl * 2.0 / rate;
  const double mfma = 2.0 * bm * bn * kspl / (4.0 * 1024.0) / 0.9;
  const double rounds = std::ceil((double)tiles * ns / kCUs);
  const double tile_bytes = (double)bm * bn * 4.0;
  if (ns == 1) return rounds * std::max(copy, mfma) + 1500.0;
  const double hbm = 2080.0;  // B/clk, the whole chip
  const double wgs = (double)tiles * ns;
  const double write = std::max(tile_bytes / 24.0, std::min(wgs, (double)kCUs) * tile_bytes / hbm);
  const double reduce = std::max(ns * tile_bytes / 24.0, wgs * tile_bytes / hbm);
  return rounds * (std::max(copy, mfma) + write) + reduce + 1500.0;
}

// Split K when the tiles alone leave CUs idle: the split count and tile size
// of least modelled cost; at least 8 stages of K per split, at most 256 MB of
// partials and one arrival counter per tile.
constexpr double kMaxPartialBytes = 256.0 * 1024 * 1024;
Plan make_plan(int M, int N, int K, bool swiglu) {
  Plan best_pl;
  double best = 1e300;
  const int kst = (K + BK - 1) / BK;  // K stages in all
  const int max_ns = std::max(1, std::min(16, kst / 8));
  for (int big = 0; big < 2; ++big) {
    if (big && M < 384) continue;
    const int bm = big ? BB : BM, bn = big ? BB : BN;
    const int cols = swiglu ? bn / 2 : bn;
    const int tiles = ((M + bm - 1) / bm) * ((N + cols - 1) / cols);
    for (int ns = 1; ns <= max_ns; ++ns) {
      if (ns > 1 && ((double)ns * tiles * bm * bn * 4.0 > kMaxPartialBytes || tiles > kWsMaxCounters))
        break;
      const double cost = plan_cost(tiles, ns, big, K);
      if (cost < best * (1.0 - 1e-9)) {
        best = cost;
        best_pl.big = big;
        best_pl.tiles = tiles;
        best_pl.ns = ns;
      }
    }
  }
  const int sps = (kst + best_pl.ns - 1) / best_pl.ns;  // stages per split
  best_pl.kr = sps * BK;
  best_pl.ns = (K + best_pl.kr - 1) / best_pl.kr;
  best_pl.grid = best_pl.tiles * best_pl.ns;
  return best_pl;
}

size_t plan_bytes(const Plan& pl) {
  if (pl.ns <= 1) return 0;
  const size_t te = pl.big ? (size_t)BB * BB : (size_t)BM * BN;
  return kWsCounterBytes + (size_t)pl.ns * pl.tiles * te * sizeof(float);
}

template <int EPI>
hipError_t launch_plan(const Plan& pl, int M, int N, int K, const uint16_t* A, int64_t lda,
                       const uint16_t* W0, const uint16_t* W1, void* out, int64_t ldo,
                       void* workspace, hipStream_t stream) {
  auto kern = pl.big ? gemm_big_kernel<EPI, 8> : gemm_kernel<EPI>;
  const int threads = pl.big ? 8 * 64 : kThreads;
  unsigned* counters = nullptr;
  float* part = nullptr;
  if (pl.ns > 1) {
    if (workspace == nullptr || pl.tiles > kWsMaxCounters) return hipErrorInvalidValue;
    counters = static_cast<unsigned*>(workspace);
    part = reinterpret_cast<float*>(static_cast<char*>(workspace) + kWsCounterBytes);
  }
  hipLaunchKernelGGL(kern, dim3(pl.grid), dim3(threads), 0, stream, M, N, K, A, lda, W0,
                     W1, out, ldo, pl.kr, counters, part);
  return hipGetLastError();
}

}  // namespace

size_t gemm_workspace_bytes(int M, int N, int K, bool swiglu) {
  return plan_bytes(make_plan(M, N, K, swiglu));
}

template <int EPI>
hipError_t gemm_launch(int M, int N, int K, const uint16_t* A, int64_t lda, const uint16_t* W0,
                       const uint16_t* W1, void* out, int64_t ldo, void* workspace,
                       hipStream_t stream) {
  const Plan pl = make_plan(M, N, K, EPI == EPI_SWIGLU);
  if (pl.grid == 0) return hipErrorInvalidValue;
  return launch_plan<EPI>(pl, M, N, K, A, lda, W0, W1, out, ldo, workspace, stream);
}

template hipError_t gemm_launch<EPI_F32>(int, int, int, const uint16_t*, int64_t,
                                         const uint16_t*, const uint16_t*, void*, int64_t, void*,
                                         hipStream_t);
template hipError_t gemm_launch<EPI_DT>(int, int, int, const uint16_t*, int64_t,
                                        const uint16_t*, const uint16_t*, void*, int64_t, void*,
                                        hipStream_t);
template hipError_t gemm_launch<EPI_SWIGLU>(int, int, int, const uint16_t*, int64_t,
                                            const uint16_t*, const uint16_t*, void*, int64_t,
                                            void*, hipStream_t);

}  // namespace tpk
