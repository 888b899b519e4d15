// Projections for many tokens: C[M, N] = A[M, K] . W[N, K]^T on bf16 MFMA
// (v_mfma_f32_32x32x16_bf16, fp32 accumulation), in two tile shapes chosen
// per call by a cost model: 128 x 128 (described here) and 256 x 128
// (described at its kernel below).
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
//   * with more than one round of tiles and a last round at most half full
//     (the unsharded gate/up at 512 tokens: 896 tiles), the whole rounds run
//     as one launch with K unsplit and the last round's tiles as a second
//     launch with K split, so that it fills the chip; each launch takes its
//     range of tiles (tile0, ntl);
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

// Scales of output columns col .. col + n - 1 (n <= 4; the rest 0).
__device__ __forceinline__ f32x4_t col_scales(const float* S, int col, int n) {
  f32x4_t v = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int e = 0; e < 4; ++e)
    if (e < n) v[e] = S[col + e];
  return v;
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
// the row-major tiles own0 and own1, or own0 alone when own1 is null), that
// split is taken from there.  With one-byte weights, S0 (and S1, the up
// rows') hold the fp32 scale of each output column, applied to the sums
// before the epilogue.
template <int EPI, int TM, int TN, int THREADS, int IQ>
__device__ __forceinline__ void finish_splits(const __amdgpu_buffer_rsrc_t pr, int64_t tbase,
                                              int64_t plane, int ns, int m0, int c0, int M,
                                              int N, void* out, int64_t ldo, int tid, int own,
                                              const f32x4_t* own0, const f32x4_t* own1,
                                              const float* S0 = nullptr,
                                              const float* S1 = nullptr) {
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
              v[i][q][e] = own1 ? own0[fi[i][q]] + own1[fi[i][q]] : own0[fi[i][q]];
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
      const int n = min(4, N - (c0 + tc[i]));
      f32x4_t v = s[i][0];
      if (S0) v *= col_scales(S0, c0 + tc[i], n);
      if constexpr (EPI == EPI_SWIGLU) {
        f32x4_t u = s[i][1];
        if (S1) u *= col_scales(S1, c0 + tc[i], n);
        v = f32x4_t{silu(v.x) * u.x, silu(v.y) * u.y, silu(v.z) * u.z, silu(v.w) * u.w};
      }
      store_out4<EPI == EPI_F32 ? EPI_F32 : EPI_DT>(out, ldo, m, c0 + tc[i], n, v);
    }
  }
}

// One launch: grid = tiles * ns workgroups of 512 threads, 160 KB of static LDS.
//   KR: K elements per split (multiple of BK); ns = ceil(K / KR).
//   counters/part: split-K workspace (unused when ns == 1).
template <int EPI>
__global__ void __launch_bounds__(kThreads)
gemm_kernel(int M, int N, int K, const uint16_t* __restrict__ A, int64_t lda,
            const uint16_t* __restrict__ W0, const uint16_t* __restrict__ W1,
            void* __restrict__ out, int64_t ldo, int KR, unsigned* __restrict__ counters,
            float* __restrict__ part, int tile0, int ntl) {
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
  const int tiles = ntl;  // this launch's tiles: tile0 .. tile0 + ntl - 1 of the product
  const int ns = (K + KR - 1) / KR;
  const int G = tiles * ns;
  int b = blockIdx.x;
  const int G8 = G & ~7;
  if (b < G8) b = (b & 7) * (G8 >> 3) + (b >> 3);
  const int split = b / tiles;
  const int tile = b % tiles;  // within the launch: arrival counter and partial slot
  const int tm = (tile0 + tile) % mt_n, tn = (tile0 + tile) / mt_n;
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

// ---------------------------------------------------------------- 256 x 128
// The same product with 256 x 128 workgroup tiles (256 activation rows, 128
// weight rows): per K element a CU copies 384 rows for 2 x 256 x 128 FLOPs, a
// quarter fewer bytes per FLOP than the 128 x 128 tile.  The per-rank shapes
// give half as many tiles, so K is split in two to fill the chip.  Its
// copies alone take a fifth less time than the 128 x 128 kernel's, but its
// MFMA and LDS work overlaps them less: measured, it ties the 128 x 128
// kernel on the TP=8 gate/up at 512 tokens (75-77 us against 80) and beats
// the 256 x 256 kernel it replaced on the TP=1 down (263-277 us split 2 ways
// against 304 split 4 ways).
//   * eight waves: a 2 x 2 grid of 128 x 64 wave tiles (4 x 2 MFMA
//     fragments, 128 fp32 accumulators per lane), twice -- the two groups of
//     four waves take alternate pairs of every stage's 16-wide K steps, so
//     the LDS bytes read per MFMA are those of a 256 x 256 tile;
//   * 64 K per stage in 128-byte tile rows (the 128 x 128 kernel's layout):
//     three 48 KB stages, two in flight.  Stages of 32 K (64-byte rows, six
//     24 KB stages) request each 128-byte line in two halves one stage apart
//     and were much slower: the TP=1 MLP at 512 tokens took 927 us against
//     723.  A 256 x 256 kernel with such rows (12.5 B/clk per CU) was
//     replaced by this one;
//   * after the K loop the second group's accumulators go to one row-major
//     [256][128] fp32 tile in LDS and the first group adds its own in place,
//     then the epilogue (or the split-K partial store) reads that tile;
//   * SwiGLU, split K and the XCD-aware order as in the 128 x 128 kernel.
constexpr int WM = 256, WN = 128, WK = 64;
constexpr int kRowW = WK * 2;                 // 128-byte tile rows
constexpr int kStageWA = WM * kRowW;          // 32 KB
constexpr int kStageW = (WM + WN) * kRowW;    // 48 KB
constexpr int SW = 3;                         // stages
constexpr int kLdsW = SW * kStageW;           // 144 KB
constexpr int kInstWA = WM / 8 / 8;           // A copy instructions per wave and stage (8 rows each)
constexpr int kInstWW = WN / 8 / 8;           // W copy instructions per wave and stage
constexpr int kInstW = kInstWA + kInstWW;
static_assert(WM * WN * 4 + 4 <= kLdsW, "the K-group tile and the arrival flag fit");

template <int EPI>
__global__ void __launch_bounds__(kThreads)
gemm_wide_kernel(int M, int N, int K, const uint16_t* __restrict__ A, int64_t lda,
                 const uint16_t* __restrict__ W0, const uint16_t* __restrict__ W1,
                 void* __restrict__ out, int64_t ldo, int KR, unsigned* __restrict__ counters,
                 float* __restrict__ part, int tile0, int ntl) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[kLdsW];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = wave >> 2;  // K group
  const int wm = (wave >> 1) & 1, wn = wave & 1;

  const int mt_n = (M + WM - 1) / WM;
  constexpr int kCols = (EPI == EPI_SWIGLU) ? WN / 2 : WN;  // output columns per tile
  const int tiles = ntl;  // this launch's tiles: tile0 .. tile0 + ntl - 1 of the product
  const int ns = (K + KR - 1) / KR;
  const int G = tiles * ns;
  int b = blockIdx.x;
  const int G8 = G & ~7;
  if (b < G8) b = (b & 7) * (G8 >> 3) + (b >> 3);
  const int split = b / tiles;
  const int tile = b % tiles;  // within the launch: arrival counter and partial slot
  const int tm = (tile0 + tile) % mt_n, tn = (tile0 + tile) / mt_n;
  const int m0 = tm * WM, c0 = tn * kCols;
  const int kb = split * KR, ke = min(K, kb + KR);

  const u32x4_t ra = rsrc_words(A + (int64_t)m0 * lda, (uint32_t)min(WM, M - m0) * (uint32_t)lda * 2u);
  const int wrows = min(kCols, N - c0);
  const u32x4_t rw0 = rsrc_words(W0 + (int64_t)c0 * K, (uint32_t)wrows * (uint32_t)K * 2u);
  const u32x4_t rw1 = rsrc_words((EPI == EPI_SWIGLU ? W1 : W0) + (int64_t)c0 * K,
                                 (uint32_t)wrows * (uint32_t)K * 2u);

  // Stage st into buffer buf: 1 KB copy instructions of 8 tile rows, first
  // the A rows, then the W rows; wave w issues A instructions w, w + 8, ...
  // and W instructions likewise.  Lane l fills slot l % 8 of row 8 q + l / 8
  // with the logical chunk that lds_off places there; past the K range, M or
  // N the offset is out of range and the slot is zero-filled.
  const int rr = lane >> 3, sl = lane & 7;
  const uint32_t lsm = lds_addr(smem);
  auto issue = [&](int st, int buf) {
    const uint32_t la = lsm + buf * kStageW;
    const int k0 = kb + st * WK;
#pragma unroll
    for (int h = 0; h < kInstWA; ++h) {
      const int q = wave + h * 8;
      const int r = q * 8 + rr;
      const int k = k0 + (sl ^ ((r >> 1) & 7)) * 8;
      const uint32_t oa = (k < ke && m0 + r < M) ? (uint32_t)r * (uint32_t)lda * 2u + (uint32_t)k * 2u
                                                 : kOob;
      lds_dma16(ra, oa, la + q * 1024);
    }
#pragma unroll
    for (int h = 0; h < kInstWW; ++h) {
      const int q = wave + h * 8;
      const int r = q * 8 + rr;  // W tile row
      const int k = k0 + (sl ^ ((r >> 1) & 7)) * 8;
      const int wr = (EPI == EPI_SWIGLU) ? (r & 63) : r;  // SwiGLU: 64 gate rows, then 64 up
      const uint32_t ow = (k < ke && wr < wrows) ? (uint32_t)wr * (uint32_t)K * 2u + (uint32_t)k * 2u
                                                 : kOob;
      lds_dma16((EPI == EPI_SWIGLU && r >= 64) ? rw1 : rw0, ow, la + kStageWA + q * 1024);
    }
  };

  // W tile rows of this wave's two 32-column fragments
  int brow[2];
  if constexpr (EPI == EPI_SWIGLU) {
    brow[0] = wn * 32;       // gate f = c0 + wn*32 + lane%32
    brow[1] = 64 + wn * 32;  // up, same f
  } else {
    brow[0] = wn * 64;
    brow[1] = wn * 64 + 32;
  }

  f32x16_t acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int NT = (ke - kb + WK - 1) / WK;
#pragma unroll
  for (int st = 0; st < SW - 1; ++st) issue(st, st);

  int buf = 0;  // kt % SW
  for (int kt = 0; kt < NT; ++kt) {
    wait_vmcnt<(SW - 2) * kInstW>();  // this wave's part of stage kt has landed
    __syncthreads();                  // everyone's has; stage kt - 1 is consumed
    const unsigned char* sa = smem + buf * kStageW;
    const unsigned char* sb = sa + kStageWA;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = (2 * g + h) * 2 + (lane >> 5);  // 16-wide K step 2g + h
      bf16x8_t af[4], bw[2];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = *reinterpret_cast<const bf16x8_t*>(sa + lds_off(wm * 128 + i * 32 + (lane & 31), c));
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bw[j] = *reinterpret_cast<const bf16x8_t*>(sb + lds_off(brow[j] + (lane & 31), c));
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bw[j], acc[i][j], 0, 0, 0);
    }
    // refill stage kt - 1's buffer after this stage's MFMAs are issued
    // (issuing it before them measured slower: the copy issue stalls them)
    issue(kt + SW - 1, buf == 0 ? SW - 1 : buf - 1);
    buf = buf == SW - 1 ? 0 : buf + 1;
  }

  wait_vmcnt<0>();  // zero-fill loads of stages past the end have landed
  __syncthreads();

  // ---- one row-major [WM][WN] fp32 tile: group 1 writes, group 0 adds
  float* T = reinterpret_cast<float*>(smem);
  if (g == 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          T[(wm * 128 + i * 32 + acc_row32(r, lane)) * WN + brow[j] + (lane & 31)] = acc[i][j][r];
  }
  __syncthreads();
  if (g == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          T[(wm * 128 + i * 32 + acc_row32(r, lane)) * WN + brow[j] + (lane & 31)] += acc[i][j][r];
  }
  __syncthreads();
  const f32x4_t* t0 = reinterpret_cast<const f32x4_t*>(smem);

  if (ns > 1) {
    const int64_t tile_elems = (int64_t)WM * WN;
    const __amdgpu_buffer_rsrc_t pr =
        make_rsrc(part, (uint32_t)((int64_t)ns * tiles * tile_elems * 4));
    const int64_t tbase = (int64_t)tile * tile_elems;
    const int64_t plane = (int64_t)tiles * tile_elems;
#pragma unroll
    for (int k = 0; k < WM * WN / 4 / kThreads; ++k) {
      const int q = tid + k * kThreads;
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, t0[q]), pr,
                                             (uint32_t)((split * plane + tbase + 4 * q) * 4), 0,
                                             kAuxSys);
    }
    int* is_last = reinterpret_cast<int*>(smem + WM * WN * 4);  // past the tile
    wait_vmcnt<0>();  // partial stores have reached memory
    __syncthreads();
    if (tid == 0) *is_last = arrive_last(counters + tile, (unsigned)ns);
    __syncthreads();
    if (!*is_last) return;
    finish_splits<EPI, WM, WN, kThreads, 8>(pr, tbase, plane, ns, m0, c0, M, N, out, ldo, tid,
                                            split, t0, nullptr);
    return;
  }

  constexpr int kQ = kCols / 4;  // items (4 output columns of one row) per tile row
#pragma unroll
  for (int k = 0; k < WM * kQ / kThreads; ++k) {
    const int idx = tid + k * kThreads;
    const int tr = idx / kQ, tc = (idx % kQ) * 4;
    const int m = m0 + tr;
    if (m >= M || c0 + tc >= N) continue;
    const int fi = (tr * WN + tc) / 4;
    f32x4_t v = t0[fi];
    if constexpr (EPI == EPI_SWIGLU) {
      const f32x4_t u = t0[fi + 16];  // up: 64 columns on
      v = f32x4_t{silu(v.x) * u.x, silu(v.y) * u.y, silu(v.z) * u.z, silu(v.w) * u.w};
    }
    store_out4<EPI == EPI_F32 ? EPI_F32 : EPI_DT>(out, ldo, m, c0 + tc, min(4, N - (c0 + tc)), v);
  }
}

// ---------------------------------------------------------------- one-byte weights
// The product with weight-only one-byte codes (OCP E4M3 or signed int8) and
// one fp32 scale per weight row, bf16 activations, for more tokens than the
// streaming kernels take: the 128 x 128 kernel's tiles, waves and K groups,
// with 128 K per stage so that a stage's code rows are whole 128-byte lines
// (activation rows are 256 bytes).  A weight tile then copies half the bytes
// of its bf16 form: 48 KB per stage for 2 x 128 x 128 x 128 FLOPs, against
// 64 KB.
//   * three 48 KB stages, two in flight; activation rows are 16 chunks of 16
//     bytes with chunk c of row r in slot c ^ (r % 16), code rows 8 chunks
//     laid out as the 128 x 128 kernel's operand rows (c ^ ((r / 2) % 8)),
//     so each 16-lane phase of an operand read covers all 64 banks once;
//   * a lane reads one whole 16-code chunk and decodes it exactly to two
//     8-element bf16 chunks (every E4M3 and int8 value is a bf16 value).
//     The two feed two MFMAs: lane half h of chunk pair p takes code chunk
//     2p + h, its low 8 codes in the first MFMA and its high 8 in the
//     second, and reads the activations of the same K (chunks 4p + 2h and
//     4p + 2h + 1 of its row) -- a fixed permutation of K within each MFMA,
//     which leaves the sums' terms unchanged;
//   * each output column's scale multiplies its sum in the epilogue (or in
//     the split-K finish), before silu(g) * u.
// Measured on the Llama TP=8 MLP share, E4M3 weights run faster than bf16
// (57 / 102 us at 128 / 512 tokens against 61 / 114): E4M3 codes decode two
// at a time straight to bf16.  int8 takes a conversion per code and runs at
// about the bf16 rate.
constexpr int QBK = 128;                         // K per stage
constexpr int kRowQA = QBK * 2;                  // 256-byte activation rows
constexpr int kRowQW = QBK;                      // 128-byte code rows
constexpr int kStageQA = BM * kRowQA;            // 32 KB
constexpr int kStageQ = kStageQA + BN * kRowQW;  // 48 KB
constexpr int SQ = 3;                            // stages
constexpr int kLdsQ = SQ * kStageQ;              // 144 KB
constexpr int kInstQA = BM * kRowQA / 1024 / 8;  // activation copy instructions per wave and stage
constexpr int kInstQW = BN * kRowQW / 1024 / 8;  // code copy instructions per wave and stage
constexpr int kInstQ = kInstQA + kInstQW;
static_assert(kRowQW == kRowB, "code rows use the 128 x 128 kernel's row layout");
static_assert(2 * BM * BN * 4 + 4 <= kLdsQ, "both K groups' tiles and the arrival flag fit");

__device__ __forceinline__ int lds_off_qa(int row, int chunk) {
  return row * kRowQA + ((chunk ^ (row & 15)) << 4);
}

template <int EPI, int WF>
__global__ void __launch_bounds__(kThreads)
gemm_q8_kernel(int M, int N, int K, const uint16_t* __restrict__ A, int64_t lda,
               const uint8_t* __restrict__ W0, const float* __restrict__ S0,
               const uint8_t* __restrict__ W1, const float* __restrict__ S1,
               void* __restrict__ out, int64_t ldo, int KR, unsigned* __restrict__ counters,
               float* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[kLdsQ];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = wave >> 2;  // K group: chunk pairs 2g, 2g + 1 of each stage
  const int wm = (wave >> 1) & 1, wn = wave & 1;

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

  const u32x4_t ra = rsrc_words(A + (int64_t)m0 * lda, (uint32_t)min(BM, M - m0) * (uint32_t)lda * 2u);
  const int wrows = min(kCols, N - c0);
  const u32x4_t rw0 = rsrc_words(W0 + (int64_t)c0 * K, (uint32_t)wrows * (uint32_t)K);
  const u32x4_t rw1 = rsrc_words((EPI == EPI_SWIGLU ? W1 : W0) + (int64_t)c0 * K,
                                 (uint32_t)wrows * (uint32_t)K);

  // Stage st into buffer buf.  Activation copies: 4 rows x 256 bytes per 1 KB
  // instruction, lane l filling slot l % 16 of row 4 q + l / 16; code copies:
  // 8 rows x 128 bytes, lane l filling slot l % 8 of row 8 q + l / 8.  Each
  // slot gets the logical chunk its layout places there; past the K range,
  // M or N the offset is out of range and the slot is zero-filled.  With one
  // M block and K a multiple of 2048 the stages start at tn % NT and wrap,
  // as in the 128 x 128 kernel.
  const uint32_t lsm = lds_addr(smem);
  const int NT = (ke - kb + QBK - 1) / QBK;
  const int rot = (mt_n == 1 && K % 2048 == 0) ? tn % NT : 0;
  auto issue = [&](int st, int buf) {
    const uint32_t la = lsm + buf * kStageQ, lb = la + kStageQA;
    int sr = st + rot;  // stages past NT - 1 start at ke: zero-filled
    if (sr >= NT) sr = st < NT ? sr - NT : NT;
    const int k0 = kb + sr * QBK;
#pragma unroll
    for (int h = 0; h < kInstQA; ++h) {
      const int q = wave + h * 8;
      const int r = q * 4 + (lane >> 4);
      const int k = k0 + ((lane & 15) ^ (r & 15)) * 8;
      const uint32_t oa = (k < ke && m0 + r < M) ? (uint32_t)r * (uint32_t)lda * 2u + (uint32_t)k * 2u
                                                 : kOob;
      lds_dma16(ra, oa, la + q * 1024);
    }
#pragma unroll
    for (int h = 0; h < kInstQW; ++h) {
      const int q = wave + h * 8;
      const int r = q * 8 + (lane >> 3);  // code tile row
      const int k = k0 + ((lane & 7) ^ ((r >> 1) & 7)) * 16;
      const int wr = (EPI == EPI_SWIGLU) ? (r & 63) : r;  // SwiGLU: 64 gate rows, then 64 up
      const uint32_t ow = (k < ke && wr < wrows) ? (uint32_t)wr * (uint32_t)K + (uint32_t)k : kOob;
      lds_dma16((EPI == EPI_SWIGLU && r >= 64) ? rw1 : rw0, ow, lb + q * 1024);
    }
  };

  // code tile rows feeding this wave's two 32-column fragments
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
  for (int st = 0; st < SQ - 1; ++st) issue(st, st);

  const int hh = lane >> 5;  // lane half: code chunk 2p + hh of a chunk pair p
  int buf = 0;               // kt % SQ
  for (int kt = 0; kt < NT; ++kt) {
    wait_vmcnt<(SQ - 2) * kInstQ>();  // this wave's part of stage kt has landed
    __syncthreads();                  // everyone's has; stage kt - 1 is consumed
    const unsigned char* sa = smem + buf * kStageQ;
    const unsigned char* sb = sa + kStageQA;
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) {
      const int p = 2 * g + pp;
      bf16x8_t wlo[2], whi[2], alo[2], ahi[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const u32x4_t w =
            *reinterpret_cast<const u32x4_t*>(sb + lds_off(brow[j] + (lane & 31), 2 * p + hh));
        u32x4_t lo, hi;
        if constexpr (WF == kWInt8)
          decode16_i8(w, lo, hi);
        else
          decode16(w, lo, hi);
        wlo[j] = __builtin_bit_cast(bf16x8_t, lo);
        whi[j] = __builtin_bit_cast(bf16x8_t, hi);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int row = wm * 64 + i * 32 + (lane & 31);
        alo[i] = *reinterpret_cast<const bf16x8_t*>(sa + lds_off_qa(row, 4 * p + 2 * hh));
        ahi[i] = *reinterpret_cast<const bf16x8_t*>(sa + lds_off_qa(row, 4 * p + 2 * hh + 1));
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(alo[i], wlo[j], acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahi[i], whi[j], acc[i][j], 0, 0, 0);
        }
    }
    // refill stage kt - 1's buffer after this stage's MFMAs are issued
    issue(kt + SQ - 1, buf == 0 ? SQ - 1 : buf - 1);
    buf = buf == SQ - 1 ? 0 : buf + 1;
  }

  wait_vmcnt<0>();  // zero-fill loads of stages past the end have landed
  __syncthreads();

  // ---- both K groups' accumulators as row-major [BM][BN] tiles in LDS
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
    // ---- split K: unscaled partial tile [BM][BN], then arrival
    const int64_t tile_elems = (int64_t)BM * BN;
    const __amdgpu_buffer_rsrc_t pr =
        make_rsrc(part, (uint32_t)((int64_t)ns * tiles * tile_elems * 4));
    const int64_t tbase = (int64_t)tile * tile_elems;
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
                                            split, t0, t1, S0, EPI == EPI_SWIGLU ? S1 : nullptr);
    return;
  }

  // ---- direct epilogue: item = 4 output columns of one row
  constexpr int kQ = kCols / 4;
#pragma unroll
  for (int k = 0; k < BM * kQ / kThreads; ++k) {
    const int idx = tid + k * kThreads;
    const int tr = idx / kQ, tc = (idx % kQ) * 4;
    const int m = m0 + tr;
    if (m >= M || c0 + tc >= N) continue;
    const int n = min(4, N - (c0 + tc));
    const int fi = (tr * BN + tc) / 4;
    f32x4_t v = (t0[fi] + t1[fi]) * col_scales(S0, c0 + tc, n);
    if constexpr (EPI == EPI_SWIGLU) {
      const f32x4_t u = (t0[fi + 16] + t1[fi + 16]) * col_scales(S1, c0 + tc, n);
      v = f32x4_t{silu(v.x) * u.x, silu(v.y) * u.y, silu(v.z) * u.z, silu(v.w) * u.w};
    }
    store_out4<EPI == EPI_F32 ? EPI_F32 : EPI_DT>(out, ldo, m, c0 + tc, n, v);
  }
}

enum Tile { kT128 = 0, kTWide = 1 };  // 128 x 128, 256 x 128

struct Plan {
  int shape = kT128;
  int tiles = 0;
  int ns = 0;  // K splits
  int kr = 0;  // K per split
  int grid = 0;
  int tile_elems = 0;
  // Split tail: with ns == 1 and more than one round of tiles, the last
  // `tail` tiles may run as a second launch with K split tail_ns ways, so
  // that a partial last round fills every CU (the first launch runs whole
  // rounds).  0: one launch.
  int tail = 0;
  int tail_ns = 0;
  int tail_kr = 0;
};

struct TileShape {
  int bm, bn;     // activation rows, weight rows
  int bk;         // K per stage
  double rate;    // copy stream of a CU next to the MFMA work, B/clk
  double wbytes;  // bytes per weight element
};

// Measured on this chip at the prefill shapes with every CU busy: the 128 x
// 128 kernel's copies run at about 21 B/clk per CU next to its MFMA work,
// the 256 x 128 kernel's at about 19.  The one-byte kernel is taken at the
// 128 x 128 kernel's rate.
constexpr int kNumShapes = 2;
constexpr TileShape kShapes[kNumShapes] = {{BM, BN, BK, 21.0, 2.0}, {WM, WN, WK, 19.0, 2.0}};
constexpr TileShape kShapeQ8 = {BM, BN, QBK, 21.0, 1.0};

// Cost model (CU cycles) for a tile shape and split count.  A workgroup's
// main loop runs at the rate its copy stream reaches next to the MFMA work,
// or at the MFMA rate if that is lower.  Workgroups run in rounds of one per
// CU; with split K each workgroup also writes its partial tile and the last
// of a tile's workgroups reads all of them, each at the slower of a CU's
// stream (about 24 B/clk) and its share of HBM (about 2 KB/clk for the chip).
double plan_cost(int tiles, int ns, const TileShape& t, int K) {
  const double kspl = std::ceil((double)K / t.bk / ns) * t.bk;  // K per split
  const double copy = (t.bm * 2.0 + t.bn * t.wbytes) * kspl / t.rate;
  const double mfma = 2.0 * t.bm * t.bn * kspl / (4.0 * 1024.0) / 0.9;
  const double rounds = std::ceil((double)tiles * ns / kCUs);
  const double tile_bytes = (double)t.bm * t.bn * 4.0;
  if (ns == 1) return rounds * std::max(copy, mfma) + 1500.0;
  const double hbm = 2080.0;  // B/clk, the whole chip
  const double wgs = (double)tiles * ns;
  const double write = std::max(tile_bytes / 24.0, std::min(wgs, (double)kCUs) * tile_bytes / hbm);
  const double reduce = std::max(ns * tile_bytes / 24.0, wgs * tile_bytes / hbm);
  return rounds * (std::max(copy, mfma) + write) + reduce + 1500.0;
}

// K range of `ns` splits: whole stages, the last split possibly shorter.
int split_kr(int K, int bk, int ns) {
  const int kst = (K + bk - 1) / bk;
  return (kst + ns - 1) / ns * bk;
}

// Split K when the tiles alone leave CUs idle: the tile shape and split
// count of least modelled cost; at least 8 stages per split, at most 256 MB
// of partials and one arrival counter per tile.  The 256-row shape needs
// M >= 384 (enough rows to fill most of a tile).  With `tail`, a plan of
// whole rounds plus a partial one may split only the partial round's tiles
// (a second launch), at the same limits.
constexpr double kMaxPartialBytes = 256.0 * 1024 * 1024;
Plan make_plan_over(const TileShape* shapes, int nshapes, int M, int N, int K, bool swiglu,
                    bool tail = false) {
  Plan best_pl;
  double best = 1e300;
  for (int shape = 0; shape < nshapes; ++shape) {
    const TileShape& t = shapes[shape];
    if (t.bm > BM && M < 384) continue;
    const int cols = swiglu ? t.bn / 2 : t.bn;
    const int tiles = ((M + t.bm - 1) / t.bm) * ((N + cols - 1) / cols);
    const int max_ns = std::max(1, std::min(16, (K + t.bk - 1) / t.bk / 8));
    for (int ns = 1; ns <= max_ns; ++ns) {
      if (ns > 1 && ((double)ns * tiles * t.bm * t.bn * 4.0 > kMaxPartialBytes || tiles > kWsMaxCounters))
        break;
      const double cost = plan_cost(tiles, ns, t, K);
      if (cost < best * (1.0 - 1e-9)) {
        best = cost;
        best_pl.shape = shape;
        best_pl.tiles = tiles;
        best_pl.ns = ns;
        best_pl.tail = best_pl.tail_ns = 0;
      }
    }
    const int rounds = (tiles + kCUs - 1) / kCUs;
    const int rest = tiles - (rounds - 1) * kCUs;  // tiles of the last round
    if (tail && rounds > 1 && 2 * rest <= kCUs && rest <= kWsMaxCounters) {
      const double whole = plan_cost((rounds - 1) * kCUs, 1, t, K);
      for (int ns = 2; ns <= max_ns && ns * rest <= kCUs; ++ns) {
        if ((double)ns * rest * t.bm * t.bn * 4.0 > kMaxPartialBytes) break;
        const double cost = whole + plan_cost(rest, ns, t, K);
        if (cost < best * (1.0 - 1e-9)) {
          best = cost;
          best_pl.shape = shape;
          best_pl.tiles = tiles;
          best_pl.ns = 1;
          best_pl.tail = rest;
          best_pl.tail_ns = ns;
        }
      }
    }
  }
  const TileShape& t = shapes[best_pl.shape];
  best_pl.kr = split_kr(K, t.bk, best_pl.ns);
  best_pl.ns = (K + best_pl.kr - 1) / best_pl.kr;
  best_pl.grid = best_pl.tiles * best_pl.ns;
  best_pl.tile_elems = t.bm * t.bn;
  if (best_pl.tail) {
    best_pl.tail_kr = split_kr(K, t.bk, best_pl.tail_ns);
    best_pl.tail_ns = (K + best_pl.tail_kr - 1) / best_pl.tail_kr;
    best_pl.grid = best_pl.tiles - best_pl.tail + best_pl.tail * best_pl.tail_ns;
  }
  return best_pl;
}

Plan make_plan(int M, int N, int K, bool swiglu) {
  return make_plan_over(kShapes, kNumShapes, M, N, K, swiglu, true);
}

Plan make_plan_q8(int M, int N, int K, bool swiglu) {
  return make_plan_over(&kShapeQ8, 1, M, N, K, swiglu);
}

size_t plan_bytes(const Plan& pl) {
  if (pl.tail) return kWsCounterBytes + (size_t)pl.tail_ns * pl.tail * pl.tile_elems * sizeof(float);
  if (pl.ns <= 1) return 0;
  return kWsCounterBytes + (size_t)pl.ns * pl.tiles * pl.tile_elems * sizeof(float);
}

// The split-K workspace of a plan: arrival counters, then the fp32 partials.
hipError_t split_buffers(const Plan& pl, void* workspace, unsigned** counters, float** part) {
  *counters = nullptr;
  *part = nullptr;
  if (pl.ns <= 1 && pl.tail == 0) return hipSuccess;
  if (workspace == nullptr || (pl.tail ? pl.tail : pl.tiles) > kWsMaxCounters)
    return hipErrorInvalidValue;
  *counters = static_cast<unsigned*>(workspace);
  *part = reinterpret_cast<float*>(static_cast<char*>(workspace) + kWsCounterBytes);
  return hipSuccess;
}

template <int EPI>
hipError_t launch_plan(const Plan& pl, int M, int N, int K, const uint16_t* A, int64_t lda,
                       const uint16_t* W0, const uint16_t* W1, void* out, int64_t ldo,
                       void* workspace, hipStream_t stream) {
  auto kern = pl.shape == kTWide ? gemm_wide_kernel<EPI> : gemm_kernel<EPI>;
  unsigned* counters;
  float* part;
  if (split_buffers(pl, workspace, &counters, &part) != hipSuccess) return hipErrorInvalidValue;
  const int head = pl.tiles - pl.tail;  // tiles of the first launch (K unsplit if tail)
  hipLaunchKernelGGL(kern, dim3(head * pl.ns), dim3(kThreads), 0, stream, M, N, K, A, lda, W0,
                     W1, out, ldo, pl.kr, counters, part, 0, head);
  if (pl.tail) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(pl.tail * pl.tail_ns), dim3(kThreads), 0, stream, M, N, K, A,
                       lda, W0, W1, out, ldo, pl.tail_kr, counters, part, head, pl.tail);
  }
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

size_t gemm_q8_workspace_bytes(int M, int N, int K, bool swiglu) {
  return plan_bytes(make_plan_q8(M, N, K, swiglu));
}

template <int EPI>
hipError_t gemm_q8_launch(int M, int N, int K, const uint16_t* A, int64_t lda, const uint8_t* W0,
                          const float* S0, const uint8_t* W1, const float* S1, void* out,
                          int64_t ldo, void* workspace, int fmt, hipStream_t stream) {
  const Plan pl = make_plan_q8(M, N, K, EPI == EPI_SWIGLU);
  if (pl.grid == 0 || K % 16) return hipErrorInvalidValue;
  unsigned* counters;
  float* part;
  if (split_buffers(pl, workspace, &counters, &part) != hipSuccess) return hipErrorInvalidValue;
  auto kern = fmt == kFmtInt8 ? gemm_q8_kernel<EPI, kWInt8> : gemm_q8_kernel<EPI, kWE4M3>;
  hipLaunchKernelGGL(kern, dim3(pl.grid), dim3(kThreads), 0, stream, M, N, K, A, lda, W0, S0, W1,
                     S1, out, ldo, pl.kr, counters, part);
  return hipGetLastError();
}

template hipError_t gemm_q8_launch<EPI_F32>(int, int, int, const uint16_t*, int64_t,
                                            const uint8_t*, const float*, const uint8_t*,
                                            const float*, void*, int64_t, void*, int, hipStream_t);
template hipError_t gemm_q8_launch<EPI_SWIGLU>(int, int, int, const uint16_t*, int64_t,
                                               const uint8_t*, const float*, const uint8_t*,
                                               const float*, void*, int64_t, void*, int,
                                               hipStream_t);

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
