// Decode attention of one rank over its KV cache.  The cache is split with
// the heads: a rank stores and reads only the KV groups of its own query
// heads (lecture "Distributed Serving", §4.4), so decode attention is a
// stream over the rank's share of the cache -- HBM-bound.
//
// Sequence b has lens[b] positions: 0 .. lens[b]-2 in the cache, the last
// one the new token, whose k and v are read from the QKV projection's output
// and also stored into the cache slot lens[b]-1 for the next step.  Caches:
// K [B, nkv, Lmax, hd], V transposed [B, nkv, hd, Lmax].
//
// Work split: one workgroup of NWV waves per (sequence, KV group, chunk of
// the positions); the chunks fill the chip when the sequences alone cannot.
// Inside a chunk the waves take rounds of 32 NWV positions, one block of 32
// per wave, on bf16 MFMA (v_mfma_f32_32x32x16_bf16) with the same transposed
// formulation as the attention core: S^T = K Q^T with the group's query
// heads as the 32 columns (all heads of a group share each K and V read),
// online softmax per head with one cross-half exchange per block, O^T +=
// V^T P^T with P^T taken from registers.  The V cache is stored transposed
// ([head_dim, positions] per sequence and group).
// A round's K rows and V^T rows are staged in LDS by direct global->LDS
// copies of whole cache lines (16-byte slots XOR-swizzled by row, so the
// MFMA operand reads are conflict-free), two rounds in flight: every wave has
// its next block requested while it computes, without holding it in
// registers.  The K rows of a block are read in an order that makes each
// lane's S^T accumulator hold consecutive positions, so the V^T operand -- 8
// positions of one head_dim row -- is one 16-byte LDS read.
// The waves merge through LDS; with several chunks, each workgroup writes
// its softmax state (max, sum, unnormalised O) to the workspace and the last
// of the sequence-group's chunks to arrive (one atomic) merges them.
#include "common.h"
#include "kernels.h"

namespace tpk {

namespace {

constexpr uint32_t kOob = 0x80000000u;  // buffer offset past any record: reads zero
constexpr int kAuxSys = 17;             // sc0 sc1: system coherent
constexpr int NWV = 4;
constexpr int kMaxChunks = 32;  // position chunks per (sequence, group)
// one per CU: measured faster than two per CU (fewer chunk states to write
// and merge) and than fewer -- B = 32 at L = 2048 / 8192: 14.7 / 31.6 us,
// against 23.4 / 40.3 with 512 workgroups and 17.0 / 42.1 with 128
constexpr int kTargetWgs = 256;
constexpr int kRP = 32 * NWV;   // positions per round: one block of 32 per wave
constexpr int kRowB = 256;      // LDS bytes per staged row: 16 slots of 16 bytes

// One round's stage: kRP K rows (head_dim padded to 128), then 32 HDT V^T
// rows of kRP positions.  Two stages; after the loop the space holds the
// waves' partial O^T for the merge.
template <int HDT>
constexpr int stage_bytes() { return (kRP + 32 * HDT) * kRowB; }
template <int HDT>
constexpr int dyn_lds_bytes() { return 2 * stage_bytes<HDT>(); }

__device__ __forceinline__ int acc_row32(int r, int lane) {
  return (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
}

// Position (within a block of 32) whose K row feeds S^T row i: bits 2 and 3
// swapped.  Accumulator elements 8 ks .. 8 ks + 7 of a lane in half h then
// hold positions 16 ks + 8 h + 0..7, consecutive, so the matching V^T operand
// of the P V step is one 16-byte load.
__device__ __forceinline__ int key_pos(int i) {
  return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1);
}

// Workspace record of one chunk: 32 heads x (hd_pad O values), then 32 (max,
// sum) pairs.
__host__ __device__ __forceinline__ int64_t rec_floats(int hdp) { return 32 * (int64_t)hdp + 64; }

template <int HDT>
// register budget of two waves per SIMD (the compiler then keeps O^T in
// VGPRs); the staging LDS leaves one workgroup per CU
__global__ void __launch_bounds__(64 * NWV) __attribute__((amdgpu_waves_per_eu(2)))
attn_decode_kernel(int nq, int nkv, int hd, int Lmax, const int* __restrict__ lens,
                   const uint16_t* __restrict__ qkv, uint16_t* __restrict__ Kc,
                   uint16_t* __restrict__ Vc, uint16_t* __restrict__ A, int NC, int Lc,
                   unsigned* __restrict__ counters, float* __restrict__ part) {
  constexpr int KS = 2 * HDT;
  constexpr int HDP = 32 * HDT;  // head_dim padded to the O^T tiles
  constexpr int SB = stage_bytes<HDT>();
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];  // the two stages
  __shared__ float fw[(kMaxChunks + 1) * 32];  // chunk merge weights, then 1/L
  __shared__ float mls[NWV][2][64];
  __shared__ int is_last;
  __shared__ u32x4_t qs[KS][64];  // the Q operand, lane-linear
  __shared__ u32x4_t knew[64];    // the new token: k chunks 0..15, v chunks 16..31

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int bg = blockIdx.x / NC, c = blockIdx.x % NC;
  const int b = bg / nkv, g = bg % nkv;
  const int G = nq / nkv;  // query heads per group
  const int N = (nq + 2 * nkv) * hd;
  const int len = min(max(lens[b], 1), Lmax);
  // scores in base 2: s = log2(e) q.k / sqrt(hd), so every exponential is
  // one exp2 (e^z = 2^(z log2 e)); the chunk states keep their maxima in it
  const float scale = 1.4426950408889634f / sqrtf((float)hd);

  // this group's cache rows, and the columns of its k and v in the qkv row
  const int64_t cache0 = ((int64_t)b * nkv + g) * Lmax * hd;
  const int kcol = (nq + g) * hd, vcol = (nq + nkv + g) * hd;

  // Q as the B operand: head h = lane % 32 of the group, chunk 2 ks + lane/32.
  // It is the same for every wave and every block, so it waits in LDS (wave
  // 0 copies it there) and is read again per block instead of holding
  // registers.  Chunk 0's wave 1 copies the new token's k and v the same way.
  // Both copies are issued ahead of the cache stream and waited on with it.
  const int h = lane & 31;
  const u32x4_t qw = rsrc_words(qkv + (int64_t)b * N, (uint32_t)N * 2u);
  if (w == 0) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int ch = 2 * ks + (lane >> 5);
      lds_dma16(qw, (h < G && ch * 8 < hd) ? (uint32_t)((g * G + h) * hd + ch * 8) * 2u : kOob,
                lds_addr(&qs[ks][0]));
    }
  }
  if (w == 1 && c == 0) {
    const int ch = lane & 15;
    lds_dma16(qw, lane < 32 && ch * 8 < hd ? (uint32_t)((lane < 16 ? kcol : vcol) + ch * 8) * 2u : kOob,
              lds_addr(&knew[0]));
  }

  f32x16_t ot[HDT];
#pragma unroll
  for (int t = 0; t < HDT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) ot[t][r] = 0.0f;
  float m = -INFINITY, l = 0.0f;

  // this chunk's cache positions [k0, k1); the new token at len-1 is folded
  // in after the loop
  const int k0 = c * Lc, k1 = min(k0 + Lc, len - 1);
  const int R = k1 > k0 ? (k1 - k0 + kRP - 1) / kRP : 0;  // rounds

  // Round r into stage r & 1, every wave a share of the copies (positions at
  // or past k1, chunks past head_dim: zero-filled, nothing fetched).  K: row
  // i = position k0 + kRP r + i, slot j holds 16-byte chunk j ^ (i & 15).
  // V^T: row d, slot j holds positions 8 (j ^ (d & 15)) .. + 7 of the
  // round; a group of 8 that runs past len-2 is masked down to its cache
  // positions when it is used (the rest of the slot may hold anything).
  constexpr int NIK = kRP * 16 / (64 * NWV);  // K copies per wave and round
  constexpr int NIV = HDP * 16 / (64 * NWV);  // V^T copies per wave and round
  const u32x4_t kr = rsrc_words(Kc + cache0, (uint32_t)Lmax * (uint32_t)hd * 2u);
  const u32x4_t vr = rsrc_words(Vc + cache0, (uint32_t)Lmax * (uint32_t)hd * 2u);
  const uint32_t l0 = lds_addr(lds);
  const int chn = hd / 8;
  auto issue_round = [&](int r) {
    const int P0 = k0 + kRP * r;
    const uint32_t base = l0 + (uint32_t)((r & 1) * SB);
#pragma unroll
    for (int i = 0; i < NIK; ++i) {
      const int q = w + NWV * i;  // 1 KB of the stage: slots 64 q .. 64 q + 63
      const int sl = q * 64 + lane;
      const int row = sl >> 4, ch = (sl & 15) ^ (row & 15);
      const int p = P0 + row;
      lds_dma16(kr, p < k1 && ch < chn ? ((uint32_t)p * (uint32_t)hd + ch * 8) * 2u : kOob,
                base + q * 1024);
    }
#pragma unroll
    for (int i = 0; i < NIV; ++i) {
      const int q = w + NWV * i;
      const int sl = q * 64 + lane;
      const int d = sl >> 4, p0 = P0 + 8 * ((sl & 15) ^ (d & 15));
      lds_dma16(vr, p0 < k1 && d < hd ? ((uint32_t)d * (uint32_t)Lmax + (uint32_t)p0) * 2u : kOob,
                base + kRP * kRowB + q * 1024);
    }
  };
  auto v_mask = [&](int kb, int ks) {  // keep positions below len-1
    const int nv = len - 1 - (kb + ks * 16 + (lane >> 5) * 8);
    u32x4_t m;
#pragma unroll
    for (int q = 0; q < 4; ++q) m[q] = nv >= 2 * q + 2 ? 0xffffffffu : nv == 2 * q + 1 ? 0xffffu : 0u;
    return m;
  };
  // One block (this wave's 32 positions of the stage): S^T = K Q^T, online
  // softmax, O^T += V^T P^T.
  auto process = [&](int kb, const unsigned char* stage) {
    const unsigned char* sk = stage + 32 * w * kRowB;  // this wave's K rows
    const unsigned char* sv = stage + kRP * kRowB;     // the round's V^T rows
    f32x16_t st;
#pragma unroll
    for (int r = 0; r < 16; ++r) st[r] = 0.0f;
    const int krow = key_pos(lane & 31);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int ch = 2 * ks + (lane >> 5);
      const bf16x8_t kv =
          *reinterpret_cast<const bf16x8_t*>(sk + krow * kRowB + ((ch ^ (krow & 15)) << 4));
      st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kv, __builtin_bit_cast(bf16x8_t, qs[ks][lane]),
                                                   st, 0, 0, 0);
    }
    float x[16];
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = kb + key_pos(acc_row32(r, lane));
      x[r] = key < k1 ? st[r] * scale : -INFINITY;
      mx = fmaxf(mx, x[r]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float mnew = fmaxf(m, mx);
    const float base = (mnew == -INFINITY) ? 0.0f : mnew;
    const float corr = __builtin_amdgcn_exp2f(m - base);
    float ps = 0.0f;
    bf16x8_t pb[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = __builtin_amdgcn_exp2f(x[r] - base);
      ps += p;
      pb[r >> 3][r & 7] = (__bf16)p;
    }
    ps += __shfl_xor(ps, 32, 64);
    l = l * corr + ps;
    m = mnew;
    // O^T is rescaled by 2^(m_old - m_new) only when some lane's max moved:
    // otherwise the factor is exactly 1 in every lane (a wave-uniform test)
    if (__builtin_amdgcn_ballot_w64(corr != 1.0f) != 0) {
#pragma unroll
      for (int t = 0; t < HDT; ++t) ot[t] *= corr;
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const u32x4_t vm = v_mask(kb, ks);
      const int pc = 4 * w + 2 * ks + (lane >> 5);  // 8-position group within the round
#pragma unroll
      for (int t = 0; t < HDT; ++t) {
        const int d = t * 32 + (lane & 31);
        const u32x4_t vv =
            *reinterpret_cast<const u32x4_t*>(sv + d * kRowB + ((pc ^ (d & 15)) << 4)) & vm;
        ot[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, vv), pb[ks],
                                                        ot[t], 0, 0, 0);
      }
    }
  };
  // Two rounds in flight.  A wave's copies are its only vector-memory
  // operations here, so "round r has landed" is "at most the NIK + NIV
  // copies of round r + 1 are outstanding", and Q and the new token (older
  // than every round) have landed once the first rounds' copies alone are.
  if (R > 0) issue_round(0);
  if (R > 1) issue_round(1);
  if (R > 1)
    wait_vmcnt<2 * (NIK + NIV)>();
  else if (R == 1)
    wait_vmcnt<NIK + NIV>();
  else
    wait_vmcnt<0>();
  __syncthreads();  // Q and the new token in LDS
  for (int r = 0; r < R; ++r) {
    if (r + 1 < R)
      wait_vmcnt<NIK + NIV>();
    else
      wait_vmcnt<0>();
    __syncthreads();  // round r staged by every wave
    const int kb = k0 + kRP * r + 32 * w;
    if (kb < k1) process(kb, lds + (r & 1) * SB);
    __syncthreads();  // every wave is done with stage r & 1
    if (r + 2 < R) issue_round(r + 2);
  }

  // ---- the new token (position len-1) into chunk 0's wave 0: one more
  //      online-softmax step with a single key, s = scale q.k_new per head
  //      (chunk 0's wave 1 meanwhile stores its k row and v column into
  //      cache slot len-1 for the next step; no copy above read that slot
  //      unmasked)
  if (c == 0 && w == 1) {
    if (lane < hd / 8)  // k: one row of the K cache
      *reinterpret_cast<u32x4_t*>(Kc + cache0 + (int64_t)(len - 1) * hd + lane * 8) = knew[lane];
    const uint16_t* vn = reinterpret_cast<const uint16_t*>(&knew[16]);
    for (int d = lane; d < hd; d += 64)  // v: one column of the transposed V cache
      Vc[cache0 + (int64_t)d * Lmax + (len - 1)] = vn[d];
  }
  if (c == 0 && w == 0) {
    float dot = 0.0f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int ch = 2 * ks + (lane >> 5);
      const u32x4_t kn = knew[ch];  // zero past head_dim
      const u32x4_t qq = qs[ks][lane];
#pragma unroll
      for (int e = 0; e < 4; ++e) dot = dot2_bf16(qq[e], kn[e], dot);
    }
    dot += __shfl_xor(dot, 32, 64);
    const float sn = dot * scale;
    const float mnew = fmaxf(m, sn);
    const float corr = exp2f(m - mnew), pn = exp2f(sn - mnew);
    l = l * corr + pn;
    m = mnew;
#pragma unroll
    for (int t = 0; t < HDT; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) {  // rows t*32 + 8 j + 4 (lane/32) + {0..3}
        const u32x4_t vc = knew[16 + 4 * t + j];  // v_new[8 (4 t + j) ..], zero past head_dim
        const u32x2_t vn = (lane >> 5) ? u32x2_t{vc[2], vc[3]} : u32x2_t{vc[0], vc[1]};
        const float vv[4] = {bf16_bits_to_f32(vn.x & 0xffffu), bf16_bits_to_f32(vn.x >> 16),
                             bf16_bits_to_f32(vn.y & 0xffffu), bf16_bits_to_f32(vn.y >> 16)};
#pragma unroll
        for (int i = 0; i < 4; ++i) ot[t][4 * j + i] = ot[t][4 * j + i] * corr + pn * vv[i];
      }
  }

  // ---- merge the waves: each leaves its (max, sum) and its O^T tiles in the
  //      stage space (free: the loop's last barrier follows the last copy's
  //      wait and every wave's reads), then wave w merges tiles t = w mod NWV
  //      of all waves, in wave order, and keeps them in its registers
  f32x4_t (*ots)[HDT][4][64] = reinterpret_cast<f32x4_t (*)[HDT][4][64]>(lds);
  static_assert(NWV * HDT * 4 * 64 * 16 <= 2 * SB, "the merge fits the stages");
  mls[w][0][lane] = m;
  mls[w][1][lane] = l;
#pragma unroll
  for (int t = 0; t < HDT; ++t)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      ots[w][t][q][lane] = f32x4_t{ot[t][4 * q], ot[t][4 * q + 1], ot[t][4 * q + 2], ot[t][4 * q + 3]};
  __syncthreads();
  {
    float mm = mls[0][0][lane];
#pragma unroll
    for (int v = 1; v < NWV; ++v) mm = fmaxf(mm, mls[v][0][lane]);
    const float base = (mm == -INFINITY) ? 0.0f : mm;
    float fv[NWV];
#pragma unroll
    for (int v = 0; v < NWV; ++v) fv[v] = exp2f(mls[v][0][lane] - base);
    l = mls[0][1][lane] * fv[0];
#pragma unroll
    for (int v = 1; v < NWV; ++v) l += mls[v][1][lane] * fv[v];
    m = mm;
#pragma unroll
    for (int t = 0; t < HDT; ++t) {
      if (t % NWV != w) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        f32x4_t o4 = ots[0][t][q][lane] * fv[0];
#pragma unroll
        for (int v = 1; v < NWV; ++v) {
          const f32x4_t ov = ots[v][t][q][lane];
#pragma unroll
          for (int e = 0; e < 4; ++e) o4[e] += ov[e] * fv[v];
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) ot[t][4 * q + e] = o4[e];
      }
    }
  }

  if (NC == 1) {  // ---- the one chunk: A = O / l, each wave its tiles
    if (h < G) {
      const float inv = 1.0f / l;
#pragma unroll
      for (int t = 0; t < HDT; ++t) {
        if (t % NWV != w) continue;
#pragma unroll
        for (int a = 0; a < 4; ++a) {  // 4 adjacent columns per 8-byte store
          const int col = t * 32 + acc_row32(4 * a, lane);
          if (col < hd)
            *reinterpret_cast<u32x2_t*>(A + (int64_t)b * (nq * hd) + (g * G + h) * hd + col) =
                u32x2_t{pack_bf16x2(ot[t][4 * a] * inv, ot[t][4 * a + 1] * inv),
                        pack_bf16x2(ot[t][4 * a + 2] * inv, ot[t][4 * a + 3] * inv)};
        }
      }
    }
    return;
  }

  // ---- several chunks: this chunk's state to the workspace, then arrival
  const int64_t rec = rec_floats(HDP);
  const int64_t nrec = (int64_t)gridDim.x;
  const __amdgpu_buffer_rsrc_t pr = make_rsrc(part, (uint32_t)(nrec * rec * 4));
  const int64_t my = (int64_t)blockIdx.x * rec;
  if (h < G) {  // lanes of padding heads (h >= G) store nothing
    // each wave its merged tiles; lane holds head h, rows t*32 + 8 j +
    // 4 (lane/32) + {0..3}: 16 bytes each
#pragma unroll
    for (int t = 0; t < HDT; ++t) {
      if (t % NWV != w) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4_t v = f32x4_t{ot[t][4 * j], ot[t][4 * j + 1], ot[t][4 * j + 2], ot[t][4 * j + 3]};
        __builtin_amdgcn_raw_buffer_store_b128(
            __builtin_bit_cast(u32x4_t, v), pr,
            (uint32_t)((my + h * HDP + t * 32 + 8 * j + 4 * (lane >> 5)) * 4), 0, kAuxSys);
      }
    }
    if (w == 0 && lane < 32) {
      const u32x2_t ml = u32x2_t{__builtin_bit_cast(uint32_t, m), __builtin_bit_cast(uint32_t, l)};
      __builtin_amdgcn_raw_buffer_store_b64(ml, pr,
                                            (uint32_t)((my + 32 * HDP + 2 * h) * 4), 0, kAuxSys);
    }
  }
  __builtin_amdgcn_s_waitcnt(0x70 | 0xF00);  // vmcnt(0): the stores have reached memory
  __syncthreads();
  if (threadIdx.x == 0) is_last = arrive_last(counters + bg, (unsigned)NC);
  __syncthreads();
  if (!is_last) return;

  // ---- the last chunk to arrive merges the NC states.  One memory round
  //      trip: each thread first issues the loads of its (head, 4 columns)
  //      item over the first 16 chunks, then the (max, sum) pairs of every
  //      chunk and real head go to LDS; per head the weights 2^(m_c - M) and
  //      1/sum follow, and each thread sums its columns over the chunks in
  //      chunk order (chunks past 16, if any, in further batches).
  const int64_t first = (int64_t)bg * NC * rec;
  const int c4n = hd / 4;  // 4-column groups per head
  const int q0 = threadIdx.x;
  const bool item = q0 < G * c4n;
  const int hh0 = item ? q0 / c4n : 0, col0 = item ? 4 * (q0 % c4n) : 0;
  u32x4_t o[16];
#pragma unroll
  for (int e = 0; e < 16; ++e)
    o[e] = __builtin_amdgcn_raw_buffer_load_b128(
        pr, item && e < NC ? (uint32_t)((first + e * rec + hh0 * HDP + col0) * 4) : kOob, 0,
        kAuxSys);
  float* mlp = reinterpret_cast<float*>(lds);  // [kMaxChunks][32] (max, sum) pairs
  static_assert(2 * kMaxChunks * 32 * 4 <= 2 * SB, "merge scratch fits");
#pragma unroll
  for (int j = 0; j < (kMaxChunks * 32) / (64 * NWV); ++j) {
    const int i = threadIdx.x + 64 * NWV * j;  // chunk i / 32, head i % 32
    const int k = i >> 5, hh = i & 31;
    const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(
        pr, k < NC && hh < G ? (uint32_t)((first + k * rec + 32 * HDP + 2 * hh) * 4) : kOob, 0,
        kAuxSys);
    const uint32_t mb = v.x, lb = v.y;  // scalars: bit_cast of a vector element misreads
    mlp[2 * i] = __builtin_bit_cast(float, mb);
    mlp[2 * i + 1] = __builtin_bit_cast(float, lb);
  }
  __syncthreads();
  if (threadIdx.x < G) {
    const int hh = threadIdx.x;
    float mm = -INFINITY;
    for (int k = 0; k < NC; ++k) mm = fmaxf(mm, mlp[2 * (k * 32 + hh)]);
    const float base = (mm == -INFINITY) ? 0.0f : mm;
    float den = 0.0f;
    for (int k = 0; k < NC; ++k) {
      const float f = exp2f(mlp[2 * (k * 32 + hh)] - base);
      fw[k * 32 + hh] = f;
      den += mlp[2 * (k * 32 + hh) + 1] * f;
    }
    fw[kMaxChunks * 32 + hh] = 1.0f / den;
  }
  __syncthreads();
  for (int q = q0; q < G * c4n; q += 64 * NWV) {
    const int hh = q / c4n, col = 4 * (q % c4n);
    f32x4_t num = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (q == q0) {  // the preloaded first 16 chunks
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (e < NC) num += __builtin_bit_cast(f32x4_t, o[e]) * fw[e * 32 + hh];
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e)
        o[e] = __builtin_amdgcn_raw_buffer_load_b128(
            pr, e < NC ? (uint32_t)((first + e * rec + hh * HDP + col) * 4) : kOob, 0, kAuxSys);
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (e < NC) num += __builtin_bit_cast(f32x4_t, o[e]) * fw[e * 32 + hh];
    }
    for (int k = 16; k < NC; k += 16) {
      u32x4_t o2[16];
#pragma unroll
      for (int e = 0; e < 16; ++e)
        o2[e] = __builtin_amdgcn_raw_buffer_load_b128(
            pr, k + e < NC ? (uint32_t)((first + (k + e) * rec + hh * HDP + col) * 4) : kOob, 0,
            kAuxSys);
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (k + e < NC) num += __builtin_bit_cast(f32x4_t, o2[e]) * fw[(k + e) * 32 + hh];
    }
    num *= fw[kMaxChunks * 32 + hh];
    u32x2_t packed;
    packed.x = pack_bf16x2(num.x, num.y);
    packed.y = pack_bf16x2(num.z, num.w);
    *reinterpret_cast<u32x2_t*>(A + (int64_t)b * (nq * hd) + (g * G + hh) * hd + col) = packed;
  }
}

struct Plan {
  int nc = 1;  // chunks per (sequence, group)
  int lc = 0;  // positions per chunk (multiple of 32)
};

Plan make_plan(int B, int nkv, int Lmax) {
  Plan pl;
  const int pairs = B * nkv;
  const int blocks = (Lmax + 31) / 32;
  const int per_wave = (blocks + NWV - 1) / NWV;  // chunks that still give each wave a block
  pl.nc = std::max(1, std::min(std::min((kTargetWgs + pairs - 1) / pairs, per_wave), kMaxChunks));
  pl.lc = ((blocks + pl.nc - 1) / pl.nc) * 32;
  pl.nc = (Lmax + pl.lc - 1) / pl.lc;
  return pl;
}

template <int HDT>
hipError_t launch_hdt(int B, int nq, int nkv, int hd, int Lmax, const int* lens,
                      const uint16_t* qkv, uint16_t* Kc, uint16_t* Vc, uint16_t* A,
                      const Plan& pl, void* workspace, hipStream_t stream) {
  unsigned* counters = static_cast<unsigned*>(workspace);
  float* part = workspace ? reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                                     kWsCounterBytes)
                          : nullptr;
  static std::atomic<uint64_t> lds_raised{0};
  const hipError_t e = dyn_lds_once(reinterpret_cast<const void*>(attn_decode_kernel<HDT>),
                                    dyn_lds_bytes<HDT>(), lds_raised);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_decode_kernel<HDT>, dim3(B * nkv * pl.nc), dim3(64 * NWV),
                     dyn_lds_bytes<HDT>(), stream,
                     nq, nkv, hd, Lmax, lens, qkv, Kc, Vc, A, pl.nc, pl.lc, counters, part);
  return hipGetLastError();
}

}  // namespace

size_t attn_decode_workspace_bytes(int B, int nkv, int hd, int Lmax) {
  const Plan pl = make_plan(B, nkv, Lmax);
  if (pl.nc <= 1) return 0;
  const int hdp = (hd + 31) / 32 * 32;
  return kWsCounterBytes + (size_t)B * nkv * pl.nc * (size_t)rec_floats(hdp) * sizeof(float);
}

hipError_t attn_decode_launch(int B, int nq, int nkv, int hd, int Lmax, const int* lens,
                              const uint16_t* qkv, uint16_t* Kc, uint16_t* Vc, uint16_t* A,
                              void* workspace, hipStream_t stream) {
  const Plan pl = make_plan(B, nkv, Lmax);
  if (pl.nc > 1 && (workspace == nullptr || B * nkv > kWsMaxCounters)) return hipErrorInvalidValue;
  switch ((hd + 31) / 32) {
    case 1: return launch_hdt<1>(B, nq, nkv, hd, Lmax, lens, qkv, Kc, Vc, A, pl, workspace, stream);
    case 2: return launch_hdt<2>(B, nq, nkv, hd, Lmax, lens, qkv, Kc, Vc, A, pl, workspace, stream);
    case 3: return launch_hdt<3>(B, nq, nkv, hd, Lmax, lens, qkv, Kc, Vc, A, pl, workspace, stream);
    case 4: return launch_hdt<4>(B, nq, nkv, hd, Lmax, lens, qkv, Kc, Vc, A, pl, workspace, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace tpk
