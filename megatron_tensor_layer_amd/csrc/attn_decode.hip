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
// Inside a chunk the waves take interleaved blocks of 32 positions on bf16
// MFMA (v_mfma_f32_32x32x16_bf16) with the same transposed formulation as
// the attention core: S^T = K Q^T with the group's query heads as the 32
// columns (all heads of a group share each K and V read), online softmax
// per head with one cross-half exchange per block, O^T += V^T P^T with P^T
// taken from registers.  The V cache is stored transposed ([head_dim,
// positions] per sequence and group), and the K rows of a block are loaded in
// an order that makes each lane's S^T accumulator hold consecutive positions,
// so the V^T operand -- 8 positions of one head_dim row -- is one 16-byte
// load straight from memory, with no transpose through LDS.
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
// and merge) -- B = 32, L = 2048: 21.2 us against 22.9; L = 8192: 37.8 against 41.6
constexpr int kTargetWgs = 256;

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
// two waves per SIMD (the compiler then keeps O^T in VGPRs), so two
// workgroups share a CU
__global__ void __launch_bounds__(64 * NWV) __attribute__((amdgpu_waves_per_eu(2)))
attn_decode_kernel(int nq, int nkv, int hd, int Lmax, const int* __restrict__ lens,
                   const uint16_t* __restrict__ qkv, uint16_t* __restrict__ Kc,
                   uint16_t* __restrict__ Vc, uint16_t* __restrict__ A, int NC, int Lc,
                   unsigned* __restrict__ counters, float* __restrict__ part) {
  constexpr int KS = 2 * HDT;
  constexpr int HDP = 32 * HDT;  // head_dim padded to the O^T tiles
  __shared__ float fw[(kMaxChunks + 1) * 32];  // chunk merge weights, then 1/L
  __shared__ float mls[NWV][2][64];
  __shared__ float ots[NWV - 1][HDT][16][64];
  __shared__ int is_last;
  __shared__ u32x4_t qs[KS][64];  // the Q operand, lane-linear

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int bg = blockIdx.x / NC, c = blockIdx.x % NC;
  const int b = bg / nkv, g = bg % nkv;
  const int G = nq / nkv;  // query heads per group
  const int N = (nq + 2 * nkv) * hd;
  const int len = min(max(lens[b], 1), Lmax);
  const float scale = 1.0f / sqrtf((float)hd);

  // new-token row of qkv and this group's cache rows
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(qkv + (int64_t)b * N, (uint32_t)N * 2u);
  const int64_t cache0 = ((int64_t)b * nkv + g) * Lmax * hd;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(Kc + cache0, (uint32_t)Lmax * (uint32_t)hd * 2u);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(Vc + cache0, (uint32_t)Lmax * (uint32_t)hd * 2u);
  const int kcol = (nq + g) * hd, vcol = (nq + nkv + g) * hd;

  // ---- the new token's k and v into cache slot len-1 (chunk 0's first wave)
  if (c == 0 && w == 0) {
    for (int ch = lane; ch < hd / 8; ch += 64) {  // k: one row of the K cache
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(qkv + (int64_t)b * N + kcol + ch * 8);
      *reinterpret_cast<u32x4_t*>(Kc + cache0 + (int64_t)(len - 1) * hd + ch * 8) = v;
    }
    for (int d = lane; d < hd; d += 64)  // v: one column of the transposed V cache
      Vc[cache0 + (int64_t)d * Lmax + (len - 1)] = qkv[(int64_t)b * N + vcol + d];
  }

  // Q as the B operand: head h = lane % 32 of the group, chunk 2 ks + lane/32.
  // It is the same for every wave and every block, so it waits in LDS (wave
  // 0 stages it) and is read again per block instead of holding registers.
  const int h = lane & 31;
  if (w == 0) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int ch = 2 * ks + (lane >> 5);
      const uint32_t off = (h < G && ch * 8 < hd) ? (uint32_t)((g * G + h) * hd + ch * 8) * 2u : kOob;
      qs[ks][lane] = buf_load16(rq, off);
    }
  }
  __syncthreads();

  f32x16_t ot[HDT];
#pragma unroll
  for (int t = 0; t < HDT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) ot[t][r] = 0.0f;
  float m = -INFINITY, l = 0.0f;

  // this chunk's cache positions [k0, k1); the new token at len-1 is folded
  // in after the loop
  const int k0 = c * Lc, k1 = min(k0 + Lc, len - 1);
  // this wave's blocks kb = k0 + 32 w, + 32 NWV, ...; the next block's K and
  // V are loaded while the current one is processed (past k1: zero)
  auto load_k = [&](int kb, bf16x8_t (&kf)[KS]) {
    const int p = kb + key_pos(lane & 31);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int ch = 2 * ks + (lane >> 5);
      const uint32_t off = (kb < k1 && p < len - 1 && ch * 8 < hd)
                               ? ((uint32_t)p * (uint32_t)hd + ch * 8) * 2u : kOob;
      kf[ks] = __builtin_bit_cast(bf16x8_t, buf_load16(rk, off));
    }
  };
  // V^T operand of 16-position step ks, tile t: head_dim row d = t*32 +
  // lane%32, positions kb + 16 ks + 8 (lane/32) + 0..7 -- the key order of
  // the S^T accumulator; past k1 or head_dim, zero.  A group of 8 that runs
  // past len-2 is masked down to its cache positions when it is used (the
  // rest of the slot may hold anything), so no load is waited on early.
  auto load_v = [&](int kb, u32x4_t (&vr)[2][HDT]) {
    const int half = lane >> 5;
#pragma unroll
    for (int t = 0; t < HDT; ++t) {
      const int d = t * 32 + (lane & 31);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int p0 = kb + ks * 16 + half * 8;
        const uint32_t off = (kb < k1 && d < hd && p0 < len - 1)
                                 ? ((uint32_t)d * (uint32_t)Lmax + (uint32_t)p0) * 2u : kOob;
        vr[ks][t] = buf_load16(rv, off);
      }
    }
  };
  auto v_mask = [&](int kb, int ks) {  // keep positions below len-1
    const int nv = len - 1 - (kb + ks * 16 + (lane >> 5) * 8);
    u32x4_t m;
#pragma unroll
    for (int q = 0; q < 4; ++q) m[q] = nv >= 2 * q + 2 ? 0xffffffffu : nv == 2 * q + 1 ? 0xffffu : 0u;
    return m;
  };
  // One block: S^T = K Q^T, online softmax, O^T += V^T P^T.  The next
  // block's K and V are loaded before the current block is processed.
  auto process = [&](int kb, const bf16x8_t (&kf)[KS], const u32x4_t (&vc)[2][HDT]) {
    f32x16_t st;
#pragma unroll
    for (int r = 0; r < 16; ++r) st[r] = 0.0f;
    asm volatile("" ::: "memory");  // read Q from LDS again: do not hold it across blocks
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks], __builtin_bit_cast(bf16x8_t, qs[ks][lane]),
                                                   st, 0, 0, 0);
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
    const float corr = expf(m - base);
    float ps = 0.0f;
    bf16x8_t pb[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = expf(x[r] - base);
      ps += p;
      pb[r >> 3][r & 7] = (__bf16)p;
    }
    ps += __shfl_xor(ps, 32, 64);
    l = l * corr + ps;
    m = mnew;
#pragma unroll
    for (int t = 0; t < HDT; ++t) ot[t] *= corr;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const u32x4_t vm = v_mask(kb, ks);
#pragma unroll
      for (int t = 0; t < HDT; ++t) {
        const u32x4_t vv = vc[ks][t] & vm;
        ot[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, vv), pb[ks],
                                                        ot[t], 0, 0, 0);
      }
    }
  };
  constexpr int kStep = 32 * NWV;
  bf16x8_t kf[KS];
  u32x4_t vr[2][HDT];
  load_k(k0 + 32 * w, kf);
  load_v(k0 + 32 * w, vr);
  for (int kb = k0 + 32 * w; kb < k1; kb += kStep) {
    bf16x8_t kc[KS];
    u32x4_t vc[2][HDT];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kc[ks] = kf[ks];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int t = 0; t < HDT; ++t) vc[ks][t] = vr[ks][t];
    load_k(kb + kStep, kf);
    load_v(kb + kStep, vr);
    process(kb, kc, vc);
  }

  // ---- the new token (position len-1) into chunk 0's wave 0: one more
  //      online-softmax step with a single key, s = scale q.k_new per head
  if (c == 0 && w == 0) {
    float dot = 0.0f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int ch = 2 * ks + (lane >> 5);
      const u32x4_t kn = buf_load16(rq, ch * 8 < hd ? (uint32_t)(kcol + ch * 8) * 2u : kOob);
      const u32x4_t qq = qs[ks][lane];
#pragma unroll
      for (int e = 0; e < 4; ++e) dot = dot2_bf16(qq[e], kn[e], dot);
    }
    dot += __shfl_xor(dot, 32, 64);
    const float sn = dot * scale;
    const float mnew = fmaxf(m, sn);
    const float corr = expf(m - mnew), pn = expf(sn - mnew);
    l = l * corr + pn;
    m = mnew;
#pragma unroll
    for (int t = 0; t < HDT; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) {  // rows t*32 + 8 j + 4 (lane/32) + {0..3}
        const int d0 = t * 32 + 8 * j + 4 * (lane >> 5);
        const u32x2_t vn = __builtin_amdgcn_raw_buffer_load_b64(
            rq, d0 < hd ? (uint32_t)(vcol + d0) * 2u : kOob, 0, 0);
        const float vv[4] = {bf16_bits_to_f32(vn.x & 0xffffu), bf16_bits_to_f32(vn.x >> 16),
                             bf16_bits_to_f32(vn.y & 0xffffu), bf16_bits_to_f32(vn.y >> 16)};
#pragma unroll
        for (int i = 0; i < 4; ++i) ot[t][4 * j + i] = ot[t][4 * j + i] * corr + pn * vv[i];
      }
  }

  // ---- merge the waves into wave 0
  if (w > 0) {
    mls[w][0][lane] = m;
    mls[w][1][lane] = l;
#pragma unroll
    for (int t = 0; t < HDT; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) ots[w - 1][t][r][lane] = ot[t][r];
  }
  __syncthreads();
  if (w == 0) {
    float mm = m;
#pragma unroll
    for (int v = 1; v < NWV; ++v) mm = fmaxf(mm, mls[v][0][lane]);
    const float base = (mm == -INFINITY) ? 0.0f : mm;
    const float f0 = expf(m - base);
    l *= f0;
#pragma unroll
    for (int t = 0; t < HDT; ++t) ot[t] *= f0;
#pragma unroll
    for (int v = 1; v < NWV; ++v) {
      const float f = expf(mls[v][0][lane] - base);
      l += mls[v][1][lane] * f;
#pragma unroll
      for (int t = 0; t < HDT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) ot[t][r] += ots[v - 1][t][r][lane] * f;
    }
    m = mm;
  }

  if (NC == 1) {  // ---- the one chunk: A = O / l
    if (w == 0 && h < G) {
      const float inv = 1.0f / l;
#pragma unroll
      for (int t = 0; t < HDT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int col = t * 32 + acc_row32(r, lane);
          if (col < hd)
            A[(int64_t)b * (nq * hd) + (g * G + h) * hd + col] = f32_to_bf16_bits(ot[t][r] * inv);
        }
    }
    return;
  }

  // ---- several chunks: this chunk's state to the workspace, then arrival
  const int64_t rec = rec_floats(HDP);
  const int64_t nrec = (int64_t)gridDim.x;
  const __amdgpu_buffer_rsrc_t pr = make_rsrc(part, (uint32_t)(nrec * rec * 4));
  const int64_t my = (int64_t)blockIdx.x * rec;
  if (w == 0 && h < G) {  // lanes of padding heads (h >= G) store nothing
    // lane holds head h, rows t*32 + 8 j + 4 (lane/32) + {0..3}: 16 bytes each
#pragma unroll
    for (int t = 0; t < HDT; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4_t v = f32x4_t{ot[t][4 * j], ot[t][4 * j + 1], ot[t][4 * j + 2], ot[t][4 * j + 3]};
        __builtin_amdgcn_raw_buffer_store_b128(
            __builtin_bit_cast(u32x4_t, v), pr,
            (uint32_t)((my + h * HDP + t * 32 + 8 * j + 4 * (lane >> 5)) * 4), 0, kAuxSys);
      }
    if (lane < 32) {
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
  //      chunk and real head go to LDS; per head the weights e^(m_c - M) and
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
  float* mlp = &ots[0][0][0][0];  // [kMaxChunks][32] (max, sum) pairs
  static_assert((NWV - 1) * HDT * 16 * 64 >= 2 * kMaxChunks * 32, "merge scratch fits");
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
      const float f = expf(mlp[2 * (k * 32 + hh)] - base);
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
  hipLaunchKernelGGL(attn_decode_kernel<HDT>, dim3(B * nkv * pl.nc), dim3(64 * NWV), 0, stream,
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
