// Attention core of one rank (test support: it joins the QKV projection to
// o_proj; it is not a projection).  Each rank computes its own heads
// completely (lecture "Distributed Serving", §4.2).
//
// One workgroup per (block of 32 query rows, local head), its waves taking
// every NWV-th block of keys and merging their softmax states at the end; on bf16 MFMA
// (v_mfma_f32_32x32x16_bf16), online softmax in fp32, computed transposed so
// that every lane owns one query:
//   * S^T = K Q^T per block of 32 keys: K rows (A operand) and the block's Q
//     (B operand, kept in registers) are both read as 16-byte chunks along
//     head_dim, as the QKV projection writes them;
//   * scale 1/sqrt(hd) (scores kept in base 2, so each exponential is one
//     exp2), causal mask inside each sequence (query i sees keys
//     s0(i)..i, s0 = the first row of its sequence); the lane holds 16 of its
//     query's 32 scores and lane ^ 32 the other 16, so the running max and
//     sum need one exchange each per key block;
//   * O^T += V^T P^T: P^T comes straight from the score registers (rounded
//     to bf16) as the B operand; the key block's V rows are staged in LDS as
//     they are loaded (16-byte chunks XOR-swizzled by key, conflict-free
//     writes), and each lane gathers its V^T operand -- 8 keys of one
//     head_dim column, in the accumulator's key order -- with 2-byte reads
//     that are conflict-free too; the per-query rescale is lane-local;
//   * head_dim up to 256 in 32-row tiles of O^T (HDT of them); columns past
//     head_dim read zero and are not stored;
//   * the next key block's K and V are loaded while the current one is
//     processed.
// Sequences of one token (decode without a cache) take a copy kernel: one
// key, weight exactly 1, A = V.
#include "common.h"
#include "kernels.h"

namespace tpk {

namespace {

constexpr uint32_t kOob = 0x80000000u;  // buffer offset past any record: reads zero

// Row (query within the block) of accumulator element r held by `lane`; the
// column (key, or output column) is lane % 32.
__device__ __forceinline__ int acc_row32(int r, int lane) {
  return (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
}


template <int HDT, int NWV>
__global__ void __launch_bounds__(64 * NWV)
attn_core_kernel(int I, int S, int nq, int nkv, int hd, const uint16_t* __restrict__ qkv,
                 uint16_t* __restrict__ A) {
  constexpr int KS = 2 * HDT;  // 16-wide steps along head_dim
  // a wave's key block of V: 32 rows of CPR 16-byte chunk slots; chunk c of
  // key k sits in slot c ^ (k mod CPR)
  constexpr int CPR = 4 * HDT <= 16 ? 16 : 32;
  __shared__ u32x4_t Vrs[NWV][32 * CPR];
  // partial results of waves 1.. for the merge: max and sum, then O^T tiles
  __shared__ float mls[NWV][2][64];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // key blocks w, w + NWV, ...
  u32x4_t* Vr = Vrs[w];
  const int i0 = blockIdx.x * 32;
  const int j = blockIdx.y;
  const int g = (j * nkv) / nq;  // KV group of local head j
  const int N = (nq + 2 * nkv) * hd;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(qkv, (uint32_t)I * (uint32_t)N * 2u);
  const int qcol = j * hd, kcol = (nq + g) * hd, vcol = (nq + nkv + g) * hd;
  // scores in base 2: s = log2(e) q.k / sqrt(hd), so every exponential is
  // one exp2 (e^z = 2^(z log2 e))
  const float scale = 1.4426950408889634f / sqrtf((float)hd);

  // 16-byte chunk c of row `row` of the head starting at `col0` (zero past
  // head_dim or past the last row)
  auto chunk_off = [&](int row, int col0, int c) -> uint32_t {
    return (c * 8 < hd && row < I) ? ((uint32_t)row * (uint32_t)N + (uint32_t)(col0 + c * 8)) * 2u
                                   : kOob;
  };

  // This lane's query (column of every accumulator below) and its sequence start
  const int qi = i0 + (lane & 31);
  const int qlo = (qi / S) * S;
  // Q of the block as the B operand: query lane%32, chunk 2 ks + lane/32
  bf16x8_t qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    qf[ks] = __builtin_bit_cast(bf16x8_t,
                                buf_load16(rq, chunk_off(qi, qcol, 2 * ks + (lane >> 5))));

  f32x16_t ot[HDT];  // O^T tiles: rows = head_dim columns, column = this lane's query
#pragma unroll
  for (int t = 0; t < HDT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) ot[t][r] = 0.0f;
  float m = -INFINITY, l = 0.0f;  // running max and sum of this lane's query

  const int last = min(i0 + 31, I - 1);
  const int first = (i0 / S) * S;
  // K fragments (A operand: key lane%32, chunk 2 ks + lane/32) and V chunks of
  // a key block; the next block's are loaded while the current one is processed
  auto load_k = [&](int kb, bf16x8_t (&kf)[KS]) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      kf[ks] = __builtin_bit_cast(
          bf16x8_t, buf_load16(rq, chunk_off(kb + (lane & 31), kcol, 2 * ks + (lane >> 5))));
  };
  auto load_v = [&](int kb, u32x4_t (&vr)[2 * HDT]) {
#pragma unroll
    for (int u = 0; u < 2 * HDT; ++u) {
      const int q = lane + 64 * u;  // chunk (key, 8-column group) of the 32 x 32 HDT tile
      vr[u] = buf_load16(rq, chunk_off(kb + q / (4 * HDT), vcol, q % (4 * HDT)));
    }
  };
  int kb = (first / 32) * 32 + 32 * w;
  bf16x8_t kf[KS];
  u32x4_t vr[2 * HDT];
  load_k(kb, kf);
  load_v(kb, vr);
  for (; kb <= last; kb += 32 * NWV) {
    // ---- S^T = K Q^T: element r holds key kb + acc_row32(r, lane)
    f32x16_t st;
#pragma unroll
    for (int r = 0; r < 16; ++r) st[r] = 0.0f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks], qf[ks], st, 0, 0, 0);
    // ---- the key block's V rows into LDS, 16 bytes per lane and chunk
#pragma unroll
    for (int u = 0; u < 2 * HDT; ++u) {
      const int q = lane + 64 * u;
      const int key = q / (4 * HDT), c = q % (4 * HDT);
      Vr[key * CPR + (c ^ (key & (CPR - 1)))] = vr[u];
    }
    // this wave's next block's loads (past the last block they read zero)
    const int nb = kb + 32 * NWV <= last ? kb + 32 * NWV : I;
    load_k(nb, kf);
    load_v(nb, vr);
    // ---- masked, scaled scores and the online softmax of this lane's query:
    //      16 of its keys here, the other 16 in lane ^ 32
    float x[16];
    float mx = -INFINITY;
    // the mask is needed only where some lane's query does not see all 32
    // keys of the block (the diagonal block, a sequence start, rows past I)
    if (__builtin_amdgcn_ballot_w64(!(kb >= qlo && kb + 31 <= qi && qi < I)) != 0) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kb + acc_row32(r, lane);
        const bool ok = key <= qi && key >= qlo && qi < I;
        x[r] = ok ? st[r] * scale : -INFINITY;
        mx = fmaxf(mx, x[r]);
      }
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        x[r] = st[r] * scale;
        mx = fmaxf(mx, x[r]);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float mnew = fmaxf(m, mx);
    const float base = (mnew == -INFINITY) ? 0.0f : mnew;  // no key seen yet
    const float corr = __builtin_amdgcn_exp2f(m - base);
    float ps = 0.0f;
    bf16x8_t pb[2];  // P^T as the B operand: 8 keys per 16-key step
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
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // ---- O^T += V^T P^T: A = V^T[32 columns][16 keys], B = P^T[16 keys][query].
    //      Element e of a lane's P^T fragment for step ks holds key
    //      16 ks + 8 (e / 4) + 4 (lane / 32) + e % 4 (the accumulator's
    //      order), so the A operand's element e is V[that key][column].
    const uint16_t* Vh = reinterpret_cast<const uint16_t*>(Vr);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int t = 0; t < HDT; ++t) {
        const int d = t * 32 + (lane & 31);
        typedef unsigned short u16x8_t __attribute__((ext_vector_type(8)));
        u16x8_t v8;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int key = 16 * ks + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
          v8[e] = Vh[(key * CPR + ((d >> 3) ^ (key & (CPR - 1)))) * 8 + (d & 7)];
        }
        const bf16x8_t vf = __builtin_bit_cast(bf16x8_t, v8);
        ot[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[ks], ot[t], 0, 0, 0);
      }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();  // the next block rewrites Vt
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  // ---- merge the waves' partial softmax states into wave 0 in halving
  //      steps (wave w takes wave w + h, h = NWV/2 .. 1):
  //      O = O_a 2^(m_a - M) + O_b 2^(m_b - M), l likewise, M = max(m_a, m_b).
  //      The partial O^T tiles pass through the V staging space, free once
  //      every wave has left the key loop.
  if constexpr (NWV > 1) {
    f32x4_t (*ots)[HDT][4][64] = reinterpret_cast<f32x4_t (*)[HDT][4][64]>(&Vrs[0][0]);
    static_assert((NWV / 2) * HDT * 4 * 64 * 16 <= (int)sizeof(Vrs), "the merge fits the V space");
    __syncthreads();  // every wave is done with its V tile
#pragma unroll
    for (int h = NWV / 2; h >= 1; h /= 2) {
      if (w >= h && w < 2 * h) {
        mls[w][0][lane] = m;
        mls[w][1][lane] = l;
#pragma unroll
        for (int t = 0; t < HDT; ++t)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            ots[w - h][t][q][lane] =
                f32x4_t{ot[t][4 * q], ot[t][4 * q + 1], ot[t][4 * q + 2], ot[t][4 * q + 3]};
      }
      __syncthreads();
      if (w < h) {
        const float m2 = mls[w + h][0][lane];
        const float mm = fmaxf(m, m2);
        const float base = (mm == -INFINITY) ? 0.0f : mm;
        const float f1 = exp2f(m - base), f2 = exp2f(m2 - base);
        l = l * f1 + mls[w + h][1][lane] * f2;
        m = mm;
#pragma unroll
        for (int t = 0; t < HDT; ++t)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const f32x4_t o2 = ots[w][t][q][lane];
#pragma unroll
            for (int e = 0; e < 4; ++e) ot[t][4 * q + e] = ot[t][4 * q + e] * f1 + o2[e] * f2;
          }
      }
      __syncthreads();  // slots and sums are free for the next step
    }
    if (w > 0) return;
  }

  // ---- A[query][column] = O / l, bf16
  if (qi < I) {  // elements 4 a .. 4 a + 3 of a tile are 4 adjacent columns: one 8-byte store
    const float inv = 1.0f / l;
#pragma unroll
    for (int t = 0; t < HDT; ++t)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int col = t * 32 + acc_row32(4 * a, lane);
        if (col < hd)  // head_dim is a multiple of 8: the 4 columns are all in or all out
          *reinterpret_cast<u32x2_t*>(A + (int64_t)qi * (nq * hd) + j * hd + col) =
              u32x2_t{pack_bf16x2(ot[t][4 * a] * inv, ot[t][4 * a + 1] * inv),
                      pack_bf16x2(ot[t][4 * a + 2] * inv, ot[t][4 * a + 3] * inv)};
      }
  }
}

// Sequences of one token: the softmax runs over a single key, whose weight is
// exactly 1, so A is the value row of the head's KV group (16 bytes per lane).
__global__ void __launch_bounds__(256)
attn_single_key_kernel(int I, int nq, int nkv, int hd, const uint16_t* __restrict__ qkv,
                       uint16_t* __restrict__ A) {
  const int cpr = hd / 8;  // 16-byte chunks per head row
  const int64_t n = (int64_t)I * nq * cpr;
  const int N = (nq + 2 * nkv) * hd;
  for (int64_t q = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; q < n;
       q += (int64_t)gridDim.x * blockDim.x) {
    const int c = (int)(q % cpr);
    const int j = (int)((q / cpr) % nq);
    const int64_t i = q / ((int64_t)cpr * nq);
    const int g = (j * nkv) / nq;
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(qkv + i * N + (nq + nkv + g) * hd + c * 8);
    *reinterpret_cast<u32x4_t*>(A + i * (int64_t)nq * hd + j * hd + c * 8) = v;
  }
}

// Waves per workgroup: 4 (8 measured no faster: each wave's block loop is
// bound by its own instruction stream, which two waves per SIMD share), 2
// above head_dim 128 (for LDS), or 1 when every sequence fits one key block.
template <int HDT>
hipError_t launch_hdt(int I, int S, int nq, int nkv, int hd, const uint16_t* qkv, uint16_t* A,
                      hipStream_t stream) {
  const dim3 grid((I + 31) / 32, nq);
  if (S <= 32) {
    hipLaunchKernelGGL((attn_core_kernel<HDT, 1>), grid, dim3(64), 0, stream, I, S, nq, nkv, hd,
                       qkv, A);
  } else if (HDT > 4) {
    hipLaunchKernelGGL((attn_core_kernel<HDT, 2>), grid, dim3(128), 0, stream, I, S, nq, nkv, hd,
                       qkv, A);
  } else {
    hipLaunchKernelGGL((attn_core_kernel<HDT, 4>), grid, dim3(256), 0, stream, I, S, nq, nkv, hd,
                       qkv, A);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t attn_core_launch(int I, int S, int nq, int nkv, int hd, const uint16_t* qkv,
                            uint16_t* A, hipStream_t stream) {
  if (S == 1) {
    const int64_t n = (int64_t)I * nq * (hd / 8);
    const int grid = (int)std::min<int64_t>((n + 255) / 256, 1024);
    hipLaunchKernelGGL(attn_single_key_kernel, dim3(grid), dim3(256), 0, stream, I, nq, nkv, hd,
                       qkv, A);
    return hipGetLastError();
  }
  switch ((hd + 31) / 32) {
    case 1: return launch_hdt<1>(I, S, nq, nkv, hd, qkv, A, stream);
    case 2: return launch_hdt<2>(I, S, nq, nkv, hd, qkv, A, stream);
    case 3: return launch_hdt<3>(I, S, nq, nkv, hd, qkv, A, stream);
    case 4: return launch_hdt<4>(I, S, nq, nkv, hd, qkv, A, stream);
    case 5: return launch_hdt<5>(I, S, nq, nkv, hd, qkv, A, stream);
    case 6: return launch_hdt<6>(I, S, nq, nkv, hd, qkv, A, stream);
    case 7: return launch_hdt<7>(I, S, nq, nkv, hd, qkv, A, stream);
    case 8: return launch_hdt<8>(I, S, nq, nkv, hd, qkv, A, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace tpk
