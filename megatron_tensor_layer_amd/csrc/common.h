// Device-side helpers shared by the gfx950 kernels of the TP-shard library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tpk {

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_t;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;

// Output epilogues of a projection.
enum Epi : int {
  EPI_F32 = 0,     // fp32 store (row-parallel partials)
  EPI_DT = 1,      // store in the input dtype (QKV)
  EPI_SWIGLU = 2,  // two weight matrices (gate, up): store silu(g) * u in dtype
};

// fp32 -> bf16 bits, round to nearest even (gfx950 v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  __bf16 b = (__bf16)f;
  return __builtin_bit_cast(uint16_t, b);
}

// Two floats to packed bf16 (lo in bits 0..15), round to nearest even: one
// v_cvt_pk_bf16_f32 (two scalar conversions and a shift-or otherwise).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
  typedef float f32x2v __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2v){lo, hi}, bf16x2v));
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) {
  return __uint_as_float(b16 << 16);
}

// Buffer resource over [base, base + bytes): raw (stride 0) addressing, so a
// 32-bit lane offset at or past `bytes` reads zero instead of memory.
// Word 3 is the gfx9-family raw-buffer format word.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// The same resource from values the compiler cannot prove wave-uniform (a
// pointer or size derived from the wave index): every word is taken from the
// first active lane, so the descriptor lives in scalar registers and the
// loads that use it need no per-lane waterfall loop.  The caller guarantees
// that the values are uniform across the wave.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc_uniform(const void* base,
                                                                     uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  const uint64_t au = ((uint64_t)hi << 32) | lo;
  return make_rsrc(reinterpret_cast<const void*>(au), __builtin_amdgcn_readfirstlane(bytes));
}

// The value unchanged, but opaque to the optimizer.  A buffer load whose
// offset is a select (an in-range offset or an out-of-range one that reads
// zero) is otherwise split into two exec-masked loads, one per arm, and the
// second arm then waits for every load in flight (vmcnt(0)) before it may
// reuse the destination registers.  With the select materialised first
// there is one load and no branch.
__device__ __forceinline__ uint32_t opaque(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}

constexpr int kAuxNT = 2;  // non-temporal hint: streamed once, do not keep in cache

// 16-byte load at byte offset `off` of a buffer resource.
template <int AUX = 0>
__device__ __forceinline__ u32x4_t buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, AUX);
}

// Sum V values per lane over the 64 lanes of a wavefront.  Afterwards lane l
// holds the total of value index l / (64 / V) in v[0].  Step S exchanges
// half of the CNT = V >> (S+1) live values with the lane 32 >> S away.
template <int V, int S>
__device__ __forceinline__ void wave_fold_step(float (&v)[V], int lane) {
  constexpr int CNT = V >> (S + 1);
  if constexpr (CNT >= 1) {
    constexpr int M = 32 >> S;
    const bool upper = (lane & M) != 0;
#pragma unroll
    for (int q = 0; q < CNT; ++q) {
      const float send = upper ? v[q] : v[q + CNT];
      const float keep = upper ? v[q + CNT] : v[q];
      v[q] = keep + __shfl_xor(send, M, 64);
    }
    wave_fold_step<V, S + 1>(v, lane);
  } else {
#pragma unroll
    for (int m = 32 >> S; m >= 1; m >>= 1) v[0] += __shfl_xor(v[0], m, 64);
  }
}

template <int V>
__device__ __forceinline__ void wave_fold(float (&v)[V], int lane) {
  static_assert(V >= 1 && V <= 64 && (V & (V - 1)) == 0, "V must be a power of two <= 64");
  wave_fold_step<V, 0>(v, lane);
}

// Split-K arrival at a tile's counter: true for the last of `ns` arrivals.
// atomicInc wraps the counter to zero on that arrival, so a finished call
// leaves every counter zero and the next call needs no reset (one atomic
// round trip per workgroup, no compare-and-swap retries under contention).
__device__ __forceinline__ bool arrive_last(unsigned* counter, unsigned ns) {
  return atomicInc(counter, ns - 1) == ns - 1;
}

// silu(z) = z / (1 + exp(-z)), fp32.
__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// 2-element bf16 dot product accumulated in fp32 (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// 16 OCP E4M3 codes -> two 8-element bf16 chunks (K 0..7, K 8..15), exact:
// every E4M3 value is a bf16 value.  v_cvt_scalef32_pk_bf16_fp8 with scale 1
// decodes two codes straight to packed bf16; on all 256 codes it gives the
// bits of v_cvt_pk_f32_fp8 followed by a bf16 conversion (NaN codes too).
__device__ __forceinline__ void decode16(const u32x4_t& w, u32x4_t& lo, u32x4_t& hi) {
  uint32_t p[8];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    p[2 * q] = __builtin_bit_cast(uint32_t,  // bytes 0, 1
                                  __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[q], 1.0f, false));
    p[2 * q + 1] = __builtin_bit_cast(uint32_t,  // bytes 2, 3
                                      __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[q], 1.0f, true));
  }
  lo = u32x4_t{p[0], p[1], p[2], p[3]};
  hi = u32x4_t{p[4], p[5], p[6], p[7]};
}

// One-byte weight codes of the weight-only variants: OCP E4M3, or signed int8.
constexpr int kFmtE4M3 = 0;
constexpr int kFmtInt8 = 1;

// 16 signed int8 codes -> two 8-element bf16 chunks (K 0..7, K 8..15), exact:
// every integer in [-128, 127] is a bf16 value.
__device__ __forceinline__ void decode16_i8(const u32x4_t& w, u32x4_t& lo, u32x4_t& hi) {
  uint32_t p[8];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int v = (int)w[q];
    p[2 * q] = pack_bf16x2((float)(int8_t)(v & 0xff), (float)(int8_t)((v >> 8) & 0xff));
    p[2 * q + 1] = pack_bf16x2((float)(int8_t)((v >> 16) & 0xff), (float)(int8_t)(v >> 24));
  }
  lo = u32x4_t{p[0], p[1], p[2], p[3]};
  hi = u32x4_t{p[4], p[5], p[6], p[7]};
}

// Weight storage of a streaming kernel's template instance: bf16, or one-byte
// codes (E4M3, int8) with one fp32 scale per row.
constexpr int kWBf16 = 0;
constexpr int kWE4M3 = 1;
constexpr int kWInt8 = 2;

// Wait until at most N vector-memory operations of this wave are in flight.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70 | 0xF00);
}

// Buffer descriptor words (raw addressing over [base, base + bytes)); kept
// in SGPRs for the asm load below.
__device__ __forceinline__ u32x4_t rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return u32x4_t{(uint32_t)a, (uint32_t)(a >> 32) & 0xffffu, bytes, 0x00020000u};
}

// 16 bytes per lane from buffer offset `voff` straight into LDS at
// lds_base + 16 * lane (buffer_load_dwordx4 ... lds; M0 holds lds_base).
// Written as asm so that the compiler does not add its own wait for it before
// every LDS read: the kernel orders these loads itself, with an explicit
// vmcnt wait and a barrier before the stage they fill is read.  No register
// is written, so nothing in flight can be overwritten.
__device__ __forceinline__ void lds_dma16(u32x4_t rsrc, uint32_t voff, uint32_t lds_base) {
  asm volatile(
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %0, %1, 0 offen lds"
      :
      : "v"(voff), "s"(rsrc), "{m0}"(__builtin_amdgcn_readfirstlane(lds_base))
      : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

}  // namespace tpk
