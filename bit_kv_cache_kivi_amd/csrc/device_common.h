// Small device helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef int v8i_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// 8 consecutive elements (bf16 or fp32) -> 8 floats.  p must be 16-byte aligned.
__device__ __forceinline__ void load8(const void* base, size_t elem, bool is_f32, float (&x)[8]) {
  if (is_f32) {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + elem);
    float4 a = p[0], b = p[1];
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  } else {
    uint4 w = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + elem);
    x[0] = bf16_lo(w.x); x[1] = bf16_hi(w.x); x[2] = bf16_lo(w.y); x[3] = bf16_hi(w.y);
    x[4] = bf16_lo(w.z); x[5] = bf16_hi(w.z); x[6] = bf16_lo(w.w); x[7] = bf16_hi(w.w);
  }
}

__device__ __forceinline__ float load1(const void* base, size_t elem, bool is_f32) {
  if (is_f32) return static_cast<const float*>(base)[elem];
  return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(base)[elem]) << 16);
}

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));

// Two floats -> two fp16 (round to nearest even) in one instruction.
__device__ __forceinline__ half2_t to_half2(float a, float b) {
  return __builtin_convertvector((float2_t){a, b}, half2_t);
}

__device__ __forceinline__ half8 to_half8(const float (&x)[8]) {
  half8 h;
#pragma unroll
  for (int i = 0; i < 8; i += 2) {
    const half2_t p = to_half2(x[i], x[i + 1]);
    h[i] = p.x;
    h[i + 1] = p.y;
  }
  return h;
}

// -1.0f in a register the compiler cannot see through, so that x - (float)h
// becomes one mixed-precision fma (v_fma_mix_f32) instead of convert + subtract.
__device__ __forceinline__ float opaque_neg_one() {
  float m = -1.0f;
  asm("" : "+s"(m));
  return m;
}

// max over the two 32-lane halves of a wave (v_permlane32_swap, no LDS).
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float sum_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

typedef short short2_t __attribute__((ext_vector_type(2)));

// x -> hi = fp16(x) and lo = bf8(2^12 * (x - hi)) (two words, byte e =
// element e; e5m2, round to nearest even).  hi + 2^-12 * lo keeps x to about
// 2^-14 of its magnitude.  x - hi is exact in fp32 and is one mixed-precision
// fma against neg_one (-1 in a register the compiler cannot see through); the
// 2^12 comes from the scaled conversion, which divides its inputs by the scale
// operand (here 2^-12).
__device__ __forceinline__ void store_hi_lo8(half8& hi, uint2& lo, const float (&x)[8], float neg_one) {
  constexpr float kLoScale = 1.0f / 4096.0f;
  half8 h;
  float l[8];
#pragma unroll
  for (int i = 0; i < 8; i += 2) {
    const half2_t p = to_half2(x[i], x[i + 1]);
    h[i] = p.x; h[i + 1] = p.y;
    l[i] = fmaf(static_cast<float>(p.x), neg_one, x[i]);
    l[i + 1] = fmaf(static_cast<float>(p.y), neg_one, x[i + 1]);
  }
  // the first conversion of each word writes its low half and the second its
  // high half, so the old value of the first is arbitrary: an input that dies
  // there, which spares a register copy
  short2_t w0 = __builtin_amdgcn_cvt_scalef32_pk_bf8_f32(__builtin_bit_cast(short2_t, l[0]), l[0], l[1], kLoScale, false);
  w0 = __builtin_amdgcn_cvt_scalef32_pk_bf8_f32(w0, l[2], l[3], kLoScale, true);
  short2_t w1 = __builtin_amdgcn_cvt_scalef32_pk_bf8_f32(__builtin_bit_cast(short2_t, l[4]), l[4], l[5], kLoScale, false);
  w1 = __builtin_amdgcn_cvt_scalef32_pk_bf8_f32(w1, l[6], l[7], kLoScale, true);
  hi = h;
  lo = make_uint2(__builtin_bit_cast(uint32_t, w0), __builtin_bit_cast(uint32_t, w1));
}

// Eight b-bit codes of a u32 as floats.  b = 4: code e at bits [4e, 4e+4);
// b = 2: code e at bits [2e, 2e+2) (the low 16 bits).  Codes are split into
// bytes first so that each float comes from one byte-convert instruction.
template <int B>
__device__ __forceinline__ void unpack8(uint32_t w, float (&c)[8]) {
  if (B == 4) {
    uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
    // keep the byte split: without the barrier the compiler folds it into
    // one bit-field extract per code (two instructions per code instead of one)
    asm("" : "+v"(lo), "+v"(hi));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      c[2 * j] = static_cast<float>((lo >> (8 * j)) & 0xFFu);
      c[2 * j + 1] = static_cast<float>((hi >> (8 * j)) & 0xFFu);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t p = (w >> (2 * j)) & 0x0303u;
      asm("" : "+v"(p));
      c[j] = static_cast<float>(p & 0xFFu);
      c[j + 4] = static_cast<float>(p >> 8);
    }
  }
}

// Workgroup barrier that orders LDS accesses only: global loads and stores in
// flight stay in flight across it (__syncthreads also waits for all of them).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

}  // namespace kvq
