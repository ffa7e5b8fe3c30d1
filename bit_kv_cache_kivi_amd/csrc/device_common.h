// Small device helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

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

__device__ __forceinline__ half8 to_half8(const float (&x)[8]) {
  half8 h;
#pragma unroll
  for (int i = 0; i < 8; ++i) h[i] = static_cast<_Float16>(x[i]);
  return h;
}

// x -> (hi, lo) fp16 pair with hi = fp16(x), lo = fp16(x - hi): hi + lo keeps
// about 22 significant bits of x.
__device__ __forceinline__ void store_hi_lo(half8& hi, half8& lo, const float (&x)[8]) {
  half8 h, l;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    h[i] = static_cast<_Float16>(x[i]);
    l[i] = static_cast<_Float16>(x[i] - static_cast<float>(h[i]));
  }
  hi = h;
  lo = l;
}

}  // namespace kvq
