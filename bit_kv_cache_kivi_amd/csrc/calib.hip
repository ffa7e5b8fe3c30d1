// Calibration kernels for reporting measured achievable peaks beside the
// published ones (they are not part of the method): a streaming copy (HBM
// bandwidth) and a loop of dense fp16 MFMAs with no memory traffic (matrix
// throughput at the clock the device holds under that load).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "../../include/kvq.h"

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Each workgroup copies a contiguous share of the n 16-byte words, eight
// nontemporal loads in flight per thread before the matching stores (the
// fastest of the copy shapes measured on MI355X); the words past the last
// whole round of the share are copied one by one.
__global__ __launch_bounds__(256) void calib_copy_kernel(u32x4* __restrict__ dst, const u32x4* __restrict__ src,
                                                         size_t n) {
  const size_t per = (n + gridDim.x - 1) / gridDim.x;
  const size_t b0 = (size_t)blockIdx.x * per;
  const size_t b1 = b0 + per < n ? b0 + per : n;
  size_t i = b0 + threadIdx.x;
  for (; i + 7 * 256 < b1; i += 8 * 256) {
    u32x4 r[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) r[k] = __builtin_nontemporal_load(src + i + k * 256);
#pragma unroll
    for (int k = 0; k < 8; ++k) __builtin_nontemporal_store(r[k], dst + i + k * 256);
  }
  for (; i < b1; i += 256) dst[i] = src[i];
}

// Each wave runs `iters` rounds of eight independent accumulation chains of
// v_mfma_f32_32x32x16_f16 (32*32*16*2 flops each); the accumulators are summed
// into one value per lane at the end so that nothing is optimised away.
__global__ __launch_bounds__(256) void calib_mfma_kernel(float* out, int iters) {
  using kvq::half8;
  using kvq::floatx16;
  half8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (_Float16)(0.001f * (float)(threadIdx.x & 7));
    b[e] = (_Float16)(0.002f * (float)(e + 1));
  }
  floatx16 acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[k][i] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[k], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += acc[k][i];
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace

extern "C" {

kvq_status kvq_calib_copy(void* d_dst, const void* d_src, size_t bytes, void* stream) {
  if (!d_dst || !d_src || (bytes & 15u) || (reinterpret_cast<uintptr_t>(d_dst) & 15u) ||
      (reinterpret_cast<uintptr_t>(d_src) & 15u))
    return KVQ_EINVAL;
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    cus = 256;
  hipLaunchKernelGGL(calib_copy_kernel, dim3(cus * 16), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<u32x4*>(d_dst), static_cast<const u32x4*>(d_src), bytes / 16);
  return hipGetLastError() == hipSuccess ? KVQ_OK : KVQ_EHIP;
}

kvq_status kvq_calib_mfma(float* d_out, int32_t workgroups, int32_t iters, void* stream) {
  if (!d_out || workgroups < 1 || iters < 1) return KVQ_EINVAL;
  hipLaunchKernelGGL(calib_mfma_kernel, dim3(workgroups), dim3(256), 0, static_cast<hipStream_t>(stream), d_out, iters);
  return hipGetLastError() == hipSuccess ? KVQ_OK : KVQ_EHIP;
}

}  // extern "C"
