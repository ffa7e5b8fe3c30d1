// K-RPBH rotation around the attention of the current block (gfx950).
//
// The rotation (SoloQ summary page, rotation paragraphs) is a permutation of
// the D channels, a Hadamard transform on each block of b consecutive
// channels, and a k x k orthogonal mix of the same channel across the
// k = D / b blocks.  When the committed values are stored rotated, the cache
// holds R v instead of v, so attention over it yields R o.  The block being
// denoised stays in full precision: its values are rotated here (fp32) so that
// they share the cache's basis, and the attention output comes back through
// the transposed rotation, R^T = P^T (I kron H) (mix^T kron I), H being
// symmetric.
//
// Forward order (fp32, compiled without contraction):
//   y = x[perm];
//   Hadamard stages h = 1, 2, ..., b/2: each pair (i, i + h) with i & h == 0
//   becomes (y_i + y_{i+h}, y_i - y_{i+h});
//   y <- y / sqrt(b) (b = 16 or 64: exact);
//   z[i*b + j] = sum over l = 0..k-1 in order of mix[i][l] * y[l*b + j].
//
// One wave per row with the row staged in LDS.  Pairs of one Hadamard stage
// are disjoint, so each lane reads and writes its own pairs; LDS operations of
// one wave complete in order, and the wave-level fences below keep the
// compiler from moving them across stages.
#include "device_common.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kRowsPerBlock = 4;   // waves per workgroup, one row each

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int D>
__device__ __forceinline__ void hadamard_stages(float* y, int block, int lane) {
  for (int h = 1; h < block; h *= 2) {
#pragma unroll
    for (int t = 0; t < (D / 2 + 63) / 64; ++t) {
      const int p = lane + 64 * t;              // pair index
      if (p < D / 2) {
        const int i = (p / h) * 2 * h + p % h;
        const float a = y[i], c = y[i + h];
        y[i] = a + c;
        y[i + h] = a - c;
      }
    }
    wave_sync();
  }
}

template <int D>
__global__ __launch_bounds__(64 * kRowsPerBlock) void blk_prep_kernel(const BlkPrepArgs a) {
#pragma clang fp contract(off)
  __shared__ float buf[kRowsPerBlock][D];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t r = (int64_t)blockIdx.x * kRowsPerBlock + w;
  if (r >= a.rows) return;
  float* y = buf[w];
  const int block = a.rot.block, k = D / block;
  const float inv_sqrt_b = block == 16 ? 0.25f : 0.125f;
#pragma unroll
  for (int t = 0; t < D / 64; ++t) {
    const int e = lane + 64 * t;
    a.k_out[r * D + e] = load1(a.k, r * D + e, a.in_f32);
    y[e] = load1(a.v, r * D + a.rot.perm[e], a.in_f32);
  }
  wave_sync();
  hadamard_stages<D>(y, block, lane);
#pragma unroll
  for (int t = 0; t < D / 64; ++t) {
    const int e = lane + 64 * t, i = e / block, j = e % block;
    float acc = a.rot.mix[i * k] * (y[j] * inv_sqrt_b);
    for (int l = 1; l < k; ++l) acc = acc + a.rot.mix[i * k + l] * (y[l * block + j] * inv_sqrt_b);
    a.v_out[r * D + e] = acc;
  }
}

template <int D>
__global__ __launch_bounds__(64 * kRowsPerBlock) void unrotate_kernel(const UnrotArgs a) {
  __shared__ float buf[kRowsPerBlock][D];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t r = (int64_t)blockIdx.x * kRowsPerBlock + w;
  if (r >= a.rows) return;
  float* y = buf[w];
  const int block = a.rot.block, k = D / block;
  const float inv_sqrt_b = block == 16 ? 0.25f : 0.125f;
  const float* z = a.src + r * D;
  // transposed mix: y[l*b + j] = sum over i of mix[i][l] * z[i*b + j]
#pragma unroll
  for (int t = 0; t < D / 64; ++t) {
    const int e = lane + 64 * t, l = e / block, j = e % block;
    float acc = 0.f;
    for (int i = 0; i < k; ++i) acc += a.rot.mix[i * k + l] * z[i * block + j];
    y[e] = acc;
  }
  wave_sync();
  hadamard_stages<D>(y, block, lane);
  // inverse permutation: x[perm[e]] = y[e]
#pragma unroll
  for (int t = 0; t < D / 64; ++t) {
    const int e = lane + 64 * t;
    const float x = y[e] * inv_sqrt_b;
    const int64_t o = r * D + a.rot.perm[e];
    if (a.out_f32) static_cast<float*>(a.out)[o] = x;
    else static_cast<uint16_t*>(a.out)[o] = (uint16_t)f32_to_bf16_bits(x);
  }
}

}  // namespace

hipError_t launch_blk_prep(const BlkPrepArgs& a, int D, hipStream_t stream) {
  if (a.rows <= 0) return hipSuccess;
  const dim3 grid((unsigned)((a.rows + kRowsPerBlock - 1) / kRowsPerBlock)), block(64 * kRowsPerBlock);
  if (D == 64) hipLaunchKernelGGL((blk_prep_kernel<64>), grid, block, 0, stream, a);
  else hipLaunchKernelGGL((blk_prep_kernel<128>), grid, block, 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_unrotate(const UnrotArgs& a, int D, hipStream_t stream) {
  if (a.rows <= 0) return hipSuccess;
  const dim3 grid((unsigned)((a.rows + kRowsPerBlock - 1) / kRowsPerBlock)), block(64 * kRowsPerBlock);
  if (D == 64) hipLaunchKernelGGL((unrotate_kernel<64>), grid, block, 0, stream, a);
  else hipLaunchKernelGGL((unrotate_kernel<128>), grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace kvq
