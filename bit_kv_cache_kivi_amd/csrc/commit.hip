// Quantize-on-commit kernel for gfx950.
//
// A committed block's keys and values are quantized once, when the block is
// committed; keys KIVI-style per channel over a 32-token group, values per
// token over G_v channels; chosen key rows stay in bf16 and are left out of
// their group's statistics (Tai et al., "KV Cache Quantization for Diffusion
// Language Models", abstract; SoloQ summary page, block-diffusion paragraph).
//
// One workgroup = two waves per (new slot, kv head): wave 0 quantizes K, wave 1
// quantizes V.  Each lane owns 8 channels x (32 / (64 / (D/8))) tokens, loaded
// with 16-byte reads that cover whole 256-byte token rows per instruction.
// Group minima/maxima come from in-lane reductions plus xor shuffles.  Codes
// are packed into a slot record staged in LDS, then the whole record leaves
// with coalesced 128-bit stores.
//
// Exactness: scale = (mx - mn) / (2^b - 1) uses IEEE division.  A code is
// rint((x - mn) / scale); the kernel first forms y = (x - mn) * rcp(scale),
// which is within a few ulp of the exact fp32 quotient, and recomputes the
// quotient by IEEE division only when y lies within 2^-12 of a rounding
// boundary (k + 1/2) or when scale lies outside [2^-100, 2^100], where rcp
// would overflow or underflow.  Away from those
// boundaries rint(y) equals rint of the exact quotient, so codes are identical
// to the plain definition.  This file is compiled with -ffp-contract=off.
#include "device_common.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

template <int KB, int VB, int D, bool F32IN>
__global__ __launch_bounds__(128) void commit_kernel(const CommitArgs a) {
  constexpr int NCG = D / 8;        // 8-channel groups per token row
  constexpr int NTQ = 64 / NCG;     // lanes along the token axis
  constexpr int TPL = kSlot / NTQ;  // tokens per lane
  constexpr uint32_t KC = kc_bytes(D, KB);
  constexpr uint32_t VC = vc_bytes(D, VB);
  constexpr uint32_t KM = kmeta_bytes(D);
  constexpr uint32_t REC_MAX = record_bytes(D, KB, VB, 32);
  static_assert(TPL % 4 == 0, "lane token count");
  __shared__ __align__(16) uint8_t rec[REC_MAX];

  const CommitTask task = a.tasks[blockIdx.x];
  const int h = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int cg = lane % NCG;
  const int tq = lane / NCG;
  const uint32_t rbytes = a.record_bytes;
  const uint32_t raw_end = KC + VC + KM + (uint32_t)(D >> a.gv_log2) * 256u;
  for (uint32_t off = raw_end + threadIdx.x * 4; off < rbytes; off += 128 * 4)
    *reinterpret_cast<uint32_t*>(rec + off) = 0u;

  // ---- load this lane's TPL token rows x 8 channels
  const void* src = wave == 0 ? a.k : a.v;
  float x[TPL][8];
#pragma unroll
  for (int k = 0; k < TPL; ++k) {
    const int t = tq * TPL + k;
    if (t < task.nvalid) {
      const size_t row = ((size_t)task.b * a.n_max + task.src_tok + t) * a.hkv + h;
      load8(src, row * D + 8 * cg, F32IN, x[k]);
    } else {
#pragma unroll
      for (int c = 0; c < 8; ++c) x[k][c] = 0.f;
    }
  }

  if (wave == 0) {
    // ================= keys: per-channel groups along the 32 tokens
    constexpr float LEV = (float)((1 << KB) - 1);
    uint32_t member = 0;
#pragma unroll
    for (int k = 0; k < TPL; ++k) {
      const int t = tq * TPL + k;
      if (t < task.nvalid && !((task.mask >> t) & 1u)) member |= 1u << k;
    }
    // protected rows: copy to the bf16 store before x is overwritten
    if (task.mask) {
#pragma unroll
      for (int k = 0; k < TPL; ++k) {
        const int t = tq * TPL + k;
        if (t < task.nvalid && ((task.mask >> t) & 1u)) {
          const int rank = task.rank_base + __popc(task.mask & ((1u << t) - 1u));
          uint4 w;
          w.x = f32_to_bf16_bits(x[k][0]) | (f32_to_bf16_bits(x[k][1]) << 16);
          w.y = f32_to_bf16_bits(x[k][2]) | (f32_to_bf16_bits(x[k][3]) << 16);
          w.z = f32_to_bf16_bits(x[k][4]) | (f32_to_bf16_bits(x[k][5]) << 16);
          w.w = f32_to_bf16_bits(x[k][6]) | (f32_to_bf16_bits(x[k][7]) << 16);
          const size_t prow = ((size_t)task.b * a.hkv + h) * a.seg.prot_cap + rank;
          *reinterpret_cast<uint4*>(a.seg.prot_rows + prow * D + 8 * cg) = w;
          if (h == 0 && cg == 0) a.seg.prot_pos[(size_t)task.b * a.seg.prot_cap + rank] = task.token_base + t;
        }
      }
    }
    float scale[8], zero[8], rcp[8];
    bool exact[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      float mn = __builtin_inff(), mx = -__builtin_inff();
#pragma unroll
      for (int k = 0; k < TPL; ++k)
        if ((member >> k) & 1u) { mn = fminf(mn, x[k][c]); mx = fmaxf(mx, x[k][c]); }
#pragma unroll
      for (int m = NCG; m < 64; m <<= 1) {
        mn = fminf(mn, __shfl_xor(mn, m));
        mx = fmaxf(mx, __shfl_xor(mx, m));
      }
      const bool any = mn <= mx;
      scale[c] = any ? (mx - mn) / LEV + 0.0f : 0.0f;
      zero[c] = any ? mn + 0.0f : 0.0f;
      rcp[c] = __builtin_amdgcn_rcpf(scale[c]);
      exact[c] = !(scale[c] >= 0x1p-100f && scale[c] <= 0x1p+100f);
#pragma unroll
      for (int k = 0; k < TPL; ++k) x[k][c] = x[k][c] - zero[c];   // d = x - mn
    }
    if (tq == 0) {
      float* ks = reinterpret_cast<float*>(rec + KC + VC) + 8 * cg;
      *reinterpret_cast<float4*>(ks) = make_float4(scale[0], scale[1], scale[2], scale[3]);
      *reinterpret_cast<float4*>(ks + 4) = make_float4(scale[4], scale[5], scale[6], scale[7]);
      *reinterpret_cast<float4*>(ks + D) = make_float4(zero[0], zero[1], zero[2], zero[3]);
      *reinterpret_cast<float4*>(ks + D + 4) = make_float4(zero[4], zero[5], zero[6], zero[7]);
    }
#pragma unroll
    for (int k = 0; k < TPL; ++k) {
      const int t = tq * TPL + k;
      uint32_t word = 0;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        uint32_t code = 0;
        if (((member >> k) & 1u) && scale[c] != 0.f) {
          const float d = x[k][c];
          float y = d * rcp[c];
          const float fr = y - floorf(y);
          if (exact[c] || fabsf(fr - 0.5f) < 0x1p-12f) y = d / scale[c];
          code = (uint32_t)fminf(fmaxf(rintf(y), 0.f), LEV);
        }
        word |= code << (KB * c);
      }
      // word-major: the word holding channel group cg of token t
      if (KB == 4) *reinterpret_cast<uint32_t*>(rec + (cg * 32 + t) * 4) = word;
      else         *reinterpret_cast<uint16_t*>(rec + ((cg >> 1) * 32 + t) * 4 + 2 * (cg & 1)) = (uint16_t)word;
    }
  } else {
    // ================= values: per-token groups along G_v channels
    constexpr float LEV = (float)((1 << VB) - 1);
    const int lanes_per_group = (1 << a.gv_log2) / 8;
    float scale[TPL], zero[TPL], rcp[TPL];
    bool exact[TPL];
#pragma unroll
    for (int k = 0; k < TPL; ++k) {
      float mn = x[k][0], mx = x[k][0];
#pragma unroll
      for (int c = 1; c < 8; ++c) { mn = fminf(mn, x[k][c]); mx = fmaxf(mx, x[k][c]); }
      for (int m = 1; m < lanes_per_group; m <<= 1) {
        mn = fminf(mn, __shfl_xor(mn, m));
        mx = fmaxf(mx, __shfl_xor(mx, m));
      }
      const bool valid = tq * TPL + k < task.nvalid;
      scale[k] = valid ? (mx - mn) / LEV + 0.0f : 0.0f;
      zero[k] = valid ? mn + 0.0f : 0.0f;
      rcp[k] = __builtin_amdgcn_rcpf(scale[k]);
      exact[k] = !(scale[k] >= 0x1p-100f && scale[k] <= 0x1p+100f);
#pragma unroll
      for (int c = 0; c < 8; ++c) x[k][c] = x[k][c] - zero[k];
    }
    if ((cg & (lanes_per_group - 1)) == 0) {
      const int g = cg / lanes_per_group;
      float* vs = reinterpret_cast<float*>(rec + KC + VC + KM + g * 256);
#pragma unroll
      for (int k = 0; k < TPL; k += 4) {
        const int t = tq * TPL + k;
        *reinterpret_cast<float4*>(vs + t) = make_float4(scale[k], scale[k + 1], scale[k + 2], scale[k + 3]);
        *reinterpret_cast<float4*>(vs + 32 + t) = make_float4(zero[k], zero[k + 1], zero[k + 2], zero[k + 3]);
      }
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int ch = 8 * cg + c;
#pragma unroll
      for (int k0 = 0; k0 < TPL; k0 += 4) {
        uint32_t chunk = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int k = k0 + i;
          uint32_t code = 0;
          if (scale[k] != 0.f) {
            const float d = x[k][c];
            float y = d * rcp[k];
            const float fr = y - floorf(y);
            if (exact[k] || fabsf(fr - 0.5f) < 0x1p-12f) y = d / scale[k];
            code = (uint32_t)fminf(fmaxf(rintf(y), 0.f), LEV);
          }
          chunk |= code << (VB * i);
        }
        // token t0 = 4-aligned group start; its place in the channel row
        const int t0 = tq * TPL + k0;
        const int mm = t0 / 16, hh = (t0 / 4) % 2, eb = 4 * ((t0 / 8) % 2);
        // word-major: word j of channel ch sits at (j * D + ch) * 4
        if (VB == 4)
          *reinterpret_cast<uint16_t*>(rec + KC + ((2 * mm + hh) * D + ch) * 4 + eb / 2) = (uint16_t)chunk;
        else
          rec[KC + (hh * D + ch) * 4 + 2 * mm + eb / 4] = (uint8_t)chunk;
      }
    }
  }
  __syncthreads();

  uint8_t* dst = a.seg.records + (((size_t)task.b * a.hkv + h) * a.seg.slot_cap + task.dst_slot) * rbytes;
  for (uint32_t off = threadIdx.x * 16; off < rbytes; off += 128 * 16)
    *reinterpret_cast<uint4*>(dst + off) = *reinterpret_cast<const uint4*>(rec + off);
  if (h == 0 && threadIdx.x == 0) {
    int4 hd = make_int4(task.nvalid, (int)task.mask, task.rank_base, task.token_base);
    *reinterpret_cast<int4*>(a.seg.headers + ((size_t)task.b * a.seg.slot_cap + task.dst_slot) * kHeaderBytes) = hd;
  }
}

template <int KB, int VB, int D, bool F32IN>
hipError_t launch_t(const CommitArgs& a, int ntasks, hipStream_t s) {
  dim3 grid(ntasks, a.hkv);
  hipLaunchKernelGGL((commit_kernel<KB, VB, D, F32IN>), grid, dim3(128), 0, s, a);
  return hipGetLastError();
}

template <int KB, int VB, int D>
hipError_t launch_d(const CommitArgs& a, int ntasks, bool f32, hipStream_t s) {
  return f32 ? launch_t<KB, VB, D, true>(a, ntasks, s) : launch_t<KB, VB, D, false>(a, ntasks, s);
}

template <int KB, int VB>
hipError_t launch_b(const CommitArgs& a, int ntasks, int D, bool f32, hipStream_t s) {
  return D == 64 ? launch_d<KB, VB, 64>(a, ntasks, f32, s) : launch_d<KB, VB, 128>(a, ntasks, f32, s);
}

}  // namespace

hipError_t launch_commit(const CommitArgs& a, int ntasks, int D, int kb, int vb, bool f32_in,
                         hipStream_t stream) {
  if (ntasks == 0) return hipSuccess;
  if (kb == 4 && vb == 4) return launch_b<4, 4>(a, ntasks, D, f32_in, stream);
  if (kb == 4 && vb == 2) return launch_b<4, 2>(a, ntasks, D, f32_in, stream);
  if (kb == 2 && vb == 4) return launch_b<2, 4>(a, ntasks, D, f32_in, stream);
  return launch_b<2, 2>(a, ntasks, D, f32_in, stream);
}

}  // namespace kvq
