// Quantize-on-commit kernel for gfx950.
//
// A committed block's keys and values are quantized once, when the block is
// committed; keys KIVI-style per channel over a 32-token group, values per
// token over G_v channels; chosen key rows stay in bf16 and are left out of
// their group's statistics (Tai et al., "KV Cache Quantization for Diffusion
// Language Models", abstract; SoloQ summary page, block-diffusion paragraph).
//
// One workgroup = four waves per (new slot, kv head): waves 0 and 1 quantize
// the keys of one half of the channels each (a key group spans the 32 tokens
// of one channel, so the halves are independent), waves 2 and 3 the values of
// one half of the tokens each (a value group spans channels of one token).
// Each lane loads 16-byte pieces of token rows; group minima and maxima come
// from in-lane reductions plus xor shuffles.  Codes are packed into a slot
// record staged in LDS, then the whole record leaves with coalesced 128-bit
// stores.
//
// Exactness: scale = (mx - mn) / (2^b - 1) uses IEEE division.  A code is
// rint(q) of the fp32 quotient q = fl((x - mn) / scale).  The kernel forms
// y = d * rcp(scale) and refines it once with the exact residual
// fma(-y, scale, d); the refined y is within one ulp of q, so rint(y) equals
// rint(q) unless y lies within 2^-19 of a rounding boundary k + 1/2 (two ulps
// or more below 16).  Only such elements -- and every element of a group whose
// scale lies outside [2^-100, 2^100], where rcp would overflow or underflow --
// are recomputed with IEEE division, on a path that runs only when some lane
// of the wave needs it.  Codes are therefore identical to the plain
// definition.  This file is compiled with -ffp-contract=off.
#include "device_common.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

// Code of one element from the refined quotient; sets 'redo' when the element
// must be recomputed with an exact division.
__device__ __forceinline__ uint32_t fast_code(float d, float scale, float rcp, float lev, bool& redo) {
  float y = d * rcp;
  const float r = fmaf(-y, scale, d);
  y = fmaf(r, rcp, y);
  redo = fabsf((y - floorf(y)) - 0.5f) <= 0x1p-19f;
  return (uint32_t)fminf(fmaxf(rintf(y), 0.f), lev);
}

__device__ __forceinline__ uint32_t exact_code(float d, float scale, float lev) {
  return (uint32_t)fminf(fmaxf(rintf(d / scale), 0.f), lev);
}

template <int KB, int VB, int D, bool F32IN>
__global__ __launch_bounds__(256) void commit_kernel(const CommitArgs a) {
  constexpr int HC = D / 2;              // channels per key wave
  constexpr int NCGK = HC / 8;           // 8-channel groups per key wave
  constexpr int NTQK = 64 / NCGK;        // key lanes along the token axis
  constexpr int TPLK = kSlot / NTQK;     // tokens per key lane
  constexpr int NCGV = D / 8;            // 8-channel groups of a value row
  constexpr int NTQV = 64 / NCGV;        // value lanes along the token axis
  constexpr int TPLV = (kSlot / 2) / NTQV;   // tokens per value lane
  constexpr uint32_t KC = kc_bytes(D, KB);
  constexpr uint32_t VC = vc_bytes(D, VB);
  constexpr uint32_t KM = kmeta_bytes(D);
  constexpr uint32_t REC_MAX = record_bytes(D, KB, VB, 32);
  static_assert(TPLK * 8 <= 32 && TPLV * 8 <= 32, "per-lane element masks are 32 bits");
  static_assert((kSlot / 2) % TPLV == 0 && TPLV % 2 == 0 && TPLV <= 4, "value token chunks");
  __shared__ __align__(16) uint8_t rec[REC_MAX];

  const CommitTask task = a.use_inline ? a.inline_tasks[blockIdx.x] : a.tasks[blockIdx.x];
  const int h = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t rbytes = a.record_bytes;
  const uint32_t raw_end = KC + VC + KM + (uint32_t)(D >> a.gv_log2) * 256u;
  // value codes are OR-ed in below: clear them, and the record's padding
  for (uint32_t off = KC + tid * 4; off < KC + VC; off += 256 * 4) *reinterpret_cast<uint32_t*>(rec + off) = 0u;
  for (uint32_t off = raw_end + tid * 4; off < rbytes; off += 256 * 4) *reinterpret_cast<uint32_t*>(rec + off) = 0u;
  __syncthreads();

  if (wave < 2) {
    // ================= keys: channels [wave*D/2, +D/2), groups along the 32 tokens
    constexpr float LEV = (float)((1 << KB) - 1);
    const int cgl = lane % NCGK, tq = lane / NCGK;
    const int cg = wave * NCGK + cgl;          // 8-channel group within the row
    float x[TPLK][8];
#pragma unroll
    for (int k = 0; k < TPLK; ++k) {
      const int t = tq * TPLK + k;
      if (t < task.nvalid) {
        const size_t row = ((size_t)task.b * a.n_max + task.src_tok + t) * a.hkv + h;
        load8(a.k, row * D + 8 * cg, F32IN, x[k]);
      } else {
#pragma unroll
        for (int c = 0; c < 8; ++c) x[k][c] = 0.f;
      }
    }
    uint32_t member = 0;
#pragma unroll
    for (int k = 0; k < TPLK; ++k) {
      const int t = tq * TPLK + k;
      if (t < task.nvalid && !((task.mask >> t) & 1u)) member |= 1u << k;
    }
    // protected rows: copy to the bf16 store
    if (task.mask) {
#pragma unroll
      for (int k = 0; k < TPLK; ++k) {
        const int t = tq * TPLK + k;
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
    uint32_t redo = 0;                         // bit 8k + c: element (token k, channel c)
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      float mn = __builtin_inff(), mx = -__builtin_inff();
#pragma unroll
      for (int k = 0; k < TPLK; ++k)
        if ((member >> k) & 1u) { mn = fminf(mn, x[k][c]); mx = fmaxf(mx, x[k][c]); }
#pragma unroll
      for (int m = NCGK; m < 64; m <<= 1) {
        mn = fminf(mn, __shfl_xor(mn, m));
        mx = fmaxf(mx, __shfl_xor(mx, m));
      }
      const bool any = mn <= mx;
      scale[c] = any ? (mx - mn) / LEV + 0.0f : 0.0f;
      zero[c] = any ? mn + 0.0f : 0.0f;
      rcp[c] = __builtin_amdgcn_rcpf(scale[c]);
      if (scale[c] != 0.f && !(scale[c] >= 0x1p-100f && scale[c] <= 0x1p+100f)) {
#pragma unroll
        for (int k = 0; k < TPLK; ++k) redo |= ((member >> k) & 1u) << (8 * k + c);
      }
    }
    if (tq == 0) {
      float* ks = reinterpret_cast<float*>(rec + KC + VC) + 8 * cg;
      *reinterpret_cast<float4*>(ks) = make_float4(scale[0], scale[1], scale[2], scale[3]);
      *reinterpret_cast<float4*>(ks + 4) = make_float4(scale[4], scale[5], scale[6], scale[7]);
      *reinterpret_cast<float4*>(ks + D) = make_float4(zero[0], zero[1], zero[2], zero[3]);
      *reinterpret_cast<float4*>(ks + D + 4) = make_float4(zero[4], zero[5], zero[6], zero[7]);
    }
    uint32_t code[TPLK][8];
#pragma unroll
    for (int k = 0; k < TPLK; ++k)
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        bool r;
        const uint32_t q = fast_code(x[k][c] - zero[c], scale[c], rcp[c], LEV, r);
        const bool live = ((member >> k) & 1u) && scale[c] != 0.f;
        code[k][c] = live ? q : 0u;
        redo |= (uint32_t)(live && r) << (8 * k + c);
      }
    if (__any(redo != 0)) {
#pragma unroll
      for (int k = 0; k < TPLK; ++k)
#pragma unroll
        for (int c = 0; c < 8; ++c)
          if ((redo >> (8 * k + c)) & 1u) code[k][c] = exact_code(x[k][c] - zero[c], scale[c], LEV);
    }
#pragma unroll
    for (int k = 0; k < TPLK; ++k) {
      const int t = tq * TPLK + k;
      uint32_t word = 0;
#pragma unroll
      for (int c = 0; c < 8; ++c) word |= code[k][c] << (KB * c);
      // word-major: the word holding channel group cg of token t
      if (KB == 4) *reinterpret_cast<uint32_t*>(rec + (cg * 32 + t) * 4) = word;
      else         *reinterpret_cast<uint16_t*>(rec + ((cg >> 1) * 32 + t) * 4 + 2 * (cg & 1)) = (uint16_t)word;
    }
  } else {
    // ================= values: tokens [16*(wave-2), +16), groups along G_v channels
    constexpr float LEV = (float)((1 << VB) - 1);
    const int cg = lane % NCGV, tq = lane / NCGV;
    const int t0 = (wave - 2) * (kSlot / 2) + tq * TPLV;   // first token of this lane
    const int lanes_per_group = (1 << a.gv_log2) / 8;
    float x[TPLV][8];
#pragma unroll
    for (int k = 0; k < TPLV; ++k) {
      const int t = t0 + k;
      if (t < task.nvalid) {
        const size_t row = ((size_t)task.b * a.n_max + task.src_tok + t) * a.hkv + h;
        load8(a.v, row * D + 8 * cg, F32IN, x[k]);
      } else {
#pragma unroll
        for (int c = 0; c < 8; ++c) x[k][c] = 0.f;
      }
    }
    float scale[TPLV], zero[TPLV], rcp[TPLV];
    uint32_t redo = 0;                         // bit 8k + c
#pragma unroll
    for (int k = 0; k < TPLV; ++k) {
      float mn = x[k][0], mx = x[k][0];
#pragma unroll
      for (int c = 1; c < 8; ++c) { mn = fminf(mn, x[k][c]); mx = fmaxf(mx, x[k][c]); }
      for (int m = 1; m < lanes_per_group; m <<= 1) {
        mn = fminf(mn, __shfl_xor(mn, m));
        mx = fmaxf(mx, __shfl_xor(mx, m));
      }
      const bool valid = t0 + k < task.nvalid;
      scale[k] = valid ? (mx - mn) / LEV + 0.0f : 0.0f;
      zero[k] = valid ? mn + 0.0f : 0.0f;
      rcp[k] = __builtin_amdgcn_rcpf(scale[k]);
      if (scale[k] != 0.f && !(scale[k] >= 0x1p-100f && scale[k] <= 0x1p+100f)) redo |= 0xFFu << (8 * k);
    }
    if ((cg & (lanes_per_group - 1)) == 0) {
      float* vs = reinterpret_cast<float*>(rec + KC + VC + KM + (cg / lanes_per_group) * 256);
#pragma unroll
      for (int k = 0; k < TPLV; k += 2) {
        *reinterpret_cast<float2*>(vs + t0 + k) = make_float2(scale[k], scale[k + 1]);
        *reinterpret_cast<float2*>(vs + 32 + t0 + k) = make_float2(zero[k], zero[k + 1]);
      }
    }
    uint32_t code[TPLV][8];
#pragma unroll
    for (int k = 0; k < TPLV; ++k)
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        bool r;
        const uint32_t q = fast_code(x[k][c] - zero[k], scale[k], rcp[k], LEV, r);
        const bool live = scale[k] != 0.f;
        code[k][c] = live ? q : 0u;
        redo |= (uint32_t)(live && r) << (8 * k + c);
      }
    if (__any(redo != 0)) {
#pragma unroll
      for (int k = 0; k < TPLV; ++k)
#pragma unroll
        for (int c = 0; c < 8; ++c)
          if ((redo >> (8 * k + c)) & 1u) code[k][c] = exact_code(x[k][c] - zero[k], scale[k], LEV);
    }
    // The lane's TPLV tokens (even-aligned, within one run of four) land in
    // one code word of each channel: token t goes to
    //   mm = t / 16, hh = (t / 4) % 2, e = (t % 4) + 4 * ((t / 8) % 2)
    //   4-bit: word 2*mm + hh, bits 4e;  2-bit: word hh, bits 2*(8*mm + e)
    // Lanes sharing a word OR their bits into it.
    const int mm = t0 / 16, hh = (t0 / 4) % 2;
    const int j = VB == 4 ? 2 * mm + hh : hh;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      uint32_t bits = 0;
#pragma unroll
      for (int k = 0; k < TPLV; ++k) {
        const int t = t0 + k;
        const int e = (t % 4) + 4 * ((t / 8) % 2);
        const int pos = VB == 4 ? 4 * e : 2 * (8 * mm + e);
        bits |= code[k][c] << pos;
      }
      atomicOr(reinterpret_cast<uint32_t*>(rec + KC) + j * D + 8 * cg + c, bits);
    }
  }
  __syncthreads();

  uint8_t* dst = a.seg.records + (((size_t)task.b * a.hkv + h) * a.seg.slot_cap + task.dst_slot) * rbytes;
  for (uint32_t off = tid * 16; off < rbytes; off += 256 * 16)
    *reinterpret_cast<uint4*>(dst + off) = *reinterpret_cast<const uint4*>(rec + off);
  if (h == 0 && tid == 0) {
    int4 hd = make_int4(task.nvalid, (int)task.mask, task.rank_base, task.token_base);
    *reinterpret_cast<int4*>(a.seg.headers + ((size_t)task.b * a.seg.slot_cap + task.dst_slot) * kHeaderBytes) = hd;
  }
}

template <int KB, int VB, int D, bool F32IN>
hipError_t launch_t(const CommitArgs& a, int ntasks, hipStream_t s) {
  dim3 grid(ntasks, a.hkv);
  hipLaunchKernelGGL((commit_kernel<KB, VB, D, F32IN>), grid, dim3(256), 0, s, a);
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
