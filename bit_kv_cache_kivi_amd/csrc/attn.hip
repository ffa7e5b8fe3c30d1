// Fused dequantize-and-attend kernel for gfx950, plus the split-K combine.
//
// The block being denoised (32 query tokens, full precision) attends without a
// mask to itself and to every cached token of the prefix (and suffix, for the
// dual cache), computed directly from the low-bit codes (MaskAhead abstract:
// Q-MaskAhead attends from low-bit KV; SoloQ summary page: bidirectional
// context revisited every step; Tai et al., abstract: prefix and dual cache).
//
// Work unit = one 32-token slot of the cache, or the block itself.  A
// workgroup (4 waves) owns one (sequence, kv head) and a contiguous range of
// units; all Hq/Hkv query heads of that kv head share every dequantized slot.
// Per unit:
//   1. the packed slot record (codes + fp32 meta) is copied HBM -> LDS with
//      coalesced 16-byte loads, prefetched into registers one unit ahead;
//   2. the 256 threads dequantize it once into fp16 MFMA operand tiles in LDS
//      (K tile: A operand of S^T = K Q^T; V tile: A operand of O^T = V^T P^T),
//      patching protected key rows from their bf16 copies;
//   3. each wave runs, for each of its query heads (32 query tokens = one
//      32-wide MFMA tile), S^T on v_mfma_f32_32x32x16_f16, an online softmax in
//      fp32 (exp2 with the softmax scale folded in), and O^T += V^T P^T.
//      Computing the transposed products lets the S accumulator registers feed
//      the PV product's B operand directly (lane = query, 16 tokens per lane).
// A split's partial (running max, sum, unnormalised O) goes to the workspace
// and the combine kernel merges splits with log-sum-exp weights; with a
// single split the workgroup writes the normalised output itself.
#include "device_common.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

template <int KB, int VB, int D, int TPW>
__global__ __launch_bounds__(256) void attn_kernel(const AttnArgs a) {
  constexpr int KS = D / 16;   // MFMA k-steps over the head dimension
  constexpr int CT = D / 32;   // 32-channel output tiles
  constexpr int CPT = D / 8;   // K channels dequantized per thread
  constexpr uint32_t KC = kc_bytes(D, KB);
  constexpr uint32_t VC = vc_bytes(D, VB);
  constexpr uint32_t KM = kmeta_bytes(D);
  constexpr uint32_t RAW_MAX = record_bytes(D, KB, VB, 32);
  constexpr int RAW_ITERS = (RAW_MAX + 256 * 16 - 1) / (256 * 16);

  __shared__ __align__(16) uint8_t raw[RAW_MAX];
  __shared__ __align__(16) half8 kop_lds[2][KS][64];   // dequantized K as fp16 hi + lo
  __shared__ __align__(16) half8 vop_lds[CT][2][64];

  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int np = a.nslots[0][b];
  const int ns = a.use_suffix ? a.nslots[1][b] : 0;
  const int U = np + ns + 1;
  const int nsplit = (U + a.split_units - 1) / a.split_units;
  if (split >= nsplit) return;
  const int u0 = split * a.split_units;
  const int u1 = min(U, u0 + a.split_units);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = a.r;
  const uint32_t rbytes = a.record_bytes;

  // ---- Q operands (B operand of S^T): lane = query token j, half hh holds
  //      channels (D/2)*hh + 8s + [0, 8) at k-step s.
  half8 qop[TPW][KS];
  {
    const int j = lane & 31, hh = lane >> 5;
#pragma unroll
    for (int ti = 0; ti < TPW; ++ti) {
      const int hl = wave + 4 * ti;
      const int hq = kvh * r + (hl < r ? hl : 0);
      const size_t row = ((size_t)b * kSlot + j) * a.hq + hq;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        float x[8];
        load8(a.q, row * D + (D / 2) * hh + 8 * s, a.q_f32, x);
        qop[ti][s] = to_half8(x);
      }
    }
  }

  float m_run[TPW], l_run[TPW];
  floatx16 o[TPW][CT];
#pragma unroll
  for (int ti = 0; ti < TPW; ++ti) {
    m_run[ti] = -__builtin_inff();
    l_run[ti] = 0.f;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[ti][ct][i] = 0.f;
  }

  // segment fields chosen by value: taking the address of the by-value kernel
  // argument would copy the whole argument block to scratch memory
  auto seg_field = [&](int seg, auto SegPtrs::*f) { return seg ? a.seg[1].*f : a.seg[0].*f; };

  // prefetch registers for the next quantized unit
  uint4 pre[RAW_ITERS];
  int pre_nvalid = 0, pre_base = 0, pre_seg = 0;
  uint32_t pre_mask = 0;
  auto prefetch = [&](int u) {
    if (u < np + ns) {
      const int seg = u < np ? 0 : 1;
      const int slot = u < np ? u : u - np;
      const int cap = seg_field(seg, &SegPtrs::slot_cap);
      const int4 hd = *reinterpret_cast<const int4*>(seg_field(seg, &SegPtrs::headers) +
                                                      ((size_t)b * cap + slot) * kHeaderBytes);
      pre_nvalid = hd.x;
      pre_mask = (uint32_t)hd.y;
      pre_base = hd.z;
      pre_seg = seg;
      const uint8_t* src = seg_field(seg, &SegPtrs::records) + (((size_t)b * a.hkv + kvh) * cap + slot) * rbytes;
#pragma unroll
      for (int i = 0; i < RAW_ITERS; ++i) {
        const uint32_t off = (tid + 256 * i) * 16;
        if (off < rbytes) pre[i] = *reinterpret_cast<const uint4*>(src + off);
      }
    }
  };

  prefetch(u0);
  for (int u = u0; u < u1; ++u) {
    int nvalid = kSlot;
    if (u < np + ns) {
      // ---------------- stage the packed record, then dequantize into LDS
      const int cur_nvalid = pre_nvalid, cur_base = pre_base;
      const uint32_t cur_mask = pre_mask;
      const uint16_t* cur_prot = seg_field(pre_seg, &SegPtrs::prot_rows);
      const int cur_pcap = seg_field(pre_seg, &SegPtrs::prot_cap);
#pragma unroll
      for (int i = 0; i < RAW_ITERS; ++i) {
        const uint32_t off = (tid + 256 * i) * 16;
        if (off < rbytes) *reinterpret_cast<uint4*>(raw + off) = pre[i];
      }
      __syncthreads();
      if (u + 1 < u1) prefetch(u + 1);
      nvalid = cur_nvalid;
      // K: thread -> token t, channels [p*CPT, (p+1)*CPT)
      {
        const int t = tid & 31, p = tid >> 5;
        const bool prot = (cur_mask >> t) & 1u;
#pragma unroll
        for (int gi = 0; gi < CPT / 8; ++gi) {
          const int cgp = p * (CPT / 8) + gi;          // 8-channel group
          float x[8];
          if (prot) {
            const int rank = cur_base + __popc(cur_mask & ((1u << t) - 1u));
            const size_t prow = ((size_t)b * cur_pcap + rank) * a.hkv + kvh;
            load8(cur_prot, prow * D + 8 * cgp, false, x);
          } else {
            uint32_t bits;
            if (KB == 4) bits = *reinterpret_cast<const uint32_t*>(raw + t * (D / 2) + 4 * cgp);
            else         bits = *reinterpret_cast<const uint16_t*>(raw + t * (D / 4) + 2 * cgp);
            const float* ks = reinterpret_cast<const float*>(raw + KC + VC) + 8 * cgp;
            const float4 s0 = *reinterpret_cast<const float4*>(ks);
            const float4 s1 = *reinterpret_cast<const float4*>(ks + 4);
            const float4 z0 = *reinterpret_cast<const float4*>(ks + D);
            const float4 z1 = *reinterpret_cast<const float4*>(ks + D + 4);
            const float sc[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
            const float zr[8] = {z0.x, z0.y, z0.z, z0.w, z1.x, z1.y, z1.z, z1.w};
#pragma unroll
            for (int e = 0; e < 8; ++e)
              x[e] = fmaf((float)((bits >> (KB * e)) & ((1u << KB) - 1u)), sc[e], zr[e]);
          }
          const int hh = cgp / (D / 16), s = cgp % (D / 16);
          store_hi_lo(kop_lds[0][s][t + 32 * hh], kop_lds[1][s][t + 32 * hh], x);
        }
      }
      // V: thread -> channel lane cl, combos (ct, mm, hh)
      {
        const int cl = tid & 31, rest = tid >> 5;
#pragma unroll
        for (int qi = 0; qi < CT / 2; ++qi) {
          const int q = rest + 8 * qi;
          const int ct = q >> 2, mm = (q >> 1) & 1, hh = q & 1;
          const int c = 32 * ct + cl;
          uint32_t bits;
          if (VB == 4) bits = *reinterpret_cast<const uint32_t*>(raw + KC + c * 16 + (2 * mm + hh) * 4);
          else         bits = *reinterpret_cast<const uint32_t*>(raw + KC + c * 8 + hh * 4) >> (16 * mm);
          const int g = c >> a.gv_log2;
          const float* vs = reinterpret_cast<const float*>(raw + KC + VC + KM + g * 256);
          const int ta = 16 * mm + 4 * hh;               // tokens ta..ta+3, ta+8..ta+11
          const float4 s0 = *reinterpret_cast<const float4*>(vs + ta);
          const float4 s1 = *reinterpret_cast<const float4*>(vs + ta + 8);
          const float4 z0 = *reinterpret_cast<const float4*>(vs + 32 + ta);
          const float4 z1 = *reinterpret_cast<const float4*>(vs + 32 + ta + 8);
          const float sc[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
          const float zr[8] = {z0.x, z0.y, z0.z, z0.w, z1.x, z1.y, z1.z, z1.w};
          float x[8];
#pragma unroll
          for (int e = 0; e < 8; ++e)
            x[e] = fmaf((float)((bits >> (VB * e)) & ((1u << VB) - 1u)), sc[e], zr[e]);
          vop_lds[ct][mm][cl + 32 * hh] = to_half8(x);
        }
      }
    } else {
      // ---------------- the full-precision block itself
      {
        const int t = tid & 31, p = tid >> 5;
        const size_t row = ((size_t)b * kSlot + t) * a.hkv + kvh;
#pragma unroll
        for (int gi = 0; gi < CPT / 8; ++gi) {
          const int cgp = p * (CPT / 8) + gi;
          float x[8];
          load8(a.k_blk, row * D + 8 * cgp, a.blk_f32, x);
          const int hh = cgp / (D / 16), s = cgp % (D / 16);
          store_hi_lo(kop_lds[0][s][t + 32 * hh], kop_lds[1][s][t + 32 * hh], x);
        }
      }
      {
        const int cl = tid & 31, rest = tid >> 5;
#pragma unroll
        for (int qi = 0; qi < CT / 2; ++qi) {
          const int q = rest + 8 * qi;
          const int ct = q >> 2, mm = (q >> 1) & 1, hh = q & 1;
          const int c = 32 * ct + cl;
          float x[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int t = 16 * mm + 4 * hh + (e & 3) + 8 * (e >> 2);
            x[e] = load1(a.v_blk, (((size_t)b * kSlot + t) * a.hkv + kvh) * D + c, a.blk_f32);
          }
          vop_lds[ct][mm][cl + 32 * hh] = to_half8(x);
        }
      }
    }
    __syncthreads();

    // ---------------- MFMA + online softmax for this wave's query heads
    // S^T = (K_hi + K_lo) Q^T: the lo part carries the bits fp16 drops from
    // the dequantized keys, so the scores keep about 22 significant bits.
    floatx16 sacc[TPW];
#pragma unroll
    for (int ti = 0; ti < TPW; ++ti)
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[ti][i] = 0.f;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const half8 kh = kop_lds[0][s][lane];
      const half8 kl = kop_lds[1][s][lane];
#pragma unroll
      for (int ti = 0; ti < TPW; ++ti) {
        if (wave + 4 * ti < r) {
          sacc[ti] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kh, qop[ti][s], sacc[ti], 0, 0, 0);
          sacc[ti] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kl, qop[ti][s], sacc[ti], 0, 0, 0);
        }
      }
    }
    half8 pop[TPW][2];
#pragma unroll
    for (int ti = 0; ti < TPW; ++ti) {
      if (wave + 4 * ti < r) {
        // sacc[i] = S[query lane%32][token 8*(i/4) + 4*(lane/32) + i%4]
        if (nvalid < kSlot) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int tok = 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
            if (tok >= nvalid) sacc[ti][i] = -__builtin_inff();
          }
        }
        float mx = sacc[ti][0];
#pragma unroll
        for (int i = 1; i < 16; ++i) mx = fmaxf(mx, sacc[ti][i]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run[ti], mx * a.scale_log2);
        const float alpha = __builtin_amdgcn_exp2f(m_run[ti] - m_new);
        m_run[ti] = m_new;
        float psum = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float pv = __builtin_amdgcn_exp2f(fmaf(sacc[ti][i], a.scale_log2, -m_new));
          psum += pv;
          pop[ti][i >> 3][i & 7] = static_cast<_Float16>(pv);
        }
        l_run[ti] = fmaf(l_run[ti], alpha, psum);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
          for (int i = 0; i < 16; ++i) o[ti][ct][i] *= alpha;
      }
    }
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      const half8 v0 = vop_lds[ct][0][lane];
      const half8 v1 = vop_lds[ct][1][lane];
#pragma unroll
      for (int ti = 0; ti < TPW; ++ti) {
        if (wave + 4 * ti < r) {
          o[ti][ct] = __builtin_amdgcn_mfma_f32_32x32x16_f16(v0, pop[ti][0], o[ti][ct], 0, 0, 0);
          o[ti][ct] = __builtin_amdgcn_mfma_f32_32x32x16_f16(v1, pop[ti][1], o[ti][ct], 0, 0, 0);
        }
      }
    }
    __syncthreads();
  }

  // ---------------- epilogue
#pragma unroll
  for (int ti = 0; ti < TPW; ++ti) {
    const int hl = wave + 4 * ti;
    if (hl >= r) continue;
    const int hq = kvh * r + hl;
    const float l_tot = l_run[ti] + __shfl_xor(l_run[ti], 32);
    const int j = lane & 31, hh = lane >> 5;
    if (nsplit == 1) {
      const float inv = 1.0f / l_tot;
      const size_t row = ((size_t)b * kSlot + j) * a.hq + hq;
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
          const int c = 32 * ct + 8 * qd + 4 * hh;
          const float v0 = o[ti][ct][4 * qd] * inv, v1 = o[ti][ct][4 * qd + 1] * inv;
          const float v2 = o[ti][ct][4 * qd + 2] * inv, v3 = o[ti][ct][4 * qd + 3] * inv;
          if (a.out_f32) {
            *reinterpret_cast<float4*>(static_cast<float*>(a.out) + row * D + c) = make_float4(v0, v1, v2, v3);
          } else {
            uint2 w;
            w.x = f32_to_bf16_bits(v0) | (f32_to_bf16_bits(v1) << 16);
            w.y = f32_to_bf16_bits(v2) | (f32_to_bf16_bits(v3) << 16);
            *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + row * D + c) = w;
          }
        }
    } else {
      const size_t idx = (((size_t)b * a.hkv + kvh) * a.max_splits + split) * r + hl;
      float* base = a.partial + idx * (size_t)(D + 2) * kSlot;
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int c = 32 * ct + 8 * (i >> 2) + 4 * hh + (i & 3);
          base[c * kSlot + j] = o[ti][ct][i];
        }
      if (hh == 0) {
        base[D * kSlot + j] = m_run[ti];
        base[(D + 1) * kSlot + j] = l_tot;
      }
    }
  }
}

// One workgroup per (query head, sequence): merges the splits of all 32 rows.
template <int D>
__global__ __launch_bounds__(256) void combine_kernel(const AttnArgs a) {
  __shared__ float w_lds[256][kSlot];
  __shared__ float out_lds[kSlot][D + 1];
  __shared__ float inv_l[kSlot];
  const int hq = blockIdx.x, b = blockIdx.y;
  const int np = a.nslots[0][b];
  const int ns = a.use_suffix ? a.nslots[1][b] : 0;
  const int U = np + ns + 1;
  const int nsplit = (U + a.split_units - 1) / a.split_units;
  if (nsplit <= 1) return;
  const int r = a.r, kvh = hq / r, hl = hq % r;
  const int tid = threadIdx.x;
  auto part = [&](int sp) {
    return a.partial + ((((size_t)b * a.hkv + kvh) * a.max_splits + sp) * r + hl) * (size_t)(D + 2) * kSlot;
  };
  if (tid < kSlot) {
    float mstar = -__builtin_inff();
    for (int sp = 0; sp < nsplit; ++sp) mstar = fmaxf(mstar, part(sp)[D * kSlot + tid]);
    float l = 0.f;
    for (int sp = 0; sp < nsplit; ++sp) {
      const float w = __builtin_amdgcn_exp2f(part(sp)[D * kSlot + tid] - mstar);
      w_lds[sp][tid] = w;
      l = fmaf(part(sp)[(D + 1) * kSlot + tid], w, l);
    }
    inv_l[tid] = 1.0f / l;
  }
  __syncthreads();
  const int j = tid & 31, cq = tid >> 5;
  for (int c = cq; c < D; c += 8) {
    float acc = 0.f;
    for (int sp = 0; sp < nsplit; ++sp) acc = fmaf(part(sp)[c * kSlot + j], w_lds[sp][j], acc);
    out_lds[j][c] = acc * inv_l[j];
  }
  __syncthreads();
  for (int idx = tid; idx < kSlot * D; idx += 256) {
    const int jj = idx / D, c = idx % D;
    const size_t o = (((size_t)b * kSlot + jj) * a.hq + hq) * D + c;
    if (a.out_f32) static_cast<float*>(a.out)[o] = out_lds[jj][c];
    else static_cast<uint16_t*>(a.out)[o] = (uint16_t)f32_to_bf16_bits(out_lds[jj][c]);
  }
}

template <int KB, int VB, int D>
hipError_t launch_kbd(const AttnArgs& a, int grid_splits, int B, hipStream_t s) {
  dim3 grid(grid_splits, a.hkv, B);
  if (a.r <= 4) hipLaunchKernelGGL((attn_kernel<KB, VB, D, 1>), grid, dim3(256), 0, s, a);
  else          hipLaunchKernelGGL((attn_kernel<KB, VB, D, 2>), grid, dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || grid_splits <= 1) return e;
  hipLaunchKernelGGL((combine_kernel<D>), dim3(a.hq, B), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int KB, int VB>
hipError_t launch_kb(const AttnArgs& a, int grid_splits, int B, int D, hipStream_t s) {
  return D == 64 ? launch_kbd<KB, VB, 64>(a, grid_splits, B, s) : launch_kbd<KB, VB, 128>(a, grid_splits, B, s);
}

}  // namespace

hipError_t launch_attention(const AttnArgs& a, int grid_splits, int B, int D, int kb, int vb,
                            hipStream_t stream) {
  if (kb == 4 && vb == 4) return launch_kb<4, 4>(a, grid_splits, B, D, stream);
  if (kb == 4 && vb == 2) return launch_kb<4, 2>(a, grid_splits, B, D, stream);
  if (kb == 2 && vb == 4) return launch_kb<2, 4>(a, grid_splits, B, D, stream);
  return launch_kb<2, 2>(a, grid_splits, B, D, stream);
}

}  // namespace kvq
