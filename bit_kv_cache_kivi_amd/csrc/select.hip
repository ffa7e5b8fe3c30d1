// Mask-query selection over the low-bit cache, for gfx950.
//
// The current block's mask queries rank the cached entries by their estimated
// contribution to the attention output, computed directly from the low-bit
// codes, and the block then attends to the top-ranked entries only (MaskAhead
// / Q-MaskAhead abstract).  The contribution of entry j of a (sequence, kv
// head) is ||v_j|| times the softmax mass that the mask queries of the group's
// query heads put on it, the softmax running over every valid cached token and
// the 32 block tokens.
//
// Two passes over the units (32-token slots) of each (sequence, kv head), in
// splits:
//   MODE 0 (stats): per (query head, query token), the maximum and the sum of
//     exp2 of the scaled scores over the split's units (the block included, in
//     the last split), written as split partials;
//   MODE 1 (score): merges the partials into the softmax normaliser, recomputes
//     the scores, turns them into probabilities, sums them over the mask queries
//     (a butterfly across the 32 lanes of a query set) and the heads, and
//     multiplies by the value norms (computed from the codes) -> one fp32
//     contribution per entry, -1 for slot positions past the valid tokens.
// A workgroup of four waves loads a unit's record into LDS (the next unit's
// loads are issued before the current one is processed), dequantizes the keys
// into fp16 MFMA operand tiles, and each wave runs S^T = K Q^T
// (v_mfma_f32_32x32x16_f16) for up to two query heads.  The ranking only needs
// the keys to fp16 precision; both passes see the same rounded scores.
//
// topk_kernel then selects, per (sequence, kv head), the k largest
// contributions exactly (ties to the lower entry) by a four-digit radix select
// on the float bits, and writes a token mask per unit and the list of units
// that hold a selected token.
#include "device_common.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxHeads = 8;   // query heads per kv head

template <int CTRL>
__device__ __forceinline__ float add_dpp(float x) {
  return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// sum over the 32 lanes of each half of the wave
__device__ __forceinline__ float sum32(float x) {
  x = add_dpp<0xB1>(x);    // quad_perm [1,0,3,2]
  x = add_dpp<0x4E>(x);    // quad_perm [2,3,0,1]
  x = add_dpp<0x141>(x);   // row_half_mirror
  x = add_dpp<0x140>(x);   // row_mirror
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

template <int KB, int VB, int D, int MODE>
__global__ __launch_bounds__(kThreads) void sel_kernel(const SelArgs a) {
  constexpr int KS = D / 16;
  constexpr int GPT = kSlot * (D / 8) / kThreads;      // (token, 8-channel group) pairs per thread
  constexpr int KTT = kSlot / GPT;
  constexpr int RPT = (48 * D / 16 + kThreads - 1) / kThreads;
  constexpr uint32_t KC = kc_bytes(D, KB), VC = vc_bytes(D, VB), KM = kmeta_bytes(D);
  static_assert(record_bytes(D, KB, VB, 32) <= 48 * D, "record fits the stage");
  __shared__ __align__(16) uint8_t rec[48 * D];
  __shared__ __align__(16) half8 kt[KS][64];
  __shared__ __align__(16) uint4 prt[GPT][kThreads];   // each thread's protected key chunks
  __shared__ float vn[kSlot];
  __shared__ float hsum[kMaxHeads][kSlot];

  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int np = a.nslots[0][b], ns = a.use_suffix ? a.nslots[1][b] : 0;
  const int NC = np + ns;                          // cached units
  const int U = NC + (MODE == 0 ? 1 : 0);          // the stats also cover the block
  const int nsplit = (U + a.split_units - 1) / a.split_units;
  if (split >= nsplit) return;
  const int u0 = split * a.split_units, u1 = min(U, u0 + a.split_units);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hkv = a.hkv, r = a.r, hq_all = a.hq;
  const uint32_t rbytes = a.record_bytes;
  const float c2 = a.scale_log2;
  const int j = lane & 31, hh = lane >> 5;
  const int kt0 = tid % KTT, kcg = tid / KTT;
  const int khh = kcg / (D / 16), kks = kcg % (D / 16);
  const SegPtrs seg0 = a.seg[0], seg1 = a.seg[1];

  // Q operands of the wave's query heads wave and wave + 4 (B operand of
  // S^T: lane = query token j, half hh holds channels (D/2)*hh + 8s + [0, 8))
  half8 qop[2][KS];
#pragma unroll
  for (int hi = 0; hi < 2; ++hi) {
    const int ci = min(wave + 4 * hi, r - 1);
    const size_t base = (((size_t)b * kSlot + j) * hq_all + kvh * r + ci) * D + (D / 2) * hh;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      float x[8];
      load8(a.q, base + 8 * s, a.q_f32, x);
      qop[hi][s] = to_half8(x);
    }
  }

  // running statistics (MODE 0) or the merged normaliser (MODE 1), per head
  float m_run[2] = {-__builtin_inff(), -__builtin_inff()}, l_run[2] = {0.f, 0.f};
  const size_t pbase = ((size_t)b * hkv + kvh) * a.max_splits;
  if (MODE == 1) {
    const int nstat = (NC + 1 + a.stats_split_units - 1) / a.stats_split_units;
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) {
      const int ci = min(wave + 4 * hi, r - 1);
      float M = -__builtin_inff();
      for (int sp = 0; sp < nstat; ++sp) M = fmaxf(M, a.partial[(((pbase + sp) * kMaxHeads + ci) * 2) * kSlot + j]);
      float L = 0.f;
      for (int sp = 0; sp < nstat; ++sp) {
        const float* pp = a.partial + (((pbase + sp) * kMaxHeads + ci) * 2) * kSlot + j;
        if (pp[0] > -__builtin_inff()) L += pp[kSlot] * __builtin_amdgcn_exp2f(pp[0] - M);
      }
      m_run[hi] = M;
      l_run[hi] = 1.0f / L;
    }
  }
  const bool qsel = (a.qmask[b] >> j) & 1u;

  // ---- unit loads: the record (16-byte chunks) and this thread's protected
  // key chunks, plus the header
  // Buffer loads: a unit past the split (or the block) gets empty resources,
  // so its loads return zeros without memory traffic and every path writes
  // the same registers.
  uint4 rc[RPT], pc[GPT];
  int4 hd;
  auto load = [&](int u) __attribute__((always_inline)) {
    const bool valid = u < min(u1, NC);
    const bool s1 = u >= np;
    const int sl = valid ? (s1 ? u - np : u) : 0;
    const int cap = s1 ? seg1.slot_cap : seg0.slot_cap;
    const int pcap = s1 ? seg1.prot_cap : seg0.prot_cap;
    const uint8_t* recp = (s1 ? seg1.records : seg0.records) + (((size_t)b * hkv + kvh) * cap + sl) * rbytes;
    const uint8_t* hdrp = (s1 ? seg1.headers : seg0.headers) + ((size_t)b * cap + sl) * kHeaderBytes;
    const uint16_t* prot = (s1 ? seg1.prot_rows : seg0.prot_rows) + ((size_t)b * hkv + kvh) * pcap * D;
    const __amdgpu_buffer_rsrc_t hr = __builtin_amdgcn_make_buffer_rsrc((void*)hdrp, 0, valid ? kHeaderBytes : 0, 0x00020000);
    const __amdgpu_buffer_rsrc_t rr = __builtin_amdgcn_make_buffer_rsrc((void*)recp, 0, valid ? (int)rbytes : 0, 0x00020000);
    const __amdgpu_buffer_rsrc_t pr_ = __builtin_amdgcn_make_buffer_rsrc(
        (void*)prot, 0, valid ? (int)min((size_t)pcap * D * 2, (size_t)0x7fffffff) : 0, 0x00020000);
    hd = __builtin_bit_cast(int4, __builtin_amdgcn_raw_buffer_load_b128(hr, 0, 0, 0));
#pragma unroll
    for (int q = 0; q < RPT; ++q)
      rc[q] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rr, (q * kThreads + tid) * 16, 0, 0));
#pragma unroll
    for (int gi = 0; gi < GPT; ++gi) {
      const int t = kt0 + KTT * gi;
      const int rank = hd.z + __popc((uint32_t)hd.y & ((1u << t) - 1u));
      const int off = ((hd.y >> t) & 1) ? (rank * D + 8 * kcg) * 2 : 0x7ff00000;
      pc[gi] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(pr_, off, 0, 0));
    }
  };

  load(u0);
  for (int u = u0; u < u1; ++u) {
    const bool blk = MODE == 0 && u == NC;
    const int4 h = blk ? make_int4(kSlot, 0, 0, 0) : hd;
    if (!blk) {
#pragma unroll
      for (int q = 0; q < RPT; ++q) {
        const uint32_t off = (uint32_t)(q * kThreads + tid) * 16u;
        if (off < rbytes) *reinterpret_cast<uint4*>(rec + off) = rc[q];
      }
#pragma unroll
      for (int gi = 0; gi < GPT; ++gi) prt[gi][tid] = pc[gi];
    }
    __syncthreads();
    load(u + 1);
    // keys -> fp16 operand tiles: tokens kt0 + KTT*gi of channel group kcg
    {
      const float* km = reinterpret_cast<const float*>(rec + KC + VC) + 8 * kcg;
      const uint32_t* words = reinterpret_cast<const uint32_t*>(rec);
#pragma unroll
      for (int gi = 0; gi < GPT; ++gi) {
        const int t = kt0 + KTT * gi;
        float x[8];
        if (blk) {
          load8(a.k_blk, (((size_t)b * kSlot + t) * hkv + kvh) * D + 8 * kcg, a.blk_f32, x);
        } else if ((h.y >> t) & 1) {
          const uint4 w = prt[gi][tid];
          x[0] = bf16_lo(w.x); x[1] = bf16_hi(w.x); x[2] = bf16_lo(w.y); x[3] = bf16_hi(w.y);
          x[4] = bf16_lo(w.z); x[5] = bf16_hi(w.z); x[6] = bf16_lo(w.w); x[7] = bf16_hi(w.w);
        } else {
          float code[8];
          const uint32_t w = KB == 4 ? words[kcg * 32 + t] : words[(kcg >> 1) * 32 + t] >> (16 * (kcg & 1));
          unpack8<KB>(w, code);
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = fmaf(code[e], km[e], km[D + e]);
        }
        kt[kks][t + 32 * khh] = to_half8(x);
      }
    }
    if (MODE == 1) {
      // value norms: token t, channels [cs * D/8, +D/8) of one value group
      const int t = tid >> 3, cs = tid & 7, c0 = cs * (D / 8);
      const int mm = t / 16, th = (t / 4) % 2, e = (t % 4) + 4 * ((t / 8) % 2);
      const int wj = VB == 4 ? 2 * mm + th : th;
      const int bit = VB == 4 ? 4 * e : 2 * (8 * mm + e);
      const float* vm = reinterpret_cast<const float*>(rec + KC + VC + KM + (c0 >> a.gv_log2) * 256);
      const float sc = vm[t], zr = vm[kSlot + t];
      const uint32_t* vw = reinterpret_cast<const uint32_t*>(rec + KC) + wj * D + c0;
      float acc = 0.f;
#pragma unroll
      for (int cc = 0; cc < D / 8; cc += 4) {
        const uint4 w4 = *reinterpret_cast<const uint4*>(vw + cc);
        const uint32_t w[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float x = fmaf((float)((w[k] >> bit) & ((1u << VB) - 1u)), sc, zr);
          acc = fmaf(x, x, acc);
        }
      }
      acc = add_dpp<0xB1>(acc);
      acc = add_dpp<0x4E>(acc);
      acc = add_dpp<0x141>(acc);
      if (cs == 0) vn[t] = sqrtf(acc);
    }
    __syncthreads();
    // scores of the wave's heads
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) {
      const int ci = wave + 4 * hi;
      if (ci < r) {
        floatx16 sacc;
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[i] = 0.f;
#pragma unroll
        for (int s = 0; s < KS; ++s) sacc = __builtin_amdgcn_mfma_f32_32x32x16_f16(kt[s][lane], qop[hi][s], sacc, 0, 0, 0);
        // sacc[i]: query j, token 8*(i/4) + 4*hh + i%4
        if (MODE == 0) {
          float sv[16], mx = -__builtin_inff();
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int tok = 8 * (i >> 2) + 4 * hh + (i & 3);
            sv[i] = tok < h.x ? sacc[i] * c2 : -__builtin_inff();
            mx = fmaxf(mx, sv[i]);
          }
          const float mn = fmaxf(m_run[hi], mx);
          if (mn > -__builtin_inff()) {
            float l = l_run[hi] * __builtin_amdgcn_exp2f(m_run[hi] - mn);
#pragma unroll
            for (int i = 0; i < 16; ++i) l += __builtin_amdgcn_exp2f(sv[i] - mn);
            l_run[hi] = l;
            m_run[hi] = mn;
          }
        } else {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int tok = 8 * (i >> 2) + 4 * hh + (i & 3);
            const float p = (qsel && tok < h.x) ? __builtin_amdgcn_exp2f(fmaf(sacc[i], c2, -m_run[hi])) * l_run[hi] : 0.f;
            const float sum = sum32(p);
            if (j == 0) hsum[ci][tok] = sum;
          }
        }
      }
    }
    __syncthreads();
    if (MODE == 1 && tid < kSlot) {
      float acc = 0.f;
      for (int ci = 0; ci < r; ++ci) acc += hsum[ci][tid];
      a.contrib[(((size_t)b * hkv + kvh) * a.ucap + u) * kSlot + tid] = tid < h.x ? vn[tid] * acc : -1.0f;
    }
  }
  if (MODE == 0) {
    // merge the two halves (the same query's two token sets) and write the partials
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) {
      const int ci = wave + 4 * hi;
      const auto pm = __builtin_amdgcn_permlane32_swap(__float_as_uint(m_run[hi]), __float_as_uint(m_run[hi]), false, false);
      const auto pl = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run[hi]), __float_as_uint(l_run[hi]), false, false);
      const float m0 = __uint_as_float(pm[0]), m1 = __uint_as_float(pm[1]);
      const float l0 = __uint_as_float(pl[0]), l1 = __uint_as_float(pl[1]);
      const float M = fmaxf(m0, m1);
      float L = 0.f;
      if (m0 > -__builtin_inff()) L += l0 * __builtin_amdgcn_exp2f(m0 - M);
      if (m1 > -__builtin_inff()) L += l1 * __builtin_amdgcn_exp2f(m1 - M);
      if (ci < r && hh == 0) {
        float* pp = a.partial + (((pbase + split) * kMaxHeads + ci) * 2) * kSlot + j;
        pp[0] = M;
        pp[kSlot] = L;
      }
    }
  }
}

// ---- exact top-k per (sequence, kv head)
constexpr int kTopkThreads = 1024;

__device__ __forceinline__ uint32_t entry_key(float c) {
  return c >= 0.f ? __float_as_uint(c) + 1u : 0u;   // valid entries above every invalid one
}

// exclusive prefix sum over the workgroup; returns the total in *total
__device__ uint32_t block_scan(uint32_t v, uint32_t* buf, uint32_t* total) {
  const int tid = threadIdx.x;
  buf[tid] = v;
  __syncthreads();
  for (int off = 1; off < kTopkThreads; off <<= 1) {
    const uint32_t add = tid >= off ? buf[tid - off] : 0u;
    __syncthreads();
    buf[tid] += add;
    __syncthreads();
  }
  const uint32_t incl = buf[tid];
  *total = buf[kTopkThreads - 1];
  __syncthreads();
  return incl - v;
}

__global__ __launch_bounds__(kTopkThreads) void topk_kernel(const TopkArgs a) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t scan[kTopkThreads];
  __shared__ uint32_t sh[4];   // prefix, remaining, nvalid
  const int kvh = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int nu = a.nunits[b];
  const int N = nu * kSlot;
  const size_t pair = (size_t)b * a.hkv + kvh;
  const float* c = a.contrib + pair * a.ucap * kSlot;
  uint32_t* mask_out = a.sel_mask + pair * a.ucap;
  int32_t* units_out = a.sel_units + pair * a.ucap;

  if (tid == 0) sh[2] = 0;
  __syncthreads();
  uint32_t nv = 0;
  for (int i = tid; i < N; i += kTopkThreads) nv += entry_key(c[i]) != 0u;
  atomicAdd(&sh[2], nv);
  __syncthreads();
  const uint32_t k = min((uint32_t)max(a.budget, 0), sh[2]);
  // radix select of the k-th largest key, most significant digit first
  uint32_t prefix = 0, pmask = 0, remaining = k;
  if (k > 0) {
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int i = tid; i < 256; i += kTopkThreads) hist[i] = 0;
      __syncthreads();
      for (int i = tid; i < N; i += kTopkThreads) {
        const uint32_t key = entry_key(c[i]);
        if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (tid == 0) {
        uint32_t cum = 0, d = 0;
        for (int dd = 255; dd >= 0; --dd) {
          if (cum + hist[dd] >= remaining) { d = (uint32_t)dd; break; }
          cum += hist[dd];
        }
        sh[0] = prefix | (d << shift);
        sh[1] = remaining - cum;
      }
      __syncthreads();
      prefix = sh[0];
      remaining = sh[1];
      pmask |= 255u << shift;
      __syncthreads();
    }
  }
  const uint32_t T = prefix, need = remaining;   // keys > T, and the first `need` keys == T
  // units [tid*UPT, (tid+1)*UPT): ties ranked in entry order
  const int UPT = (nu + kTopkThreads - 1) / kTopkThreads;
  const int ub = tid * UPT, ue = min(nu, ub + UPT);
  uint32_t ties = 0;
  if (k > 0)
    for (int i = ub * kSlot; i < ue * kSlot; ++i) ties += entry_key(c[i]) == T;
  uint32_t tot;
  uint32_t rank = block_scan(ties, scan, &tot);
  uint32_t nonzero = 0;
  for (int u = ub; u < ue; ++u) {
    uint32_t m = 0;
    if (k > 0) {
      for (int t = 0; t < kSlot; ++t) {
        const uint32_t key = entry_key(c[u * kSlot + t]);
        bool s = key > T;
        if (key == T) { s = rank < need; ++rank; }
        m |= (s ? 1u : 0u) << t;
      }
    }
    mask_out[u] = m;
    nonzero += m != 0u;
  }
  uint32_t pos = block_scan(nonzero, scan, &tot);
  for (int u = ub; u < ue; ++u)
    if (mask_out[u] != 0u) units_out[pos++] = u;
  if (tid == 0) a.sel_count[pair] = (int32_t)tot;
}

template <int KB, int VB, int D>
hipError_t launch_sel_kbd(const SelArgs& a, int mode, int grid_splits, int B, hipStream_t s) {
  const dim3 grid(grid_splits, a.hkv, B);
  if (mode == 0) hipLaunchKernelGGL((sel_kernel<KB, VB, D, 0>), grid, dim3(kThreads), 0, s, a);
  else           hipLaunchKernelGGL((sel_kernel<KB, VB, D, 1>), grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

template <int KB, int VB>
hipError_t launch_sel_kb(const SelArgs& a, int mode, int grid_splits, int B, int D, hipStream_t s) {
  return D == 64 ? launch_sel_kbd<KB, VB, 64>(a, mode, grid_splits, B, s)
                 : launch_sel_kbd<KB, VB, 128>(a, mode, grid_splits, B, s);
}

}  // namespace

hipError_t launch_select(const SelArgs& a, int mode, int grid_splits, int B, int D, int kb, int vb,
                         hipStream_t stream) {
  if (grid_splits <= 0) return hipSuccess;
  if (kb == 4 && vb == 4) return launch_sel_kb<4, 4>(a, mode, grid_splits, B, D, stream);
  if (kb == 4 && vb == 2) return launch_sel_kb<4, 2>(a, mode, grid_splits, B, D, stream);
  if (kb == 2 && vb == 4) return launch_sel_kb<2, 4>(a, mode, grid_splits, B, D, stream);
  return launch_sel_kb<2, 2>(a, mode, grid_splits, B, D, stream);
}

hipError_t launch_topk(const TopkArgs& a, int B, hipStream_t stream) {
  hipLaunchKernelGGL(topk_kernel, dim3(a.hkv, B), dim3(kTopkThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace kvq
