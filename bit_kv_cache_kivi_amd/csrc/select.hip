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
//     the scores as S = Q K^T (a lane per token), turns them into
//     probabilities, sums them over the mask queries (in-lane, then across the
//     two lane halves) and the heads, and
//     multiplies by the value norms (computed from the codes) -> one fp32
//     contribution per entry, -1 for slot positions past the valid tokens.
// A workgroup of eight waves loads a unit's record into LDS (the next unit's
// loads are issued before the current one is processed), dequantizes the keys
// into fp16 MFMA operand tiles, and wave w runs S^T = K Q^T
// (v_mfma_f32_32x32x16_f16) for query head w of the group.  The workgroup
// barriers order LDS only (a plain workgroup barrier would also wait for the
// prefetch loads in flight).  The ranking only needs
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

constexpr int kWaves = 8;                 // one query head per wave
constexpr int kThreads = 64 * kWaves;
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
  constexpr int NPAIR = kSlot * (D / 8);                 // (token, 8-channel group) pairs of a unit
  static_assert(NPAIR <= kThreads, "one pair per thread");
  constexpr int RPT = (48 * D / 16 + kThreads - 1) / kThreads;
  constexpr int VLANES = kThreads / kSlot;               // threads per token for the value norms
  constexpr int VCH = D / VLANES;                        // channels per thread
  static_assert(VLANES == 16 && VCH % 4 == 0, "value-norm mapping");
  constexpr uint32_t KC = kc_bytes(D, KB), VC = vc_bytes(D, VB), KM = kmeta_bytes(D);
  static_assert(record_bytes(D, KB, VB, 32) <= 48 * D, "record fits the stage");
  __shared__ __align__(16) uint8_t rec[48 * D];
  __shared__ __align__(16) half8 kt[KS][64];
  __shared__ __align__(16) uint4 prt[kThreads];          // each thread's protected key chunk
  __shared__ float vn[kSlot];
  __shared__ __align__(16) int4 hdrs[kMaxSelSplit];    // the split's unit headers
  __shared__ float hsum[kWaves][kSlot];                  // per wave (head): P summed over the mask queries
  __shared__ __align__(16) float mq[kWaves][kSlot];      // MODE 1: per head and query, the maximum
  __shared__ __align__(16) float lq[kWaves][kSlot];      // and the weight 1/sum (0 outside the mask)

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
  const bool kpair = tid < NPAIR;                  // this thread dequantizes (token kt0, group kcg)
  const int kt0 = tid % kSlot, kcg = tid / kSlot;
  const int khh = kcg / (D / 16), kks = kcg % (D / 16);
  const SegPtrs seg0 = a.seg[0], seg1 = a.seg[1];
  const bool head = wave < r;                      // wave w runs query head w of the group
  const int ci = min(wave, r - 1);

  // Q operand of the wave's head (B operand of S^T: lane = query token j,
  // half hh holds channels (D/2)*hh + 8s + [0, 8) at k-step s)
  half8 qop[KS];
  {
    const size_t base = (((size_t)b * kSlot + j) * hq_all + kvh * r + ci) * D + (D / 2) * hh;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      float x[8];
      load8(a.q, base + 8 * s, a.q_f32, x);
      qop[s] = to_half8(x);
    }
  }

  // running statistics (MODE 0) or the merged normaliser (MODE 1)
  float m_run = -__builtin_inff(), l_run = 0.f;
  const size_t pbase = ((size_t)b * hkv + kvh) * a.max_splits;
  if (MODE == 1) {
    // merge the stats pass's split partials, eight splits' loads at a time
    // (indices clamped; repeats are masked out), so that each batch costs
    // one memory latency
    const int nstat = (NC + 1 + a.stats_split_units - 1) / a.stats_split_units;
    constexpr int kBatch = 8;
    float M = -__builtin_inff(), L = 0.f;
    for (int sp0 = 0; sp0 < nstat; sp0 += kBatch) {
      float mv[kBatch], lv[kBatch];
#pragma unroll
      for (int q = 0; q < kBatch; ++q) {
        const float* pp = a.partial + (((pbase + min(sp0 + q, nstat - 1)) * kMaxHeads + ci) * 2) * kSlot + j;
        mv[q] = pp[0];
        lv[q] = pp[kSlot];
      }
#pragma unroll
      for (int q = 0; q < kBatch; ++q) {
        if (sp0 + q < nstat && mv[q] > -__builtin_inff()) {
          const float mn = fmaxf(M, mv[q]);
          L = L * __builtin_amdgcn_exp2f(M - mn) + lv[q] * __builtin_amdgcn_exp2f(mv[q] - mn);
          M = mn;
        }
      }
    }
    // queries outside the mask get weight 0
    if (hh == 0) {
      mq[wave][j] = M;
      lq[wave][j] = ((a.qmask[b] >> j) & 1u) ? 1.0f / L : 0.f;
    }
  }

  // ---- unit loads: the record (16-byte chunks) and this thread's protected
  // key chunk.  Buffer loads: a unit past the split (or the block) gets empty
  // resources, so its loads return zeros without memory traffic and every
  // path writes the same registers.
  // two units in flight: a unit's loads are issued two units before it is
  // processed (register sets indexed by the unrolled position)
  constexpr int NPF = 2;
  struct Pre { uint4 rc[RPT]; uint4 pc; int4 hd; };
  Pre pre[NPF];
  auto load = [&](int u, Pre& p) __attribute__((always_inline)) {
    const bool valid = u < min(u1, NC);
    const bool s1 = u >= np;
    const int sl = valid ? (s1 ? u - np : u) : 0;
    const int cap = s1 ? seg1.slot_cap : seg0.slot_cap;
    const int pcap = s1 ? seg1.prot_cap : seg0.prot_cap;
    const uint8_t* recp = (s1 ? seg1.records : seg0.records) + (((size_t)b * hkv + kvh) * cap + sl) * rbytes;
    const uint16_t* prot = (s1 ? seg1.prot_rows : seg0.prot_rows) + ((size_t)b * hkv + kvh) * pcap * D;
    const __amdgpu_buffer_rsrc_t rr = __builtin_amdgcn_make_buffer_rsrc((void*)recp, 0, valid ? (int)rbytes : 0, 0x00020000);
    const __amdgpu_buffer_rsrc_t pr_ = __builtin_amdgcn_make_buffer_rsrc(
        (void*)prot, 0, valid ? (int)min((size_t)pcap * D * 2, (size_t)0x7fffffff) : 0, 0x00020000);
    const int4 hd = valid ? hdrs[u - u0] : make_int4(0, 0, 0, 0);
    p.hd = hd;
#pragma unroll
    for (int q = 0; q < RPT; ++q)
      p.rc[q] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rr, (q * kThreads + tid) * 16, 0, 0));
    const int rank = hd.z + __popc((uint32_t)hd.y & ((1u << kt0) - 1u));
    const int off = (kpair && ((hd.y >> kt0) & 1)) ? (rank * D + 8 * kcg) * 2 : 0x7ff00000;
    p.pc = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(pr_, off, 0, 0));
  };

  // the split's headers, read once: a unit's protected-row loads depend on its
  // header, and a global read of it per unit would stall the prefetch
  for (int i = tid; i < min(u1, NC) - u0; i += kThreads) {
    const int u = u0 + i;
    const bool s1 = u >= np;
    const int sl = s1 ? u - np : u;
    const int cap = s1 ? seg1.slot_cap : seg0.slot_cap;
    hdrs[i] = *reinterpret_cast<const int4*>((s1 ? seg1.headers : seg0.headers) + ((size_t)b * cap + sl) * kHeaderBytes);
  }
  lds_barrier();
#pragma unroll
  for (int k = 0; k < NPF; ++k) load(u0 + k, pre[k]);
  for (int ub = u0; ub < u1; ub += NPF)
#pragma unroll
  for (int k = 0; k < NPF; ++k) {
    const int u = ub + k;
    if (u >= u1) break;
    const bool blk = MODE == 0 && u == NC;
    const int4 h = blk ? make_int4(kSlot, 0, 0, 0) : pre[k].hd;
    if (!blk) {
#pragma unroll
      for (int q = 0; q < RPT; ++q) {
        const uint32_t off = (uint32_t)(q * kThreads + tid) * 16u;
        if (off < rbytes) *reinterpret_cast<uint4*>(rec + off) = pre[k].rc[q];
      }
      prt[tid] = pre[k].pc;
    }
    lds_barrier();
    load(u + NPF, pre[k]);
    // keys -> fp16 operand tiles: token kt0 of channel group kcg
    if (kpair) {
      const float* km = reinterpret_cast<const float*>(rec + KC + VC) + 8 * kcg;
      const uint32_t* words = reinterpret_cast<const uint32_t*>(rec);
      const int t = kt0;
      float x[8];
      if (blk) {
        load8(a.k_blk, (((size_t)b * kSlot + t) * hkv + kvh) * D + 8 * kcg, a.blk_f32, x);
      } else if ((h.y >> t) & 1) {
        const uint4 w = prt[tid];
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
    if (MODE == 1) {
      // value norms: token t, channels [cs * VCH, +VCH) of one value group
      const int t = tid / VLANES, cs = tid % VLANES, c0 = cs * VCH;
      const int mm = t / 16, th = (t / 4) % 2, e = (t % 4) + 4 * ((t / 8) % 2);
      const int wj = VB == 4 ? 2 * mm + th : th;
      const int bit = VB == 4 ? 4 * e : 2 * (8 * mm + e);
      const float* vm = reinterpret_cast<const float*>(rec + KC + VC + KM + (c0 >> a.gv_log2) * 256);
      const float sc = vm[t], zr = vm[kSlot + t];
      const uint32_t* vw = reinterpret_cast<const uint32_t*>(rec + KC) + wj * D + c0;
      float acc = 0.f;
#pragma unroll
      for (int cc = 0; cc < VCH; cc += 4) {
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
      acc = add_dpp<0x140>(acc);
      if (cs == 0) vn[t] = sqrtf(acc);
    }
    lds_barrier();
    // scores of the wave's head
    if (head) {
      floatx16 sacc;
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[i] = 0.f;
      // MODE 0: S^T = K Q^T, sacc[i] = S[query j][token 8*(i/4) + 4*hh + i%4];
      // MODE 1: S = Q K^T (the same operand registers, swapped),
      // sacc[i] = S[query 8*(i/4) + 4*hh + i%4][token j]
#pragma unroll
      for (int s = 0; s < KS; ++s)
        sacc = MODE == 0 ? __builtin_amdgcn_mfma_f32_32x32x16_f16(kt[s][lane], qop[s], sacc, 0, 0, 0)
                         : __builtin_amdgcn_mfma_f32_32x32x16_f16(qop[s], kt[s][lane], sacc, 0, 0, 0);
      if (MODE == 0) {
        float sv[16], mx = -__builtin_inff();
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int tok = 8 * (i >> 2) + 4 * hh + (i & 3);
          sv[i] = tok < h.x ? sacc[i] * c2 : -__builtin_inff();
          mx = fmaxf(mx, sv[i]);
        }
        const float mn = fmaxf(m_run, mx);
        if (mn > -__builtin_inff()) {
          float l = l_run * __builtin_amdgcn_exp2f(m_run - mn);
#pragma unroll
          for (int i = 0; i < 16; ++i) l += __builtin_amdgcn_exp2f(sv[i] - mn);
          l_run = l;
          m_run = mn;
        }
      } else {
        // MODE 1 computes S = Q K^T (lane = token, 16 queries per lane), so the
        // sum over queries is in-lane; the queries' maxima and weights come
        // from LDS (four consecutive queries per read)
        float acc = 0.f;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const float4 m4 = *reinterpret_cast<const float4*>(&mq[ci][8 * g + 4 * hh]);
          const float4 l4 = *reinterpret_cast<const float4*>(&lq[ci][8 * g + 4 * hh]);
          acc = fmaf(__builtin_amdgcn_exp2f(fmaf(sacc[4 * g], c2, -m4.x)), l4.x, acc);
          acc = fmaf(__builtin_amdgcn_exp2f(fmaf(sacc[4 * g + 1], c2, -m4.y)), l4.y, acc);
          acc = fmaf(__builtin_amdgcn_exp2f(fmaf(sacc[4 * g + 2], c2, -m4.z)), l4.z, acc);
          acc = fmaf(__builtin_amdgcn_exp2f(fmaf(sacc[4 * g + 3], c2, -m4.w)), l4.w, acc);
        }
        const auto ps = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc), __float_as_uint(acc), false, false);
        if (hh == 0) hsum[wave][j] = __uint_as_float(ps[0]) + __uint_as_float(ps[1]);
      }
    }
    lds_barrier();
    if (MODE == 1 && wave == 0) {
      // entry contributions (lanes 0..31), and the unit's sum over its valid
      // entries (a butterfly over those lanes)
      float cv = 0.f;
      if (lane < kSlot) {
        float acc = 0.f;
        for (int w = 0; w < r; ++w) acc += hsum[w][lane];
        const bool ok = lane < h.x;
        cv = ok ? vn[lane] * acc : 0.f;
        a.contrib[(((size_t)b * hkv + kvh) * a.ucap + u) * kSlot + lane] = ok ? cv : -1.0f;
      }
      const float us = sum32(cv);
      if (lane == 0) a.unit_contrib[((size_t)b * hkv + kvh) * a.ucap + u] = us;
    }
  }
  if (MODE == 0) {
    // merge the two halves (the same query's two token sets) and write the partials
    const auto pm = __builtin_amdgcn_permlane32_swap(__float_as_uint(m_run), __float_as_uint(m_run), false, false);
    const auto pl = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run), __float_as_uint(l_run), false, false);
    const float m0 = __uint_as_float(pm[0]), m1 = __uint_as_float(pm[1]);
    const float l0 = __uint_as_float(pl[0]), l1 = __uint_as_float(pl[1]);
    const float M = fmaxf(m0, m1);
    float L = 0.f;
    if (m0 > -__builtin_inff()) L += l0 * __builtin_amdgcn_exp2f(m0 - M);
    if (m1 > -__builtin_inff()) L += l1 * __builtin_amdgcn_exp2f(m1 - M);
    if (head && hh == 0) {
      float* pp = a.partial + (((pbase + split) * kMaxHeads + ci) * 2) * kSlot + j;
      pp[0] = M;
      pp[kSlot] = L;
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
  constexpr int kTopkWaves = kTopkThreads / 64;
  __shared__ uint32_t hist[kTopkWaves][256];   // per-wave histograms: same-digit keys do not all contend for one word
  __shared__ uint32_t scan[kTopkThreads];
  __shared__ uint32_t sh[4];   // prefix, remaining, candidates
  const int kvh = blockIdx.x, b = blockIdx.y, tid = threadIdx.x, wave = tid >> 6;
  const int nu = a.nunits[b];
  const size_t pair = (size_t)b * a.hkv + kvh;
  const float* c = a.contrib + pair * a.ucap * kSlot;
  const bool units = a.granularity == kSlot;
  // candidates: entries, or whole units ranked by their sums
  const float* key_src = units ? a.unit_contrib + pair * a.ucap : c;
  const int N = units ? nu : nu * kSlot;
  uint32_t* mask_out = a.sel_mask + pair * a.ucap;
  int32_t* units_out = a.sel_units + pair * a.ucap;

  if (tid == 0) sh[2] = 0;
  __syncthreads();
  uint32_t nv = 0;
  for (int i = tid; i < N; i += kTopkThreads) nv += entry_key(key_src[i]) != 0u;
  atomicAdd(&sh[2], nv);
  __syncthreads();
  const uint32_t k = min((uint32_t)max(a.budget, 0), sh[2]);
  // radix select of the k-th largest key, most significant digit first
  uint32_t prefix = 0, pmask = 0, remaining = k;
  if (k > 0) {
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int i = tid; i < kTopkWaves * 256; i += kTopkThreads) (&hist[0][0])[i] = 0;
      __syncthreads();
      for (int i = tid; i < N; i += kTopkThreads) {
        const uint32_t key = entry_key(key_src[i]);
        if ((key & pmask) == prefix) atomicAdd(&hist[wave][(key >> shift) & 255u], 1u);
      }
      __syncthreads();
      // counts per digit, then suffix sums (digits above d) by a log-step scan
      // over 256 threads; the digit d with above(d) < remaining <= above(d) +
      // count(d) holds the k-th key
      uint32_t cnt = 0;
      if (tid < 256) {
        for (int w = 0; w < kTopkWaves; ++w) cnt += hist[w][tid];
        scan[tid] = cnt;
      }
      __syncthreads();
      for (int off = 1; off < 256; off <<= 1) {
        const uint32_t add = (tid < 256 && tid + off < 256) ? scan[tid + off] : 0u;
        __syncthreads();
        if (tid < 256) scan[tid] += add;
        __syncthreads();
      }
      if (tid < 256) {
        const uint32_t incl = scan[tid], above = incl - cnt;
        if (above < remaining && remaining <= incl) {
          sh[0] = prefix | ((uint32_t)tid << shift);
          sh[1] = remaining - above;
        }
      }
      __syncthreads();
      prefix = sh[0];
      remaining = sh[1];
      pmask |= 255u << shift;
      __syncthreads();
    }
  }
  const uint32_t T = prefix, need = remaining;   // keys > T, and the first `need` keys == T
  // units [tid*UPT, (tid+1)*UPT): ties ranked in entry (or unit) order
  const int UPT = (nu + kTopkThreads - 1) / kTopkThreads;
  const int ub = tid * UPT, ue = min(nu, ub + UPT);
  uint32_t ties = 0;
  if (k > 0) {
    if (units) {
      for (int u = ub; u < ue; ++u) ties += entry_key(key_src[u]) == T;
    } else {
      for (int i = ub * kSlot; i < ue * kSlot; ++i) ties += entry_key(c[i]) == T;
    }
  }
  uint32_t tot;
  uint32_t rank = block_scan(ties, scan, &tot);
  uint32_t nonzero = 0;
  for (int u = ub; u < ue; ++u) {
    uint32_t m = 0;
    if (k > 0) {
      if (units) {
        const uint32_t key = entry_key(key_src[u]);
        bool s = key > T;
        if (key == T) { s = rank < need; ++rank; }
        if (s)
          for (int t = 0; t < kSlot; ++t) m |= (c[u * kSlot + t] >= 0.f ? 1u : 0u) << t;
      } else {
        for (int t = 0; t < kSlot; ++t) {
          const uint32_t key = entry_key(c[u * kSlot + t]);
          bool s = key > T;
          if (key == T) { s = rank < need; ++rank; }
          m |= (s ? 1u : 0u) << t;
        }
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
