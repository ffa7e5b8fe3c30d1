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
// into the same operands as the attention kernel -- an fp16 hi tile and an
// e5m2 lo tile of 2^12 (x - hi) -- and wave w runs S^T = K Q^T for query head w
// of the group: hi on v_mfma_f32_32x32x16_f16, lo against an e4m3 copy of Q on
// the scaled fp8 MFMA (E8M0 scale 2^-12 on the lo side).  The scores then
// carry the keys to about 2^-14 of their size, as in attention, so the ranking
// follows the exact contributions closely.  The workgroup barriers order LDS
// only (a plain workgroup barrier would also wait for the prefetch loads in
// flight).
//
// topk_kernel then selects, per (sequence, kv head), the k largest
// contributions exactly (ties to the lower entry) by a four-digit radix select
// on the float bits, and writes a token mask per unit and the list of units
// that hold a selected token.
#include "device_common.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kWaves = 8;                 // consumer waves: one query head per wave
constexpr int kProd = 4;                  // producer waves (one per SIMD)
constexpr int kPThreads = 64 * kProd;
constexpr int kThreads = 64 * (kProd + kWaves);
constexpr int kMaxHeads = kSelHeads;   // query heads per kv head

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
__global__ __launch_bounds__(kThreads, 1) void sel_kernel(const SelArgs a) {
  constexpr int KS = D / 16;
  constexpr int NPAIR = kSlot * (D / 8);                 // (token, 8-channel group) pairs of a unit
  constexpr int PPT = NPAIR / kPThreads;                 // pairs per producer thread
  static_assert(PPT >= 1 && PPT * kPThreads == NPAIR, "pairs per producer thread");
  constexpr int RPT = (48 * D / 16 + kPThreads - 1) / kPThreads;   // 16-byte record chunks per producer thread
  constexpr int VLANES = kPThreads / kSlot;              // producer threads per token for the value norms
  constexpr int VCH = D / VLANES;                        // channels per thread
  static_assert(VLANES == 8 && VCH % 4 == 0, "value-norm mapping");
  constexpr uint32_t KC = kc_bytes(D, KB), VC = vc_bytes(D, VB), KM = kmeta_bytes(D);
  static_assert(record_bytes(D, KB, VB, 32) <= 48 * D, "record fits the stage");
  // double-buffered by unit parity: unit u's record and protected chunks are
  // staged in [u & 1], its key operand tiles in [u & 1]
  __shared__ __align__(16) uint8_t rec[2][48 * D];
  __shared__ __align__(16) half8 kt[2][KS][64];
  // key lo tiles (e5m2): byte j of lane l of 64-channel block k holds channel
  // 64k + 32(l/32) + j of token l%32 (the attention kernel's layout)
  __shared__ __align__(16) uint4 klt[2][D / 64][2][64];
  __shared__ __align__(16) uint4 prt[2][PPT][kPThreads];  // each producer thread's protected key chunks
  __shared__ float vn[3][kSlot];                         // MODE 1: value norms, by unit % 3
  __shared__ __align__(16) int4 hdrs[kMaxSelSplit];    // the split's unit headers
  __shared__ float hsum[2][kWaves][kSlot];               // MODE 1: per head, P summed over the mask queries
  __shared__ __align__(16) float mq[kWaves][kSlot];      // MODE 1: per head and query, the maximum
  __shared__ __align__(16) float lq[kWaves][kSlot];      // and the weight 1/sum (0 outside the mask)

  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int np = a.nslots[0][b], ns = a.use_suffix ? a.nslots[1][b] : 0;
  const int NC = np + ns;                          // cached units
  const int U = NC + (MODE == 0 ? 1 : 0);          // the stats also cover the block
  const int nsplit = (U + a.split_units - 1) / a.split_units;
  if (split >= nsplit) return;
  const int u0 = split * a.split_units, u1 = min(U, u0 + a.split_units);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool producer = wave < kProd;
  const int hkv = a.hkv, r = a.r;
  const int j = lane & 31, hh = lane >> 5;
  const SegPtrs seg0 = a.seg[0], seg1 = a.seg[1];

  // the split's headers, read once: a unit's protected-row loads depend on its
  // header, and a global read of it per unit would stall the prefetch
  for (int i = tid; i < min(u1, NC) - u0; i += kThreads) {
    const int u = u0 + i;
    const bool s1 = u >= np;
    const int sl = s1 ? u - np : u;
    const int cap = s1 ? seg1.slot_cap : seg0.slot_cap;
    hdrs[i] = *reinterpret_cast<const int4*>((s1 ? seg1.headers : seg0.headers) + ((size_t)b * cap + sl) * kHeaderBytes);
  }

  const int writer_wave = r < kWaves ? kProd + r : kProd - 1;
  const bool writer = MODE == 1 && wave == writer_wave;
  // MODE 1, the writer wave: entry contributions of unit u (lanes 0..31)
  // and the unit's sum over its valid entries (a butterfly over those lanes).
  // The writer is the consumer wave left without a query head when r < 8
  // (it has no MFMA work), else the last producer wave.  The heads' sums are
  // read all at once (independent LDS reads) and the unused ones dropped.
  auto contribute = [&](int u) __attribute__((always_inline)) {
    const int4 h = hdrs[u - u0];
    float cv = 0.f;
    if (lane < kSlot) {
      float hs[kWaves];
#pragma unroll
      for (int w = 0; w < kWaves; ++w) hs[w] = hsum[u & 1][w][lane];
      float acc = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) acc += w < r ? hs[w] : 0.f;
      const bool ok = lane < h.x;
      cv = ok ? vn[u % 3][lane] * acc : 0.f;
      a.contrib[(((size_t)b * hkv + kvh) * a.ucap + u) * kSlot + lane] = ok ? cv : -1.0f;
    }
    const float us = sum32(cv);
    if (lane == 0) a.unit_contrib[((size_t)b * hkv + kvh) * a.ucap + u] = us;
  };

  // Pipeline, one barrier per unit.  In interval u the consumer waves (one per
  // query head) score unit u from the operand tiles kt[u & 1] while the
  // producer waves dequantize unit u + 1 into the other tiles (and, MODE 1,
  // compute its value norms), stage unit u + 2's record from the registers its
  // loads arrived in, issue the loads of unit u + 4, and write unit u - 1's
  // contributions.  Prologue: the headers, then units u0 and u0 + 1 staged,
  // then unit u0 dequantized (three barriers on both sides).
  if (producer) {
    const int ptid = tid;                          // 0 .. kPThreads - 1
    const uint32_t rbytes = a.record_bytes;
    const float neg_one = opaque_neg_one();
    // the block's keys (the stats pass's last split), read before the loop:
    // a global load inside it would make every unit wait for the prefetch
    // loads issued before it
    float xblk[PPT][8];
#pragma unroll
    for (int q = 0; q < PPT; ++q)
#pragma unroll
      for (int e = 0; e < 8; ++e) xblk[q][e] = 0.f;
    if (MODE == 0 && u1 > NC) {
#pragma unroll
      for (int q = 0; q < PPT; ++q) {
        const int p = ptid + kPThreads * q, t = p % kSlot, cg = p / kSlot;
        load8(a.k_blk, (((size_t)b * kSlot + t) * hkv + kvh) * D + 8 * cg, a.blk_f32, xblk[q]);
      }
    }
    struct Pre { uint4 rc[RPT]; uint4 pc[PPT]; };
    Pre pre[2];
    // buffer loads: a unit past the split (or the block) gets empty
    // resources, so its loads return zeros without memory traffic
    auto load = [&](int u, Pre& pr) __attribute__((always_inline)) {
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
#pragma unroll
      for (int q = 0; q < RPT; ++q)
        pr.rc[q] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rr, (q * kPThreads + ptid) * 16, 0, 0));
#pragma unroll
      for (int q = 0; q < PPT; ++q) {
        const int p = ptid + kPThreads * q, t = p % kSlot, cg = p / kSlot;
        const int rank = hd.z + __popc((uint32_t)hd.y & ((1u << t) - 1u));
        const int off = ((hd.y >> t) & 1) ? (rank * D + 8 * cg) * 2 : 0x7ff00000;
        pr.pc[q] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(pr_, off, 0, 0));
      }
    };
    // Wait for this unit's loads only: the next unit's RPT + PPT loads (and,
    // for the wave writing contributions, its two stores of the last
    // interval, issued after them) stay in flight.  Stated once, before the
    // conditional stores, so that the compiler adds no wait of its own there.
    constexpr int kLoadsPerUnit = RPT + PPT;
    static_assert(kLoadsPerUnit + 2 < 16, "vmcnt field");
    auto stage = [&](int u, const Pre& pr) __attribute__((always_inline)) {
      if (writer) __builtin_amdgcn_s_waitcnt(0xF70 | (kLoadsPerUnit + 2));
      else        __builtin_amdgcn_s_waitcnt(0xF70 | kLoadsPerUnit);
      if (MODE == 0 && u == NC) return;
      uint8_t* rs = rec[u & 1];
#pragma unroll
      for (int q = 0; q < RPT; ++q) {
        const uint32_t off = (uint32_t)(q * kPThreads + ptid) * 16u;
        if (off < rbytes) *reinterpret_cast<uint4*>(rs + off) = pr.rc[q];
      }
#pragma unroll
      for (int q = 0; q < PPT; ++q) prt[u & 1][q][ptid] = pr.pc[q];
    };
    // keys of unit u -> fp16 hi / e5m2 lo operand tiles, one (token, channel
    // group) pair at a time
    // Branch-free: every LDS read of both pairs (code word, scales, zeros,
    // protected chunk) is issued before any arithmetic, so the pairs share one
    // LDS latency; a protected token then takes its bf16 row instead of the
    // dequantized codes.
    auto dequant = [&](int u) __attribute__((always_inline)) {
      const bool blk = MODE == 0 && u == NC;       // uniform
      const uint32_t pmask = blk ? 0u : (uint32_t)hdrs[u - u0].y;
      const uint8_t* rs = rec[u & 1];
      const uint32_t* words = reinterpret_cast<const uint32_t*>(rs);
      uint32_t cw[PPT];
      uint4 pw[PPT];
      float4 sc0[PPT], sc1[PPT], zr0[PPT], zr1[PPT];
#pragma unroll
      for (int q = 0; q < PPT; ++q) {
        const int p = ptid + kPThreads * q, t = p % kSlot, cg = p / kSlot;
        const float* km = reinterpret_cast<const float*>(rs + KC + VC) + 8 * cg;
        cw[q] = KB == 4 ? words[cg * 32 + t] : words[(cg >> 1) * 32 + t] >> (16 * (cg & 1));
        pw[q] = prt[u & 1][q][ptid];
        sc0[q] = *reinterpret_cast<const float4*>(km);
        sc1[q] = *reinterpret_cast<const float4*>(km + 4);
        zr0[q] = *reinterpret_cast<const float4*>(km + D);
        zr1[q] = *reinterpret_cast<const float4*>(km + D + 4);
      }
#pragma unroll
      for (int q = 0; q < PPT; ++q) {
        const int p = ptid + kPThreads * q, t = p % kSlot, cg = p / kSlot;
        const int khh = cg / (D / 16), kks = cg % (D / 16);
        float code[8], x[8];
        unpack8<KB>(cw[q], code);
        const float sc[8] = {sc0[q].x, sc0[q].y, sc0[q].z, sc0[q].w, sc1[q].x, sc1[q].y, sc1[q].z, sc1[q].w};
        const float zr[8] = {zr0[q].x, zr0[q].y, zr0[q].z, zr0[q].w, zr1[q].x, zr1[q].y, zr1[q].z, zr1[q].w};
        const uint4 w = pw[q];
        const float pr[8] = {bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y),
                             bf16_lo(w.z), bf16_hi(w.z), bf16_lo(w.w), bf16_hi(w.w)};
        const bool prot = (pmask >> t) & 1u;
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = blk ? xblk[q][e] : prot ? pr[e] : fmaf(code[e], sc[e], zr[e]);
        store_hi_lo8(kt[u & 1][kks][t + 32 * khh],
                     reinterpret_cast<uint2*>(&klt[u & 1][cg >> 3][(cg >> 1) & 1][t + 32 * ((cg >> 2) & 1)])[cg & 1], x,
                     neg_one);
      }
    };
    // MODE 1: value norms of unit u: token t, channels [cs * VCH, +VCH) of
    // one value group, summed over the token's VLANES adjacent lanes
    auto norms = [&](int u) __attribute__((always_inline)) {
      const uint8_t* rs = rec[u & 1];
      const int t = ptid / VLANES, cs = ptid % VLANES, c0 = cs * VCH;
      const int mm = t / 16, th = (t / 4) % 2, e = (t % 4) + 4 * ((t / 8) % 2);
      const int wj = VB == 4 ? 2 * mm + th : th;
      const int bit = VB == 4 ? 4 * e : 2 * (8 * mm + e);
      const float* vm = reinterpret_cast<const float*>(rs + KC + VC + KM + (c0 >> a.gv_log2) * 256);
      const float sc = vm[t], zr = vm[kSlot + t];
      const uint32_t* vw = reinterpret_cast<const uint32_t*>(rs + KC) + wj * D + c0;
      // sum over the lane's channels of (code * sc + zr)^2 = sc^2 S2 + 2 sc zr
      // S1 + VCH zr^2, with the code sums S1 and S2 exact in integers (one
      // bit-field extract, one add and one 24-bit multiply-add per code)
      uint32_t s1 = 0, s2 = 0;
#pragma unroll
      for (int cc = 0; cc < VCH; cc += 4) {
        const uint4 w4 = *reinterpret_cast<const uint4*>(vw + cc);
        const uint32_t w[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t cd = __builtin_amdgcn_ubfe(w[k], (uint32_t)bit, (uint32_t)VB);
          s1 += cd;
          s2 += cd * cd;
        }
      }
      float acc = fmaf(sc * sc, (float)s2, fmaf(2.0f * sc * zr, (float)s1, (float)VCH * zr * zr));
      acc = add_dpp<0xB1>(acc);    // quad_perm [1,0,3,2]
      acc = add_dpp<0x4E>(acc);    // quad_perm [2,3,0,1]
      acc = add_dpp<0x141>(acc);   // row_half_mirror: the 8 lanes of the token
      // (the sum of squares cannot be negative; rounding of the expanded form can make it so)
      if (cs == 0) vn[u % 3][t] = sqrtf(fmaxf(acc, 0.f));
    };
    lds_barrier();                                   // headers
    load(u0, pre[0]);
    load(u0 + 1, pre[1]);
    stage(u0, pre[0]);
    load(u0 + 2, pre[0]);
    stage(u0 + 1, pre[1]);
    load(u0 + 3, pre[1]);
    lds_barrier();                                   // units u0, u0 + 1 staged
    dequant(u0);
    if (MODE == 1) norms(u0);
    lds_barrier();                                   // unit u0's operands
    // pk holds the loads of unit u + 2 (the two register sets alternate, named
    // statically so that both stay in registers)
    auto interval = [&](int u, Pre& pk) __attribute__((always_inline)) {
      if (u + 1 < u1) {
        dequant(u + 1);
        if (MODE == 1) norms(u + 1);
      }
      if (u + 2 < u1) stage(u + 2, pk);
      load(u + 4, pk);
      if (writer && u > u0) contribute(u - 1);
      lds_barrier();
    };
    // whole pairs, so that the loop is re-entered only after the second set's
    // loads (the compiler then keeps the first set's wait at one unit's
    // loads), and an odd last unit
    int ub = u0;
    for (; ub + 1 < u1; ub += 2) {
      interval(ub, pre[0]);
      interval(ub + 1, pre[1]);
    }
    if (ub < u1) interval(ub, pre[0]);
    if (writer) contribute(u1 - 1);
    return;
  }

  // ---- consumer waves: query head kvh * r + ci
  const int ci = wave - kProd;
  const bool head = ci < r;
  const int cq = min(ci, r - 1);
  const float c2 = a.scale_log2;
  // Q operand of the wave's head (B operand of S^T: lane = query token j,
  // half hh holds channels (D/2)*hh + 8s + [0, 8) at k-step s), and its e4m3
  // copy for the lo product (block k holds channels 64k + 32*hh + [0, 32))
  constexpr int KB8 = D / 64;
  half8 qop[KS];
  v8i_t q8[KB8];
  {
    const size_t row = (((size_t)b * kSlot + j) * a.hq + kvh * r + cq) * D;
    const size_t base = row + (D / 2) * hh;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      float x[8];
      load8(a.q, base + 8 * s, a.q_f32, x);
      qop[s] = to_half8(x);
    }
#pragma unroll
    for (int k = 0; k < KB8; ++k) {
#pragma unroll
      for (int w8 = 0; w8 < 4; ++w8) {
        float x[8];
        load8(a.q, row + 64 * k + 32 * hh + 8 * w8, a.q_f32, x);
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          uint32_t d = __builtin_amdgcn_cvt_pk_fp8_f32(x[4 * h2], x[4 * h2 + 1], 0u, false);
          d = __builtin_amdgcn_cvt_pk_fp8_f32(x[4 * h2 + 2], x[4 * h2 + 3], d, true);
          q8[k][2 * w8 + h2] = (int)d;
        }
      }
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
        const float* pp = a.partial + (((pbase + min(sp0 + q, nstat - 1)) * kMaxHeads + cq) * 2) * kSlot + j;
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
      mq[ci][j] = M;
      lq[ci][j] = ((a.qmask[b] >> j) & 1u) ? 1.0f / L : 0.f;
    }
  }
  lds_barrier();                                     // headers
  lds_barrier();                                     // units u0, u0 + 1 staged
  lds_barrier();                                     // unit u0's operands
  for (int u = u0; u < u1; ++u) {
    const int4 h = (MODE == 0 && u == NC) ? make_int4(kSlot, 0, 0, 0) : hdrs[u - u0];
    if (head) {
      floatx16 sacc;
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[i] = 0.f;
      // MODE 0: S^T = K Q^T, sacc[i] = S[query j][token 8*(i/4) + 4*hh + i%4];
      // MODE 1: S = Q K^T (the same operand registers, swapped),
      // sacc[i] = S[query 8*(i/4) + 4*hh + i%4][token j]
#pragma unroll
      for (int s = 0; s < KS; ++s)
        sacc = MODE == 0 ? __builtin_amdgcn_mfma_f32_32x32x16_f16(kt[u & 1][s][lane], qop[s], sacc, 0, 0, 0)
                         : __builtin_amdgcn_mfma_f32_32x32x16_f16(qop[s], kt[u & 1][s][lane], sacc, 0, 0, 0);
      // + 2^-12 K_lo' Q8^T (bf8 x e4m3; the E8M0 scale 2^-12 on the lo side)
#pragma unroll
      for (int kk = 0; kk < KB8; ++kk) {
        const uint4 l0 = klt[u & 1][kk][0][lane], l1 = klt[u & 1][kk][1][lane];
        const v8i_t kl = v8i_t{(int)l0.x, (int)l0.y, (int)l0.z, (int)l0.w, (int)l1.x, (int)l1.y, (int)l1.z, (int)l1.w};
        sacc = MODE == 0 ? __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kl, q8[kk], sacc, 1, 0, 0, 127 - 12, 0, 127)
                         : __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(q8[kk], kl, sacc, 0, 1, 0, 127, 0, 127 - 12);
      }
      if (MODE == 0) {
        float mx = -__builtin_inff();
#pragma unroll
        for (int i = 0; i < 16; ++i) {   // scaled scores in place
          const int tok = 8 * (i >> 2) + 4 * hh + (i & 3);
          sacc[i] = tok < h.x ? sacc[i] * c2 : -__builtin_inff();
          mx = fmaxf(mx, sacc[i]);
        }
        const float mn = fmaxf(m_run, mx);
        if (mn > -__builtin_inff()) {
          float l = l_run * __builtin_amdgcn_exp2f(m_run - mn);
#pragma unroll
          for (int i = 0; i < 16; ++i) l += __builtin_amdgcn_exp2f(sacc[i] - mn);
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
        if (hh == 0) hsum[u & 1][ci][j] = __uint_as_float(ps[0]) + __uint_as_float(ps[1]);
      }
    }
    if (writer && u > u0) contribute(u - 1);
    lds_barrier();
  }
  if (writer) contribute(u1 - 1);
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
constexpr int kTopkLdsKeys = 32 * 1024;   // keys kept in LDS (128 KB); more are re-read from memory
constexpr int kTopkSmallN = 512;          // up to this many keys, ranks are counted directly

__device__ __forceinline__ uint32_t entry_key(float c) {
  return c >= 0.f ? __float_as_uint(c) + 1u : 0u;   // valid entries above every invalid one
}

// inclusive prefix sum over the 64 lanes of a wave (lane i gets the sum of
// lanes 0..i), by six shuffle-and-add steps
__device__ __forceinline__ uint32_t wave_scan(uint32_t v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t u = (uint32_t)__shfl_up((int)v, off, 64);
    v += lane >= off ? u : 0u;
  }
  return v;
}

// exclusive prefix sum over the workgroup (wave scans, then a scan of the
// wave totals by wave 0); returns the total in *total.  buf holds at least
// kTopkThreads / 64 + 1 words.
__device__ uint32_t block_scan(uint32_t v, uint32_t* buf, uint32_t* total) {
  constexpr int kW = kTopkThreads / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint32_t incl = wave_scan(v);
  if (lane == 63) buf[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    const uint32_t t = lane < kW ? buf[lane] : 0u;
    const uint32_t ti = wave_scan(t);
    if (lane < kW) buf[lane] = ti - t;      // exclusive offset of wave `lane`
    if (lane == kW - 1) buf[kW] = ti;       // the total
  }
  __syncthreads();
  const uint32_t r = buf[wave] + incl - v;
  *total = buf[kW];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(kTopkThreads) void topk_kernel(const TopkArgs a) {
  constexpr int kTopkWaves = kTopkThreads / 64;
  __shared__ uint32_t hist[kTopkWaves][256];   // per-wave histograms: same-digit keys do not all contend for one word
  __shared__ uint32_t scan[kTopkThreads];
  __shared__ uint32_t sh[5];   // prefix and remaining of even and odd radix passes, then the valid count
  __shared__ __align__(16) uint32_t keys[kTopkLdsKeys];
  __shared__ uint8_t selb[kTopkSmallN];        // few keys: selected or not
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

  // the keys, read from global memory once: in LDS when they fit, so the four
  // radix passes and the tie pass do not each pay a memory latency
  const bool in_lds = N <= kTopkLdsKeys;
  auto key_at = [&](int i) __attribute__((always_inline)) {
    return in_lds ? keys[i] : entry_key(key_src[i]);
  };
  if (tid == 0) sh[4] = 0;
  uint32_t nv = 0;
  for (int i = tid; i < N; i += kTopkThreads) {
    const uint32_t key = entry_key(key_src[i]);
    if (in_lds) keys[i] = key;
    nv += key != 0u;
  }
  nv = wave_scan(nv);          // the wave's count in lane 63: one LDS atomic per wave
  __syncthreads();
  if ((tid & 63) == 63) atomicAdd(&sh[4], nv);
  __syncthreads();
  const uint32_t k = min((uint32_t)max(a.budget, 0), sh[4]);
  // Few keys (unit granularity): each key's rank counted against every other
  // key in LDS (broadcast reads), kept when the rank is below k.  Otherwise a
  // radix select of the k-th largest key, most significant digit first.
  // (The keys are read four at a time, sixteen per iteration, and past N the
  // array holds zeros, which rank below every valid key.)
  const bool small = in_lds && N <= kTopkSmallN;
  if (small) {
    for (int i = N + tid; i < ((N + 15) & ~15); i += kTopkThreads) keys[i] = 0u;
    __syncthreads();
    for (int i = tid; i < N; i += kTopkThreads) {
      const uint32_t ki = keys[i];
      uint32_t rk = 0;
      for (int q0 = 0; q0 < N; q0 += 16) {
        uint4 kv[4];
#pragma unroll
        for (int g = 0; g < 4; ++g) kv[g] = *reinterpret_cast<const uint4*>(&keys[q0 + 4 * g]);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const uint32_t kq[4] = {kv[g].x, kv[g].y, kv[g].z, kv[g].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int q = q0 + 4 * g + e;
            rk += (kq[e] > ki || (kq[e] == ki && q < i)) ? 1u : 0u;
          }
        }
      }
      selb[i] = (ki != 0u && rk < k) ? 1 : 0;
    }
    __syncthreads();
  }
  uint32_t prefix = 0, pmask = 0, remaining = k;
  if (k > 0 && !small) {
    // Two barriers per pass: each wave clears and fills its own histogram (in
    // order, so without a barrier between), and the passes alternate between
    // two result slots, so that a pass's search never overwrites the slot
    // the previous pass's result is still read from.
    for (int shift = 24; shift >= 0; shift -= 8) {
      const int slot = (shift >> 2) & 2;        // 24, 8 -> 2; 16, 0 -> 0
#pragma unroll
      for (int i = 0; i < 4; ++i) hist[wave][(tid & 63) + 64 * i] = 0;
      for (int i = tid; i < N; i += kTopkThreads) {
        const uint32_t key = key_at(i);
        if ((key & pmask) == prefix) atomicAdd(&hist[wave][(key >> shift) & 255u], 1u);
      }
      __syncthreads();
      // counts per digit, then, in wave 0 (lane l holds digits 255 - 4l ..
      // 252 - 4l, highest first), the counts of the digits above each one; the
      // digit d with above(d) < remaining <= above(d) + count(d) holds the
      // k-th key
      if (wave == 0) {
        uint32_t cnt[4], sum = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int d = 255 - 4 * (tid & 63) - e;
          cnt[e] = 0;
          for (int w = 0; w < kTopkWaves; ++w) cnt[e] += hist[w][d];
          sum += cnt[e];
        }
        uint32_t above = wave_scan(sum) - sum;   // counts of the lanes holding higher digits
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int d = 255 - 4 * (tid & 63) - e;
          if (above < remaining && remaining <= above + cnt[e]) {
            sh[slot] = prefix | ((uint32_t)d << shift);
            sh[slot + 1] = remaining - above;
          }
          above += cnt[e];
        }
      }
      __syncthreads();
      prefix = sh[slot];
      remaining = sh[slot + 1];
      pmask |= 255u << shift;
    }
  }
  const uint32_t T = prefix, need = remaining;   // keys > T, and the first `need` keys == T
  // units [tid*UPT, (tid+1)*UPT): ties ranked in entry (or unit) order
  const int UPT = (nu + kTopkThreads - 1) / kTopkThreads;
  const int ub = tid * UPT, ue = min(nu, ub + UPT);
  uint32_t ties = 0;
  if (k > 0 && !small) {
    if (units) {
      for (int u = ub; u < ue; ++u) ties += key_at(u) == T;
    } else {
      for (int i = ub * kSlot; i < ue * kSlot; ++i) ties += key_at(i) == T;
    }
  }
  uint32_t tot;
  // (the direct ranking leaves no ties to order: no scan)
  uint32_t rank = (k > 0 && !small) ? block_scan(ties, scan, &tot) : 0u;
  // each thread's masks, for its unit-list pass: in LDS (the histograms are
  // no longer read) when they fit, else read back from memory
  uint32_t* mlds = &hist[0][0];
  const bool m_in_lds = nu <= kTopkWaves * 256;
  uint32_t nonzero = 0;
  for (int u = ub; u < ue; ++u) {
    uint32_t m = 0;
    if (k > 0) {
      if (units) {
        bool s;
        if (small) {
          s = selb[u] != 0;
        } else {
          const uint32_t key = key_at(u);
          s = key > T;
          if (key == T) { s = rank < need; ++rank; }
        }
        if (s) {
          // the unit's valid tokens (contribution >= 0), eight 16-byte loads
          const float4* c4 = reinterpret_cast<const float4*>(c + (size_t)u * kSlot);
          float4 cv[kSlot / 4];
#pragma unroll
          for (int g = 0; g < kSlot / 4; ++g) cv[g] = c4[g];
#pragma unroll
          for (int g = 0; g < kSlot / 4; ++g)
            m |= ((cv[g].x >= 0.f ? 1u : 0u) | (cv[g].y >= 0.f ? 2u : 0u) | (cv[g].z >= 0.f ? 4u : 0u) |
                  (cv[g].w >= 0.f ? 8u : 0u)) << (4 * g);
        }
      } else {
        for (int t = 0; t < kSlot; ++t) {
          bool s;
          if (small) {
            s = selb[u * kSlot + t] != 0;
          } else {
            const uint32_t key = key_at(u * kSlot + t);
            s = key > T;
            if (key == T) { s = rank < need; ++rank; }
          }
          m |= (s ? 1u : 0u) << t;
        }
      }
    }
    mask_out[u] = m;
    if (m_in_lds) mlds[u] = m;
    nonzero += m != 0u;
  }
  uint32_t pos = block_scan(nonzero, scan, &tot);
  for (int u = ub; u < ue; ++u)
    if ((m_in_lds ? mlds[u] : mask_out[u]) != 0u) units_out[pos++] = u;
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
