// Quantizer of one 32-token slot of one kv head, shared by the persistent
// commit kernel (commit.hip) and by the attention kernel's fused commit of the
// current block (attn.hip).
//
// A committed block's keys and values are quantized once, when the block is
// committed; keys KIVI-style per channel over a 32-token group, values per
// token over G_v channels; chosen key rows stay in bf16 and are left out of
// their group's statistics (Tai et al., "KV Cache Quantization for Diffusion
// Language Models", abstract; SoloQ summary page, block-diffusion paragraph).
//
// Four waves (256 threads) quantize one slot: waves 0 and 1 the keys of one
// half of the channels each (a key group spans the 32 tokens of one channel,
// so the halves are independent), waves 2 and 3 the values of one half of the
// tokens each (a value group spans channels of one token).  Each lane holds
// 16-byte pieces of token rows.
//
// Every step is shaped to cost few vector instructions per element:
//   - group minima and maxima: in-lane min3/max3, then, for values, DPP steps
//     between the lanes of a group, and for keys a transposed exchange through
//     LDS that leaves each lane with the 8 or 16 partial results of one channel;
//   - one lane per group computes the group's scale with an IEEE division and
//     publishes scale, zero and a reciprocal through LDS;
//   - per element: subtract, multiply by the reciprocal, round, and a
//     distance-to-boundary test (below); key codes are packed with
//     v_cvt_pk_u8_f32, value codes with shift-or, and each lane writes its
//     part of the code words to the LDS record with plain stores (no atomics,
//     no clearing), so a slot needs one workgroup barrier.
// The record then leaves with coalesced 128-bit stores.
//
// Exactness: scale = (mx - mn) / (2^b - 1) uses IEEE division.  A code is
// rint(q) of the fp32 quotient q = fl((x - mn) / scale).  The quantizer forms
// y = fl(d * rcp(scale)) with v_rcp_f32 (1 ulp): for q < 16,
// |y - q| < 16 * 1.5 * 2^-23 + 2^-21 < 2^-18, so rint(y) equals rint(q) unless
// y lies within 2^-18 of a rounding boundary k + 1/2.  An element with
// |y - rint(y)| >= 1/2 - 2^-17 takes its code from an IEEE division instead
// (with bf16 inputs about 0.2% of elements do: exact ties are common), and a
// wave in which some group's scale lies outside [2^-100, 2^100] (where rcp
// would overflow or underflow) recomputes all its codes that way.  For members
// of a group d lies in [0, mx - mn], so y < LEV + 1/2 and rint(y) needs no
// clamp; elements that are not members (protected or padding tokens) are
// masked to code 0.  Codes are therefore identical to the plain definition.
// Every function body below turns floating-point contraction off: the
// quantizer must round exactly as written, whichever file includes it.
#pragma once

#include <type_traits>

#include "device_common.h"
#include "kvq_internal.h"

namespace kvq {
namespace slotq {

// min/max of three floats.  In IEEE mode a quiet-NaN operand is ignored, so
// elements left out of a group are set to NaN before the reduction.
__device__ __forceinline__ float vmin3(float a, float b, float c) {
  float r;
  asm("v_min3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ float vmax3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
// One DPP step of a min/max reduction over groups of consecutive lanes, in
// place on N minima and N maxima.  The leading s_nop covers the DPP read-after-
// write and exec-write hazards of whatever the compiler placed before the block.
#define KVQ_DMIN(i, C) "v_min_f32_dpp %" #i ", %" #i ", %" #i " " C " row_mask:0xf bank_mask:0xf\n\t"
#define KVQ_DMAX(i, C) "v_max_f32_dpp %" #i ", %" #i ", %" #i " " C " row_mask:0xf bank_mask:0xf\n\t"
template <int N>
struct DppMinMax;
template <>
struct DppMinMax<4> {
  template <int S>
  __device__ __forceinline__ static void step(float (&mn)[4], float (&mx)[4]) {
#define KVQ_STEP4(C)                                                                                    \
  asm("s_nop 4\n\t" KVQ_DMIN(0, C) KVQ_DMIN(1, C) KVQ_DMIN(2, C) KVQ_DMIN(3, C) KVQ_DMAX(4, C)          \
          KVQ_DMAX(5, C) KVQ_DMAX(6, C) KVQ_DMAX(7, C)                                                  \
      : "+v"(mn[0]), "+v"(mn[1]), "+v"(mn[2]), "+v"(mn[3]), "+v"(mx[0]), "+v"(mx[1]), "+v"(mx[2]),   \
        "+v"(mx[3]))
    if (S == 0) KVQ_STEP4("quad_perm:[1,0,3,2]");
    if (S == 1) KVQ_STEP4("quad_perm:[2,3,0,1]");
    if (S == 2) KVQ_STEP4("row_half_mirror");
    if (S == 3) KVQ_STEP4("row_mirror");
#undef KVQ_STEP4
  }
};
template <>
struct DppMinMax<2> {
  template <int S>
  __device__ __forceinline__ static void step(float (&mn)[2], float (&mx)[2]) {
#define KVQ_STEP2(C)                                                                  \
  asm("s_nop 4\n\t" KVQ_DMIN(0, C) KVQ_DMIN(1, C) KVQ_DMAX(2, C) KVQ_DMAX(3, C)       \
      : "+v"(mn[0]), "+v"(mn[1]), "+v"(mx[0]), "+v"(mx[1]))
    if (S == 0) KVQ_STEP2("quad_perm:[1,0,3,2]");
    if (S == 1) KVQ_STEP2("quad_perm:[2,3,0,1]");
    if (S == 2) KVQ_STEP2("row_half_mirror");
    if (S == 3) KVQ_STEP2("row_mirror");
#undef KVQ_STEP2
  }
};
#undef KVQ_DMIN
#undef KVQ_DMAX

// x | (x of lane i ^ 8 within each 16-lane row)
__device__ __forceinline__ uint32_t or_lane_xor8(uint32_t x) {
  uint32_t r;
  asm("s_nop 4\n\tv_or_b32_dpp %0, %1, %1 row_ror:8 row_mask:0xf bank_mask:0xf" : "=v"(r) : "v"(x));
  return r;
}

// Orders LDS traffic between the lanes of one wave (same-wave LDS accesses
// execute in order; this only keeps the compiler from moving them).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <typename T>
__device__ __forceinline__ T pick(bool c, T a, T b) { return c ? a : b; }

// scale and zero of a group from its minimum and maximum (NaN when the group
// has no member), and the reciprocal the fast path multiplies by
struct GroupParams {
  float scale, zero, rcp;
  bool bad;   // scale outside [2^-100, 2^100]: codes need the exact path
};
template <int B>
__device__ __forceinline__ GroupParams group_params(float mn, float mx, bool valid) {
#pragma clang fp contract(off)
  constexpr float LEV = (float)((1 << B) - 1);
  GroupParams p;
  const bool any = valid && mn <= mx;
  p.scale = any ? (mx - mn) / LEV + 0.0f : 0.0f;
  p.zero = any ? mn + 0.0f : 0.0f;
  p.bad = p.scale != 0.f && !(p.scale >= 0x1p-100f && p.scale <= 0x1p+100f);
  p.rcp = p.scale == 0.f ? 0.f : __builtin_amdgcn_rcpf(p.scale);
  return p;
}

// The plain definition, branch-free (the division is done for scale == 0 too,
// by 1, and its result dropped).
__device__ __forceinline__ float exact_code(float d, float scale, float lev) {
#pragma clang fp contract(off)
  const float q = fminf(fmaxf(rintf(d / (scale == 0.f ? 1.f : scale)), 0.f), lev);
  return scale == 0.f ? 0.f : q;
}

constexpr float kNearHalf = 0.5f - 0x1p-17f;

// fp16 metadata: scale and zero rounded to fp16 (nearest even), canonical +0,
// and the reciprocal of the rounded scale
__device__ __forceinline__ GroupParams to_h16(GroupParams p) {
#pragma clang fp contract(off)
  p.scale = (float)(_Float16)p.scale + 0.0f;
  p.zero = (float)(_Float16)p.zero + 0.0f;
  p.bad = p.scale != 0.f && !(p.scale >= 0x1p-100f && p.scale <= 0x1p+100f);
  p.rcp = p.scale == 0.f ? 0.f : __builtin_amdgcn_rcpf(p.scale);
  return p;
}

// x of lane (lane ^ M) within each 32-lane half (ds_swizzle, bit-mask mode)
template <int M>
__device__ __forceinline__ float swz_xor(float x) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x1F | (M << 10)));
}

}  // namespace slotq

// Where one slot's quantizer reads and writes: the commit's source rows and
// the destination segment.
struct SlotIO {
  const void* k;        // [B, n_max, Hkv, D]
  const void* v;
  SegPtrs seg;
  int32_t n_max;
  int32_t hkv;
  int32_t gv_log2;
  uint32_t record_bytes;
};

// The record format: FMT 0 integer codes with fp32 scale and zero; 1 MX FP4;
// 2 integer codes with fp16 scale and zero (codes against the rounded pair).
// ROT: values are K-RPBH-rotated before quantization (permutation and mix in
// the LDS arrays rperm / rmix, filled by the caller).
template <int KB, int VB, int D, bool F32IN, bool ROT, int FMT>
struct SlotQuant {
  static constexpr int HC = D / 2;              // channels per key wave
  static constexpr int NCGK = HC / 8;           // 8-channel groups per key wave
  static constexpr int NTQK = 64 / NCGK;        // key lanes along the token axis
  static constexpr int TPLK = kSlot / NTQK;     // tokens per key lane
  static constexpr int NCGV = D / 8;            // 8-channel groups of a value row
  static constexpr int NTQV = 64 / NCGV;        // value lanes along the token axis
  static constexpr int TPLV = (kSlot / 2) / NTQV;   // tokens per value lane
  static constexpr int TPL = TPLK > TPLV ? TPLK : TPLV;
  static constexpr int ES = F32IN ? 4 : 2;      // input element bytes
  static constexpr int PPR = F32IN ? 2 : 1;     // 16-byte pieces per 8-channel row piece
  static constexpr uint32_t KC = kc_bytes(D, KB);
  static constexpr uint32_t VC = vc_bytes(D, VB);
  static constexpr bool MX = FMT == 1, H16 = FMT == 2;
  // MX FP4 records: one scale byte per key channel and per (value group, token);
  // fp16 metadata: half the bytes of fp32 scales and zeros
  static constexpr uint32_t KM = MX ? D : H16 ? kmeta_bytes(D) / 2 : kmeta_bytes(D);
  static constexpr uint32_t REC_MAX = MX ? (KC + VC + 2 * D + 255) / 256 * 256
                                         : H16 ? (KC + VC + KM + (D / 32) * 128 + 255) / 256 * 256
                                               : record_bytes(D, KB, VB, 32);
  static constexpr int TST = 9 * NTQK;          // padded row of the key statistics exchange
  static_assert(NTQK == 8 || NTQK == 16, "key lanes per channel group");
  static_assert(TPLK == 2 || TPLK == 4, "key tokens per lane");
  static_assert(TPLV == 2 || TPLV == 4, "value tokens per lane");
  static_assert(TPLK == TPLV, "key and value lanes hold the same number of rows");
  static constexpr int NST = (REC_MAX + 256 * 16 - 1) / (256 * 16);   // 16-byte record stores per thread

  // LDS of one slot in flight (the record itself is passed separately, so the
  // persistent kernel can alternate two)
  struct Lds {
    float kx[2][2][NCGK * TST];      // key partial min/max: [wave][min|max][cgl][channel][tq]
    float krcp[D];                   // key reciprocals per channel
    float vrcp[D / 32][kSlot];       // value reciprocals per (group, token)
    // fp16 metadata: the rounded scales and zeros as fp32 for the code step
    float kmf[H16 ? 2 * D : 4];
    float vmf[H16 ? D / 32 : 1][H16 ? 2 * kSlot : 4];
    // rotation only: the value rows of each value wave, the permutation and the mix
    float vrow[2][ROT ? kSlot / 2 : 1][ROT ? D : 4];
    int32_t rperm[ROT ? D : 4];
    float rmix[ROT ? 64 : 4];
  };

  // This lane's 16-byte pieces of its token rows.
  struct Raw { uint4 p[TPL][PPR]; };

  Lds& s;
  const SlotIO& io;
  int h;                // kv head of the item being processed (set by the caller)
  int tid, lane, wave;
  bool keys;
  int cg, tq, t0, nrows;
  const void* src;
  uint32_t raw_end;

  // lane geometry: a key lane holds tokens tq*TPLK + k of channel group cg
  // (the NTQK lanes of a channel group are consecutive); a value lane holds
  // tokens t0 + k of channel group cg (the lanes of a value group are consecutive)
  __device__ __forceinline__ SlotQuant(Lds& lds, const SlotIO& sio, int head, int thread)
      : s(lds), io(sio), h(head), tid(thread) {
    lane = tid & 63;
    wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    keys = wave < 2;
    cg = keys ? wave * NCGK + lane / NTQK : lane % NCGV;
    tq = keys ? lane % NTQK : lane / NCGV;
    t0 = keys ? tq * TPLK : (wave - 2) * (kSlot / 2) + tq * TPLV;
    nrows = keys ? TPLK : TPLV;
    src = keys ? io.k : io.v;
    raw_end = MX ? KC + VC + 2 * D : KC + VC + KM + (uint32_t)(D >> io.gv_log2) * (H16 ? 128u : 256u);
  }

  // the record bytes past the last field are zero (written once per buffer)
  __device__ __forceinline__ void clear_tail(uint8_t* rec) const {
    for (uint32_t off = raw_end + tid * 4; off < io.record_bytes; off += 256 * 4)
      *reinterpret_cast<uint32_t*>(rec + off) = 0u;
  }

  // This lane's row pieces of a task (buffer loads: rows past the task's valid
  // tokens, and a task that is not live, read as zeros without traffic).
  __device__ __forceinline__ void fetch(bool live, const CommitTask& task, Raw& raw) const {
    const uint8_t* base = static_cast<const uint8_t*>(src) +
                          (((size_t)task.b * io.n_max + task.src_tok) * io.hkv) * D * ES;
    const int nbytes = live ? task.nvalid * io.hkv * D * ES : 0;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, nbytes, 0x00020000);
#pragma unroll
    for (int k = 0; k < TPL; ++k)
#pragma unroll
      for (int j = 0; j < PPR; ++j) {
        const int off = k < nrows ? ((t0 + k) * io.hkv + h) * D * ES + 8 * cg * ES + 16 * j : 0x7ff00000;
        raw.p[k][j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
      }
  }

  __device__ __forceinline__ static void unpack_row(const Raw& raw, int k, float (&x)[8]) {
    if (F32IN) {
      const uint4 p0 = raw.p[k][0], p1 = raw.p[k][PPR - 1];
      x[0] = __uint_as_float(p0.x); x[1] = __uint_as_float(p0.y); x[2] = __uint_as_float(p0.z); x[3] = __uint_as_float(p0.w);
      x[4] = __uint_as_float(p1.x); x[5] = __uint_as_float(p1.y); x[6] = __uint_as_float(p1.z); x[7] = __uint_as_float(p1.w);
    } else {
      const uint4 w = raw.p[k][0];
      x[0] = bf16_lo(w.x); x[1] = bf16_hi(w.x); x[2] = bf16_lo(w.y); x[3] = bf16_hi(w.y);
      x[4] = bf16_lo(w.z); x[5] = bf16_hi(w.z); x[6] = bf16_lo(w.w); x[7] = bf16_hi(w.w);
    }
  }

  // ================= keys: protected rows go to the bf16 store as they are
  __device__ __forceinline__ void store_protected(const CommitTask& task, const float (&x)[TPL][8]) const {
#pragma unroll
    for (int k = 0; k < TPLK; ++k) {
      const int t = t0 + k;
      if (t < task.nvalid && ((task.mask >> t) & 1u)) {
        const int rank = task.rank_base + __popc(task.mask & ((1u << t) - 1u));
        uint4 w;
        w.x = f32_to_bf16_bits(x[k][0]) | (f32_to_bf16_bits(x[k][1]) << 16);
        w.y = f32_to_bf16_bits(x[k][2]) | (f32_to_bf16_bits(x[k][3]) << 16);
        w.z = f32_to_bf16_bits(x[k][4]) | (f32_to_bf16_bits(x[k][5]) << 16);
        w.w = f32_to_bf16_bits(x[k][6]) | (f32_to_bf16_bits(x[k][7]) << 16);
        const size_t prow = ((size_t)task.b * io.hkv + h) * io.seg.prot_cap + rank;
        *reinterpret_cast<uint4*>(io.seg.prot_rows + prow * D + 8 * cg) = w;
        if (h == 0 && cg == 0) io.seg.prot_pos[(size_t)task.b * io.seg.prot_cap + rank] = task.token_base + t;
      }
    }
  }

  // Code of one element: y = d * rcp rounded, or the exact division when y
  // lies near a rounding boundary (rare; the branch is skipped when no lane
  // of the wave needs it).
  __device__ __forceinline__ static float code_of(float d, float rcp, float scale, float lev) {
#pragma clang fp contract(off)
    const float y = d * rcp;
    float r = rintf(y);
    if (fabsf(y - r) >= slotq::kNearHalf) r = slotq::exact_code(d, scale, lev);
    return r;
  }

  // ================= keys: channels [wave*D/2, +D/2), groups along the 32 tokens
  __device__ __forceinline__ void process_keys(const CommitTask& task, float (&x)[TPL][8], uint8_t* rec) const {
#pragma clang fp contract(off)
    using namespace slotq;
    constexpr float LEV = (float)((1 << KB) - 1);
    uint32_t member = 0;
#pragma unroll
    for (int k = 0; k < TPLK; ++k) {
      const int t = t0 + k;
      if (t < task.nvalid && !((task.mask >> t) & 1u)) member |= 1u << k;
    }
    if (task.mask != 0u || task.nvalid < kSlot) {
      // tokens outside the group take no part in its statistics or codes
#pragma unroll
      for (int k = 0; k < TPLK; ++k)
#pragma unroll
        for (int c = 0; c < 8; ++c) x[k][c] = ((member >> k) & 1u) ? x[k][c] : __builtin_nanf("");
    }
    // partial min/max over the lane's tokens, exchanged transposed through
    // LDS: lane (cgl, tq) then reduces channel tq % 8 of its channel group
    const int cgl = lane / NTQK;
    float* kmn = s.kx[wave][0] + cgl * TST;
    float* kmx = s.kx[wave][1] + cgl * TST;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const float mn = vmin3(x[0][c], x[1][c], x[TPLK - 1][c]);
      const float mx = vmax3(x[0][c], x[1][c], x[TPLK - 1][c]);
      kmn[c * NTQK + tq] = TPLK == 4 ? vmin3(mn, x[TPLK - 2][c], x[TPLK - 2][c]) : mn;
      kmx[c * NTQK + tq] = TPLK == 4 ? vmax3(mx, x[TPLK - 2][c], x[TPLK - 2][c]) : mx;
    }
    wave_lds_sync();
    const int ch = tq & 7;
    float gmn, gmx;
    {
      const float4* pn = reinterpret_cast<const float4*>(kmn + ch * NTQK);
      const float4* px = reinterpret_cast<const float4*>(kmx + ch * NTQK);
      float4 n = pn[0], m = px[0];
      gmn = vmin3(n.x, n.y, n.z); gmn = vmin3(gmn, n.w, n.w);
      gmx = vmax3(m.x, m.y, m.z); gmx = vmax3(gmx, m.w, m.w);
#pragma unroll
      for (int j = 1; j < NTQK / 4; ++j) {
        n = pn[j]; m = px[j];
        gmn = vmin3(gmn, n.x, n.y); gmn = vmin3(gmn, n.z, n.w);
        gmx = vmax3(gmx, m.x, m.y); gmx = vmax3(gmx, m.z, m.w);
      }
    }
    if constexpr (MX) {
      // MX FP4: one E8M0 byte per channel, s = max(E(amax) - 2, 0), codes
      // E2M1(x * 2^(127 - s)) by the hardware conversion (round to nearest
      // even, saturating at 6; the power-of-two scaling is exact)
      const bool any = gmn <= gmx;
      const float amax = any ? fmaxf(-gmn, gmx) : 0.f;
      const uint32_t eb = (__float_as_uint(amax) >> 23) & 0xFFu;
      const uint32_t sb = eb > 2u ? eb - 2u : 0u;
      if (tq < 8) {
        rec[KC + VC + 8 * cg + ch] = (uint8_t)sb;
        s.krcp[8 * cg + ch] = amax > 0.f ? __uint_as_float((254u - sb) << 23) : 0.f;
      }
      wave_lds_sync();
      float mul[8];
      {
        const float4 m0 = *reinterpret_cast<const float4*>(s.krcp + 8 * cg);
        const float4 m1 = *reinterpret_cast<const float4*>(s.krcp + 8 * cg + 4);
        mul[0] = m0.x; mul[1] = m0.y; mul[2] = m0.z; mul[3] = m0.w;
        mul[4] = m1.x; mul[5] = m1.y; mul[6] = m1.z; mul[7] = m1.w;
      }
      uint32_t zm = 0;   // channels of an all-zero group keep code 0 (also for -0 inputs)
#pragma unroll
      for (int c = 0; c < 8; ++c) zm |= (mul[c] != 0.f ? 0xFu : 0u) << (4 * c);
      uint32_t word[TPLK];
#pragma unroll
      for (int k = 0; k < TPLK; ++k) {
        uint32_t w = 0;   // byte j: channels 2j (low nibble) and 2j + 1
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[k][0] * mul[0], x[k][1] * mul[1], 1.0f, 0);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[k][2] * mul[2], x[k][3] * mul[3], 1.0f, 1);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[k][4] * mul[4], x[k][5] * mul[5], 1.0f, 2);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[k][6] * mul[6], x[k][7] * mul[7], 1.0f, 3);
        word[k] = ((member >> k) & 1u) ? (w & zm) : 0u;
      }
      if (TPLK == 4) *reinterpret_cast<uint4*>(rec + (cg * 32 + t0) * 4) = make_uint4(word[0], word[1], word[TPLK - 2], word[TPLK - 1]);
      else           *reinterpret_cast<uint2*>(rec + (cg * 32 + t0) * 4) = make_uint2(word[0], word[TPLK - 1]);
    } else {
      const GroupParams gp = H16 ? to_h16(group_params<KB>(gmn, gmx, true)) : group_params<KB>(gmn, gmx, true);
      float* kscale = H16 ? s.kmf : reinterpret_cast<float*>(rec + KC + VC);
      if (tq < 8) {
        kscale[8 * cg + ch] = gp.scale;
        kscale[D + 8 * cg + ch] = gp.zero;
        s.krcp[8 * cg + ch] = gp.rcp;
        if constexpr (H16) {
          _Float16* k16 = reinterpret_cast<_Float16*>(rec + KC + VC);
          k16[8 * cg + ch] = (_Float16)gp.scale;
          k16[D + 8 * cg + ch] = (_Float16)gp.zero;
        }
      }
      wave_lds_sync();
      // scales stay in LDS: only the rare exact path reads them
      float zero[8], rcp[8];
      {
        const float4 z0 = *reinterpret_cast<const float4*>(kscale + D + 8 * cg);
        const float4 z1 = *reinterpret_cast<const float4*>(kscale + D + 8 * cg + 4);
        const float4 r0 = *reinterpret_cast<const float4*>(s.krcp + 8 * cg);
        const float4 r1 = *reinterpret_cast<const float4*>(s.krcp + 8 * cg + 4);
        zero[0] = z0.x; zero[1] = z0.y; zero[2] = z0.z; zero[3] = z0.w;
        zero[4] = z1.x; zero[5] = z1.y; zero[6] = z1.z; zero[7] = z1.w;
        rcp[0] = r0.x; rcp[1] = r0.y; rcp[2] = r0.z; rcp[3] = r0.w;
        rcp[4] = r1.x; rcp[5] = r1.y; rcp[6] = r1.z; rcp[7] = r1.w;
      }
      // codes of token k: channel c in bits [KB*c, KB*c + KB) of its word
      uint32_t word[TPLK];
#pragma unroll
      for (int k = 0; k < TPLK; ++k) {
        uint32_t p[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          float rc = code_of(x[k][c] - zero[c], rcp[c], kscale[8 * cg + c], LEV);
          if constexpr (H16) rc = fminf(fmaxf(rc, 0.f), LEV);   // the rounded zero may lie above the minimum
          if (KB == 4) p[c & 1] = __builtin_amdgcn_cvt_pk_u8_f32(rc, c >> 1, p[c & 1]);
          else         p[c & 3] = __builtin_amdgcn_cvt_pk_u8_f32(rc, c >> 2, p[c & 3]);
        }
        const uint32_t w = KB == 4 ? (p[0] | (p[1] << 4)) : (p[0] | (p[1] << 2) | (p[2] << 4) | (p[3] << 6));
        word[k] = ((member >> k) & 1u) ? w : 0u;
      }
      if (__any(gp.bad)) {
#pragma unroll
        for (int k = 0; k < TPLK; ++k) {
          uint32_t w = 0;
#pragma unroll
          for (int c = 0; c < 8; ++c) {
            const float q = exact_code(x[k][c] - zero[c], kscale[8 * cg + c], LEV);
            w |= (uint32_t)q << (KB * c);
          }
          word[k] = ((member >> k) & 1u) ? w : 0u;
        }
      }
      // word-major: the word holding channel group cg of token t.  4-bit: the
      // lane's TPLK tokens are consecutive words, written at once (a wide write
      // also avoids the bank conflicts of lanes 32 words apart)
      if (KB == 4) {
        if (TPLK == 4) *reinterpret_cast<uint4*>(rec + (cg * 32 + t0) * 4) = make_uint4(word[0], word[1], word[TPLK - 2], word[TPLK - 1]);
        else           *reinterpret_cast<uint2*>(rec + (cg * 32 + t0) * 4) = make_uint2(word[0], word[TPLK - 1]);
      } else {
#pragma unroll
        for (int k = 0; k < TPLK; ++k)
          *reinterpret_cast<uint16_t*>(rec + ((cg >> 1) * 32 + t0 + k) * 4 + 2 * (cg & 1)) = (uint16_t)word[k];
      }
    }
  }

  // ================= values: K-RPBH rotation of the lane's rows (SoloQ summary
  // page, rotation paragraphs), in the fp32 order
  //   y = x[perm]; Hadamard stages h = 1, 2, ..., b/2, each pair (i, i + h)
  //   with i & h == 0 becoming (y_i + y_{i+h}, y_i - y_{i+h}); y <- y / sqrt(b);
  //   z[i*b + j] = sum over l = 0..k-1 in order of mix[i][l] * y[l*b + j]
  // (products rounded, then added: no contraction).  A lane holds positions
  // 8*cg .. 8*cg + 7 of its rows; stages h < 8 stay in the lane, stages h >= 8
  // pair it with the lane whose cg differs in bit h / 8 (the lanes of one row
  // are consecutive), and the mix reads the rows back from LDS.
  template <int M>
  __device__ __forceinline__ void rot_cross(float (&x)[TPL][8]) const {
#pragma clang fp contract(off)
    const bool upper = (cg & M) != 0;
#pragma unroll
    for (int k = 0; k < TPLV; ++k)
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const float o = slotq::swz_xor<M>(x[k][c]);
        x[k][c] = upper ? o - x[k][c] : x[k][c] + o;
      }
  }
  __device__ __forceinline__ void rotate_values(float (&x)[TPL][8], int block) const {
#pragma clang fp contract(off)
    using namespace slotq;
    float* rows = &s.vrow[wave - 2][0][0];
    const int lr0 = tq * TPLV;
    const int nb = D / block;
    wave_lds_sync();
#pragma unroll
    for (int k = 0; k < TPLV; ++k) {
      float4* p = reinterpret_cast<float4*>(rows + (lr0 + k) * D + 8 * cg);
      p[0] = make_float4(x[k][0], x[k][1], x[k][2], x[k][3]);
      p[1] = make_float4(x[k][4], x[k][5], x[k][6], x[k][7]);
    }
    wave_lds_sync();
    int pm[8];
    {
      const int4 q0 = *reinterpret_cast<const int4*>(s.rperm + 8 * cg);
      const int4 q1 = *reinterpret_cast<const int4*>(s.rperm + 8 * cg + 4);
      pm[0] = q0.x; pm[1] = q0.y; pm[2] = q0.z; pm[3] = q0.w;
      pm[4] = q1.x; pm[5] = q1.y; pm[6] = q1.z; pm[7] = q1.w;
    }
#pragma unroll
    for (int k = 0; k < TPLV; ++k)
#pragma unroll
      for (int c = 0; c < 8; ++c) x[k][c] = rows[(lr0 + k) * D + pm[c]];
#pragma unroll
    for (int hs = 1; hs < 8; hs *= 2)
#pragma unroll
      for (int k = 0; k < TPLV; ++k)
#pragma unroll
        for (int c = 0; c < 8; ++c)
          if ((c & hs) == 0) {
            const float u = x[k][c], w = x[k][c + hs];
            x[k][c] = u + w;
            x[k][c + hs] = u - w;
          }
    rot_cross<1>(x);
    if (block == 64) {
      rot_cross<2>(x);
      rot_cross<4>(x);
    }
    const float inv_sqrt_b = block == 16 ? 0.25f : 0.125f;
#pragma unroll
    for (int k = 0; k < TPLV; ++k)
#pragma unroll
      for (int c = 0; c < 8; ++c) x[k][c] = x[k][c] * inv_sqrt_b;
    if (nb == 1) {
      const float m0 = s.rmix[0];
#pragma unroll
      for (int k = 0; k < TPLV; ++k)
#pragma unroll
        for (int c = 0; c < 8; ++c) x[k][c] = m0 * x[k][c];
      return;
    }
    wave_lds_sync();
#pragma unroll
    for (int k = 0; k < TPLV; ++k) {
      float4* p = reinterpret_cast<float4*>(rows + (lr0 + k) * D + 8 * cg);
      p[0] = make_float4(x[k][0], x[k][1], x[k][2], x[k][3]);
      p[1] = make_float4(x[k][4], x[k][5], x[k][6], x[k][7]);
    }
    wave_lds_sync();
    const int bi = (8 * cg) / block;               // the lane's block
    const int col = (8 * cg) % block;              // its first position inside the block
    const float* mrow = s.rmix + bi * nb;
#pragma unroll
    for (int k = 0; k < TPLV; ++k) {
      const float* rw = rows + (lr0 + k) * D + col;
      float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      for (int l = 0; l < nb; ++l) {
        const float4 y0 = *reinterpret_cast<const float4*>(rw + l * block);
        const float4 y1 = *reinterpret_cast<const float4*>(rw + l * block + 4);
        const float ml = mrow[l];
        const float y[8] = {y0.x, y0.y, y0.z, y0.w, y1.x, y1.y, y1.z, y1.w};
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[c] = l == 0 ? ml * y[c] : acc[c] + ml * y[c];
      }
#pragma unroll
      for (int c = 0; c < 8; ++c) x[k][c] = acc[c];
    }
  }

  // ================= values: tokens [16*(wave-2), +16), groups along G_v channels
  __device__ __forceinline__ void process_values(const CommitTask& task, float (&x)[TPL][8], uint8_t* rec,
                                                 int rot_block) const {
#pragma clang fp contract(off)
    using namespace slotq;
    constexpr float LEV = (float)((1 << VB) - 1);
    if constexpr (ROT) rotate_values(x, rot_block);
    const int lpg = (1 << io.gv_log2) / 8;     // lanes per value group (4, 8 or 16)
    float mn[TPLV], mx[TPLV];
#pragma unroll
    for (int k = 0; k < TPLV; ++k) {
      float n = vmin3(x[k][0], x[k][1], x[k][2]), m = vmax3(x[k][0], x[k][1], x[k][2]);
      n = vmin3(n, x[k][3], x[k][4]); m = vmax3(m, x[k][3], x[k][4]);
      n = vmin3(n, x[k][5], x[k][6]); m = vmax3(m, x[k][5], x[k][6]);
      mn[k] = vmin3(n, x[k][7], x[k][7]); mx[k] = vmax3(m, x[k][7], x[k][7]);
    }
    DppMinMax<TPLV>::template step<0>(mn, mx);
    DppMinMax<TPLV>::template step<1>(mn, mx);
    if (lpg >= 8) DppMinMax<TPLV>::template step<2>(mn, mx);
    if (lpg >= 16) DppMinMax<TPLV>::template step<3>(mn, mx);
    // lane gl of a group computes token gl % TPLV of the lane's tokens
    const int gl = cg & (lpg - 1);
    const int g = cg / lpg;
    const int kk = gl & (TPLV - 1);
    float smn, smx;
    if (TPLV == 4) {
      const float n01 = pick((kk & 1) != 0, mn[1], mn[0]), n23 = pick((kk & 1) != 0, mn[TPLV - 1], mn[TPLV - 2]);
      const float m01 = pick((kk & 1) != 0, mx[1], mx[0]), m23 = pick((kk & 1) != 0, mx[TPLV - 1], mx[TPLV - 2]);
      smn = pick((kk & 2) != 0, n23, n01);
      smx = pick((kk & 2) != 0, m23, m01);
    } else {
      smn = pick((kk & 1) != 0, mn[TPLV - 1], mn[0]);
      smx = pick((kk & 1) != 0, mx[TPLV - 1], mx[0]);
    }
    uint32_t bits[8];
    if constexpr (MX) {
      // MX FP4: per (token, 32-channel group) one E8M0 byte, codes as for keys
      const bool any = t0 + kk < task.nvalid && smn <= smx;
      const float amax = any ? fmaxf(-smn, smx) : 0.f;
      const uint32_t eb = (__float_as_uint(amax) >> 23) & 0xFFu;
      const uint32_t sb = eb > 2u ? eb - 2u : 0u;
      if (gl < TPLV) {
        rec[KC + VC + KM + g * kSlot + t0 + kk] = (uint8_t)sb;
        s.vrcp[g][t0 + kk] = amax > 0.f ? __uint_as_float((254u - sb) << 23) : 0.f;
      }
      wave_lds_sync();
#pragma unroll
      for (int c = 0; c < 8; ++c) bits[c] = 0u;
#pragma unroll
      for (int k = 0; k < TPLV; ++k) {
        const float m = s.vrcp[g][t0 + k];
        uint32_t w = 0;   // byte j: channels 2j (low nibble) and 2j + 1
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[k][0] * m, x[k][1] * m, 1.0f, 0);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[k][2] * m, x[k][3] * m, 1.0f, 1);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[k][4] * m, x[k][5] * m, 1.0f, 2);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[k][6] * m, x[k][7] * m, 1.0f, 3);
        if (m == 0.f) w = 0u;
#pragma unroll
        for (int c = 0; c < 8; ++c) bits[c] |= ((w >> (4 * c)) & 0xFu) << (4 * k);
      }
    } else {
      const GroupParams gp = H16 ? to_h16(group_params<VB>(smn, smx, t0 + kk < task.nvalid))
                                 : group_params<VB>(smn, smx, t0 + kk < task.nvalid);
      float* vs = H16 ? &s.vmf[g][0] : reinterpret_cast<float*>(rec + KC + VC + KM + g * 256);
      if (gl < TPLV) {
        vs[t0 + kk] = gp.scale;
        vs[32 + t0 + kk] = gp.zero;
        s.vrcp[g][t0 + kk] = gp.rcp;
        if constexpr (H16) {
          _Float16* v16 = reinterpret_cast<_Float16*>(rec + KC + VC + KM + g * 128);
          v16[t0 + kk] = (_Float16)gp.scale;
          v16[32 + t0 + kk] = (_Float16)gp.zero;
        }
      }
      wave_lds_sync();
      // scales stay in LDS: only the rare exact path reads them
      float zero[TPLV], rcp[TPLV];
      if (TPLV == 4) {
        const float4 z = *reinterpret_cast<const float4*>(vs + 32 + t0);
        const float4 r = *reinterpret_cast<const float4*>(&s.vrcp[g][t0]);
        zero[0] = z.x; zero[1] = z.y; zero[TPLV - 2] = z.z; zero[TPLV - 1] = z.w;
        rcp[0] = r.x; rcp[1] = r.y; rcp[TPLV - 2] = r.z; rcp[TPLV - 1] = r.w;
      } else {
        const float2 z = *reinterpret_cast<const float2*>(vs + 32 + t0);
        const float2 r = *reinterpret_cast<const float2*>(&s.vrcp[g][t0]);
        zero[0] = z.x; zero[TPLV - 1] = z.y;
        rcp[0] = r.x; rcp[TPLV - 1] = r.y;
      }
      // The lane's TPLV consecutive tokens land next to each other in one code
      // word of each channel: token t goes to
      //   mm = t / 16, hh = (t / 4) % 2, e = (t % 4) + 4 * ((t / 8) % 2)
      //   4-bit: word 2*mm + hh, bits 4e;  2-bit: word hh, bits 2*(8*mm + e)
      // bits[c] holds the lane's codes of channel c from bit 0 on.
      // 4-bit: tokens k = 0, 2 go to bytes 0, 1 of pe and k = 1, 3 to those
      // of po (v_cvt_pk_u8_f32), so pe | po << 4 has token k at bits 4k
      uint32_t pe[8], po[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) bits[c] = pe[c] = po[c] = 0u;
#pragma unroll
      for (int k = 0; k < TPLV; ++k) {
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          float rc = code_of(x[k][c] - zero[k], rcp[k], vs[t0 + k], LEV);
          if constexpr (H16) rc = fminf(fmaxf(rc, 0.f), LEV);
          if (VB == 4) {
            if (k & 1) po[c] = __builtin_amdgcn_cvt_pk_u8_f32(rc, k >> 1, po[c]);
            else       pe[c] = __builtin_amdgcn_cvt_pk_u8_f32(rc, k >> 1, pe[c]);
          } else {
            bits[c] |= (uint32_t)rc << (VB * k);
          }
        }
      }
      if (VB == 4) {
#pragma unroll
        for (int c = 0; c < 8; ++c) bits[c] = pe[c] | (po[c] << 4);
      }
      if (__any(gp.bad)) {
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          uint32_t b = 0;
#pragma unroll
          for (int k = 0; k < TPLV; ++k) b |= (uint32_t)exact_code(x[k][c] - zero[k], vs[t0 + k], LEV) << (VB * k);
          bits[c] = b;
        }
      }
    }
    const int mm = t0 / 16, hh = (t0 / 4) % 2;
    const int e0 = (t0 % 4) + 4 * ((t0 / 8) % 2);
    const int j = VB == 4 ? 2 * mm + hh : hh;
    const int p0 = VB == 4 ? 4 * e0 : 2 * (8 * mm + e0);   // bit of the lane's first token
    uint8_t* vw = rec + KC + (j * D + 8 * cg) * 4 + p0 / 8;
    if (VB == 4 && TPLV == 4) {
      // lane L (< 32) and lane L + 32 hold the two 16-bit halves of the same
      // words (tokens t0 and t0 + 8); one swap per channel pair c, c + 4 gives
      // the lower lane words c and the upper lane words c + 4 as r[0] | r[1] << 16
      uint32_t wv[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const auto r = __builtin_amdgcn_permlane32_swap(bits[c], bits[c + 4], false, false);
        wv[c] = r[0] | (r[1] << 16);
      }
      const int hi = lane >= 32;
      *reinterpret_cast<uint4*>(rec + KC + (j * D + 8 * cg + 4 * hi) * 4) = make_uint4(wv[0], wv[1], wv[2], wv[3]);
    } else {
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        if (VB * TPLV == 16) {
          *reinterpret_cast<uint16_t*>(vw + 4 * c) = (uint16_t)bits[c];
        } else if (VB * TPLV == 8) {
          vw[4 * c] = (uint8_t)bits[c];
        } else {
          // two 2-bit codes per lane: a byte holds the codes of this lane and
          // of the lane with the neighbouring token pair (lane ^ 8 in the row)
          const uint32_t both = or_lane_xor8(bits[c] << (p0 % 8));
          if (p0 % 8 == 0) vw[4 * c] = (uint8_t)both;
        }
      }
    }
  }

  // The record, and the slot header (written by kv head 0, thread 0), leave
  // with 128-bit buffer stores; every thread issues the same number of stores
  // (lanes past the record, and the header store of all but one thread, fall
  // outside their resource and are dropped).
  static constexpr int kStoreNT = 2;   // buffer-store cache policy: nt
  __device__ __forceinline__ void copy_out(const CommitTask& task, const uint8_t* rec) const {
    const uint32_t rbytes = io.record_bytes;
    uint8_t* dst = io.seg.records + (((size_t)task.b * io.hkv + h) * io.seg.slot_cap + task.dst_slot) * rbytes;
    const __amdgpu_buffer_rsrc_t rr = __builtin_amdgcn_make_buffer_rsrc(dst, 0, rbytes, 0x00020000);
    // records are stored with the non-temporal hint (cache policy bit nt):
    // nothing reads them again in this kernel, and a prefill commit that left
    // them dirty in L2 waited longer at the kernel boundary (about 2% per call)
#pragma unroll
    for (int r = 0; r < NST; ++r) {
      const uint32_t off = (r * 256 + tid) * 16;
      const uint4 val = *reinterpret_cast<const uint4*>(rec + (off < REC_MAX ? off : REC_MAX - 16));
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned int, val), rr, off < rbytes ? off : 0x7ff00000u, 0, kStoreNT);
    }
    uint8_t* hdst = io.seg.headers + ((size_t)task.b * io.seg.slot_cap + task.dst_slot) * kHeaderBytes;
    const __amdgpu_buffer_rsrc_t hr = __builtin_amdgcn_make_buffer_rsrc(hdst, 0, kHeaderBytes, 0x00020000);
    const int4 hd = make_int4(task.nvalid, (int)task.mask, task.rank_base, task.token_base);
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned int, hd), hr,
                                           (h == 0 && tid == 0) ? 0u : 0x7ff00000u, 0, 0);
  }
};

}  // namespace kvq
