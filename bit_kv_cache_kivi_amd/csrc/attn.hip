// Fused dequantize-and-attend kernel for gfx950, plus the split-K combine.
//
// The block being denoised (32 query tokens, full precision) attends without a
// mask to itself and to every cached token of the prefix (and suffix, for the
// dual cache), computed directly from the low-bit codes (MaskAhead abstract:
// Q-MaskAhead attends from low-bit KV; SoloQ summary page: bidirectional
// context revisited every step; Tai et al., abstract: prefix and dual cache).
//
// Work unit = one 32-token slot of the cache, or the block itself (the last
// unit of the split that holds it).  A workgroup owns one (sequence, kv head)
// and a contiguous range of units, and is split into two roles:
//   * 4 producer waves (one per SIMD) stream the packed slot records and the
//     protected bf16 key rows from HBM (buffer loads into registers, three
//     units ahead), stage them in LDS, and dequantize each unit into MFMA
//     operand tiles: K as hi = fp16(x) plus an e5m2 lo part holding
//     2^12 (x - hi), V as fp16;
//   * one consumer wave per query head of the kv head (32 query tokens = one
//     32-wide MFMA tile) runs S^T = K Q^T (hi on v_mfma_f32_32x32x16_f16, lo
//     against an e4m3 copy of Q on the scaled fp8 MFMA), an online
//     softmax in fp32 (exp2 with the scale folded in; the reference maximum is
//     raised only when the running maximum exceeds it by more than 2^8, so O is
//     rarely rescaled) and O^T += V^T P^T.  The transposed products let the S
//     accumulators feed the PV B operand directly (lane = query, 16 tokens per
//     lane).
// A slot is dequantized once per workgroup and shared by all query heads
// through LDS.  One barrier per unit: in interval i producers store unit i+1,
// issue the loads of unit i+3 and dequantize unit i, while consumers work on
// units i-2 and i-1.  Consumers 0..3 first issue the PV of unit i-2 and the
// scores of unit i-1 to the MFMA pipe, then run the softmax of unit i-1;
// consumers 4..7 first run the softmax of unit i-2, then its PV and the
// scores of unit i-1.  On each SIMD one consumer's MFMA work thus overlaps
// the other consumer's softmax and the producer's dequantization.
// A split's partial (reference maximum, sum and O: fp32 unnormalised for an
// fp32 output, fp16 normalised for a 16-bit one) goes to the workspace and a
// merge kernel combines the splits with log-sum-exp weights; a single split
// writes the normalised output itself.  With rotated values and a 16-bit
// output every pair goes through the merge, which also rotates the output
// back.  Optionally the final per-row maximum and sum are written as well
// (the selection's softmax statistics), and the workgroup holding a block can
// also commit it (the one-launch step).
#include <cstring>
#include <mutex>

#include "commit_slot.h"
#include "device_common.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kMaxUnits = 256;     // units per split (the host keeps splits within this)
constexpr float kRescaleSlack = 8.0f;
constexpr int kProducerWaves = 4;
constexpr int kProducerThreads = kProducerWaves * 64;

template <class T>
__device__ __forceinline__ T pick(bool c, T x, T y) { return c ? x : y; }

// A split's partial for a 16-bit output: O normalised by the split's sum, as
// fp16 quads [D / 4][32 rows][4 channels], then per row the reference
// maximum, the sum and the power of two the row was scaled by (int32).
template <int D>
struct PartialH16 {
  static constexpr size_t kStats = (size_t)D * kSlot * 2;
  static constexpr size_t kBytes = kStats + 3 * kSlot * 4;
};

template <int D>
struct Shape {
  static constexpr int KS = D / 16;                  // MFMA k-steps over the head dimension
  static constexpr int CT = D / 32;                  // 32-channel output tiles
  static constexpr int NKG = kSlot * (D / 8);        // (token, 8-channel group) pairs of K
  static constexpr int NVC = D * 4;                  // (channel, token-octet) pairs of V
  static constexpr int GPT = NKG / kProducerThreads; // K groups per producer thread
  static constexpr int VPT = NVC / kProducerThreads; // V pairs per producer thread
  // one LDS stage holds a slot record (at most 48*D bytes) or the block as
  // fp32 K rows followed by fp16 V rows (192*D bytes)
  static constexpr int STAGE = 192 * D;
  static constexpr int RPT = (48 * D / 16 + kProducerThreads - 1) / kProducerThreads;   // record chunks per thread
  static_assert(NKG % kProducerThreads == 0 && NVC % kProducerThreads == 0, "thread mapping");
  static_assert(RPT >= GPT, "the block's K rows use the record prefetch slots");
};

// Fused commit of the block (SoloQ summary page, block-diffusion paragraph:
// the block's keys and values are quantized once, when it is committed): the
// four producer waves of the workgroup that attended with the block quantize
// its first cvalid[b] tokens for kv head kvh into prefix slot nslots[0][b]
// once their pipeline is done, with the same per-slot quantizer as the commit
// kernel, in LDS the pipeline no longer reads.  The slot's protected rank and
// token bases continue those of the previous slot's header (0 for the first
// slot).  Ends with one workgroup barrier before the record leaves; the
// consumer waves match it.
template <int KB, int VB, int D, bool F32IN, int FMT>
__device__ __forceinline__ void commit_block(uint8_t* lds_base, size_t lds_bytes, const AttnArgs& a, int b, int kvh,
                                             int tid) {
  using Q = SlotQuant<KB, VB, D, F32IN, false, FMT>;
  constexpr size_t kLds = (sizeof(typename Q::Lds) + 15) / 16 * 16;
  (void)lds_bytes;
  auto& lds = *reinterpret_cast<typename Q::Lds*>(lds_base);
  uint8_t* rec = lds_base + kLds;
  const SlotIO io{a.k_blk, a.v_blk, a.seg[0], kSlot, a.hkv, a.gv_log2, a.record_bytes};
  Q q(lds, io, kvh, tid);
  CommitTask task;
  task.b = b;
  task.dst_slot = a.nslots[0][b];
  task.src_tok = 0;
  task.nvalid = a.cvalid[b];
  task.mask = a.cmask[b];
  task.rank_base = 0;
  task.token_base = 0;
  task.pad = 0;
  if (task.dst_slot > 0) {
    const int4 ph = *reinterpret_cast<const int4*>(a.seg[0].headers +
                                                   ((size_t)b * a.seg[0].slot_cap + task.dst_slot - 1) * kHeaderBytes);
    task.rank_base = __builtin_amdgcn_readfirstlane(ph.z + __popc((uint32_t)ph.y));
    task.token_base = __builtin_amdgcn_readfirstlane(ph.w + ph.x);
  }
  q.clear_tail(rec);
  typename Q::Raw raw;
  q.fetch(true, task, raw);
  float x[Q::TPL][8];
#pragma unroll
  for (int k = 0; k < Q::TPL; ++k) Q::unpack_row(raw, k, x[k]);
  if (q.keys) {
    if (task.mask != 0u) q.store_protected(task, x);
    q.process_keys(task, x, rec);
  } else {
    q.process_values(task, x, rec, 0);
  }
  __syncthreads();
  q.copy_out(task, rec);
}

// CEN (values stored in a rotated basis): a value is dequantized as
// (code - cm) * scale with cm the middle code, (2^vb - 1) / 2, and the offset
// zero + cm * scale of each (token, channel group) is summed apart in fp32,
// weighted by the same fp16 probabilities as the PV product.  A dequantized
// value then rounds to fp16 with an error that is odd in the code around cm,
// instead of one shared by every channel with the same code; those shared
// errors would line up with the constant vector that the transposed
// Hadamard transform concentrates into one channel per block.
// MX (MX FP4 records): codes are E2M1 with one E8M0 scale byte per key
// channel and per (value group of 32 channels, token); the hardware converts
// the codes to fp16 exactly and a packed fp16 multiply applies the power-of-two
// scales, so the keys need no lo part (it is stored as zero).
// H16 (integer codes with fp16 scales and zeros): the producers read the
// half-width metadata and widen it to fp32 before the same fused multiply-add.
template <int KB, int VB, int D, int NC, bool CEN, int FMT>
__global__ __launch_bounds__((NC + kProducerWaves) * 64) void attn_kernel(const AttnArgs a) {
  using S = Shape<D>;
  constexpr int KS = S::KS, CT = S::CT, GPT = S::GPT, VPT = S::VPT, RPT = S::RPT;
  constexpr int NPT = kProducerThreads;
  constexpr uint32_t KC = kc_bytes(D, KB);
  constexpr uint32_t VC = vc_bytes(D, VB);
  constexpr bool MX = FMT == 1, H16 = FMT == 2;
  constexpr uint32_t KM = MX ? D : H16 ? kmeta_bytes(D) / 2 : kmeta_bytes(D);
  static_assert(record_bytes(D, KB, VB, 32) <= 48 * D, "record fits a stage");
  static_assert(!MX || (KB == 4 && VB == 4), "MX FP4 codes are 4-bit");
  static_assert(!(H16 && CEN), "fp16 metadata is not combined with rotated values");

  __shared__ __align__(16) uint8_t rawbuf[2][S::STAGE];      // packed slot records / the block
  __shared__ __align__(16) uint4 prtbuf[2][GPT][NPT];        // a producer thread's protected-row chunks
  __shared__ __align__(16) half8 kop[2][KS][64];             // key hi tiles: [buffer][k-step][lane]
  __shared__ __align__(16) uint4 klo[2][D / 64][2][64];      // key lo tiles (bf8): [buffer][64-channel block][16-byte half][lane]
  __shared__ __align__(16) half8 vop[3][CT][2][64];          // [buffer][channel tile][k-half][lane]
  __shared__ __align__(16) int4 hdr[kMaxUnits];
  __shared__ __align__(16) float zoff[CEN ? 3 : 1][CEN ? D / 32 : 1][kSlot];   // value offsets (CEN)
  // CEN: per consumer lane, the sum of P times the value offsets of each
  // channel group (kept in LDS: the consumers have no registers to spare)
  __shared__ __align__(16) float zsum[CEN ? NC : 1][CEN ? D / 32 : 1][64];
  constexpr float kCm = 0.5f * (float)((1 << VB) - 1);

  int split_i, kvh_i, b_i;
  if (a.num_wg) {
    const uint32_t e = a.wg[blockIdx.x];
    split_i = e & 0xff; kvh_i = (e >> 8) & 0xff; b_i = e >> 16;
  } else {
    split_i = blockIdx.x; kvh_i = blockIdx.y; b_i = blockIdx.z;
  }
  const int split = split_i, kvh = kvh_i, b = b_i;
  // Kernel-argument fields as locals: lambdas below capture these, never the
  // argument struct itself (capturing it by reference would copy the whole
  // struct to scratch memory).
  const int hkv = a.hkv, hq_all = a.hq, gv_log2 = a.gv_log2;
  const bool blk_f32 = a.blk_f32, q_f32 = a.q_f32;
  const void* const q_ptr = a.q;
  const void* const k_blk = a.k_blk;
  const void* const v_blk = a.v_blk;
  const SegPtrs seg0 = a.seg[0], seg1 = a.seg[1];
  // both counts read unconditionally, so the two loads overlap
  const int np = a.nslots[0][b], ns_all = a.nslots[1][b];
  const int ns = a.use_suffix ? ns_all : 0;
  // With a selection, the units are the listed cached units (prefix slots
  // numbered first, then suffix slots) and each carries a token mask.
  const int32_t* const sel_units = a.sel_units;
  const uint32_t* const sel_mask = a.sel_mask;
  const size_t sel_base = ((size_t)b * hkv + kvh) * a.sel_ucap;
  const int U = (a.sel_count ? a.sel_count[b * hkv + kvh] : np + ns) + 1;   // cached units + the block
  const int nsplit = (U + a.split_units - 1) / a.split_units;
  if (split >= nsplit) return;
  const int u0 = split * a.split_units;
  const int u1 = min(U, u0 + a.split_units);
  const int nq = min(u1, U - 1) - u0;        // slot units of this split
  const bool has_block = u1 == U;
  const int NU = nq + (has_block ? 1 : 0);   // units; the block, if here, is unit nq
  // this workgroup also commits the block (uniform)
  const bool fuse = a.commit_blk && has_block && a.cvalid[b] > 0;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool producer = wave < kProducerWaves;
  const int ci = wave - kProducerWaves;      // consumer index = query head kvh*r + ci
  const bool late = NC > 4 && ci >= 4;
  const int r = a.r;
  const uint32_t rbytes = a.record_bytes;
  const float c2 = a.scale_log2;


  // ---------------- prologues (run inside the role branches below): headers
  // and the block's raw rows (producers), Q operands (consumers)
  half8 qop[KS];
  v8i_t q8[D / 64];

  // ---------------- producers: register prefetch of one unit -- the slot
  // record (16-byte chunks, as laid out in memory) and this thread's chunks of
  // protected bf16 key rows.  Buffer loads: their range check turns reads past
  // a segment, or of rows a thread does not need, into zeros without memory
  // traffic, so every thread issues the same loads per unit and they stay
  // independent in-flight loads.  The descriptor of a unit's segment is
  // rebuilt per unit from values passed through readfirstlane: a descriptor
  // chosen by a select is taken as divergent and would force a per-lane loop
  // around every load.
  const uint8_t* rec_base0 = seg0.records + ((size_t)b * hkv + kvh) * seg0.slot_cap * rbytes;
  const uint8_t* rec_base1 = seg1.records + ((size_t)b * hkv + kvh) * seg1.slot_cap * rbytes;
  const int rec_n0 = (int)min((size_t)seg0.slot_cap * rbytes, (size_t)0x7fffffff);
  const int rec_n1 = (int)min((size_t)seg1.slot_cap * rbytes, (size_t)0x7fffffff);
  const uint16_t* prot_base0 = seg0.prot_rows + ((size_t)b * hkv + kvh) * seg0.prot_cap * D;
  const uint16_t* prot_base1 = seg1.prot_rows + ((size_t)b * hkv + kvh) * seg1.prot_cap * D;
  const int prot_n0 = (int)min((size_t)seg0.prot_cap * D * 2, (size_t)0x7fffffff);
  const int prot_n1 = (int)min((size_t)seg1.prot_cap * D * 2, (size_t)0x7fffffff);
  auto uniform_rsrc = [](const void* p, int n) __attribute__((always_inline)) {
    const uint64_t v = (uint64_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return __builtin_amdgcn_make_buffer_rsrc((void*)(((uint64_t)hi << 32) | lo), 0,
                                             __builtin_amdgcn_readfirstlane(n), 0x00020000);
  };
  struct Pre { uint4 rec[RPT]; uint4 prt[GPT]; uint32_t mask; };
  // Producer thread -> work mapping.  K: the thread's GPT (token, 8-channel
  // group) pairs share the group (tokens kt0 + KTT*gi of group kcg), so the
  // group's scales and zeros are read once.  V: the thread's VPT (channel,
  // token octet) pairs share the octet vcombo and the channel group, so the
  // tokens' scales and zeros are read once.  With value groups of 64 or more
  // channels, lane j takes channels j%32 + 32*(vi + VPT*(j/32)), so that
  // consecutive lanes write consecutive operand rows (no LDS bank conflicts);
  // with 32-channel groups, channels VPT*j + vi.
  constexpr int KTT = kSlot / GPT;
  static_assert(D / VPT == 64, "one V channel set per lane");
  const int kt0 = tid % KTT, kcg = tid / KTT;
  const int vcombo = tid / 64;
  int vch[VPT];
#pragma unroll
  for (int vi = 0; vi < VPT; ++vi)
    vch[vi] = gv_log2 >= 6 ? (lane & 31) + 32 * (vi + VPT * (lane >> 5)) : VPT * lane + vi;
  constexpr int kOutOfRange = 0x7ff00000;
  bool rec_chunk[RPT];
#pragma unroll
  for (int j = 0; j < RPT; ++j) rec_chunk[j] = (uint32_t)(j * NPT + tid) * 16u < rbytes;
  // Loads are issued unconditionally (units past the slots read out of range)
  // so that every path has the same number of loads in flight.
  // The block unit (bf16 input) takes the same loads: its K rows through the
  // record descriptor slots and its V rows through the protected-row slots.
  const uint8_t* kblk_base = static_cast<const uint8_t*>(k_blk) + ((size_t)b * kSlot * hkv + kvh) * D * 2;
  const uint8_t* vblk_base = static_cast<const uint8_t*>(v_blk) + ((size_t)b * kSlot * hkv + kvh) * D * 2;
  const int blk_n = kSlot * hkv * D * 2;
  const int blk_row = hkv * D * 2;                 // bytes between the block's token rows
  auto load_unit = [&](int q, Pre& pr, const int4 h) __attribute__((always_inline)) {
    const bool valid = q < nq;
    const bool blk_unit = has_block && q == nq && !blk_f32;
    // header word 0: segment << 16 | slot (the same LDS word in every lane)
    const int hx = __builtin_amdgcn_readfirstlane(h.x);
    const int sg = valid ? (hx >> 16) : 0;
    // (selects on values: a conditional on the captured lvalues would select
    // their addresses and keep them in scratch memory)
    const __amdgpu_buffer_rsrc_t rr =
        uniform_rsrc(pick(blk_unit, (const void*)kblk_base, pick(sg, (const void*)rec_base1, (const void*)rec_base0)),
                     pick(blk_unit, blk_n, pick(sg, rec_n1, rec_n0)));
    const __amdgpu_buffer_rsrc_t prr =
        uniform_rsrc(pick(blk_unit, (const void*)vblk_base, pick(sg, (const void*)prot_base1, (const void*)prot_base0)),
                     pick(blk_unit, blk_n, pick(sg, prot_n1, prot_n0)));
    const int rbase = (hx & 0xffff) * (int)rbytes;
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
      const int idx = j * NPT + tid;
      const int boff = j < GPT ? (kt0 + KTT * j) * blk_row + kcg * 16 : kOutOfRange;
      const int off = blk_unit ? boff : (valid && rec_chunk[j]) ? rbase + idx * 16 : kOutOfRange;
      pr.rec[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rr, off, 0, 0));
    }
    // header read by the caller (clamped index) and masked by a select, so no
    // branch splits the loads of a unit
    const uint32_t mask = valid ? (uint32_t)h.y : 0u;
    pr.mask = mask;
#pragma unroll
    for (int gi = 0; gi < GPT; ++gi) {
      const int t = kt0 + KTT * gi, cg = kcg;
      const int rank = h.z + __popc(mask & ((1u << t) - 1u));
      const int poff = blk_unit ? t * blk_row + cg * 16
                                : ((mask >> t) & 1u) ? (rank * D + 8 * cg) * 2 : kOutOfRange;
      pr.prt[gi] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(prr, poff, 0, 0));
    }
  };
  // Wait for the oldest unit's loads (the newer unit's RPT + GPT loads may stay
  // in flight).  Stating the wait once, before the conditional stores, keeps
  // the compiler from adding waits later where it reuses these registers.
  constexpr int kLoadsPerUnit = RPT + GPT;
  static_assert(kLoadsPerUnit < 16, "vmcnt field");
  auto store_unit = [&](int q, const Pre& pr) __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0xF70 | kLoadsPerUnit);   // vmcnt(kLoadsPerUnit), others unconstrained
    uint8_t* stage = rawbuf[q & 1];
    if (q < nq) {
#pragma unroll
      for (int j = 0; j < RPT; ++j)
        if (rec_chunk[j]) *reinterpret_cast<uint4*>(stage + (j * NPT + tid) * 16) = pr.rec[j];
#pragma unroll
      for (int gi = 0; gi < GPT; ++gi) {
        const int t = kt0 + KTT * gi;
        if ((pr.mask >> t) & 1u) prtbuf[q & 1][gi][tid] = pr.prt[gi];
      }
    } else if (q == nq && has_block) {
      // the block: K rows as fp32 [32][D], then V rows as fp16 [32][D]; bf16
      // rows arrived through the prefetch registers, fp32 rows are read here
      float* kst = reinterpret_cast<float*>(stage);
      _Float16* vst = reinterpret_cast<_Float16*>(stage + kSlot * D * 4);
#pragma unroll
      for (int gi = 0; gi < GPT; ++gi) {
        const int t = kt0 + KTT * gi, cg = kcg;
        float kx[8], vx[8];
        if (blk_f32) {
          const size_t e = (((size_t)b * kSlot + t) * hkv + kvh) * D + 8 * cg;
          load8(k_blk, e, true, kx);
          load8(v_blk, e, true, vx);
        } else {
          const uint4 k0 = pr.rec[gi], v0 = pr.prt[gi];
          kx[0] = bf16_lo(k0.x); kx[1] = bf16_hi(k0.x); kx[2] = bf16_lo(k0.y); kx[3] = bf16_hi(k0.y);
          kx[4] = bf16_lo(k0.z); kx[5] = bf16_hi(k0.z); kx[6] = bf16_lo(k0.w); kx[7] = bf16_hi(k0.w);
          vx[0] = bf16_lo(v0.x); vx[1] = bf16_hi(v0.x); vx[2] = bf16_lo(v0.y); vx[3] = bf16_hi(v0.y);
          vx[4] = bf16_lo(v0.z); vx[5] = bf16_hi(v0.z); vx[6] = bf16_lo(v0.w); vx[7] = bf16_hi(v0.w);
        }
        float* kd = kst + t * D + 8 * cg;
        *reinterpret_cast<float4*>(kd) = make_float4(kx[0], kx[1], kx[2], kx[3]);
        *reinterpret_cast<float4*>(kd + 4) = make_float4(kx[4], kx[5], kx[6], kx[7]);
        *reinterpret_cast<half8*>(vst + t * D + 8 * cg) = to_half8(vx);
      }
    }
  };

  // ---------------- producers: dequantize unit q into K buffer q & 1 and
  // V buffer q % 3.  dq_fetch issues every LDS read of a unit (code words,
  // scales and zeros, the protected chunks) at the start of an interval, so
  // that their latency overlaps the stores and loads of other units;
  // dequant does the arithmetic.  The reads are unconditional (the addresses
  // stay inside the stage whatever it holds); values a unit does not use are
  // ignored.
  const float neg_one = opaque_neg_one();
  const int khh = kcg / (D / 16), kks = kcg % (D / 16);
  const int vmm = vcombo >> 1, vhh = vcombo & 1;
  const int vta = 16 * vmm + 4 * vhh;       // value tokens vta..vta+3, vta+8..vta+11
  // the 8-byte lo part of channel group cg, token t: byte j of lane l of
  // 64-channel block k holds channel 64k + 32(l/32) + j of token l%32
  auto klo_part = [&](int kb, int cg, int t) __attribute__((always_inline)) -> uint2& {
    return reinterpret_cast<uint2*>(&klo[kb][cg >> 3][(cg >> 1) & 1][t + 32 * ((cg >> 2) & 1)])[cg & 1];
  };
  struct DqIn {
    uint32_t kw[GPT]; uint4 kp[GPT]; float4 ks[2], kz[2]; uint32_t vw[VPT]; float4 vs[2], vz[2]; uint2 kb8, vb8;
    uint4 ksh, kzh; uint2 vsh[2], vzh[2];   // fp16 metadata
  };
  auto dq_fetch = [&](int q, DqIn& d) __attribute__((always_inline)) {
    const uint8_t* rawS = rawbuf[q & 1];
    const uint32_t* words = reinterpret_cast<const uint32_t*>(rawS);
    // K: tokens kt0 + KTT*gi of channel group kcg; their codes are word kcg
    // (4-bit) or half kcg % 2 of word kcg / 2 (2-bit) of the token's word column.
    if constexpr (MX) {
      d.kb8 = *reinterpret_cast<const uint2*>(rawS + KC + VC + 8 * kcg);     // the 8 channels' scale bytes
    } else if constexpr (H16) {
      const uint8_t* kmeta = rawS + KC + VC + 16 * kcg;                      // 8 fp16 scales, then 8 zeros at +2D bytes
      d.ksh = *reinterpret_cast<const uint4*>(kmeta);
      d.kzh = *reinterpret_cast<const uint4*>(kmeta + 2 * D);
    } else {
      const float* kmeta = reinterpret_cast<const float*>(rawS + KC + VC) + 8 * kcg;
      d.ks[0] = *reinterpret_cast<const float4*>(kmeta);
      d.ks[1] = *reinterpret_cast<const float4*>(kmeta + 4);
      d.kz[0] = *reinterpret_cast<const float4*>(kmeta + D);
      d.kz[1] = *reinterpret_cast<const float4*>(kmeta + D + 4);
    }
#pragma unroll
    for (int gi = 0; gi < GPT; ++gi) {
      const int t = kt0 + KTT * gi;
      d.kw[gi] = KB == 4 ? words[kcg * 32 + t] : words[(kcg >> 1) * 32 + t];
      d.kp[gi] = prtbuf[q & 1][gi][tid];
    }
    // V: channels vch[vi] of token octet (vmm, vhh); 4-bit: word 2vmm+vhh of
    // the channel; 2-bit: half vmm of word vhh.
    if constexpr (MX) {
      // scale bytes of tokens vta..vta+3 and vta+8..vta+11 of the channels' group
      const uint8_t* vb = rawS + KC + VC + KM + (vch[0] >> 5) * kSlot;
      d.vb8 = make_uint2(*reinterpret_cast<const uint32_t*>(vb + vta), *reinterpret_cast<const uint32_t*>(vb + vta + 8));
    } else if constexpr (H16) {
      // per token: 32 fp16 scales, then 32 fp16 zeros
      const _Float16* vs = reinterpret_cast<const _Float16*>(rawS + KC + VC + KM + (vch[0] >> gv_log2) * 128);
      d.vsh[0] = *reinterpret_cast<const uint2*>(vs + vta);
      d.vsh[1] = *reinterpret_cast<const uint2*>(vs + vta + 8);
      d.vzh[0] = *reinterpret_cast<const uint2*>(vs + 32 + vta);
      d.vzh[1] = *reinterpret_cast<const uint2*>(vs + 32 + vta + 8);
    } else {
      const float* vs = reinterpret_cast<const float*>(rawS + KC + VC + KM + (vch[0] >> gv_log2) * 256);
      d.vs[0] = *reinterpret_cast<const float4*>(vs + vta);
      d.vs[1] = *reinterpret_cast<const float4*>(vs + vta + 8);
      d.vz[0] = *reinterpret_cast<const float4*>(vs + 32 + vta);
      d.vz[1] = *reinterpret_cast<const float4*>(vs + 32 + vta + 8);
    }
#pragma unroll
    for (int vi = 0; vi < VPT; ++vi)
      d.vw[vi] = VB == 4 ? words[KC / 4 + (2 * vmm + vhh) * D + vch[vi]] : words[KC / 4 + vhh * D + vch[vi]];
  };
  auto dequant = [&](int q, uint32_t mask, const DqIn& d) __attribute__((always_inline)) {
    const uint8_t* rawS = rawbuf[q & 1];
    const int kb = q & 1, vbuf = q % 3;
    if (MX && q < nq) {
      // scale pairs 2^(s - 127) as fp16 (exact within the fp16 range; the
      // scale of an all-zero group, byte 0, reads as 0)
      auto pairs = [](uint2 b8, half2_t (&sp)[4]) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t w = j < 2 ? b8.x : b8.y;
          const uint32_t b0 = (w >> (16 * (j & 1))) & 0xFFu, b1 = (w >> (16 * (j & 1) + 8)) & 0xFFu;
          sp[j] = to_half2(__uint_as_float(b0 << 23), __uint_as_float(b1 << 23));
        }
      };
      auto fp4x8 = [](uint32_t w, const half2_t (&sp)[4]) __attribute__((always_inline)) {
        half8 h;
        half2_t p;
        p = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * sp[0]; h[0] = p.x; h[1] = p.y;
        p = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * sp[1]; h[2] = p.x; h[3] = p.y;
        p = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * sp[2]; h[4] = p.x; h[5] = p.y;
        p = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * sp[3]; h[6] = p.x; h[7] = p.y;
        return h;
      };
      half2_t ksp[4];
      pairs(d.kb8, ksp);
#pragma unroll
      for (int gi = 0; gi < GPT; ++gi) {
        const int t = kt0 + KTT * gi;
        if ((mask >> t) & 1u) {
          const uint4 w = d.kp[gi];
          float x[8];
          x[0] = bf16_lo(w.x); x[1] = bf16_hi(w.x); x[2] = bf16_lo(w.y); x[3] = bf16_hi(w.y);
          x[4] = bf16_lo(w.z); x[5] = bf16_hi(w.z); x[6] = bf16_lo(w.w); x[7] = bf16_hi(w.w);
          store_hi_lo8(kop[kb][kks][t + 32 * khh], klo_part(kb, kcg, t), x, neg_one);
        } else {
          // key word: channel 8*kcg + c at bits 4c
          kop[kb][kks][t + 32 * khh] = fp4x8(d.kw[gi], ksp);
          klo_part(kb, kcg, t) = make_uint2(0u, 0u);
        }
      }
      // value word of channel c: token e (vta + e % 4 + 8 * (e / 4)) at bits 4e
      half2_t vsp[4];
      pairs(d.vb8, vsp);
#pragma unroll
      for (int vi = 0; vi < VPT; ++vi) {
        const int c = vch[vi];
        vop[vbuf][c >> 5][vmm][(c & 31) + 32 * vhh] = fp4x8(d.vw[vi], vsp);
      }
    } else if (q < nq) {
      // widen two fp16 values packed in a word
      auto h2f = [](uint32_t w, float& lo, float& hi) __attribute__((always_inline)) {
        lo = (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
        hi = (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
      };
      float ksc[8], kzr[8];
      if constexpr (H16) {
        h2f(d.ksh.x, ksc[0], ksc[1]); h2f(d.ksh.y, ksc[2], ksc[3]); h2f(d.ksh.z, ksc[4], ksc[5]); h2f(d.ksh.w, ksc[6], ksc[7]);
        h2f(d.kzh.x, kzr[0], kzr[1]); h2f(d.kzh.y, kzr[2], kzr[3]); h2f(d.kzh.z, kzr[4], kzr[5]); h2f(d.kzh.w, kzr[6], kzr[7]);
      } else {
        const float4 a0 = d.ks[0], a1 = d.ks[1], z0 = d.kz[0], z1 = d.kz[1];
        ksc[0] = a0.x; ksc[1] = a0.y; ksc[2] = a0.z; ksc[3] = a0.w; ksc[4] = a1.x; ksc[5] = a1.y; ksc[6] = a1.z; ksc[7] = a1.w;
        kzr[0] = z0.x; kzr[1] = z0.y; kzr[2] = z0.z; kzr[3] = z0.w; kzr[4] = z1.x; kzr[5] = z1.y; kzr[6] = z1.z; kzr[7] = z1.w;
      }
#pragma unroll
      for (int gi = 0; gi < GPT; ++gi) {
        const int t = kt0 + KTT * gi;
        float x[8];
        if ((mask >> t) & 1u) {
          const uint4 w = d.kp[gi];
          x[0] = bf16_lo(w.x); x[1] = bf16_hi(w.x); x[2] = bf16_lo(w.y); x[3] = bf16_hi(w.y);
          x[4] = bf16_lo(w.z); x[5] = bf16_hi(w.z); x[6] = bf16_lo(w.w); x[7] = bf16_hi(w.w);
        } else {
          float code[8];
          unpack8<KB>(KB == 4 ? d.kw[gi] : d.kw[gi] >> (16 * (kcg & 1)), code);
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = fmaf(code[e], ksc[e], kzr[e]);
        }
        store_hi_lo8(kop[kb][kks][t + 32 * khh], klo_part(kb, kcg, t), x, neg_one);
      }
      float vsc[8], vzr[8];
      if constexpr (H16) {
        h2f(d.vsh[0].x, vsc[0], vsc[1]); h2f(d.vsh[0].y, vsc[2], vsc[3]); h2f(d.vsh[1].x, vsc[4], vsc[5]); h2f(d.vsh[1].y, vsc[6], vsc[7]);
        h2f(d.vzh[0].x, vzr[0], vzr[1]); h2f(d.vzh[0].y, vzr[2], vzr[3]); h2f(d.vzh[1].x, vzr[4], vzr[5]); h2f(d.vzh[1].y, vzr[6], vzr[7]);
      } else {
        const float4 a0 = d.vs[0], a1 = d.vs[1], z0 = d.vz[0], z1 = d.vz[1];
        vsc[0] = a0.x; vsc[1] = a0.y; vsc[2] = a0.z; vsc[3] = a0.w; vsc[4] = a1.x; vsc[5] = a1.y; vsc[6] = a1.z; vsc[7] = a1.w;
        vzr[0] = z0.x; vzr[1] = z0.y; vzr[2] = z0.z; vzr[3] = z0.w; vzr[4] = z1.x; vzr[5] = z1.y; vzr[6] = z1.z; vzr[7] = z1.w;
      }
      if constexpr (CEN) {
#pragma unroll
        for (int e = 0; e < 8; ++e) vzr[e] = -kCm * vsc[e];
        if (tid < (D >> gv_log2) * kSlot) {
          const int g = tid / kSlot, t = tid % kSlot;
          const float* vm = reinterpret_cast<const float*>(rawS + KC + VC + KM + g * 256);
          zoff[vbuf][g][t] = fmaf(kCm, vm[t], vm[kSlot + t]);
        }
      }
#pragma unroll
      for (int vi = 0; vi < VPT; ++vi) {
        const int c = vch[vi];
        float code[8];
        unpack8<VB>(VB == 4 ? d.vw[vi] : d.vw[vi] >> (16 * vmm), code);
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = fmaf(code[e], vsc[e], vzr[e]);
        vop[vbuf][c >> 5][vmm][(c & 31) + 32 * vhh] = to_half8(x);
      }
    } else if (q == nq && has_block) {
      const float* kst = reinterpret_cast<const float*>(rawS);
      const _Float16* vst = reinterpret_cast<const _Float16*>(rawS + kSlot * D * 4);
#pragma unroll
      for (int gi = 0; gi < GPT; ++gi) {
        const int t = kt0 + KTT * gi, cg = kcg;
        const float4 x0 = *reinterpret_cast<const float4*>(kst + t * D + 8 * cg);
        const float4 x1 = *reinterpret_cast<const float4*>(kst + t * D + 8 * cg + 4);
        const float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
        store_hi_lo8(kop[kb][kks][t + 32 * khh], klo_part(kb, cg, t), x, neg_one);
      }
#pragma unroll
      for (int vi = 0; vi < VPT; ++vi) {
        const int c = vch[vi];
        half8 v;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = vst[(vta + (e & 3) + 8 * (e >> 2)) * D + c];
        vop[vbuf][c >> 5][vmm][(c & 31) + 32 * vhh] = v;
      }
      if constexpr (CEN) {
        if (tid < (D / 32) * kSlot) zoff[vbuf][tid / kSlot][tid % kSlot] = 0.f;   // the block is not quantized
      }
    }
  };

  // ---------------- consumers: scores of unit q (part 1) and softmax + PV of
  // unit q (part 2)
  float m_ref = -__builtin_inff(), l_run = 0.f;
  floatx16 o[CT];                            // zeroed once the Q operands are built
  floatx16 sacc;
  // The operand tiles are read from LDS a few k-steps ahead of the MFMAs
  // that use them (the scheduling barriers pin the interleave; left alone
  // the compiler issues each read right before its MFMA and waits for it).
  // S^T = K_hi Q^T (fp16, v_mfma_f32_32x32x16_f16) + 2^-12 K_lo' Q8^T (bf8 x
  // e4m3, v_mfma_scale_f32_32x32x64_f8f6f4 with an E8M0 scale of 2^-12 on K_lo')
  constexpr int KB8 = D / 64;
  auto scores = [&](int q) __attribute__((always_inline)) {
    const int kb = q & 1;
    half8 kh[KS];
    v8i_t kl[KB8];
#pragma unroll
    for (int s = 0; s < KS; ++s) kh[s] = kop[kb][s][lane];
#pragma unroll
    for (int k = 0; k < KB8; ++k) {
      const uint4 l0 = klo[kb][k][0][lane];
      const uint4 l1 = klo[kb][k][1][lane];
      kl[k] = v8i_t{(int)l0.x, (int)l0.y, (int)l0.z, (int)l0.w, (int)l1.x, (int)l1.y, (int)l1.z, (int)l1.w};
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) sacc[i] = 0.f;
#pragma unroll
    for (int s = 0; s < KS; ++s) sacc = __builtin_amdgcn_mfma_f32_32x32x16_f16(kh[s], qop[s], sacc, 0, 0, 0);
#pragma unroll
    for (int k = 0; k < KB8; ++k)
      sacc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kl[k], q8[k], sacc, 1, 0, 0, 127 - 12, 0, 127);
    constexpr int NR = KS + 2 * KB8, NM = KS + KB8, AHEAD = 4;
    __builtin_amdgcn_sched_group_barrier(0x100, AHEAD, 0);    // LDS reads ahead
#pragma unroll
    for (int k = 0; k < NR - AHEAD; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);      // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);      // next LDS read
    }
    __builtin_amdgcn_sched_group_barrier(0x008, NM - (NR - AHEAD), 0);
  };
  // tmask (the unit's attended tokens: valid, and selected if a selection is
  // used) is read from the header one phase ahead by the caller, so its LDS
  // latency stays off the softmax path.
  // softmax of the scores in sacc: P (fp16, the PV B operand) into pop; the
  // running maximum, sum and O are updated.
  auto softmax = [&](uint32_t tmask, half8 (&pop)[2]) __attribute__((always_inline)) {
    // sacc[i] = S[query lane%32][token 8*(i/4) + 4*(lane/32) + i%4]
    if (tmask != ~0u) {
      // the lane's tokens 4*(lane/32) + {0..3, 8..11, 16..19, 24..27}: bits at
      // fixed positions once the mask is shifted by 4*(lane/32)
      const uint32_t mm = tmask >> (4 * (lane >> 5));
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (!((mm >> (8 * (i >> 2) + (i & 3))) & 1u)) sacc[i] = -__builtin_inff();
    }
    float mx = fmaxf(fmaxf(sacc[0], sacc[1]), sacc[2]);
#pragma unroll
    for (int i = 3; i < 15; i += 2) mx = fmaxf(fmaxf(mx, sacc[i]), sacc[i + 1]);
    mx = max_halves(fmaxf(mx, sacc[15]));
    const float ms = mx * c2;
    const bool need = ms > m_ref + kRescaleSlack;
    if (__any(need)) {
      const float m_new = need ? ms : m_ref;
      const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);
      m_ref = m_new;
      l_run *= alpha;
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[ct][i] *= alpha;
      if constexpr (CEN) {
#pragma unroll
        for (int g = 0; g < D / 32; ++g)
          if (g < (D >> gv_log2)) zsum[ci][g][lane] *= alpha;
      }
    }
    const float mneg = -m_ref;
    // P is rounded to fp16 for the PV product; the row sum takes the same
    // rounded values (v_dot2_f32_f16 against (1, 1)), so numerator and
    // denominator see identical weights.
    float psum = l_run;
    const half2_t ones = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
    for (int i = 0; i < 16; i += 2) {
      const half2_t pp = to_half2(__builtin_amdgcn_exp2f(fmaf(sacc[i], c2, mneg)),
                                  __builtin_amdgcn_exp2f(fmaf(sacc[i + 1], c2, mneg)));
      pop[i >> 3][i & 7] = pp.x;
      pop[i >> 3][(i & 7) + 1] = pp.y;
      psum = __builtin_amdgcn_fdot2(pp, ones, psum, false);
    }
    l_run = psum;
  };
  // CEN: zsum[g] += sum over the lane's 16 tokens of P (fp16, as in the PV
  // product) times the offset of the token's group g; token of P entry i is
  // 8*(i/4) + 4*(lane/32) + i%4
  auto zacc = [&](int q, const half8 (&pop)[2]) __attribute__((always_inline)) {
    if constexpr (CEN) {
      const int ng = D >> gv_log2;
#pragma unroll
      for (int g = 0; g < D / 32; ++g) {
        if (g < ng) {
          const float* zp = &zoff[q % 3][g][4 * (lane >> 5)];
          float acc = zsum[ci][g][lane];
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            const float4 z = *reinterpret_cast<const float4*>(zp + 8 * m);
            const half8& pp = pop[m >> 1];
            const int i0 = (4 * m) & 7;
            acc = fmaf((float)pp[i0], z.x, acc);
            acc = fmaf((float)pp[i0 + 1], z.y, acc);
            acc = fmaf((float)pp[i0 + 2], z.z, acc);
            acc = fmaf((float)pp[i0 + 3], z.w, acc);
          }
          zsum[ci][g][lane] = acc;
        }
      }
    }
  };
  auto pv = [&](const half8 (&va)[CT][2], const half8 (&pop)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
      o[ct] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va[ct][0], pop[0], o[ct], 0, 0, 0);
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
      o[ct] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va[ct][1], pop[1], o[ct], 0, 0, 0);
  };
  // V operands of unit q, k-half kh
  auto read_v = [&](int q, int kh, half8 (&va)[CT][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) va[ct][kh] = vop[q % 3][ct][kh][lane];
  };

  // ---------------- pipeline.  Interval i: producers store unit i+1 (register
  // set (i+1) & 1), load unit i+3 into the freed set and dequantize unit i;
  // early consumers run the PV of unit i-2 and the scores and softmax of unit
  // i-1; late consumers run the softmax and PV of unit i-2 and the scores of
  // unit i-1.  Producers and consumers run separate loops with the same
  // barrier count (the branch is uniform per wave), so neither role holds the
  // other's loop-carried registers.
  // intervals: unit q is dequantized in interval q and its PV runs in
  // interval q + 2, so NU + 2 intervals, rounded up to even so that the
  // producer loop (unrolled by two for its two register sets) has no
  // conditional half: a conditional half would merge register states at the
  // latch and force waits on in-flight loads
  const int n_int = (NU + 3) & ~1;
  if (producer) {
      // unit headers in LDS: (segment << 16 | slot, protected mask, first
      // protected rank, attended-token mask)
      for (int i = tid; i < nq; i += NPT) {
        const int cu = sel_units ? sel_units[sel_base + u0 + i] : u0 + i;
        const int seg = cu < np ? 0 : 1, sl = cu < np ? cu : cu - np;
        const uint8_t* hb = seg ? seg1.headers : seg0.headers;
        const int cap = seg ? seg1.slot_cap : seg0.slot_cap;
        const int4 h = *reinterpret_cast<const int4*>(hb + ((size_t)b * cap + sl) * kHeaderBytes);
        uint32_t tm = h.x >= kSlot ? ~0u : (1u << h.x) - 1u;
        if (sel_mask) tm &= sel_mask[sel_base + cu];
        hdr[i] = make_int4((seg << 16) | sl, h.y, h.z, (int)tm);
      }
      if (tid == 0 && has_block) hdr[nq] = make_int4(0, 0, 0, -1);
    __syncthreads();                         // headers in LDS
    auto hdr_at = [&](int q) { return hdr[min(q, kMaxUnits - 1)]; };
    Pre pre0, pre1;
    load_unit(0, pre0, hdr_at(0));
    load_unit(1, pre1, hdr_at(1));
    store_unit(0, pre0);
    uint32_t dmask = pre0.mask;              // protected mask of the unit dequantized next
    load_unit(2, pre0, hdr_at(2));
    __syncthreads();
    // Interval order: LDS reads of the header of the unit to load (first, so
    // that waiting for it does not wait for the rest) and of the unit to
    // dequantize; store the next unit (its loads have landed); the
    // dequantization arithmetic, as soon as its reads land (it then runs while
    // the early consumers' MFMAs do, and is done before their softmax); last,
    // the loads three units ahead.
    for (int i = 0; i < n_int; i += 2) {
      const int4 h3 = hdr_at(i + 3);
      __builtin_amdgcn_sched_barrier(0);
      DqIn d;
      dq_fetch(i, d);
      store_unit(i + 1, pre1);
      const uint32_t m1 = pre1.mask;
      if (i < NU) dequant(i, dmask, d);
      load_unit(i + 3, pre1, h3);
      __syncthreads();
      const int4 h4 = hdr_at(i + 4);
      __builtin_amdgcn_sched_barrier(0);
      dq_fetch(i + 1, d);
      store_unit(i + 2, pre0);
      const uint32_t m0 = pre0.mask;
      if (i + 1 < NU) dequant(i + 1, m1, d);
      dmask = m0;
      load_unit(i + 4, pre0, h4);
      __syncthreads();
    }
    if (fuse) {
      // the pipeline's last barrier has passed: the producers own rawbuf
      static_assert(sizeof(typename SlotQuant<KB, VB, D, true, false, FMT>::Lds) + 16 +
                        SlotQuant<KB, VB, D, true, false, FMT>::REC_MAX <= sizeof(rawbuf),
                    "the fused commit fits the staging buffers");
      uint8_t* base = &rawbuf[0][0];
      if constexpr (CEN) {
        // rotated values: the block's rows are the fp32 keys and the rotated
        // values staged for this launch (the same rotation, in the same
        // order, as the commit kernel applies), quantized without rotating
        commit_block<KB, VB, D, true, FMT>(base, sizeof(rawbuf), a, b, kvh, tid);
      } else {
        if (blk_f32) commit_block<KB, VB, D, true, FMT>(base, sizeof(rawbuf), a, b, kvh, tid);
        else         commit_block<KB, VB, D, false, FMT>(base, sizeof(rawbuf), a, b, kvh, tid);
      }
    }
    return;
  }
  // Q operands.  Q is the B operand of S^T: lane = query token j; half hh
  // holds channels (D/2)*hh + 8s + [0, 8) at k-step s.  Q8, Q in e4m3 for the
  // key lo product: block k holds channels 64k + 32*hh + [0, 32) (the lo-tile
  // layout).  The fp16 operands of bf16 Q are loaded before the two prologue
  // barriers and converted after them, so the fetch overlaps the producers'
  // header reads and first unit loads (the first scores come an interval
  // later); the barriers order LDS only, so the loads stay in flight across
  // them.  fp32 Q (twice the registers) is loaded and converted after them.
  {
    const int j = lane & 31, hh = lane >> 5;
    const int hq = kvh * r + ci;
    const size_t base = (((size_t)b * kSlot + j) * hq_all + hq) * D + (D / 2) * hh;
    const size_t row = (((size_t)b * kSlot + j) * hq_all + kvh * r + min(ci, r - 1)) * D;
    auto q8_pack = [&](int k, const float (&x)[32]) __attribute__((always_inline)) {
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        uint32_t d = __builtin_amdgcn_cvt_pk_fp8_f32(x[4 * w], x[4 * w + 1], 0u, false);
        d = __builtin_amdgcn_cvt_pk_fp8_f32(x[4 * w + 2], x[4 * w + 3], d, true);
        q8[k][w] = (int)d;
      }
    };
    uint4 raw[KS];
    if (!q_f32) {
      const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(q_ptr) + base);
#pragma unroll
      for (int s = 0; s < KS; ++s) raw[s] = p[s];
    }
    if constexpr (CEN) {
      if (ci < r) {
#pragma unroll
        for (int g = 0; g < D / 32; ++g) zsum[ci][g][lane] = 0.f;
      }
    }
    // the producers' header barrier and prologue barrier
    lds_barrier();
    lds_barrier();
    if (q_f32) {
      float4 rf[KS][2];
      const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(q_ptr) + base);
#pragma unroll
      for (int s = 0; s < KS; ++s) { rf[s][0] = p[2 * s]; rf[s][1] = p[2 * s + 1]; }
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const float x[8] = {rf[s][0].x, rf[s][0].y, rf[s][0].z, rf[s][0].w,
                            rf[s][1].x, rf[s][1].y, rf[s][1].z, rf[s][1].w};
        qop[s] = to_half8(x);
      }
#pragma unroll
      for (int k = 0; k < KB8; ++k) {
        const float4* p8 = reinterpret_cast<const float4*>(static_cast<const float*>(q_ptr) + row + 64 * k + 32 * hh);
        float x[32];
#pragma unroll
        for (int v = 0; v < 8; ++v) {
          const float4 t = p8[v];
          x[4 * v] = t.x; x[4 * v + 1] = t.y; x[4 * v + 2] = t.z; x[4 * v + 3] = t.w;
        }
        q8_pack(k, x);
      }
    } else {
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const float x[8] = {bf16_lo(raw[s].x), bf16_hi(raw[s].x), bf16_lo(raw[s].y), bf16_hi(raw[s].y),
                            bf16_lo(raw[s].z), bf16_hi(raw[s].z), bf16_lo(raw[s].w), bf16_hi(raw[s].w)};
        qop[s] = to_half8(x);
      }
#pragma unroll
      for (int k = 0; k < KB8; ++k) {
        // the same rows as the fp16 operands, read again in the lo-tile layout
        // (from L2: this wave has just fetched them)
        const uint4* p8 = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(q_ptr) + row + 64 * k + 32 * hh);
        float x[32];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const uint4 t = p8[v];
          x[8 * v] = bf16_lo(t.x); x[8 * v + 1] = bf16_hi(t.x); x[8 * v + 2] = bf16_lo(t.y); x[8 * v + 3] = bf16_hi(t.y);
          x[8 * v + 4] = bf16_lo(t.z); x[8 * v + 5] = bf16_hi(t.z); x[8 * v + 6] = bf16_lo(t.w); x[8 * v + 7] = bf16_hi(t.w);
        }
        q8_pack(k, x);
      }
    }
  }
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[ct][i] = 0.f;
  if (ci >= r) {
    for (int i = 0; i < n_int; ++i) __syncthreads();
    if (fuse) __syncthreads();   // the fused commit's barrier
    return;
  }
  half8 pop[2], va[CT][2];
  if (late) {
    // Interval i: softmax and PV of unit i-2, then the scores of unit i-1.
    uint32_t nv = ~0u;
    for (int i = 0; i < n_int; ++i) {
      // The late consumers' softmax and PV are the longest path of an
      // interval (their V tiles and MFMAs queue behind the early consumers'
      // scores); a higher issue priority on the SIMD for that phase shortens it.
      __builtin_amdgcn_s_setprio(2);
      if (i >= 2 && i - 2 < NU) {
        if constexpr (CEN) {
          // the offset sums first: with the V tiles in flight as well, the
          // wave would run out of registers
          softmax(nv, pop);
          zacc(i - 2, pop);
          read_v(i - 2, 0, va);
        } else {
          read_v(i - 2, 0, va);
          softmax(nv, pop);
        }
        read_v(i - 2, 1, va);
        pv(va, pop);
      }
      __builtin_amdgcn_s_setprio(0);
      if (i >= 1 && i - 1 < NU) {
        nv = (uint32_t)hdr[i - 1].w;
        scores(i - 1);
      }
      __syncthreads();
    }
  } else {
    // Interval i: PV of unit i-2 (P kept from the previous interval) and the
    // scores of unit i-1 go to the MFMA pipe back to back, then the softmax
    // of unit i-1; the late consumer on the same SIMD runs its softmax first
    // and its MFMAs second, so the two alternate between vector ALU and MFMA.
    for (int i = 0; i < n_int; ++i) {
      if (i >= 2 && i - 2 < NU) {
        read_v(i - 2, 1, va);
        pv(va, pop);
        // the second-half reads, then the MFMAs (left alone, the compiler
        // issues each read right before its MFMA and waits for it)
        __builtin_amdgcn_sched_group_barrier(0x100, CT, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 2 * CT, 0);
      }
      if (i >= 1 && i - 1 < NU) {
        const uint32_t nv = (uint32_t)hdr[i - 1].w;
        scores(i - 1);
        softmax(nv, pop);
        zacc(i - 1, pop);
        // first V k-half of unit i-1 for the next interval's PV, in flight
        // across the barrier
        __builtin_amdgcn_sched_barrier(0);
        read_v(i - 1, 0, va);
      }
      // A consumer only reads LDS, so its barrier needs no release fence and
      // the reads above stay in flight across it (a unit's V tile is rewritten
      // three intervals after it is produced); the acquire fence keeps the
      // next interval's reads below the barrier.
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    }
  }

  // ---------------- epilogue (consumers)
  const int hq = kvh * r + ci;
  const float l_tot = sum_halves(l_run);
  const int j = lane & 31, hh = lane >> 5;
  if constexpr (CEN) {
    // the offsets' contribution, common to every channel of a group
    float zt[D / 32];
#pragma unroll
    for (int g = 0; g < D / 32; ++g) zt[g] = g < (D >> gv_log2) ? sum_halves(zsum[ci][g][lane]) : 0.f;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      const int gct = (32 * ct) >> gv_log2;
      float z = zt[0];
#pragma unroll
      for (int g = 1; g < D / 32; ++g) z = gct == g ? zt[g] : z;
#pragma unroll
      for (int i = 0; i < 16; ++i) o[ct][i] += z;
    }
  }
  if (nsplit == 1 && !a.force_partials) {
    const float inv = 1.0f / l_tot;
    const size_t row = ((size_t)b * kSlot + j) * hq_all + hq;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        const int c = 32 * ct + 8 * qd + 4 * hh;
        const float v0 = o[ct][4 * qd] * inv, v1 = o[ct][4 * qd + 1] * inv;
        const float v2 = o[ct][4 * qd + 2] * inv, v3 = o[ct][4 * qd + 3] * inv;
        if (a.out_f32) {
          *reinterpret_cast<float4*>(static_cast<float*>(a.out) + row * D + c) = make_float4(v0, v1, v2, v3);
        } else {
          uint2 w;
          w.x = f32_to_bf16_bits(v0) | (f32_to_bf16_bits(v1) << 16);
          w.y = f32_to_bf16_bits(v2) | (f32_to_bf16_bits(v3) << 16);
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + row * D + c) = w;
        }
      }
    if (a.row_stats && hh == 0) {
      float* rs = a.row_stats + (((size_t)b * hkv + kvh) * kSelHeads + ci) * 2 * kSlot + j;
      rs[0] = m_ref;
      rs[kSlot] = l_tot;
    }
  } else if (!a.out_f32) {
    // 16-bit output: the split's O normalised by its own sum and scaled by a
    // power of two per row (row maximum in [2^14, 2^15)), in fp16, so the
    // hand-off to the combine costs half the bytes of fp32 and its rounding
    // (at most 2^-11 of the row maximum) stays below the bf16 output's
    const size_t pidx = (((size_t)b * hkv + kvh) * a.max_splits + split) * r + ci;
    uint8_t* base = reinterpret_cast<uint8_t*>(a.partial) + pidx * PartialH16<D>::kBytes;
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    float mx = 0.f;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, fabsf(o[ct][i]));
    const int sh = 15 - __builtin_amdgcn_frexp_expf(max_halves(mx) * inv);
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        const int cq = 8 * ct + 2 * qd + hh;      // channels 4cq .. 4cq+3
        const _Float16 h0 = (_Float16)__builtin_amdgcn_ldexpf(o[ct][4 * qd] * inv, sh);
        const _Float16 h1 = (_Float16)__builtin_amdgcn_ldexpf(o[ct][4 * qd + 1] * inv, sh);
        const _Float16 h2 = (_Float16)__builtin_amdgcn_ldexpf(o[ct][4 * qd + 2] * inv, sh);
        const _Float16 h3 = (_Float16)__builtin_amdgcn_ldexpf(o[ct][4 * qd + 3] * inv, sh);
        uint2 w;
        w.x = (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
        w.y = (uint32_t)__builtin_bit_cast(uint16_t, h2) | ((uint32_t)__builtin_bit_cast(uint16_t, h3) << 16);
        *reinterpret_cast<uint2*>(base + ((size_t)cq * kSlot + j) * 8) = w;
      }
    if (hh == 0) {
      float* stats = reinterpret_cast<float*>(base + PartialH16<D>::kStats);
      stats[j] = m_ref;
      stats[kSlot + j] = l_tot;
      stats[2 * kSlot + j] = __int_as_float(-sh);
    }
  } else {
    const size_t pidx = (((size_t)b * hkv + kvh) * a.max_splits + split) * r + ci;
    float* base = a.partial + pidx * (size_t)(D + 2) * kSlot;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int c = 32 * ct + 8 * (i >> 2) + 4 * hh + (i & 3);
        base[c * kSlot + j] = o[ct][i];
      }
    if (hh == 0) {
      base[D * kSlot + j] = m_ref;
      base[(D + 1) * kSlot + j] = l_tot;
    }
  }
  if (fuse) __syncthreads();   // the fused commit's barrier
}

// One workgroup per (query head, sequence, 32-channel chunk): merges the
// splits of all 32 rows for those channels.  Thread -> (query tokens
// 4jq..4jq+3, one channel), jq fastest, so each 16-byte load of a wave covers
// whole 128-byte rows of the partials.  Every thread loads, for a batch of up
// to kBatch splits at once, its partial O values together with the reference
// maxima and row sums of its four rows (the 32 threads of a row group load
// the same maxima and sums: one request per wave), so a batch costs one
// memory latency and no barrier; batches past the first rescale what has
// been summed when the maximum grows.  The result is transposed through LDS
// for row-contiguous output stores.
template <int D>
__global__ __launch_bounds__(256) void combine_kernel(const AttnArgs a) {
  constexpr int CW = 32;        // channels per workgroup
  constexpr int kBatch = 8;     // splits loaded at once
  __shared__ __align__(16) float out_lds[kSlot][CW + 4];
  const int hq = blockIdx.x, b = blockIdx.y, c0 = blockIdx.z * CW;
  // both counts read unconditionally, so the two loads overlap
  const int np = a.nslots[0][b], ns_all = a.nslots[1][b];
  const int ns = a.use_suffix ? ns_all : 0;
  const int r = a.r, kvh = hq / r, hl = hq % r;
  const int U = (a.sel_count ? a.sel_count[b * a.hkv + kvh] : np + ns) + 1;
  const int nsplit = (U + a.split_units - 1) / a.split_units;
  if (nsplit <= 1) return;
  const int tid = threadIdx.x;
  const size_t pstride = (size_t)r * (D + 2) * kSlot;           // one split's partial
  const float* p0 = a.partial + ((((size_t)b * a.hkv + kvh) * a.max_splits) * r + hl) * (size_t)(D + 2) * kSlot;
  const int jq = tid & 7, c = tid >> 3;
  const float* po = p0 + (size_t)(c0 + c) * kSlot + 4 * jq;     // O of channel c0 + c, rows 4jq..
  const float* pm = p0 + (size_t)D * kSlot + 4 * jq;            // maxima, then sums, of the same rows
  constexpr float kNegInf = -__builtin_inff();
  float mst[4] = {kNegInf, kNegInf, kNegInf, kNegInf};
  float l[4] = {0.f, 0.f, 0.f, 0.f}, acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < nsplit; s0 += kBatch) {
    float4 v[kBatch], mv[kBatch], lv[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const size_t off = (size_t)min(s0 + u, nsplit - 1) * pstride;   // clamped repeats are masked below
      v[u] = *reinterpret_cast<const float4*>(po + off);
      mv[u] = *reinterpret_cast<const float4*>(pm + off);
      lv[u] = *reinterpret_cast<const float4*>(pm + off + kSlot);
    }
    float mn[4] = {mst[0], mst[1], mst[2], mst[3]};
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {          // clamped repeats change no maximum
      mn[0] = fmaxf(mn[0], mv[u].x); mn[1] = fmaxf(mn[1], mv[u].y);
      mn[2] = fmaxf(mn[2], mv[u].z); mn[3] = fmaxf(mn[3], mv[u].w);
    }
    // a row whose maximum is still -inf has only empty splits so far: weight 0
    auto wt = [](float m, float ref) __attribute__((always_inline)) {
      return ref == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(m - ref);
    };
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float sc = wt(mst[k], mn[k]);
      l[k] *= sc;
      acc[k] *= sc;
      mst[k] = mn[k];
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      if (s0 + u < nsplit) {
        const float w0 = wt(mv[u].x, mst[0]), w1 = wt(mv[u].y, mst[1]);
        const float w2 = wt(mv[u].z, mst[2]), w3 = wt(mv[u].w, mst[3]);
        l[0] = fmaf(lv[u].x, w0, l[0]); l[1] = fmaf(lv[u].y, w1, l[1]);
        l[2] = fmaf(lv[u].z, w2, l[2]); l[3] = fmaf(lv[u].w, w3, l[3]);
        acc[0] = fmaf(v[u].x, w0, acc[0]); acc[1] = fmaf(v[u].y, w1, acc[1]);
        acc[2] = fmaf(v[u].z, w2, acc[2]); acc[3] = fmaf(v[u].w, w3, acc[3]);
      }
    }
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) out_lds[4 * jq + k][c] = acc[k] / l[k];
  if (a.row_stats && blockIdx.z == 0 && c == 0) {
    float* rs = a.row_stats + (((size_t)b * a.hkv + kvh) * kSelHeads + hl) * 2 * kSlot + 4 * jq;
    *reinterpret_cast<float4*>(rs) = make_float4(mst[0], mst[1], mst[2], mst[3]);
    *reinterpret_cast<float4*>(rs + kSlot) = make_float4(l[0], l[1], l[2], l[3]);
  }
  __syncthreads();
  // row jj of this head: channels c0 + 4*(tid % 8) .. +3
  const int jj = tid >> 3, cc = 4 * (tid & 7);
  const size_t o = (((size_t)b * kSlot + jj) * a.hq + hq) * D + c0 + cc;
  const float4 res = *reinterpret_cast<const float4*>(&out_lds[jj][cc]);
  if (a.out_f32) {
    *reinterpret_cast<float4*>(static_cast<float*>(a.out) + o) = res;
  } else {
    uint2 w;
    w.x = f32_to_bf16_bits(res.x) | (f32_to_bf16_bits(res.y) << 16);
    w.y = f32_to_bf16_bits(res.z) | (f32_to_bf16_bits(res.w) << 16);
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + o) = w;
  }
}

// The same merge over fp16 partials (16-bit output).  Thread -> (query token
// j, channel quad q), j fastest, so each 8-byte load of a wave covers two
// whole quads of 32 rows (512 contiguous bytes).  A split's weight is its sum
// times 2^(m - max), times the power of two its row was scaled by.
template <int D>
__global__ __launch_bounds__(256) void combine_h16_kernel(const AttnArgs a) {
  constexpr int CW = 32;        // channels per workgroup
  constexpr int kBatch = 8;     // splits loaded at once
  __shared__ __align__(16) float out_lds[kSlot][CW + 4];
  const int hq = blockIdx.x, b = blockIdx.y, c0 = blockIdx.z * CW;
  const int np = a.nslots[0][b], ns_all = a.nslots[1][b];
  const int ns = a.use_suffix ? ns_all : 0;
  const int r = a.r, kvh = hq / r, hl = hq % r;
  const int U = (a.sel_count ? a.sel_count[b * a.hkv + kvh] : np + ns) + 1;
  const int nsplit = (U + a.split_units - 1) / a.split_units;
  if (nsplit <= 1) return;
  const int tid = threadIdx.x;
  const int j = tid & 31, q = tid >> 5;
  const size_t pstride = (size_t)r * PartialH16<D>::kBytes;     // one split's partials
  const uint8_t* p0 = reinterpret_cast<const uint8_t*>(a.partial) +
                      ((((size_t)b * a.hkv + kvh) * a.max_splits) * r + hl) * PartialH16<D>::kBytes;
  const uint8_t* po = p0 + ((size_t)(c0 / 4 + q) * kSlot + j) * 8;
  const float* ps = reinterpret_cast<const float*>(p0 + PartialH16<D>::kStats) + j;
  constexpr float kNegInf = -__builtin_inff();
  float mst = kNegInf, l = 0.f, acc[4] = {0.f, 0.f, 0.f, 0.f};
  auto wt = [](float m, float ref) __attribute__((always_inline)) {
    return ref == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(m - ref);
  };
  for (int s0 = 0; s0 < nsplit; s0 += kBatch) {
    uint2 v[kBatch];
    float mv[kBatch], lv[kBatch];
    int ev[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const size_t off = (size_t)min(s0 + u, nsplit - 1) * pstride;   // clamped repeats are masked below
      v[u] = *reinterpret_cast<const uint2*>(po + off);
      const float* st = reinterpret_cast<const float*>(reinterpret_cast<const uint8_t*>(ps) + off);
      mv[u] = st[0];
      lv[u] = st[kSlot];
      ev[u] = __float_as_int(st[2 * kSlot]);
    }
    float mn = mst;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) mn = fmaxf(mn, mv[u]);   // clamped repeats change no maximum
    const float sc = wt(mst, mn);
    l *= sc;
#pragma unroll
    for (int k = 0; k < 4; ++k) acc[k] *= sc;
    mst = mn;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      if (s0 + u < nsplit) {
        const float w = wt(mv[u], mst) * lv[u];
        const float wo = __builtin_amdgcn_ldexpf(w, ev[u]);
        l += w;
        acc[0] = fmaf((float)__builtin_bit_cast(_Float16, (uint16_t)(v[u].x & 0xFFFFu)), wo, acc[0]);
        acc[1] = fmaf((float)__builtin_bit_cast(_Float16, (uint16_t)(v[u].x >> 16)), wo, acc[1]);
        acc[2] = fmaf((float)__builtin_bit_cast(_Float16, (uint16_t)(v[u].y & 0xFFFFu)), wo, acc[2]);
        acc[3] = fmaf((float)__builtin_bit_cast(_Float16, (uint16_t)(v[u].y >> 16)), wo, acc[3]);
      }
    }
  }
  const float inv = 1.0f / l;
  if (a.row_stats && blockIdx.z == 0 && q == 0) {
    float* rs = a.row_stats + (((size_t)b * a.hkv + kvh) * kSelHeads + hl) * 2 * kSlot + j;
    rs[0] = mst;
    rs[kSlot] = l;
  }
  *reinterpret_cast<float4*>(&out_lds[j][4 * q]) = make_float4(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
  __syncthreads();
  // row jj of this head: channels c0 + 4*(tid % 8) .. +3
  const int jj = tid >> 3, cc = 4 * (tid & 7);
  const size_t o = (((size_t)b * kSlot + jj) * a.hq + hq) * D + c0 + cc;
  const float4 res = *reinterpret_cast<const float4*>(&out_lds[jj][cc]);
  uint2 w;
  w.x = f32_to_bf16_bits(res.x) | (f32_to_bf16_bits(res.y) << 16);
  w.y = f32_to_bf16_bits(res.z) | (f32_to_bf16_bits(res.w) << 16);
  *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + o) = w;
}

// The fp16-partial merge of a cache with rotated values (16-bit output): one
// workgroup per (query head, sequence) holds all D channels of the head's 32
// rows, so after the merge it applies the transposed rotation R^T = P^T
// (I kron H) (mix^T kron I) to each row in LDS and writes the output in the
// caller's basis (one partial when the pair has one split).  A row belongs to
// D / 4 consecutive lanes of one wave, so the Hadamard stages need only
// wave-level ordering.
struct RotCombineArgs {
  const float* partial;
  void* out;
  float* row_stats;
  const int32_t* sel_count;
  int32_t hq, hkv, r, split_units, max_splits, use_suffix;
  uint16_t nslots[2][KVQ_MAX_BATCH];
  int32_t block;                 // Hadamard block b
  float mix[64];                 // k x k, k = D / b
  uint8_t perm_inv[128];         // output channel c takes rotated coordinate perm_inv[c]
};

__device__ __forceinline__ void row_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int D>
__global__ __launch_bounds__(64 * D / 8) void combine_rot_kernel(const RotCombineArgs a) {
  constexpr int kBatch = 8;     // splits loaded at once
  constexpr int TPR = D / 4;    // threads per row in the rotation (four channels each)
  __shared__ __align__(16) float zb[kSlot][D + 4];   // merged rows (rotated basis)
  __shared__ __align__(16) float yb[kSlot][D + 4];   // after the transposed mix
  const int hq = blockIdx.x, b = blockIdx.y;
  const int np = a.nslots[0][b], ns_all = a.nslots[1][b];
  const int ns = a.use_suffix ? ns_all : 0;
  const int r = a.r, kvh = hq / r, hl = hq % r;
  const int U = (a.sel_count ? a.sel_count[b * a.hkv + kvh] : np + ns) + 1;
  const int nsplit = (U + a.split_units - 1) / a.split_units;
  const int chunk = threadIdx.x >> 8, tid = threadIdx.x & 255;
  const int j = tid & 31, q = tid >> 5;
  const int c0 = chunk * 32;
  const size_t pstride = (size_t)r * PartialH16<D>::kBytes;
  const uint8_t* p0 = reinterpret_cast<const uint8_t*>(a.partial) +
                      ((((size_t)b * a.hkv + kvh) * a.max_splits) * r + hl) * PartialH16<D>::kBytes;
  const uint8_t* po = p0 + ((size_t)(c0 / 4 + q) * kSlot + j) * 8;
  const float* ps = reinterpret_cast<const float*>(p0 + PartialH16<D>::kStats) + j;
  float mst = -__builtin_inff(), l = 0.f, acc[4] = {0.f, 0.f, 0.f, 0.f};
  auto wt = [](float m, float ref) __attribute__((always_inline)) {
    return ref == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(m - ref);
  };
  for (int s0 = 0; s0 < nsplit; s0 += kBatch) {
    uint2 v[kBatch];
    float mv[kBatch], lv[kBatch];
    int ev[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const size_t off = (size_t)min(s0 + u, nsplit - 1) * pstride;   // clamped repeats are masked below
      v[u] = *reinterpret_cast<const uint2*>(po + off);
      const float* st = reinterpret_cast<const float*>(reinterpret_cast<const uint8_t*>(ps) + off);
      mv[u] = st[0];
      lv[u] = st[kSlot];
      ev[u] = __float_as_int(st[2 * kSlot]);
    }
    float mn = mst;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) mn = fmaxf(mn, mv[u]);
    const float sc = wt(mst, mn);
    l *= sc;
#pragma unroll
    for (int k = 0; k < 4; ++k) acc[k] *= sc;
    mst = mn;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      if (s0 + u < nsplit) {
        const float w = wt(mv[u], mst) * lv[u];
        const float wo = __builtin_amdgcn_ldexpf(w, ev[u]);
        l += w;
        acc[0] = fmaf((float)__builtin_bit_cast(_Float16, (uint16_t)(v[u].x & 0xFFFFu)), wo, acc[0]);
        acc[1] = fmaf((float)__builtin_bit_cast(_Float16, (uint16_t)(v[u].x >> 16)), wo, acc[1]);
        acc[2] = fmaf((float)__builtin_bit_cast(_Float16, (uint16_t)(v[u].y & 0xFFFFu)), wo, acc[2]);
        acc[3] = fmaf((float)__builtin_bit_cast(_Float16, (uint16_t)(v[u].y >> 16)), wo, acc[3]);
      }
    }
  }
  const float inv = 1.0f / l;
  if (a.row_stats && chunk == 0 && q == 0) {
    float* rs = a.row_stats + (((size_t)b * a.hkv + kvh) * kSelHeads + hl) * 2 * kSlot + j;
    rs[0] = mst;
    rs[kSlot] = l;
  }
  *reinterpret_cast<float4*>(&zb[j][c0 + 4 * q]) = make_float4(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
  __syncthreads();
  // row rr, lane-in-row e0 (TPR lanes of one wave per row)
  const int rr = threadIdx.x / TPR, e0 = threadIdx.x % TPR;
  const int blk = a.block, k = D / blk;
  // transposed mix: y[l*b + i] = sum over m of mix[m][l] * z[m*b + i]
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int e = e0 + TPR * t, lb = e / blk, i = e % blk;
    float acc_m = 0.f;
    for (int m = 0; m < k; ++m) acc_m = fmaf(a.mix[m * k + lb], zb[rr][m * blk + i], acc_m);
    yb[rr][e] = acc_m;
  }
  row_sync();
  for (int h = 1; h < blk; h *= 2) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int p = e0 + TPR * t;                // pair index
      const int i = (p / h) * 2 * h + p % h;
      const float x = yb[rr][i], y = yb[rr][i + h];
      yb[rr][i] = x + y;
      yb[rr][i + h] = x - y;
    }
    row_sync();
  }
  // output channels c .. c + 3 of the row: x[c] = y[perm_inv[c]] / sqrt(b)
  const float inv_sqrt_b = blk == 16 ? 0.25f : 0.125f;
  const int c = 4 * e0;
  const float x0 = yb[rr][a.perm_inv[c]] * inv_sqrt_b, x1 = yb[rr][a.perm_inv[c + 1]] * inv_sqrt_b;
  const float x2 = yb[rr][a.perm_inv[c + 2]] * inv_sqrt_b, x3 = yb[rr][a.perm_inv[c + 3]] * inv_sqrt_b;
  uint2 w;
  w.x = f32_to_bf16_bits(x0) | (f32_to_bf16_bits(x1) << 16);
  w.y = f32_to_bf16_bits(x2) | (f32_to_bf16_bits(x3) << 16);
  const size_t o = (((size_t)b * kSlot + rr) * a.hq + hq) * D + c;
  *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + o) = w;
}

template <int KB, int VB, int D>
hipError_t launch_kbd(const AttnArgs& a, int grid_splits, int B, hipStream_t s, const RotParams* unrot) {
  const dim3 grid = a.num_wg ? dim3(a.num_wg) : dim3(grid_splits, a.hkv, B);
  const dim3 block((kProducerWaves + a.r) * 64);   // producers + one consumer per query head
  bool done = false;
  if constexpr (KB == 4 && VB == 4) {
    if (a.fmt == 1) {
      if (a.r <= 4) hipLaunchKernelGGL((attn_kernel<KB, VB, D, 4, false, 1>), grid, block, 0, s, a);
      else          hipLaunchKernelGGL((attn_kernel<KB, VB, D, 8, false, 1>), grid, block, 0, s, a);
      done = true;
    }
  }
  if (done) {
  } else if (a.fmt == 2) {
    if (a.r <= 4) hipLaunchKernelGGL((attn_kernel<KB, VB, D, 4, false, 2>), grid, block, 0, s, a);
    else          hipLaunchKernelGGL((attn_kernel<KB, VB, D, 8, false, 2>), grid, block, 0, s, a);
  } else if (a.v_centred) {
    if (a.r <= 4) hipLaunchKernelGGL((attn_kernel<KB, VB, D, 4, true, 0>), grid, block, 0, s, a);
    else          hipLaunchKernelGGL((attn_kernel<KB, VB, D, 8, true, 0>), grid, block, 0, s, a);
  } else {
    if (a.r <= 4) hipLaunchKernelGGL((attn_kernel<KB, VB, D, 4, false, 0>), grid, block, 0, s, a);
    else          hipLaunchKernelGGL((attn_kernel<KB, VB, D, 8, false, 0>), grid, block, 0, s, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.force_partials) {
    RotCombineArgs c;
    std::memset(&c, 0, sizeof(c));
    c.partial = a.partial;
    c.out = a.out;
    c.row_stats = a.row_stats;
    c.sel_count = a.sel_count;
    c.hq = a.hq; c.hkv = a.hkv; c.r = a.r;
    c.split_units = a.split_units; c.max_splits = a.max_splits; c.use_suffix = a.use_suffix;
    std::memcpy(c.nslots, a.nslots, sizeof(c.nslots));
    c.block = unrot->block;
    const int k = D / unrot->block;
    for (int i = 0; i < k * k; ++i) c.mix[i] = unrot->mix[i];
    for (int i = 0; i < D; ++i) c.perm_inv[unrot->perm[i]] = (uint8_t)i;
    hipLaunchKernelGGL((combine_rot_kernel<D>), dim3(a.hq, B), dim3(64 * D / 8), 0, s, c);
    return hipGetLastError();
  }
  if (grid_splits <= 1) return e;
  if (a.out_f32) hipLaunchKernelGGL((combine_kernel<D>), dim3(a.hq, B, D / 32), dim3(256), 0, s, a);
  else           hipLaunchKernelGGL((combine_h16_kernel<D>), dim3(a.hq, B, D / 32), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int KB, int VB>
hipError_t launch_kb(const AttnArgs& a, int grid_splits, int B, int D, hipStream_t s, const RotParams* unrot) {
  return D == 64 ? launch_kbd<KB, VB, 64>(a, grid_splits, B, s, unrot) : launch_kbd<KB, VB, 128>(a, grid_splits, B, s, unrot);
}

}  // namespace

// Workspace of kvq_block_attn_noalloc: split partials and rotation staging.
// Each device holds its own copy for the life of the process; every call on a
// device shares it, so calls that overlap on one device race.
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

hipError_t noalloc_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));   // the current device's copy
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_attention(const AttnArgs& a, int grid_splits, int B, int D, int kb, int vb,
                            hipStream_t stream, const RotParams* unrot) {
  if (a.force_partials && !unrot) return hipErrorInvalidValue;
  if (kb == 4 && vb == 4) return launch_kb<4, 4>(a, grid_splits, B, D, stream, unrot);
  if (kb == 4 && vb == 2) return launch_kb<4, 2>(a, grid_splits, B, D, stream, unrot);
  if (kb == 2 && vb == 4) return launch_kb<2, 4>(a, grid_splits, B, D, stream, unrot);
  return launch_kb<2, 2>(a, grid_splits, B, D, stream, unrot);
}

}  // namespace kvq
