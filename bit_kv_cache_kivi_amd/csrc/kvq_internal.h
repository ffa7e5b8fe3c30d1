// Internal declarations shared by the host library and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/kvq.h"

namespace kvq {

constexpr int kSlot = 32;         // tokens per slot = K group = block length
constexpr int kHeaderBytes = 16;  // slot header

// One new slot of a commit: tokens [src_tok, src_tok + nvalid) of sequence b.
struct CommitTask {
  int32_t b;
  int32_t dst_slot;    // slot index inside the segment
  int32_t src_tok;     // first token row in the commit's input
  int32_t nvalid;      // 1..32
  uint32_t mask;       // protected tokens of the slot
  int32_t rank_base;   // rank of its first protected row
  int32_t token_base;  // segment position of its first token
  int32_t pad;
};
static_assert(sizeof(CommitTask) == 32, "task layout");

struct SegPtrs {
  uint8_t* records;     // [B][Hkv][slot_cap] records
  uint8_t* headers;     // [B][slot_cap] 16-byte headers
  uint16_t* prot_rows;  // [B][Hkv][prot_cap][D] bf16 bits
  int32_t* prot_pos;    // [B][prot_cap]
  int32_t slot_cap;
  int32_t prot_cap;
};

constexpr int kInlineTasks = 64;  // commits with at most this many new slots pass their tasks by value

// K-RPBH value rotation: permutation of the D channels, Hadamard transform on
// blocks of `block` channels, k x k mix (k = D / block, row-major) across the
// blocks.  block == 0: no rotation.
struct RotParams {
  int32_t block;
  int32_t perm[128];
  float mix[64];
};

struct CommitArgs {
  const void* k;        // [B, n_max, Hkv, D]
  const void* v;
  const CommitTask* tasks;  // device task table (used when use_inline == 0)
  SegPtrs seg;
  int32_t n_max;
  int32_t hkv;
  int32_t gv_log2;
  uint32_t record_bytes;
  int32_t use_inline;
  int32_t num_cus;          // compute units of the device (sizes the persistent grid)
  RotParams rot;            // values are rotated before quantization when rot.block != 0
  int32_t fmt;              // record format: 0 integer, 1 MX FP4, 2 integer with fp16 metadata
  CommitTask inline_tasks[kInlineTasks];
};
static_assert(sizeof(CommitArgs) <= 4096, "commit launch arguments fit the kernel-argument segment");

constexpr int kMaxWgTable = 256;  // attention workgroups listed in the launch arguments

struct AttnArgs {
  const void* q;        // [B, 32, Hq, D]
  const void* k_blk;    // [B, 32, Hkv, D]
  const void* v_blk;
  void* out;            // [B, 32, Hq, D]
  float* partial;       // split-K partials
  SegPtrs seg[2];
  float scale_log2;     // softmax_scale * log2(e)
  int32_t hq, hkv, r;
  int32_t q_f32, blk_f32, out_f32;
  int32_t gv_log2;
  uint32_t record_bytes;
  int32_t split_units;  // units (slots + block) per split
  int32_t max_splits;
  int32_t use_suffix;
  int32_t v_centred;    // values in a rotated basis: dequantized around the middle code
  int32_t fmt;          // record format: 0 integer, 1 MX FP4, 2 integer with fp16 metadata
  // selection (all null without one): per (b, kv head) the number of listed
  // units, the listed cached units, and each cached unit's selected tokens
  const int32_t* sel_count;
  const int32_t* sel_units;
  const uint32_t* sel_mask;
  int32_t sel_ucap;
  uint16_t nslots[2][KVQ_MAX_BATCH];   // per-sequence slot counts of both segments
  // Fused commit of the block (commit_blk != 0): after its attention work,
  // the workgroup that holds the block of (b, kv head) quantizes the block's
  // first cvalid[b] tokens into prefix slot nslots[0][b], with protected
  // tokens cmask[b] (rank and token bases follow the previous slot's header).
  int32_t commit_blk;
  uint32_t cmask[KVQ_MAX_BATCH];
  uint8_t cvalid[KVQ_MAX_BATCH];
  // Workgroup list of a one-dimensional grid: entry i = split | kvh << 8 |
  // b << 16 for workgroup i, only splits that hold units.  num_wg == 0: a
  // (splits, Hkv, B) grid instead, whose workgroups past a sequence's splits
  // exit at once.
  int32_t num_wg;
  // Row statistics (null: not written): per (b, kv head, head of the group,
  // query token) the softmax reference maximum (log2 units, scores times
  // scale_log2) and the sum of exp2(score - maximum) over every attended
  // token, fp32 [B][Hkv][kSelHeads][2][32], written by the workgroup that
  // finishes the row (the attention itself with one split, else the combine)
  float* row_stats;
  // Rotated values with a 16-bit output: every (sequence, kv head) hands its
  // splits (one included) to the merge as fp16 partials, and the merge also
  // applies the transposed rotation
  int32_t force_partials;
  uint32_t wg[kMaxWgTable];
};
static_assert(sizeof(AttnArgs) <= 4096, "attention launch arguments fit the kernel-argument segment");

// The current block's keys converted to fp32 and its values rotated, rows
// [B * 32 * Hkv] of D (the attention then sees the rotated value basis).
struct BlkPrepArgs {
  const void* k;
  const void* v;
  float* k_out;
  float* v_out;
  int64_t rows;
  int32_t in_f32;
  RotParams rot;
};

// Transposed rotation of attention output rows [B * 32 * Hq] of D (fp32) into
// the caller's output.
struct UnrotArgs {
  const float* src;
  void* out;
  int64_t rows;
  int32_t out_f32;
  RotParams rot;
};

constexpr int kMaxSelSplit = 64;  // units per split of a selection pass
constexpr int kSelHeads = 8;      // query heads per kv head in the selection's row statistics

// Mask-query selection: the stats pass (MODE 0) and the score pass (MODE 1)
// run over the cached units of every (sequence, kv head) in splits of
// split_units units; MODE 0 also covers the block (the last unit).
struct SelArgs {
  const void* q;        // [B, 32, Hq, D]
  const void* k_blk;    // [B, 32, Hkv, D]
  SegPtrs seg[2];
  float* partial;       // per split: [B][Hkv][max_splits][8 heads][2][32] (maximum, sum)
  float* contrib;       // [B][Hkv][ucap * 32]; -1 for invalid entries
  float* unit_contrib;  // [B][Hkv][ucap]: sum over each unit's valid entries
  float scale_log2;
  int32_t hq, hkv, r, q_f32, blk_f32, gv_log2;
  uint32_t record_bytes;
  int32_t split_units;        // this pass
  int32_t stats_split_units;  // the stats pass (the score pass merges its partials)
  int32_t max_splits;
  int32_t use_suffix;
  int32_t ucap;               // prefix_slots + suffix_slots
  uint32_t qmask[KVQ_MAX_BATCH];
  uint16_t nslots[2][KVQ_MAX_BATCH];
};
static_assert(sizeof(SelArgs) <= 4096, "selection launch arguments fit the kernel-argument segment");

// Exact top-k of the contributions per (sequence, kv head), ties to the lower
// entry; writes per-unit token masks, the list of units with a selected
// token, and its length.
struct TopkArgs {
  const float* contrib;
  const float* unit_contrib;
  int32_t granularity;  // 1: entries ranked one by one; 32: whole units by their sums
  uint32_t* sel_mask;   // [B][Hkv][ucap]
  int32_t* sel_units;   // [B][Hkv][ucap]
  int32_t* sel_count;   // [B][Hkv]
  int32_t hkv, ucap, budget;
  int32_t nunits[KVQ_MAX_BATCH];    // cached units of each sequence (prefix + suffix if used)
};

// Record field offsets for (D, kb, vb, G_v): see include/kvq.h.
__host__ __device__ constexpr uint32_t kc_bytes(int D, int kb) { return kSlot * D * kb / 8; }
__host__ __device__ constexpr uint32_t vc_bytes(int D, int vb) { return D * vb * 4; }
__host__ __device__ constexpr uint32_t kmeta_bytes(int D) { return 2 * D * 4; }
__host__ __device__ constexpr uint32_t vmeta_bytes(int D, int gv) { return (D / gv) * 2 * kSlot * 4; }
__host__ __device__ constexpr uint32_t record_bytes(int D, int kb, int vb, int gv) {
  return (kc_bytes(D, kb) + vc_bytes(D, vb) + kmeta_bytes(D) + vmeta_bytes(D, gv) + 255u) / 256u * 256u;
}
// MX FP4 records: 4-bit codes, one scale byte per key channel and per (value group, token)
__host__ __device__ constexpr uint32_t record_bytes_mx(int D) {
  return (kc_bytes(D, 4) + vc_bytes(D, 4) + 2u * D + 255u) / 256u * 256u;
}
// integer codes with fp16 scales and zeros
__host__ __device__ constexpr uint32_t record_bytes_h16(int D, int kb, int vb, int gv) {
  return (kc_bytes(D, kb) + vc_bytes(D, vb) + kmeta_bytes(D) / 2 + vmeta_bytes(D, gv) / 2 + 255u) / 256u * 256u;
}

// Launchers (defined in the .hip files); return the launch status.
hipError_t launch_commit(const CommitArgs& a, int ntasks, int D, int kb, int vb, bool f32_in,
                         hipStream_t stream);
// unrot: with a.force_partials, the rotation whose transpose the merge applies
hipError_t launch_attention(const AttnArgs& a, int grid_splits, int B, int D, int kb, int vb,
                            hipStream_t stream, const RotParams* unrot = nullptr);
hipError_t launch_blk_prep(const BlkPrepArgs& a, int D, hipStream_t stream);
hipError_t launch_select(const SelArgs& a, int mode, int grid_splits, int B, int D, int kb, int vb,
                         hipStream_t stream);
hipError_t launch_topk(const TopkArgs& a, int B, hipStream_t stream);
hipError_t launch_unrotate(const UnrotArgs& a, int D, hipStream_t stream);

// The allocation-free attention's workspace: a file-scope device array of
// kNoAllocScratchBytes (attn.hip), one per device, whose device address is
// looked up once per device (hipGetSymbolAddress, with that device current).
constexpr size_t kNoAllocScratchBytes = KVQ_NOALLOC_SCRATCH_BYTES;
hipError_t noalloc_scratch(void** ptr);

}  // namespace kvq
