/*
 * kvq.h — C ABI of a low-bit KV cache for block-diffusion language models on
 * AMD Instinct MI355X (gfx950).
 *
 * Two operations make up the path:
 *
 *  1. kvq_commit: when a block of tokens is finished, its keys and values are
 *     quantized once into packed 2- or 4-bit codes and appended to a per-layer
 *     cache.  Keys use KIVI-style asymmetric quantization with one (scale, zero)
 *     per channel over a group of 32 consecutive tokens; values use one
 *     (scale, zero) per token over a group of G_v consecutive channels.  A
 *     per-layer set of key token rows chosen by the caller is kept in bf16 and is
 *     excluded from quantization.
 *     Sources: Tai et al., "KV Cache Quantization for Diffusion Language Models"
 *     (Findings of EMNLP 2026, ACL Anthology record, abstract: KIVI adapted to
 *     prefix and dual cache reuse; KProtect keeps chosen per-layer K-cache
 *     entries in high precision while values use standard low-bit quantization);
 *     "SoloQ: Calibration-Free Quantization for Diffusion Language Models"
 *     (summary page, paragraph on block diffusion: KV entries are quantized only
 *     when a block is committed, the block being denoised stays in full
 *     precision, keys use KIVI-style per-channel asymmetric quantization).
 *
 *  2. kvq_block_attn: the block still being denoised (32 query tokens per
 *     sequence, full precision) attends bidirectionally to itself and to the
 *     quantized prefix cache, optionally also to a quantized suffix cache of
 *     masked future tokens ("dual cache").  Attention is computed directly from
 *     the low-bit codes; no full-precision copy of the cache is materialised.
 *     Sources: MaskAhead / Q-MaskAhead abstract (attention directly from low-bit
 *     KV, cache attended at every denoising step); SoloQ summary page (a
 *     diffusion LM revisits bidirectional context at every denoising step);
 *     Elastic-Cache abstract, observation (1) (distant MASK tokens can be cached
 *     block-wise beyond the active window), for the suffix segment.
 *
 * The pages give no formula; the quantizer is the plain asymmetric min/max one,
 * evaluated in IEEE fp32 in this order:
 *     mn = min(group), mx = max(group)
 *     scale = (mx - mn) / (2^b - 1)   (fp32 subtract, fp32 division), then + 0.0f
 *     zero  = mn + 0.0f               (both stored as canonical +0 when zero)
 *     code  = scale == 0 ? 0 : clamp(rint((x - mn) / scale), 0, 2^b - 1)
 *             (fp32 subtract, fp32 division, round half to even)
 * Dequantized value: code * scale + zero.
 *
 * ------------------------------------------------------------------------
 * Ownership, threading and errors
 * ------------------------------------------------------------------------
 *  - The caller owns all device memory: the cache buffer handed to kvq_create
 *    (kvq_required_bytes bytes, 256-byte aligned), inputs and outputs.  The
 *    library never allocates device memory.  Commits of more than 64 slots
 *    take their task table from a ring of eight pinned host tables (read by
 *    the commit kernel directly from host memory) with eight events, one ring
 *    per device shared by every handle and thread (calls on it are
 *    serialised by a lock), created by the first such commit, grown to the
 *    largest table a handle needs (32 bytes x batch x the larger segment's
 *    slot capacity, per table) and held until the process ends.  No other
 *    call allocates anything.
 *  - Pointers named d_* are device pointers; h_* are host pointers read only
 *    during the call.  `stream` is a hipStream_t (NULL = default stream).
 *  - Calls are asynchronous and stream-ordered, with one exception: a commit of
 *    more than 64 slots (a prefill) reuses one of the eight pinned task tables
 *    and blocks the calling thread until the kernel that last read that table
 *    has finished, i.e. only while eight such commits (of any handle) are
 *    still in flight on the device; growing the ring waits for all eight.
 *    All calls on one handle must be
 *    issued on one stream or be ordered by the caller.  A handle is not
 *    thread-safe.
 *  - Every call returns a kvq_status.  All argument checks run on the host
 *    before any device work; on any error the cache is unchanged.
 *    kvq_last_error() gives a thread-local detail string for the last failure.
 *
 * ------------------------------------------------------------------------
 * Packed cache layout (part of the ABI; little-endian)
 * ------------------------------------------------------------------------
 * A cache has two segments: PREFIX (committed blocks) and SUFFIX (the masked
 * future tokens of the dual cache).  Each segment holds, per sequence, a list of
 * slots; a slot holds the tokens of one 32-token quantization group.  Each
 * commit starts a new slot at its first token; its last slot may be partial and
 * is never reopened.
 *
 * Slot record, one per (segment, sequence b, kv head h, slot s), located at
 *     records_offset[seg] + ((b * Hkv + h) * slot_cap[seg] + s) * record_bytes
 *   Kc    at kc_offset    (= 0): D*kb/32 word columns of 32 tokens; word w
 *         of token t is the u32 at byte (w*32 + t)*4.  Word w holds channels
 *         [w*32/kb, (w+1)*32/kb); channel c sits at bits [kb*(c mod 32/kb), +kb).
 *   Vc    at vc_offset    (= 32*D*kb/8): vb word rows of D channels; word j of
 *         channel c is the u32 at byte (j*D + c)*4.  Token t of channel c is
 *         placed by
 *             mm = t / 16,  h = (t / 4) % 2,  e = (t % 4) + 4 * ((t / 8) % 2)
 *         vb = 4: word 2*mm + h, bits [4e, 4e+4)
 *         vb = 2: word h,        bits [2*(8*mm + e), +2)
 *         (this order puts the 8 tokens one MFMA lane consumes in one u32, and
 *         the word-major order lets consecutive threads read consecutive words).
 *   Kmeta at kmeta_offset (= vc_offset + 4*D*vb): fp32 scale[D], fp32 zero[D].
 *   Vmeta at vmeta_offset (= kmeta_offset + 8*D): for each channel group
 *         g < D/G_v: fp32 scale[32 tokens], fp32 zero[32 tokens].
 *   record_bytes = the above rounded up to a multiple of 256.
 *   Codes of invalid tokens (past the slot's count) are 0, and so are their V
 *   scale/zero; codes of protected tokens in Kc are 0 and protected tokens do not
 *   enter the per-channel K statistics.  A channel group with no contributing
 *   token has scale = zero = 0.
 *
 * Slot header, one per (segment, b, s), 16 bytes at
 *     headers_offset[seg] + (b * slot_cap[seg] + s) * 16:
 *   int32 nvalid     tokens in the slot (1..32)
 *   uint32 prot_mask bit t set <=> token t of the slot is protected
 *   int32 prot_base  rank of the slot's first protected row in the segment
 *   int32 token_base segment position of the slot's first token
 *
 * Protected K rows, per (segment, b): rank r in [0, nprot) in ascending
 * position order (a slot's rows for one kv head are contiguous):
 *   bf16 rows at prot_rows_offset[seg] + ((b * Hkv + h) * prot_cap[seg] + r) * D * 2
 *   int32 position at prot_pos_offset[seg] + (b * prot_cap[seg] + r) * 4
 * A protected token's row in slot s is rank prot_base + popcount(prot_mask & ((1<<t)-1)).
 *
 * MX FP4 records (kv_format = KVQ_FMT_MXFP4; k_bits = v_bits = 4, G_v = 32,
 * no value rotation, no selection).  A hardware-native 4-bit floating-point
 * format with per-block scales (SoloQ abstract and summary page: NVFP4; here
 * the OCP microscaling FP4 that gfx950 converts natively):
 *   codes: E2M1 (sign << 3 | index into {0, .5, 1, 1.5, 2, 3, 4, 6}) at the
 *          4-bit positions of Kc and Vc above;
 *   Kmeta at kmeta_offset: one E8M0 byte s per key channel (D bytes);
 *   Vmeta at vmeta_offset: per 32-channel group g, one byte per token (32 bytes);
 *   record_bytes = (32*D + 2*D) rounded up to a multiple of 256.
 * A group (key: one channel over the slot's valid, unprotected tokens; value: 32
 * channels of a valid token) with largest magnitude amax gets
 *   s = max(E(amax) - 2, 0), E(amax) the biased exponent field of amax in fp32,
 *   code = E2M1 round-to-nearest-even (saturating at 6) of x * 2^(127 - s),
 *   sign from the sign bit of x; a group with amax = 0 (or no member) has s = 0
 *   and codes 0.  Dequantized value: e2m1(code) * 2^(s - 127).
 *
 * fp16 metadata (kv_format = KVQ_FMT_INT_H16; no value rotation, no selection).
 * An engineering variant of the same quantizer (the pages fix no width for
 * the quantization constants): the integer codes above with every scale and
 * zero stored in fp16, which halves the metadata bytes:
 *   Kmeta at kmeta_offset: fp16 scale[D], then fp16 zero[D];
 *   Vmeta at vmeta_offset: per channel group g (D / G_v of them, 128 bytes
 *          apart): fp16 scale[32 tokens], then fp16 zero[32 tokens];
 *   record_bytes = (Kc + Vc + 4*D + 128 * D / G_v) rounded up to 256.
 * scale16 and zero16 are the fp32 scale and zero above rounded to fp16 (nearest,
 * ties to even; -0 stored as +0), and the codes are taken against that pair:
 *   code = scale16 == 0 ? 0 : clamp(rint((x - zero16) / scale16), 0, 2^b - 1)
 * (fp32 subtraction and correctly rounded division), so code * scale16 + zero16
 * is the stored reconstruction.  Group values must lie within the fp16 range
 * (|x| <= 65504); a group whose scale or zero overflows fp16 gets unspecified codes.
 */
#ifndef KVQ_H_
#define KVQ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVQ_ABI_VERSION 7
#define KVQ_SLOT_TOKENS 32   /* K group size along tokens = block length */
#define KVQ_MAX_BATCH 256

typedef enum {
  KVQ_OK = 0,
  KVQ_EINVAL = 1,       /* malformed argument (null, out of range, unsorted list, ...) */
  KVQ_EUNSUPPORTED = 2, /* well-formed but outside the supported set */
  KVQ_ECAPACITY = 3,    /* the commit would exceed a slot or protected-row capacity */
  KVQ_EHIP = 4          /* a HIP runtime call failed; see kvq_last_error() */
} kvq_status;

typedef enum { KVQ_F32 = 0, KVQ_BF16 = 1 } kvq_dtype;
typedef enum { KVQ_PREFIX = 0, KVQ_SUFFIX = 1 } kvq_segment;

typedef struct {
  int32_t batch;             /* B, 1..KVQ_MAX_BATCH                                 */
  int32_t num_kv_heads;      /* Hkv >= 1                                            */
  int32_t head_dim;          /* D in {64, 128}                                      */
  int32_t k_bits, v_bits;    /* each in {2, 4}                                      */
  int32_t k_group_tokens;    /* must be 32                                          */
  int32_t v_group_channels;  /* G_v in {32, 64, 128}, G_v <= D, D % G_v == 0        */
  int32_t prefix_slots;      /* slot capacity per sequence, 1..65535                */
  int32_t suffix_slots;      /* 0..65535 (0 = no suffix segment)                    */
  int32_t prefix_protected;  /* protected-row capacity per sequence, >= 0           */
  int32_t suffix_protected;  /* >= 0                                                */
  int32_t max_q_heads;       /* largest Hq passed to kvq_block_attn (Hq % Hkv == 0) */
  int32_t max_splits;        /* split-K partial capacity per (b, kv head); 0 = 32   */
  int32_t v_rotation_block;  /* 0 = values stored as they are; 16 or 64 = K-RPBH      */
                             /* rotated values (see kvq_set_v_rotation), D % b == 0 */
  int32_t protect_sink;      /* != 0: a prefix commit that starts a sequence (segment  */
                             /* position 0) also protects that first token's key row, */
                             /* counted against prefix_protected (SoloQ summary page, */
                             /* paragraph on keeping the attention sink in full       */
                             /* precision, which matters at 2-bit KV)                 */
  int32_t kv_format;         /* KVQ_FMT_INT (0): the asymmetric integer codes above;   */
                             /* KVQ_FMT_MXFP4 (1): see "MX FP4 records" below;         */
                             /* KVQ_FMT_INT_H16 (2): see "fp16 metadata" below         */
} kvq_config;

enum { KVQ_FMT_INT = 0, KVQ_FMT_MXFP4 = 1, KVQ_FMT_INT_H16 = 2 };

typedef struct {
  uint64_t total_bytes;          /* == kvq_required_bytes                          */
  uint64_t record_bytes;
  uint64_t kc_offset, vc_offset, kmeta_offset, vmeta_offset; /* within a record   */
  uint64_t records_offset[2];
  uint64_t headers_offset[2];
  uint64_t prot_rows_offset[2];
  uint64_t prot_pos_offset[2];
  int32_t slot_cap[2];
  int32_t prot_cap[2];
  uint64_t workspace_offset, workspace_bytes; /* attention split-K partials       */
  uint64_t rotation_offset, rotation_bytes;   /* rotated-value attention staging:
                                                 block K and V in fp32, then the
                                                 rotated output; 0 bytes when
                                                 v_rotation_block == 0            */
  /* Selection results (kvq_select), ucap = prefix_slots + suffix_slots cached
   * units per (b, kv head), numbered prefix slots first, then suffix slots:   */
  uint64_t sel_contrib_offset; /* fp32 [B][Hkv][ucap][32] contribution per entry,
                                  -1 at slot positions past the valid tokens   */
  uint64_t sel_unit_offset;    /* fp32 [B][Hkv][ucap] sum of each unit's valid
                                  entries' contributions                       */
  uint64_t sel_mask_offset;    /* uint32 [B][Hkv][ucap] selected tokens per unit */
  uint64_t sel_units_offset;   /* int32 [B][Hkv][ucap] units with a selected
                                  token, ascending                             */
  uint64_t sel_count_offset;   /* int32 [B][Hkv] length of that list          */
  uint64_t sel_stats_offset;   /* fp32 [B][Hkv][8][2][32] kvq_attend_select's
                                  softmax statistics per (query head of the
                                  group, query token): reference maximum of
                                  score * softmax_scale * log2(e), then the
                                  sum of exp2(that - maximum)                 */
} kvq_layout;

typedef struct kvq_cache kvq_cache;

/* Bytes of device memory a cache with this configuration needs; 0 if the
 * configuration is invalid or unsupported (see kvq_last_error). */
size_t kvq_required_bytes(const kvq_config* cfg);

/* Fills *out with the region offsets of a cache with this configuration. */
kvq_status kvq_get_layout(const kvq_config* cfg, kvq_layout* out);

/* Creates a handle over d_buf (device, >= kvq_required_bytes, 256-byte aligned,
 * must outlive the handle).  Host-only: touches no device memory.  The cache
 * starts empty; nothing in d_buf needs initialising. */
kvq_status kvq_create(const kvq_config* cfg, void* d_buf, size_t buf_bytes, kvq_cache** out);

/* Frees the host-side handle (host memory only; the device's shared task-table
 * ring stays).  Waits for nothing.  NULL is accepted. */
kvq_status kvq_destroy(kvq_cache* c);

/* Quantize-on-commit.  Appends, for every sequence b, the first h_ntok[b]
 * tokens of d_k / d_v (each [B, n_max, Hkv, D] contiguous, dtype in_dtype,
 * 16-byte aligned) to segment `segment` as ceil(h_ntok[b] / 32) new slots.
 * h_ntok: host [B], each in 0..n_max, or NULL for n_max everywhere.
 * Protected rows: host CSR h_prot_off [B+1] (h_prot_off[0] == 0, non-decreasing)
 * and h_prot_idx, positions relative to this commit's first token, strictly
 * increasing within each sequence and < h_ntok[b]; both NULL for none.
 * reset_segment != 0 first empties the segment for every sequence (used to
 * replace the dual cache's suffix wholesale).
 * Errors: KVQ_EINVAL for malformed arguments, KVQ_ECAPACITY if a sequence would
 * exceed slot or protected capacity; the cache is unchanged in both cases. */
kvq_status kvq_commit(kvq_cache* c, int32_t segment, int32_t reset_segment,
                      const void* d_k, const void* d_v, int32_t in_dtype, int32_t n_max,
                      const int32_t* h_ntok, const int32_t* h_prot_off, const int32_t* h_prot_idx,
                      void* stream);

/* Fused dequantize-and-attend of the current block.
 * d_q [B, L, Hq, D], d_k_blk / d_v_blk [B, L, Hkv, D] (dtype blk_dtype),
 * d_out [B, L, Hq, D] (dtype out_dtype), all contiguous and 16-byte aligned;
 * L must be 32; Hq % Hkv == 0, Hq <= max_q_heads.  Query head hq uses kv head
 * hq / (Hq / Hkv).  Every query token attends, without a mask, to all L block
 * tokens, every valid prefix token and, if use_suffix != 0, every valid suffix
 * token; a protected prefix/suffix key is its stored bf16 row.  Scores are
 * q.k * softmax_scale.  MFMA operands are fp16, accumulation fp32.
 * Inputs must be finite with |x| < 65504 (the fp16 operand range). */
kvq_status kvq_block_attn(kvq_cache* c, int32_t use_suffix,
                          const void* d_q, int32_t num_q_heads, int32_t q_dtype,
                          const void* d_k_blk, const void* d_v_blk, int32_t blk_dtype,
                          int32_t block_len, float softmax_scale,
                          void* d_out, int32_t out_dtype, void* stream);

/* kvq_block_attn for callers that cannot allocate or touch workspace they do
 * not own (code under stream capture, tight serving loops, harnesses that
 * forbid allocation): the same arguments, kernels and results (outputs
 * bit-identical to kvq_block_attn's), but the split partials and, with value
 * rotation, the rotation staging live in a device array owned by the library,
 * of KVQ_NOALLOC_SCRATCH_BYTES, that each device holds until the process
 * ends; the cache buffer's workspace region is not touched.  The call
 * allocates nothing (no hipMalloc, no host allocation).  Every call on one
 * device shares that array, so calls that overlap on one device (other
 * streams, other handles, other threads) race and must be ordered by the
 * caller.  A launch whose workspace would exceed the array returns
 * KVQ_ECAPACITY before any device work (the default split plan needs at most
 * 256 workgroups x (Hq/Hkv) x (D + 2) x 32 x 4 bytes, about 34 MB at Hq/Hkv = 8,
 * D = 128). */
#define KVQ_NOALLOC_SCRATCH_BYTES (64u << 20)
kvq_status kvq_block_attn_noalloc(kvq_cache* c, int32_t use_suffix,
                                  const void* d_q, int32_t num_q_heads, int32_t q_dtype,
                                  const void* d_k_blk, const void* d_v_blk, int32_t blk_dtype,
                                  int32_t block_len, float softmax_scale,
                                  void* d_out, int32_t out_dtype, void* stream);

/* Mask-query selection (MaskAhead / Q-MaskAhead abstract: the current block's
 * mask queries rank the cached KV entries by their estimated contribution to
 * the attention output; the quantized variant ranks and attends directly from
 * the low-bit cache).  For every sequence b and kv head h, entry j (a valid
 * cached token: prefix slots, then suffix slots if use_suffix) gets
 *     c_j = ||v_j|| * sum over the query heads of h and the mask queries t of
 *           softmax_t(j),
 * v_j its dequantized value row and softmax_t the attention distribution of
 * block query t over all valid cached tokens and the 32 block tokens (scores
 * q.k * softmax_scale, keys dequantized to fp16).  Mask queries: block tokens
 * whose bit is set in h_query_mask[b] (host [B]; NULL = all 32).  The
 * min(budget, valid entries) largest contributions of each (b, h) are
 * selected, ties to the lower entry (entry number 32 * unit + position).
 * granularity = 32 ranks whole units (32-token slots) by the sum of their
 * entries' contributions instead and keeps every valid entry of the
 * min(budget, units) top units, ties to the lower unit; granularity = 1 is the
 * per-entry ranking.
 * Arguments as for kvq_block_attn (d_q, d_k_blk; no values are read from the
 * block); budget >= 0 (entries, or units with granularity 32).  Results go to the selection region of the cache buffer
 * (see kvq_layout) and stay valid until the next commit. */
kvq_status kvq_select(kvq_cache* c, int32_t use_suffix, const void* d_q, int32_t num_q_heads, int32_t q_dtype,
                      const void* d_k_blk, int32_t blk_dtype, int32_t block_len, float softmax_scale,
                      const uint32_t* h_query_mask, int32_t budget, int32_t granularity, void* stream);

/* kvq_block_attn restricted to the last selection: every query token attends
 * to all 32 block tokens and to the selected cached entries only.  Arguments
 * as for kvq_block_attn; use_suffix must equal the selection's.  KVQ_EINVAL if
 * no selection was made since the last commit. */
kvq_status kvq_block_attn_selected(kvq_cache* c, int32_t use_suffix, const void* d_q, int32_t num_q_heads,
                                   int32_t q_dtype, const void* d_k_blk, const void* d_v_blk, int32_t blk_dtype,
                                   int32_t block_len, float softmax_scale, void* d_out, int32_t out_dtype,
                                   void* stream);

/* Full attention and selection from one pass over the cache: the first
 * denoising step of a block attends to the whole cache and, from the same
 * softmax, ranks the entries that its later steps attend to (MaskAhead /
 * Q-MaskAhead abstract: the mask queries' attention mass decides which KV
 * entries the block keeps).  Equivalent to kvq_block_attn(c, use_suffix, d_q,
 * ..., d_out, out_dtype, stream) followed by kvq_select(c, use_suffix, d_q,
 * ..., h_query_mask, budget, granularity, stream) with the same arguments: the
 * output is kvq_block_attn's (bit-identical), and the selection follows
 * kvq_select's definition, except that the softmax normaliser of each query
 * row is the one the attention computed (its reference maximum and its sum
 * of the probabilities as rounded to fp16 for the PV product: each term
 * within 2^-11 relative or 2^-25 absolute of its exact value) instead of one
 * from a separate statistics pass over the cache.  The attention
 * writes these statistics to the sel_stats region of the cache buffer, then
 * the selection's scoring pass and its top-k run on `stream`.  Arguments are
 * checked before anything is launched; the cache's records must be in the
 * integer format (as for kvq_select).  Calls on one handle must not overlap. */
kvq_status kvq_attend_select(kvq_cache* c, int32_t use_suffix, const void* d_q, int32_t num_q_heads,
                             int32_t q_dtype, const void* d_k_blk, const void* d_v_blk, int32_t blk_dtype,
                             int32_t block_len, float softmax_scale, void* d_out, int32_t out_dtype,
                             const uint32_t* h_query_mask, int32_t budget, int32_t granularity, void* stream);

/* Attend, then commit the same block, in one call (SoloQ summary page,
 * commit-time KV quantization paragraph: the block being denoised stays in
 * full precision and is quantized when it is committed; reading: its last
 * denoising step attends with its own K and V, which are then committed).
 * Equivalent to kvq_block_attn(c, use_suffix, d_q, ..., stream) followed by
 * kvq_commit(c, KVQ_PREFIX, 0, d_k_blk, d_v_blk, blk_dtype, block_len, h_ntok,
 * h_prot_off, h_prot_idx, stream), with the same arguments and results: the
 * output is that of the attention over the cache as it was before the call.
 * It is one launch on `stream`: the workgroup that attends with the block of
 * (sequence b, kv head h) also quantizes that block's keys and values for kv
 * head h into the next prefix slot once its attention work is done (the new
 * slot is one no attention of the call reads).  For a cache with value
 * rotation the launch quantizes the block's values from the rotated copy the
 * attention reads (computed in the same order as kvq_commit's rotation, so
 * the records are the same bytes).  The commit is checked
 * before anything is launched: on an error the cache is unchanged.  Calls on
 * one handle must not overlap. */
kvq_status kvq_attend_commit(kvq_cache* c, int32_t use_suffix, const void* d_q, int32_t num_q_heads,
                             int32_t q_dtype, const void* d_k_blk, const void* d_v_blk, int32_t blk_dtype,
                             int32_t block_len, float softmax_scale, void* d_out, int32_t out_dtype,
                             const int32_t* h_ntok, const int32_t* h_prot_off, const int32_t* h_prot_idx,
                             void* stream);

/* Host mirror of a segment's lengths: any of the [B] arrays may be NULL. */
kvq_status kvq_segment_info(const kvq_cache* c, int32_t segment,
                            int32_t* h_ntok, int32_t* h_nslots, int32_t* h_nprot);

/* K-RPBH value rotation (SoloQ summary page, rotation paragraphs: a random
 * permutation of the channels, a Hadamard transform on blocks of b consecutive
 * channels, then a k x k random orthogonal mix of the same channel across the
 * k = D / b blocks; block-diffusion paragraph: values follow the activation path,
 * so they are rotated before they are quantized).  Only for a cache created with
 * v_rotation_block = b != 0, and only while both segments are empty (before the
 * first commit, or after both were reset); every commit and attention call of
 * such a cache fails with KVQ_EINVAL until the rotation is set.
 *   h_perm: host int32 [D], a permutation of 0..D-1 (rotated channel e takes
 *           input channel h_perm[e]);
 *   h_mix:  host fp32 [k * k], row-major, orthogonal (|M^T M - I| <= 1e-4 in every
 *           entry), finite.
 * Both are copied into the handle.  With the rotation set, kvq_commit quantizes
 * R v instead of v, computed in fp32 in this order:
 *     y = v[perm];  Hadamard stages h = 1, 2, ..., b/2: each pair (i, i + h) with
 *     i & h == 0 becomes (y_i + y_{i+h}, y_i - y_{i+h});  y <- y / sqrt(b);
 *     z[i*b + j] = sum over l = 0..k-1, in that order, of mix[i][l] * y[l*b + j]
 *     (each product rounded, then added; no fused multiply-add);
 * and kvq_block_attn rotates the block's values the same way, attends in the
 * rotated basis and returns R^T of the result, so its output approximates the
 * attention over the unrotated values.  The Hadamard block is normalised by
 * 1/sqrt(b); no length correction is applied. */
kvq_status kvq_set_v_rotation(kvq_cache* c, const int32_t* h_perm, const float* h_mix);

/* Attention work split: slots per split-K chunk (0 = automatic). */
kvq_status kvq_set_split_slots(kvq_cache* c, int32_t slots_per_split);

const char* kvq_status_str(kvq_status s);
const char* kvq_last_error(void);
int32_t kvq_abi_version(void);

/* Calibration kernels, used to report measured achievable peaks beside the
 * published ones; they are not part of the method.
 *   kvq_calib_copy: copies `bytes` (a multiple of 16; both pointers 16-byte
 *     aligned device memory) from d_src to d_dst with a streaming grid-stride
 *     kernel; timing it gives the achievable HBM bandwidth (2 * bytes moved).
 *   kvq_calib_mfma: `workgroups` workgroups of four waves, each wave issuing
 *     iters x 8 independent v_mfma_f32_32x32x16_f16 (32768 flops each) with no
 *     memory traffic, and one float per thread to d_out (workgroups * 256
 *     floats); timing it gives the achievable dense fp16 MFMA rate.
 * Asynchronous on `stream`; KVQ_EINVAL for bad arguments, KVQ_EHIP if the
 * launch fails. */
kvq_status kvq_calib_copy(void* d_dst, const void* d_src, size_t bytes, void* stream);
kvq_status kvq_calib_mfma(float* d_out, int32_t workgroups, int32_t iters, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H_ */
