// Host side of the C ABI: configuration checks, buffer layout, host mirror of
// segment lengths, commit task tables and kernel launches.  All argument checks
// run before any device work, so a failing call leaves the cache unchanged.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "kvq_internal.h"

using kvq::CommitTask;

constexpr int kMaxSplitUnits = 256;   // units one attention workgroup can hold headers for

namespace {

thread_local std::string g_err;

kvq_status fail(kvq_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

uint64_t align256(uint64_t x) { return (x + 255u) / 256u * 256u; }

int ilog2(int x) {
  int l = 0;
  while ((1 << l) < x) ++l;
  return l;
}

kvq_status check_config(const kvq_config* c) {
  if (!c) return fail(KVQ_EINVAL, "config is NULL");
  if (c->batch < 1 || c->batch > KVQ_MAX_BATCH) return fail(KVQ_EINVAL, "batch %d outside 1..%d", c->batch, KVQ_MAX_BATCH);
  if (c->num_kv_heads < 1 || c->num_kv_heads > 4096) return fail(KVQ_EINVAL, "num_kv_heads %d", c->num_kv_heads);
  if (c->head_dim != 64 && c->head_dim != 128) return fail(KVQ_EUNSUPPORTED, "head_dim %d (supported: 64, 128)", c->head_dim);
  if ((c->k_bits != 2 && c->k_bits != 4) || (c->v_bits != 2 && c->v_bits != 4))
    return fail(KVQ_EUNSUPPORTED, "k_bits %d / v_bits %d (supported: 2, 4)", c->k_bits, c->v_bits);
  if (c->k_group_tokens != kvq::kSlot) return fail(KVQ_EUNSUPPORTED, "k_group_tokens %d (supported: 32)", c->k_group_tokens);
  const int gv = c->v_group_channels;
  if ((gv != 32 && gv != 64 && gv != 128) || gv > c->head_dim)
    return fail(KVQ_EUNSUPPORTED, "v_group_channels %d (supported: 32, 64, 128, <= head_dim)", gv);
  if (c->prefix_slots < 1 || c->prefix_slots > 65535) return fail(KVQ_EINVAL, "prefix_slots %d outside 1..65535", c->prefix_slots);
  if (c->suffix_slots < 0 || c->suffix_slots > 65535) return fail(KVQ_EINVAL, "suffix_slots %d outside 0..65535", c->suffix_slots);
  if (c->prefix_protected < 0 || c->suffix_protected < 0) return fail(KVQ_EINVAL, "negative protected capacity");
  if (c->prefix_protected > c->prefix_slots * kvq::kSlot || c->suffix_protected > c->suffix_slots * kvq::kSlot)
    return fail(KVQ_EINVAL, "protected capacity exceeds the segment's token capacity");
  if (c->max_q_heads < c->num_kv_heads || c->max_q_heads % c->num_kv_heads != 0)
    return fail(KVQ_EINVAL, "max_q_heads %d must be a positive multiple of num_kv_heads %d", c->max_q_heads, c->num_kv_heads);
  if (c->max_q_heads / c->num_kv_heads > 8)
    return fail(KVQ_EUNSUPPORTED, "query heads per kv head %d (supported: <= 8)", c->max_q_heads / c->num_kv_heads);
  if (c->max_splits < 0 || c->max_splits > 256) return fail(KVQ_EINVAL, "max_splits %d outside 0..256", c->max_splits);
  if (c->v_rotation_block != 0 && c->v_rotation_block != 16 && c->v_rotation_block != 64)
    return fail(KVQ_EUNSUPPORTED, "v_rotation_block %d (supported: 0, 16, 64)", c->v_rotation_block);
  if (c->v_rotation_block > c->head_dim)
    return fail(KVQ_EUNSUPPORTED, "v_rotation_block %d exceeds head_dim %d", c->v_rotation_block, c->head_dim);
  if (c->kv_format != KVQ_FMT_INT && c->kv_format != KVQ_FMT_MXFP4 && c->kv_format != KVQ_FMT_INT_H16)
    return fail(KVQ_EUNSUPPORTED, "kv_format %d", c->kv_format);
  if (c->kv_format == KVQ_FMT_INT_H16 && c->v_rotation_block != 0)
    return fail(KVQ_EUNSUPPORTED, "fp16 metadata is not combined with value rotation");
  if (c->kv_format == KVQ_FMT_MXFP4 &&
      (c->k_bits != 4 || c->v_bits != 4 || c->v_group_channels != 32 || c->v_rotation_block != 0))
    return fail(KVQ_EUNSUPPORTED, "MX FP4 needs k_bits = v_bits = 4, v_group_channels = 32 and no value rotation");
  return KVQ_OK;
}

void compute_layout(const kvq_config* c, kvq_layout* L) {
  memset(L, 0, sizeof(*L));
  const uint64_t B = c->batch, H = c->num_kv_heads, D = c->head_dim;
  const bool mx = c->kv_format == KVQ_FMT_MXFP4, h16 = c->kv_format == KVQ_FMT_INT_H16;
  const uint64_t R = mx ? kvq::record_bytes_mx((int)D)
                   : h16 ? kvq::record_bytes_h16((int)D, c->k_bits, c->v_bits, c->v_group_channels)
                         : kvq::record_bytes((int)D, c->k_bits, c->v_bits, c->v_group_channels);
  L->record_bytes = R;
  L->kc_offset = 0;
  L->vc_offset = kvq::kc_bytes((int)D, c->k_bits);
  L->kmeta_offset = L->vc_offset + kvq::vc_bytes((int)D, c->v_bits);
  L->vmeta_offset = L->kmeta_offset + (mx ? D : h16 ? kvq::kmeta_bytes((int)D) / 2 : kvq::kmeta_bytes((int)D));
  uint64_t off = 0;
  for (int s = 0; s < 2; ++s) {
    const uint64_t cap = s == 0 ? c->prefix_slots : c->suffix_slots;
    const uint64_t pcap = s == 0 ? c->prefix_protected : c->suffix_protected;
    L->slot_cap[s] = (int32_t)cap;
    L->prot_cap[s] = (int32_t)pcap;
    L->records_offset[s] = off;   off += align256(B * H * cap * R);
    L->headers_offset[s] = off;   off += align256(B * cap * kvq::kHeaderBytes);
    L->prot_rows_offset[s] = off; off += align256(B * pcap * H * D * 2);
    L->prot_pos_offset[s] = off;  off += align256(B * pcap * 4);
  }
  const uint64_t splits = c->max_splits ? c->max_splits : 32;
  const uint64_t rmax = c->max_q_heads / c->num_kv_heads;
  L->workspace_offset = off;
  L->workspace_bytes = align256(B * H * splits * rmax * (D + 2) * kvq::kSlot * 4);
  off += L->workspace_bytes;
  L->rotation_offset = off;
  L->rotation_bytes = c->v_rotation_block
                          ? align256(2 * B * kvq::kSlot * H * D * 4) + align256(B * kvq::kSlot * (uint64_t)c->max_q_heads * D * 4)
                          : 0;
  off += L->rotation_bytes;
  // selection results: contributions per entry, token masks and unit lists
  // per cached unit, and the list lengths
  const uint64_t ucap = (uint64_t)c->prefix_slots + (uint64_t)c->suffix_slots;
  L->sel_contrib_offset = off; off += align256(B * H * ucap * kvq::kSlot * 4);
  L->sel_unit_offset = off;    off += align256(B * H * ucap * 4);
  L->sel_mask_offset = off;    off += align256(B * H * ucap * 4);
  L->sel_units_offset = off;   off += align256(B * H * ucap * 4);
  L->sel_count_offset = off;   off += align256(B * H * 4);
  // kvq_attend_select: the attention's softmax statistics per query row
  L->sel_stats_offset = off;   off += align256(B * H * kvq::kSelHeads * 2 * kvq::kSlot * 4);
  L->total_bytes = off;
}

struct SegMirror {
  std::vector<int32_t> ntok, nslots, nprot;
};

}  // namespace

struct kvq_cache {
  kvq_config cfg;
  kvq_layout lay;
  uint8_t* dbuf;
  SegMirror seg[2];
  int32_t split_slots = 0;
  bool dev_ready = false;
  int device = 0;                  // the device current at the first device call
  size_t task_bytes = 0;           // the largest task table of this handle
  int num_cus = 0;                 // compute units of the device (sizes the grids)
  std::vector<CommitTask> tasks;
  kvq::RotParams rot{};            // value rotation (rot.block == 0 until set)
  // the last selection: valid while no commit has happened since
  uint64_t commit_gen = 0, sel_gen = 0;
  bool sel_valid = false;
  int sel_use_suffix = 0, sel_budget = 0;
};

namespace {


// Task tables of large commits, in pinned host memory shared by every handle
// on a device: the commit kernel reads its table straight from host memory
// (each workgroup's first tasks in one parallel read), so no copy operation
// sits on the stream ahead of it.  One ring per device, so that the tables a
// process rewrites stay in the CPU's caches however many handles (one per
// layer, say) take turns: a table written cold costs a memory round trip per
// line, tens of microseconds for a prefill's table.  ev[k] marks the end of
// the last kernel that read table k; a commit blocks its thread only when the
// table it needs is still being read, i.e. when kSlots large commits are in
// flight on the device.  Grown (after every table's kernel has finished) to
// the largest table a handle can need; held until the process ends.
struct StageRing {
  static constexpr int kSlots = 8;
  std::mutex mu;
  uint8_t* h = nullptr;
  size_t slot_bytes = 0;
  hipEvent_t ev[kSlots] = {};
  bool used[kSlots] = {};
  int next = 0;
};
constexpr int kMaxDevices = 64;

StageRing& stage_ring(int dev) {
  static StageRing rings[kMaxDevices];
  return rings[dev];
}

// With R.mu held: a slot of at least `bytes`, free for rewriting.
kvq_status ring_slot(StageRing& R, size_t bytes, uint8_t** slot, int* k) {
  hipError_t e = hipSuccess;
  if (!R.ev[0]) {
    for (int i = 0; i < StageRing::kSlots; ++i) {
      e = hipEventCreateWithFlags(&R.ev[i], hipEventDisableTiming);
      if (e != hipSuccess) {
        for (int j = 0; j < i; ++j) (void)hipEventDestroy(R.ev[j]);
        for (int j = 0; j < StageRing::kSlots; ++j) R.ev[j] = nullptr;
        return fail(KVQ_EHIP, "hipEventCreate: %s", hipGetErrorString(e));
      }
    }
  }
  if (bytes > R.slot_bytes) {
    for (int i = 0; i < StageRing::kSlots; ++i) {
      if (R.used[i]) {
        e = hipEventSynchronize(R.ev[i]);
        if (e != hipSuccess) return fail(KVQ_EHIP, "hipEventSynchronize: %s", hipGetErrorString(e));
        R.used[i] = false;
      }
    }
    if (R.h) (void)hipHostFree(R.h);
    R.h = nullptr;
    R.slot_bytes = 0;
    e = hipHostMalloc(reinterpret_cast<void**>(&R.h), StageRing::kSlots * bytes, hipHostMallocDefault);
    if (e != hipSuccess) {
      R.h = nullptr;
      return fail(KVQ_EHIP, "hipHostMalloc: %s", hipGetErrorString(e));
    }
    R.slot_bytes = bytes;
    R.next = 0;
  }
  const int i = R.next;
  if (R.used[i]) {
    e = hipEventSynchronize(R.ev[i]);
    if (e != hipSuccess) return fail(KVQ_EHIP, "hipEventSynchronize: %s", hipGetErrorString(e));
    R.used[i] = false;
  }
  *slot = R.h + (size_t)i * R.slot_bytes;
  *k = i;
  return KVQ_OK;
}

// Device properties the launches need; allocates nothing.
kvq_status ensure_device(kvq_cache* c) {
  if (c->dev_ready) return KVQ_OK;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(KVQ_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(KVQ_EUNSUPPORTED, "device %d (this library handles 0..%d)", dev, kMaxDevices - 1);
  if (hipDeviceGetAttribute(&c->num_cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c->num_cus <= 0)
    c->num_cus = 256;
  const size_t maxcap = std::max(c->cfg.prefix_slots, c->cfg.suffix_slots);
  c->task_bytes = ((size_t)c->cfg.batch * maxcap * sizeof(CommitTask) + 255) & ~(size_t)255;
  c->device = dev;
  c->dev_ready = true;
  return KVQ_OK;
}

kvq::SegPtrs seg_ptrs(const kvq_cache* c, int s) {
  kvq::SegPtrs p;
  p.records = c->dbuf + c->lay.records_offset[s];
  p.headers = c->dbuf + c->lay.headers_offset[s];
  p.prot_rows = reinterpret_cast<uint16_t*>(c->dbuf + c->lay.prot_rows_offset[s]);
  p.prot_pos = reinterpret_cast<int32_t*>(c->dbuf + c->lay.prot_pos_offset[s]);
  p.slot_cap = c->lay.slot_cap[s];
  p.prot_cap = c->lay.prot_cap[s];
  return p;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" {

int32_t kvq_abi_version(void) { return KVQ_ABI_VERSION; }

const char* kvq_status_str(kvq_status s) {
  switch (s) {
    case KVQ_OK: return "ok";
    case KVQ_EINVAL: return "invalid argument";
    case KVQ_EUNSUPPORTED: return "unsupported configuration";
    case KVQ_ECAPACITY: return "capacity exceeded";
    case KVQ_EHIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* kvq_last_error(void) { return g_err.c_str(); }

size_t kvq_required_bytes(const kvq_config* cfg) {
  if (check_config(cfg) != KVQ_OK) return 0;
  kvq_layout L;
  compute_layout(cfg, &L);
  return L.total_bytes;
}

kvq_status kvq_get_layout(const kvq_config* cfg, kvq_layout* out) {
  kvq_status s = check_config(cfg);
  if (s != KVQ_OK) return s;
  if (!out) return fail(KVQ_EINVAL, "layout output is NULL");
  compute_layout(cfg, out);
  return KVQ_OK;
}

kvq_status kvq_create(const kvq_config* cfg, void* d_buf, size_t buf_bytes, kvq_cache** out) {
  kvq_status s = check_config(cfg);
  if (s != KVQ_OK) return s;
  if (!out) return fail(KVQ_EINVAL, "output handle pointer is NULL");
  if (!d_buf) return fail(KVQ_EINVAL, "device buffer is NULL");
  if (reinterpret_cast<uintptr_t>(d_buf) & 255u) return fail(KVQ_EINVAL, "device buffer is not 256-byte aligned");
  kvq_layout L;
  compute_layout(cfg, &L);
  if (buf_bytes < L.total_bytes)
    return fail(KVQ_EINVAL, "device buffer has %zu bytes, %llu needed", buf_bytes, (unsigned long long)L.total_bytes);
  kvq_cache* c = new (std::nothrow) kvq_cache();
  if (!c) return fail(KVQ_EINVAL, "out of host memory");
  c->cfg = *cfg;
  c->lay = L;
  c->dbuf = static_cast<uint8_t*>(d_buf);
  for (int i = 0; i < 2; ++i) {
    c->seg[i].ntok.assign(cfg->batch, 0);
    c->seg[i].nslots.assign(cfg->batch, 0);
    c->seg[i].nprot.assign(cfg->batch, 0);
  }
  *out = c;
  return KVQ_OK;
}

kvq_status kvq_destroy(kvq_cache* c) {
  if (!c) return KVQ_OK;
  delete c;
  return KVQ_OK;
}

kvq_status kvq_segment_info(const kvq_cache* c, int32_t segment, int32_t* h_ntok, int32_t* h_nslots,
                            int32_t* h_nprot) {
  if (!c) return fail(KVQ_EINVAL, "handle is NULL");
  if (segment != KVQ_PREFIX && segment != KVQ_SUFFIX) return fail(KVQ_EINVAL, "segment %d", segment);
  const SegMirror& m = c->seg[segment];
  const size_t n = (size_t)c->cfg.batch * sizeof(int32_t);
  if (h_ntok) memcpy(h_ntok, m.ntok.data(), n);
  if (h_nslots) memcpy(h_nslots, m.nslots.data(), n);
  if (h_nprot) memcpy(h_nprot, m.nprot.data(), n);
  return KVQ_OK;
}

kvq_status kvq_set_v_rotation(kvq_cache* c, const int32_t* h_perm, const float* h_mix) {
  if (!c) return fail(KVQ_EINVAL, "handle is NULL");
  const int b = c->cfg.v_rotation_block, D = c->cfg.head_dim;
  if (b == 0) return fail(KVQ_EINVAL, "cache was created without value rotation (v_rotation_block = 0)");
  if (!h_perm || !h_mix) return fail(KVQ_EINVAL, "permutation and mix must be non-NULL");
  for (int s = 0; s < 2; ++s)
    for (int i = 0; i < c->cfg.batch; ++i)
      if (c->seg[s].nslots[i] != 0) return fail(KVQ_EINVAL, "the rotation can only change while both segments are empty");
  std::vector<int> seen(D, 0);
  for (int e = 0; e < D; ++e) {
    const int p = h_perm[e];
    if (p < 0 || p >= D || seen[p]) return fail(KVQ_EINVAL, "h_perm is not a permutation of 0..%d", D - 1);
    seen[p] = 1;
  }
  const int k = D / b;
  for (int i = 0; i < k * k; ++i)
    if (!std::isfinite(h_mix[i])) return fail(KVQ_EINVAL, "h_mix has a non-finite entry");
  for (int i = 0; i < k; ++i)
    for (int j = 0; j < k; ++j) {
      double g = 0.0;
      for (int l = 0; l < k; ++l) g += (double)h_mix[l * k + i] * h_mix[l * k + j];
      if (std::fabs(g - (i == j ? 1.0 : 0.0)) > 1e-4) return fail(KVQ_EINVAL, "h_mix is not orthogonal");
    }
  kvq::RotParams r{};
  r.block = b;
  for (int e = 0; e < D; ++e) r.perm[e] = h_perm[e];
  for (int i = 0; i < k * k; ++i) r.mix[i] = h_mix[i];
  c->rot = r;
  return KVQ_OK;
}

kvq_status kvq_set_split_slots(kvq_cache* c, int32_t slots_per_split) {
  if (!c) return fail(KVQ_EINVAL, "handle is NULL");
  if (slots_per_split < 0) return fail(KVQ_EINVAL, "slots_per_split %d", slots_per_split);
  c->split_slots = slots_per_split;
  return KVQ_OK;
}

}  // extern "C"

namespace {

// A validated commit: the task table is in c->tasks; ntok and nprot_add are
// what the host mirror gains once the commit is launched.
struct CommitPlan {
  int segment = 0, reset = 0, in_dtype = 0, n_max = 0;
  const void* k = nullptr;
  const void* v = nullptr;
  std::vector<int32_t> ntok, nprot_add;
};

// Every check of a commit, and its task table; no device work, no change to the mirror.
kvq_status commit_plan(kvq_cache* c, int32_t segment, int32_t reset_segment, const void* d_k, const void* d_v,
                       int32_t in_dtype, int32_t n_max, const int32_t* h_ntok, const int32_t* h_prot_off,
                       const int32_t* h_prot_idx, CommitPlan& plan) {
  if (!c) return fail(KVQ_EINVAL, "handle is NULL");
  const kvq_config& cfg = c->cfg;
  const int B = cfg.batch;
  if (segment != KVQ_PREFIX && segment != KVQ_SUFFIX) return fail(KVQ_EINVAL, "segment %d", segment);
  if (segment == KVQ_SUFFIX && cfg.suffix_slots == 0) return fail(KVQ_EINVAL, "cache has no suffix segment");
  if (in_dtype != KVQ_F32 && in_dtype != KVQ_BF16) return fail(KVQ_EINVAL, "in_dtype %d", in_dtype);
  if (n_max < 0) return fail(KVQ_EINVAL, "n_max %d", n_max);
  if (cfg.v_rotation_block != 0 && c->rot.block == 0) return fail(KVQ_EINVAL, "value rotation is not set");
  if (h_prot_idx && !h_prot_off) return fail(KVQ_EINVAL, "protected index list given without offsets");
  std::vector<int32_t> ntok(B);
  int64_t total = 0;
  for (int b = 0; b < B; ++b) {
    ntok[b] = h_ntok ? h_ntok[b] : n_max;
    if (ntok[b] < 0 || ntok[b] > n_max) return fail(KVQ_EINVAL, "h_ntok[%d] = %d outside 0..%d", b, ntok[b], n_max);
    total += ntok[b];
  }
  if (total > 0) {
    if (!d_k || !d_v) return fail(KVQ_EINVAL, "k or v is NULL");
    if (!aligned16(d_k) || !aligned16(d_v)) return fail(KVQ_EINVAL, "k and v must be 16-byte aligned");
  }
  if (h_prot_off) {
    if (h_prot_off[0] != 0) return fail(KVQ_EINVAL, "h_prot_off[0] must be 0");
    for (int b = 0; b < B; ++b) {
      if (h_prot_off[b + 1] < h_prot_off[b]) return fail(KVQ_EINVAL, "h_prot_off decreases at %d", b);
      if (h_prot_off[b + 1] > h_prot_off[b] && !h_prot_idx) return fail(KVQ_EINVAL, "h_prot_idx is NULL");
      // one branch-free pass: position i must lie in prev + 1 .. ntok - 1
      uint32_t bad = 0;
      int lo = 0;
      for (int i = h_prot_off[b]; i < h_prot_off[b + 1]; ++i) {
        const int p = h_prot_idx[i];
        bad |= (uint32_t)((uint32_t)p - (uint32_t)lo >= (uint32_t)ntok[b] - (uint32_t)lo);
        lo = p + 1;
      }
      if (bad) {
        for (int i = h_prot_off[b]; i < h_prot_off[b + 1]; ++i) {
          const int p = h_prot_idx[i];
          if (p < 0 || p >= ntok[b])
            return fail(KVQ_EINVAL, "protected position %d of sequence %d outside 0..%d", p, b, ntok[b] - 1);
          if (i > h_prot_off[b] && p <= h_prot_idx[i - 1])
            return fail(KVQ_EINVAL, "protected positions of sequence %d are not strictly increasing", b);
        }
      }
    }
  }
  SegMirror& m = c->seg[segment];
  // attention-sink protection: a prefix commit that starts a sequence also
  // protects its first token (merged into the caller's sorted list)
  std::vector<int32_t> sink_off, sink_idx;
  if (cfg.protect_sink && segment == KVQ_PREFIX) {
    bool any = false;
    for (int b = 0; b < B; ++b) any = any || ((reset_segment || m.ntok[b] == 0) && ntok[b] > 0);
    if (any) {
      sink_off.assign(B + 1, 0);
      for (int b = 0; b < B; ++b) {
        const int n = h_prot_off ? h_prot_off[b + 1] - h_prot_off[b] : 0;
        const int32_t* p = n ? h_prot_idx + h_prot_off[b] : nullptr;
        if ((reset_segment || m.ntok[b] == 0) && ntok[b] > 0 && (n == 0 || p[0] != 0)) sink_idx.push_back(0);
        for (int i = 0; i < n; ++i) sink_idx.push_back(p[i]);
        sink_off[b + 1] = (int32_t)sink_idx.size();
      }
      h_prot_off = sink_off.data();
      h_prot_idx = sink_idx.empty() ? nullptr : sink_idx.data();
    }
  }
  const int cap = c->lay.slot_cap[segment], pcap = c->lay.prot_cap[segment];
  for (int b = 0; b < B; ++b) {
    const int base_slots = reset_segment ? 0 : m.nslots[b];
    const int base_prot = reset_segment ? 0 : m.nprot[b];
    const int add_slots = (ntok[b] + kvq::kSlot - 1) / kvq::kSlot;
    const int add_prot = h_prot_off ? h_prot_off[b + 1] - h_prot_off[b] : 0;
    if (base_slots + add_slots > cap)
      return fail(KVQ_ECAPACITY, "sequence %d needs %d slots, segment capacity is %d", b, base_slots + add_slots, cap);
    if (base_prot + add_prot > pcap)
      return fail(KVQ_ECAPACITY, "sequence %d needs %d protected rows, capacity is %d", b, base_prot + add_prot, pcap);
  }

  // ---- task table
  // one task per 32-token slot; the protected positions (validated above)
  // set their slot's mask bits, and a slot's first rank is the running count
  auto& tasks = c->tasks;
  size_t ntasks = 0;
  for (int b = 0; b < B; ++b) ntasks += (size_t)((ntok[b] + kvq::kSlot - 1) / kvq::kSlot);
  tasks.resize(ntasks);
  size_t t0 = 0;
  for (int b = 0; b < B; ++b) {
    const int base_slots = reset_segment ? 0 : m.nslots[b];
    const int tok0 = reset_segment ? 0 : m.ntok[b];
    const int nsl = (ntok[b] + kvq::kSlot - 1) / kvq::kSlot;
    CommitTask* tb = tasks.data() + t0;
    for (int j = 0; j < nsl; ++j) {
      CommitTask& t = tb[j];
      t.b = b;
      t.dst_slot = base_slots + j;
      t.src_tok = j * kvq::kSlot;
      t.nvalid = std::min(kvq::kSlot, ntok[b] - t.src_tok);
      t.mask = 0;
      t.token_base = tok0 + t.src_tok;
      t.pad = 0;
    }
    if (h_prot_off) {
      for (int i = h_prot_off[b]; i < h_prot_off[b + 1]; ++i) {
        const int p = h_prot_idx[i];
        tb[p / kvq::kSlot].mask |= 1u << (p % kvq::kSlot);
      }
    }
    int rank = reset_segment ? 0 : m.nprot[b];
    for (int j = 0; j < nsl; ++j) {
      tb[j].rank_base = rank;
      rank += __builtin_popcount(tb[j].mask);
    }
    t0 += (size_t)nsl;
  }
  plan.segment = segment;
  plan.reset = reset_segment;
  plan.in_dtype = in_dtype;
  plan.n_max = n_max;
  plan.k = d_k;
  plan.v = d_v;
  plan.ntok = ntok;
  plan.nprot_add.assign(B, 0);
  for (int b = 0; b < B; ++b) plan.nprot_add[b] = h_prot_off ? h_prot_off[b + 1] - h_prot_off[b] : 0;
  return KVQ_OK;
}

void commit_mirror(kvq_cache* c, const CommitPlan& plan);

// Launches a planned commit on st and updates the host mirror.
kvq_status commit_run(kvq_cache* c, const CommitPlan& plan, hipStream_t st) {
  const kvq_config& cfg = c->cfg;
  const int B = cfg.batch;
  const int segment = plan.segment, reset_segment = plan.reset, in_dtype = plan.in_dtype, n_max = plan.n_max;
  const void* d_k = plan.k;
  const void* d_v = plan.v;
  const std::vector<int32_t>& ntok = plan.ntok;
  SegMirror& m = c->seg[segment];
  auto& tasks = c->tasks;
  if (!tasks.empty()) {
    kvq_status s = ensure_device(c);
    if (s != KVQ_OK) return s;
    kvq::CommitArgs a;          // about 2 KB with the inline task table; the launch copies it
    memset(&a, 0, sizeof(a));
    hipError_t e = hipSuccess;
    // large commits: the ring's lock is held from taking a table to recording
    // its event, so tables and events are handed out in launch order
    std::unique_lock<std::mutex> lock;
    StageRing* ring = nullptr;
    int slot = -1;
    if ((int)tasks.size() <= kvq::kInlineTasks) {
      // small commits (one block per sequence) pass the tasks by value
      a.use_inline = 1;
      memcpy(a.inline_tasks, tasks.data(), tasks.size() * sizeof(CommitTask));
      a.tasks = nullptr;
    } else {
      ring = &stage_ring(c->device);
      lock = std::unique_lock<std::mutex>(ring->mu);
      uint8_t* hs = nullptr;
      s = ring_slot(*ring, std::max(c->task_bytes, tasks.size() * sizeof(CommitTask)), &hs, &slot);
      if (s != KVQ_OK) return s;
      memcpy(hs, tasks.data(), tasks.size() * sizeof(CommitTask));
      a.use_inline = 0;
      a.tasks = reinterpret_cast<const CommitTask*>(hs);   // device-accessible pinned memory
    }
    a.k = d_k;
    a.v = d_v;
    a.num_cus = c->num_cus;
    a.rot = c->rot;
    a.fmt = cfg.kv_format;
    a.seg = seg_ptrs(c, segment);
    a.n_max = n_max;
    a.hkv = cfg.num_kv_heads;
    a.gv_log2 = ilog2(cfg.v_group_channels);
    a.record_bytes = (uint32_t)c->lay.record_bytes;
    e = kvq::launch_commit(a, (int)tasks.size(), cfg.head_dim, cfg.k_bits, cfg.v_bits, in_dtype == KVQ_F32, st);
    if (e != hipSuccess) return fail(KVQ_EHIP, "commit launch: %s", hipGetErrorString(e));
    if (ring) {
      e = hipEventRecord(ring->ev[slot], st);
      if (e != hipSuccess) return fail(KVQ_EHIP, "hipEventRecord: %s", hipGetErrorString(e));
      ring->used[slot] = true;
      ring->next = (slot + 1) % StageRing::kSlots;
    }
  }

  commit_mirror(c, plan);
  return KVQ_OK;
}

// Updates the host mirror for a planned commit that has been launched.
void commit_mirror(kvq_cache* c, const CommitPlan& plan) {
  const int B = c->cfg.batch;
  const int segment = plan.segment, reset_segment = plan.reset;
  const std::vector<int32_t>& ntok = plan.ntok;
  SegMirror& m = c->seg[segment];
  if (reset_segment || !c->tasks.empty()) ++c->commit_gen;
  for (int b = 0; b < B; ++b) {
    if (reset_segment) { m.ntok[b] = 0; m.nslots[b] = 0; m.nprot[b] = 0; }
    m.ntok[b] += ntok[b];
    m.nslots[b] += (ntok[b] + kvq::kSlot - 1) / kvq::kSlot;
    m.nprot[b] += plan.nprot_add[b];
  }
}

}  // namespace

extern "C" {

kvq_status kvq_commit(kvq_cache* c, int32_t segment, int32_t reset_segment, const void* d_k, const void* d_v,
                      int32_t in_dtype, int32_t n_max, const int32_t* h_ntok, const int32_t* h_prot_off,
                      const int32_t* h_prot_idx, void* stream) {
  CommitPlan plan;
  kvq_status s = commit_plan(c, segment, reset_segment, d_k, d_v, in_dtype, n_max, h_ntok, h_prot_off, h_prot_idx, plan);
  if (s != KVQ_OK) return s;
  return commit_run(c, plan, static_cast<hipStream_t>(stream));
}

}  // extern "C"

namespace {

// fused: a planned commit of this same block into the prefix (one slot per
// sequence), carried out by the attention launch itself.
kvq_status block_attn_impl(kvq_cache* c, int32_t use_suffix, const void* d_q, int32_t num_q_heads, int32_t q_dtype,
                           const void* d_k_blk, const void* d_v_blk, int32_t blk_dtype, int32_t block_len,
                           float softmax_scale, void* d_out, int32_t out_dtype, void* stream, bool selected,
                           const CommitPlan* fused = nullptr, bool noalloc = false, float* row_stats = nullptr) {
  if (!c) return fail(KVQ_EINVAL, "handle is NULL");
  const kvq_config& cfg = c->cfg;
  const int B = cfg.batch, H = cfg.num_kv_heads;
  if (use_suffix && cfg.suffix_slots == 0) return fail(KVQ_EINVAL, "cache has no suffix segment");
  if (block_len != kvq::kSlot) return fail(KVQ_EUNSUPPORTED, "block_len %d (supported: 32)", block_len);
  if (num_q_heads < H || num_q_heads % H != 0 || num_q_heads > cfg.max_q_heads)
    return fail(KVQ_EINVAL, "num_q_heads %d must be a multiple of %d and <= %d", num_q_heads, H, cfg.max_q_heads);
  if ((q_dtype != KVQ_F32 && q_dtype != KVQ_BF16) || (blk_dtype != KVQ_F32 && blk_dtype != KVQ_BF16) ||
      (out_dtype != KVQ_F32 && out_dtype != KVQ_BF16))
    return fail(KVQ_EINVAL, "dtype must be KVQ_F32 or KVQ_BF16");
  if (!d_q || !d_k_blk || !d_v_blk || !d_out) return fail(KVQ_EINVAL, "q, k_blk, v_blk and out must be non-NULL");
  if (!aligned16(d_q) || !aligned16(d_k_blk) || !aligned16(d_v_blk) || !aligned16(d_out))
    return fail(KVQ_EINVAL, "q, k_blk, v_blk and out must be 16-byte aligned");
  if (!std::isfinite(softmax_scale) || softmax_scale <= 0.f) return fail(KVQ_EINVAL, "softmax_scale must be finite and > 0");
  if (cfg.v_rotation_block != 0 && c->rot.block == 0) return fail(KVQ_EINVAL, "value rotation is not set");
  if (selected) {
    if (!c->sel_valid || c->sel_gen != c->commit_gen)
      return fail(KVQ_EINVAL, "no selection for the cache as it stands (kvq_select after the last commit)");
    if ((use_suffix ? 1 : 0) != c->sel_use_suffix)
      return fail(KVQ_EINVAL, "use_suffix %d differs from the selection's", use_suffix);
  }

  const int max_splits = cfg.max_splits ? cfg.max_splits : 32;
  int max_units = 0;
  int64_t total_units = 0;
  kvq::AttnArgs a;
  memset(&a, 0, sizeof(a));
  // units per sequence: its cached slots (or, with a selection, at most the
  // budget of them: each selected entry lies in one slot) plus the block
  std::vector<int> ub(B);
  for (int b = 0; b < B; ++b) {
    const int np = c->seg[0].nslots[b], ns = use_suffix ? c->seg[1].nslots[b] : 0;
    a.nslots[0][b] = (uint16_t)np;
    a.nslots[1][b] = (uint16_t)(use_suffix ? ns : 0);
    const int U = (selected ? std::min(c->sel_budget, np + ns) : np + ns) + 1;
    ub[b] = U;
    max_units = std::max(max_units, U);
    total_units += U;
  }
  kvq_status hs = ensure_device(c);
  if (hs != KVQ_OK) return hs;
  int split_units;
  if (c->split_slots > 0) {
    split_units = c->split_slots;
  } else {
    // The kernel holds one workgroup per compute unit, so the grid should fit
    // in one round: the smallest split length (at least 8 units) whose
    // workgroups, summed over every (sequence, kv head) pair, do not exceed
    // the CU count.  Ragged batches need this count per sequence: a length
    // from the total alone leaves a second, mostly idle round.  When even one
    // split per pair exceeds the CUs, split the total evenly instead.
    const std::vector<int>& units = ub;
    auto groups = [&](int su) {
      int64_t n = 0;
      for (int b = 0; b < B; ++b) n += (units[b] + su - 1) / su;
      return n * H;
    };
    const int64_t cus = c->num_cus;
    if (groups(std::max(max_units, 8)) > cus) {
      split_units = (int)std::max<int64_t>(8, (total_units * H + cus - 1) / cus);
    } else {
      int lo = 8, hi = std::max(max_units, 8);      // groups(hi) <= cus; find the smallest such length
      while (lo < hi) {
        const int mid = (lo + hi) / 2;
        if (groups(mid) <= cus) hi = mid; else lo = mid + 1;
      }
      split_units = lo;
    }
  }
  split_units = std::max(split_units, (max_units + max_splits - 1) / max_splits);
  split_units = std::min(split_units, kMaxSplitUnits);
  if ((int64_t)split_units * max_splits < max_units)
    return fail(KVQ_EUNSUPPORTED, "%d attended units per sequence exceed max_splits %d x %d units", max_units,
                max_splits, kMaxSplitUnits);
  const int grid_splits = (max_units + split_units - 1) / split_units;

  // Workspace: split partials [b][kvh][split][head][D+2][32] fp32, then (value
  // rotation) the block's fp32 K and rotated V and the rotated output.  In
  // the cache buffer; for the allocation-free call, in the device's scratch
  // array, with the split stride cut to this launch's split count.
  const int D = cfg.head_dim;
  const size_t blk_elems = (size_t)B * kvq::kSlot * H * D;
  uint8_t* rot_ws = c->dbuf + c->lay.rotation_offset;
  // rotated values, 16-bit output: the merge applies the transposed rotation
  // (every pair hands its splits to it, one included); an fp32 output keeps
  // the fp32 partials and a separate unrotation
  const bool rot_merge = c->rot.block != 0 && out_dtype == KVQ_BF16;
  a.partial = reinterpret_cast<float*>(c->dbuf + c->lay.workspace_offset);
  a.max_splits = max_splits;
  if (noalloc) {
    const size_t part = (grid_splits > 1 || rot_merge)
                            ? align256((uint64_t)B * H * grid_splits * (num_q_heads / H) * (D + 2) * kvq::kSlot * 4)
                            : 0;
    const size_t rot = c->rot.block ? align256(2 * blk_elems * 4) + align256((uint64_t)B * kvq::kSlot * num_q_heads * D * 4)
                                    : 0;
    if (part + rot > kvq::kNoAllocScratchBytes)
      return fail(KVQ_ECAPACITY, "this call needs %zu bytes of workspace; the allocation-free scratch holds %zu",
                  part + rot, kvq::kNoAllocScratchBytes);
    void* base = nullptr;
    hipError_t e = kvq::noalloc_scratch(&base);
    if (e != hipSuccess) return fail(KVQ_EHIP, "scratch address: %s", hipGetErrorString(e));
    a.partial = static_cast<float*>(base);
    a.max_splits = grid_splits;
    rot_ws = static_cast<uint8_t*>(base) + part;
  }
  a.q = d_q;
  a.k_blk = d_k_blk;
  a.v_blk = d_v_blk;
  a.out = d_out;
  a.seg[0] = seg_ptrs(c, 0);
  a.seg[1] = seg_ptrs(c, 1);
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  a.hq = num_q_heads;
  a.hkv = H;
  a.r = num_q_heads / H;
  a.q_f32 = q_dtype == KVQ_F32;
  a.blk_f32 = blk_dtype == KVQ_F32;
  a.out_f32 = out_dtype == KVQ_F32;
  a.gv_log2 = ilog2(cfg.v_group_channels);
  a.record_bytes = (uint32_t)c->lay.record_bytes;
  a.split_units = split_units;
  a.use_suffix = use_suffix ? 1 : 0;
  a.fmt = cfg.kv_format;
  a.row_stats = row_stats;
  if (fused) {
    // one task per committing sequence: slot nslots[0][b], first token 0
    a.commit_blk = 1;
    for (const CommitTask& t : c->tasks) {
      if (t.dst_slot != c->seg[0].nslots[t.b] || t.src_tok != 0 || t.nvalid < 1 || t.nvalid > kvq::kSlot ||
          t.rank_base != c->seg[0].nprot[t.b] || t.token_base != c->seg[0].ntok[t.b])
        return fail(KVQ_EINVAL, "internal: the block commit of sequence %d is not one slot after the cache", t.b);
      a.cmask[t.b] = t.mask;
      a.cvalid[t.b] = (uint8_t)t.nvalid;
    }
  }
  if (selected) {
    a.sel_count = reinterpret_cast<const int32_t*>(c->dbuf + c->lay.sel_count_offset);
    a.sel_units = reinterpret_cast<const int32_t*>(c->dbuf + c->lay.sel_units_offset);
    a.sel_mask = reinterpret_cast<const uint32_t*>(c->dbuf + c->lay.sel_mask_offset);
    a.sel_ucap = cfg.prefix_slots + cfg.suffix_slots;
  }
  // One-dimensional grid of exactly the workgroups that hold units, when they
  // fit the launch-argument list: with one workgroup per CU, workgroups that
  // exit at once still take dispatch slots, and an uneven spread of the
  // working ones over the XCDs can leave some of them for a second round.
  {
    int64_t n = 0;
    for (int b = 0; b < B; ++b) n += (int64_t)H * ((ub[b] + split_units - 1) / split_units);
    a.num_wg = 0;
    if (n <= kvq::kMaxWgTable && grid_splits <= 256 && H <= 256) {
      // Workgroup i starts on XCD i % kXcds.  All splits of one (sequence,
      // kv head) go to one XCD, so the block's queries (read by every split)
      // come from HBM once and from that XCD's L2 after: each (sequence, kv
      // head) joins the XCD with the fewest workgroups so far, and the table
      // interleaves the XCDs' lists (a list that runs out early is filled
      // from the longest one).
      constexpr int kXcds = 8;
      uint32_t bin[kXcds][kvq::kMaxWgTable];
      int cnt[kXcds] = {0}, next[kXcds] = {0};
      for (int b = 0; b < B; ++b) {
        const int ns = (ub[b] + split_units - 1) / split_units;
        for (int h = 0; h < H; ++h) {
          int x = 0;
          for (int y = 1; y < kXcds; ++y)
            if (cnt[y] < cnt[x]) x = y;
          for (int sp = 0; sp < ns; ++sp) bin[x][cnt[x]++] = (uint32_t)sp | ((uint32_t)h << 8) | ((uint32_t)b << 16);
        }
      }
      for (int i = 0; i < (int)n; ++i) {
        int x = i % kXcds;
        if (next[x] == cnt[x]) {
          for (int y = 0; y < kXcds; ++y)
            if (cnt[y] - next[y] > cnt[x] - next[x]) x = y;
        }
        a.wg[i] = bin[x][next[x]++];
      }
      a.num_wg = (int32_t)n;
    }
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  float* rot_o = nullptr;
  if (c->rot.block != 0) {
    // rotated values: the block's values join the cache's basis (keys are
    // converted alongside, so that both block operands are fp32), attention
    // writes R o in fp32, and the transposed rotation gives o
    float* ws = reinterpret_cast<float*>(rot_ws);
    const size_t blk = blk_elems;
    kvq::BlkPrepArgs p;
    memset(&p, 0, sizeof(p));
    p.k = d_k_blk;
    p.v = d_v_blk;
    p.k_out = ws;
    p.v_out = ws + blk;
    p.rows = (int64_t)B * kvq::kSlot * H;
    p.in_f32 = blk_dtype == KVQ_F32;
    p.rot = c->rot;
    hipError_t e = kvq::launch_blk_prep(p, D, st);
    if (e != hipSuccess) return fail(KVQ_EHIP, "block rotation launch: %s", hipGetErrorString(e));
    rot_o = reinterpret_cast<float*>(rot_ws + align256(2 * blk * 4));
    a.k_blk = p.k_out;
    a.v_blk = p.v_out;
    a.blk_f32 = 1;
    a.v_centred = 1;
    if (rot_merge) {
      a.force_partials = 1;
    } else {
      a.out = rot_o;
      a.out_f32 = 1;
    }
  }
  hipError_t e = kvq::launch_attention(a, grid_splits, B, D, cfg.k_bits, cfg.v_bits, st,
                                       rot_merge ? &c->rot : nullptr);
  if (e != hipSuccess) return fail(KVQ_EHIP, "attention launch: %s", hipGetErrorString(e));
  if (rot_o && !rot_merge) {
    kvq::UnrotArgs u;
    memset(&u, 0, sizeof(u));
    u.src = rot_o;
    u.out = d_out;
    u.rows = (int64_t)B * kvq::kSlot * num_q_heads;
    u.out_f32 = out_dtype == KVQ_F32;
    u.rot = c->rot;
    e = kvq::launch_unrotate(u, D, st);
    if (e != hipSuccess) return fail(KVQ_EHIP, "output rotation launch: %s", hipGetErrorString(e));
  }
  return KVQ_OK;
}

// Argument checks of a selection (kvq_select, kvq_attend_select).
kvq_status select_check(kvq_cache* c, int32_t use_suffix, const void* d_q, int32_t num_q_heads, int32_t q_dtype,
                        const void* d_k_blk, int32_t blk_dtype, int32_t block_len, float softmax_scale,
                        int32_t budget, int32_t granularity) {
  if (!c) return fail(KVQ_EINVAL, "handle is NULL");
  if (granularity != 1 && granularity != kvq::kSlot) return fail(KVQ_EINVAL, "granularity %d (1 or 32)", granularity);
  const kvq_config& cfg = c->cfg;
  const int H = cfg.num_kv_heads;
  if (use_suffix && cfg.suffix_slots == 0) return fail(KVQ_EINVAL, "cache has no suffix segment");
  if (block_len != kvq::kSlot) return fail(KVQ_EUNSUPPORTED, "block_len %d (supported: 32)", block_len);
  if (num_q_heads < H || num_q_heads % H != 0 || num_q_heads > cfg.max_q_heads)
    return fail(KVQ_EINVAL, "num_q_heads %d must be a multiple of %d and <= %d", num_q_heads, H, cfg.max_q_heads);
  if ((q_dtype != KVQ_F32 && q_dtype != KVQ_BF16) || (blk_dtype != KVQ_F32 && blk_dtype != KVQ_BF16))
    return fail(KVQ_EINVAL, "dtype must be KVQ_F32 or KVQ_BF16");
  if (!d_q || !d_k_blk) return fail(KVQ_EINVAL, "q and k_blk must be non-NULL");
  if (!aligned16(d_q) || !aligned16(d_k_blk)) return fail(KVQ_EINVAL, "q and k_blk must be 16-byte aligned");
  if (!std::isfinite(softmax_scale) || softmax_scale <= 0.f) return fail(KVQ_EINVAL, "softmax_scale must be finite and > 0");
  if (budget < 0) return fail(KVQ_EINVAL, "budget %d", budget);
  if (cfg.kv_format != KVQ_FMT_INT) return fail(KVQ_EUNSUPPORTED, "selection reads integer-format records only");
  return ensure_device(c);
}

// The selection's launches: the statistics pass (unless row_stats holds the
// attention's per-row softmax statistics), the scoring pass and the top-k.
kvq_status select_run(kvq_cache* c, int32_t use_suffix, const void* d_q, int32_t num_q_heads, int32_t q_dtype,
                      const void* d_k_blk, int32_t blk_dtype, float softmax_scale, const uint32_t* h_query_mask,
                      int32_t budget, int32_t granularity, void* stream, float* row_stats) {
  const kvq_config& cfg = c->cfg;
  const int B = cfg.batch, H = cfg.num_kv_heads;
  const int max_splits = cfg.max_splits ? cfg.max_splits : 32;
  const int ucap = cfg.prefix_slots + cfg.suffix_slots;
  kvq::SelArgs a;
  memset(&a, 0, sizeof(a));
  int max_nc = 0;
  int64_t total_nc = 0;
  for (int b = 0; b < B; ++b) {
    const int np = c->seg[0].nslots[b], ns = use_suffix ? c->seg[1].nslots[b] : 0;
    a.nslots[0][b] = (uint16_t)np;
    a.nslots[1][b] = (uint16_t)ns;
    a.qmask[b] = h_query_mask ? h_query_mask[b] : 0xFFFFFFFFu;
    max_nc = std::max(max_nc, np + ns);
    total_nc += np + ns;
  }
  // split lengths: one workgroup per compute unit over all (sequence, kv
  // head) pairs (each workgroup pipelines its units; one fits a CU at D =
  // 128), at least 4 units, and the stats pass within the partial capacity of
  // max_splits per pair
  const int64_t cus = c->num_cus;
  auto split_len = [&](int64_t total, int maxu) {
    int su = (int)std::max<int64_t>(4, (total * H + cus - 1) / cus);
    return std::min(std::max(su, (maxu + max_splits - 1) / max_splits), kvq::kMaxSelSplit);
  };
  const int su_stats = split_len(total_nc + B, max_nc + 1);
  const int su_score = split_len(total_nc, max_nc);
  if (!row_stats && (int64_t)su_stats * max_splits < max_nc + 1)
    return fail(KVQ_EUNSUPPORTED, "%d cached units per sequence exceed max_splits %d x %d units", max_nc, max_splits,
                kvq::kMaxSelSplit);
  a.q = d_q;
  a.k_blk = d_k_blk;
  a.seg[0] = seg_ptrs(c, 0);
  a.seg[1] = seg_ptrs(c, 1);
  a.partial = reinterpret_cast<float*>(c->dbuf + c->lay.workspace_offset);
  a.contrib = reinterpret_cast<float*>(c->dbuf + c->lay.sel_contrib_offset);
  a.unit_contrib = reinterpret_cast<float*>(c->dbuf + c->lay.sel_unit_offset);
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  a.hq = num_q_heads;
  a.hkv = H;
  a.r = num_q_heads / H;
  a.q_f32 = q_dtype == KVQ_F32;
  a.blk_f32 = blk_dtype == KVQ_F32;
  a.gv_log2 = ilog2(cfg.v_group_channels);
  a.record_bytes = (uint32_t)c->lay.record_bytes;
  a.stats_split_units = su_stats;
  a.max_splits = max_splits;
  a.use_suffix = use_suffix ? 1 : 0;
  a.ucap = ucap;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int D = cfg.head_dim;
  hipError_t e = hipSuccess;
  if (row_stats) {
    // the attention's statistics: one "split" that covers every unit
    a.partial = row_stats;
    a.max_splits = 1;
    a.stats_split_units = max_nc + 1;
  } else {
    a.split_units = su_stats;
    e = kvq::launch_select(a, 0, (max_nc + 1 + su_stats - 1) / su_stats, B, D, cfg.k_bits, cfg.v_bits, st);
    if (e != hipSuccess) return fail(KVQ_EHIP, "selection stats launch: %s", hipGetErrorString(e));
  }
  a.split_units = su_score;
  e = kvq::launch_select(a, 1, (max_nc + su_score - 1) / su_score, B, D, cfg.k_bits, cfg.v_bits, st);
  if (e != hipSuccess) return fail(KVQ_EHIP, "selection score launch: %s", hipGetErrorString(e));
  kvq::TopkArgs t;
  memset(&t, 0, sizeof(t));
  t.contrib = a.contrib;
  t.unit_contrib = a.unit_contrib;
  t.granularity = granularity;
  t.sel_mask = reinterpret_cast<uint32_t*>(c->dbuf + c->lay.sel_mask_offset);
  t.sel_units = reinterpret_cast<int32_t*>(c->dbuf + c->lay.sel_units_offset);
  t.sel_count = reinterpret_cast<int32_t*>(c->dbuf + c->lay.sel_count_offset);
  t.hkv = H;
  t.ucap = ucap;
  t.budget = budget;
  for (int b = 0; b < B; ++b) t.nunits[b] = (uint16_t)(a.nslots[0][b] + a.nslots[1][b]);
  e = kvq::launch_topk(t, B, st);
  if (e != hipSuccess) return fail(KVQ_EHIP, "top-k launch: %s", hipGetErrorString(e));
  c->sel_valid = true;
  c->sel_gen = c->commit_gen;
  c->sel_use_suffix = use_suffix ? 1 : 0;
  c->sel_budget = budget;
  return KVQ_OK;
}


}  // namespace

extern "C" {

kvq_status kvq_block_attn(kvq_cache* c, int32_t use_suffix, const void* d_q, int32_t num_q_heads, int32_t q_dtype,
                          const void* d_k_blk, const void* d_v_blk, int32_t blk_dtype, int32_t block_len,
                          float softmax_scale, void* d_out, int32_t out_dtype, void* stream) {
  return block_attn_impl(c, use_suffix, d_q, num_q_heads, q_dtype, d_k_blk, d_v_blk, blk_dtype, block_len,
                         softmax_scale, d_out, out_dtype, stream, false);
}

kvq_status kvq_block_attn_noalloc(kvq_cache* c, int32_t use_suffix, const void* d_q, int32_t num_q_heads,
                                  int32_t q_dtype, const void* d_k_blk, const void* d_v_blk, int32_t blk_dtype,
                                  int32_t block_len, float softmax_scale, void* d_out, int32_t out_dtype,
                                  void* stream) {
  return block_attn_impl(c, use_suffix, d_q, num_q_heads, q_dtype, d_k_blk, d_v_blk, blk_dtype, block_len,
                         softmax_scale, d_out, out_dtype, stream, false, nullptr, true);
}

kvq_status kvq_block_attn_selected(kvq_cache* c, int32_t use_suffix, const void* d_q, int32_t num_q_heads,
                                   int32_t q_dtype, const void* d_k_blk, const void* d_v_blk, int32_t blk_dtype,
                                   int32_t block_len, float softmax_scale, void* d_out, int32_t out_dtype,
                                   void* stream) {
  return block_attn_impl(c, use_suffix, d_q, num_q_heads, q_dtype, d_k_blk, d_v_blk, blk_dtype, block_len,
                         softmax_scale, d_out, out_dtype, stream, true);
}

kvq_status kvq_attend_commit(kvq_cache* c, int32_t use_suffix, const void* d_q, int32_t num_q_heads, int32_t q_dtype,
                             const void* d_k_blk, const void* d_v_blk, int32_t blk_dtype, int32_t block_len,
                             float softmax_scale, void* d_out, int32_t out_dtype, const int32_t* h_ntok,
                             const int32_t* h_prot_off, const int32_t* h_prot_idx, void* stream) {
  // the commit is checked before anything is launched; the attention checks
  // its own arguments before its launches, and reads the cache as it was
  CommitPlan plan;
  kvq_status s = commit_plan(c, KVQ_PREFIX, 0, d_k_blk, d_v_blk, blk_dtype, block_len, h_ntok, h_prot_off,
                             h_prot_idx, plan);
  if (s != KVQ_OK) return s;
  // one launch: the workgroup holding each (sequence, kv head)'s block also
  // commits it (with rotated values, from the rotated copy of the block that
  // the attention reads)
  s = block_attn_impl(c, use_suffix, d_q, num_q_heads, q_dtype, d_k_blk, d_v_blk, blk_dtype, block_len,
                      softmax_scale, d_out, out_dtype, stream, false, &plan);
  if (s != KVQ_OK) return s;
  commit_mirror(c, plan);
  return KVQ_OK;
}

kvq_status kvq_select(kvq_cache* c, int32_t use_suffix, const void* d_q, int32_t num_q_heads, int32_t q_dtype,
                      const void* d_k_blk, int32_t blk_dtype, int32_t block_len, float softmax_scale,
                      const uint32_t* h_query_mask, int32_t budget, int32_t granularity, void* stream) {
  kvq_status s = select_check(c, use_suffix, d_q, num_q_heads, q_dtype, d_k_blk, blk_dtype, block_len, softmax_scale,
                              budget, granularity);
  if (s != KVQ_OK) return s;
  return select_run(c, use_suffix, d_q, num_q_heads, q_dtype, d_k_blk, blk_dtype, softmax_scale, h_query_mask, budget,
                    granularity, stream, nullptr);
}

kvq_status kvq_attend_select(kvq_cache* c, int32_t use_suffix, const void* d_q, int32_t num_q_heads,
                             int32_t q_dtype, const void* d_k_blk, const void* d_v_blk, int32_t blk_dtype,
                             int32_t block_len, float softmax_scale, void* d_out, int32_t out_dtype,
                             const uint32_t* h_query_mask, int32_t budget, int32_t granularity, void* stream) {
  // the selection's arguments are checked before the attention launches;
  // the attention checks its own before any of its launches
  kvq_status s = select_check(c, use_suffix, d_q, num_q_heads, q_dtype, d_k_blk, blk_dtype, block_len, softmax_scale,
                              budget, granularity);
  if (s != KVQ_OK) return s;
  float* stats = reinterpret_cast<float*>(c->dbuf + c->lay.sel_stats_offset);
  s = block_attn_impl(c, use_suffix, d_q, num_q_heads, q_dtype, d_k_blk, d_v_blk, blk_dtype, block_len,
                      softmax_scale, d_out, out_dtype, stream, false, nullptr, false, stats);
  if (s != KVQ_OK) return s;
  return select_run(c, use_suffix, d_q, num_q_heads, q_dtype, d_k_blk, blk_dtype, softmax_scale, h_query_mask, budget,
                    granularity, stream, stats);
}

}  // extern "C"
