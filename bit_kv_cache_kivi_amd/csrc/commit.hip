// Quantize-on-commit kernel for gfx950.
//
// A committed block's keys and values are quantized once, when the block is
// committed (Tai et al., "KV Cache Quantization for Diffusion Language Models",
// abstract; SoloQ summary page, block-diffusion paragraph).  The quantizer of
// one slot of one kv head is in commit_slot.h; this kernel runs it over every
// new slot of a commit.
//
// A persistent grid of four-wave workgroups; each takes a contiguous range of
// (slot, kv head) items and loops over it.  Each lane loads the next item's
// 16-byte row pieces before quantizing the current one, so HBM reads stay in
// flight while a slot is processed; the record buffers alternate, so an item's
// stores into one buffer never race the previous item's copy-out of the
// other.  This file is compiled with -ffp-contract=off.
#include <algorithm>

#include "commit_slot.h"

namespace kvq {
namespace {

constexpr int kTaskLds = 16;   // tasks of a workgroup kept in LDS (large commits)

// Work items are (slot, kv head) pairs, item = task * Hkv + head; workgroup bx
// takes the contiguous range [bx * n / G, (bx + 1) * n / G), so the kv heads
// of one slot mostly go to the same workgroup and a task descriptor is read
// once for all of them.
template <int KB, int VB, int D, bool F32IN, bool ROT, int FMT>
__global__ __launch_bounds__(256, (F32IN || ROT) ? 3 : 4) void commit_kernel(const CommitArgs a, int ntasks) {
  using Q = SlotQuant<KB, VB, D, F32IN, ROT, FMT>;
  __shared__ __align__(16) uint8_t recbuf[2][Q::REC_MAX];
  __shared__ __align__(16) typename Q::Lds lds;
  __shared__ __align__(16) CommitTask tlds[kTaskLds];

  const int tid = threadIdx.x;
  const int bx = blockIdx.x;
  const int G = gridDim.x;
  const int hkv = a.hkv;
  const int nitems = ntasks * hkv;
  const int beg = (int)((int64_t)bx * nitems / G);
  const int end = (int)((int64_t)(bx + 1) * nitems / G);
  const int task0 = beg / hkv;
  const SlotIO io{a.k, a.v, a.seg, a.n_max, a.hkv, a.gv_log2, a.record_bytes};
  Q q(lds, io, 0, tid);

  // the record bytes past the last field stay zero in both buffers
  q.clear_tail(recbuf[0]);
  q.clear_tail(recbuf[1]);
  if constexpr (ROT) {
    for (int e = tid; e < D; e += 256) lds.rperm[e] = a.rot.perm[e];
    for (int e = tid; e < 64; e += 256) lds.rmix[e] = a.rot.mix[e];
  }
  // A table in pinned host memory: the workgroup's tasks (first kTaskLds)
  // arrive with one parallel read, so the slot loop never waits on a
  // host-memory round trip (a scalar load there would also hold up every LDS
  // wait, which shares its counter).
  if (!a.use_inline) {
    const int ntl = end > beg ? (end - 1) / hkv - task0 + 1 : 0;
    const int nl = ntl < kTaskLds ? ntl : kTaskLds;
    if (tid < 2 * nl) {
      const int k = tid >> 1, half = tid & 1;
      reinterpret_cast<uint4*>(&tlds[k])[half] = reinterpret_cast<const uint4*>(a.tasks + task0 + k)[half];
    }
  }
  __syncthreads();

  // Task descriptors: kernel arguments (small commits), LDS, or, past the
  // first kTaskLds tasks of a workgroup, scalar loads of the host table.
  // Fields are made wave-uniform so that addresses built from them stay scalar.
  typedef const __attribute__((address_space(4))) int32_t* ConstWords;
  auto task_at = [&](int t) __attribute__((always_inline)) {
    CommitTask r;
    if (a.use_inline) {
      r = a.inline_tasks[t];
    } else if (t - task0 < kTaskLds) {
      const CommitTask u = tlds[t - task0];
      r.b = __builtin_amdgcn_readfirstlane(u.b);
      r.dst_slot = __builtin_amdgcn_readfirstlane(u.dst_slot);
      r.src_tok = __builtin_amdgcn_readfirstlane(u.src_tok);
      r.nvalid = __builtin_amdgcn_readfirstlane(u.nvalid);
      r.mask = (uint32_t)__builtin_amdgcn_readfirstlane((int)u.mask);
      r.rank_base = __builtin_amdgcn_readfirstlane(u.rank_base);
      r.token_base = __builtin_amdgcn_readfirstlane(u.token_base);
      r.pad = 0;
    } else {
      const ConstWords w = (ConstWords)(uintptr_t)(a.tasks + t);
      r.b = w[0]; r.dst_slot = w[1]; r.src_tok = w[2]; r.nvalid = w[3];
      r.mask = (uint32_t)w[4]; r.rank_base = w[5]; r.token_base = w[6]; r.pad = 0;
    }
    return r;
  };

  // ---- item loop: the next item's rows are fetched before the current item
  // is processed; the record buffers alternate, so an item's stores into one
  // buffer never race the previous item's copy-out of the other.  Key and
  // value waves run separate copies of the loop (same barrier count, the
  // branch is uniform per wave), so neither holds the other's registers.
  // Every thread issues the same number of stores (see copy_out), so the wait
  // for the next item's rows, which were loaded before these stores, is a
  // fixed count.
  auto run = [&](const bool role_keys) __attribute__((always_inline)) {
    typename Q::Raw raw;
    int t = task0, hh = beg - task0 * hkv;      // the current item's task and head
    CommitTask cur = task_at(t);
    q.h = hh;
    q.fetch(beg < end, cur, raw);
    {
      // stores that fall outside their resource, in the shape of copy_out:
      // the loop is then entered with the same pending loads and stores as
      // from its back edge, and its waits stay at the fixed store count
      const __amdgpu_buffer_rsrc_t none = __builtin_amdgcn_make_buffer_rsrc(a.seg.headers, 0, 0, 0x00020000);
      const __attribute__((ext_vector_type(4))) unsigned int z = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int r = 0; r < Q::NST + 1; ++r) __builtin_amdgcn_raw_buffer_store_b128(z, none, 0x7ff00000u + 16u * r, 0, 0);
    }
    int it = 0;
    for (int i = beg; i < end; ++i, ++it) {
      // unpack this item's rows, then reuse their registers for the next
      // item's loads
      float x[Q::TPL][8];
#pragma unroll
      for (int k = 0; k < Q::TPL; ++k) Q::unpack_row(raw, k, x[k]);
      const CommitTask task = cur;
      const int h = hh;
      q.h = h;
      // stores of data-dependent count go before the next loads (see copy_out)
      if (role_keys && task.mask != 0u) q.store_protected(task, x);
      const bool more = i + 1 < end;
      const bool wrap = h + 1 == hkv;
      const int tn = more && wrap ? t + 1 : t;
      const CommitTask next = task_at(tn);
      q.h = more ? (wrap ? 0 : h + 1) : h;
      q.fetch(more, next, raw);
      q.h = h;
      uint8_t* rec = recbuf[it & 1];
      if (role_keys) q.process_keys(task, x, rec);
      else           q.process_values(task, x, rec, a.rot.block);
      lds_barrier();
      q.copy_out(task, rec);
      cur = next;
      t = tn;
      hh = more ? (wrap ? 0 : h + 1) : h;
    }
  };
  if (q.keys) run(true);
  else        run(false);
}

// Persistent grid: as many workgroups as the device holds at once (the
// kernel's occupancy per CU times the CU count), or one per item when there
// are fewer items; each workgroup loops over its range of items.
template <int KB, int VB, int D, bool F32IN, bool ROT, int FMT>
hipError_t launch_t(const CommitArgs& a, int ntasks, hipStream_t s) {
  static const int per_cu = [] {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, commit_kernel<KB, VB, D, F32IN, ROT, FMT>, 256, 0) != hipSuccess ||
        n < 1)
      n = 1;
    return n;
  }();
  const int64_t nitems = (int64_t)ntasks * a.hkv;
  dim3 grid((unsigned)std::min<int64_t>(nitems, (int64_t)per_cu * a.num_cus));
  hipLaunchKernelGGL((commit_kernel<KB, VB, D, F32IN, ROT, FMT>), grid, dim3(256), 0, s, a, ntasks);
  return hipGetLastError();
}

template <int KB, int VB, int D>
hipError_t launch_d(const CommitArgs& a, int ntasks, bool f32, hipStream_t s) {
  if constexpr (KB == 4 && VB == 4) {
    if (a.fmt == 1)
      return f32 ? launch_t<KB, VB, D, true, false, 1>(a, ntasks, s) : launch_t<KB, VB, D, false, false, 1>(a, ntasks, s);
  }
  if (a.fmt == 2)
    return f32 ? launch_t<KB, VB, D, true, false, 2>(a, ntasks, s) : launch_t<KB, VB, D, false, false, 2>(a, ntasks, s);
  if (a.rot.block != 0)
    return f32 ? launch_t<KB, VB, D, true, true, 0>(a, ntasks, s) : launch_t<KB, VB, D, false, true, 0>(a, ntasks, s);
  return f32 ? launch_t<KB, VB, D, true, false, 0>(a, ntasks, s) : launch_t<KB, VB, D, false, false, 0>(a, ntasks, s);
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
