"""Throughput of the low-bit block-diffusion KV cache hot path on one MI355X.

One step = one denoising step of one layer for a whole batch, as a
block-diffusion decoder runs it once per block (SoloQ summary page,
block-diffusion paragraph; Tai et al., abstract): the current 32-token block
attends to itself and to the whole quantized prefix cache, and the finished
block is quantized and appended (3 of its key rows kept in bf16).  The step is
one kvq_attend_commit call, a single launch in which the workgroup holding each
(sequence, kv head)'s block also commits it.  The same work as two calls
(kvq_commit of the block, then kvq_block_attn) is timed afterwards
(``ms_per_step_separate_calls``).
Steps rotate over a stack of per-layer caches (28 layers, as in a Dream-7B
model) so that every call reads its cache from HBM rather than from the
256 MB Infinity Cache.

Prints one JSON line; ``value`` is query tokens per second over the timed
steps (B * 32 query tokens per step).  Inputs are seeded synthetic tensors with
the layer shapes (no weights or datasets are used).
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

PEAK_HBM_GBS = 8000.0      # MI355X HBM3E, GB/s
PEAK_F16_TFLOPS = 2500.0   # MI355X dense fp16/bf16 MFMA, TFLOP/s

# HBM bytes of one attention launch on this workload, from rocprofv3 --pmc
# FETCH_SIZE and WRITE_SIZE passes (median KiB per dispatch over the rotation),
# scaled by what the same counters read for a plain copy of 256 MiB
# (bench.py --calibrate-copy 256: FETCH_SIZE reads 131084 KiB for 262144 KiB
# moved, WRITE_SIZE 262144).  Valid only for the kernel source they were taken
# on (its SHA-256); any other source reports null.
_FETCH_SCALE = 262144.0 / 131084.0
_WRITE_SCALE = 1.0
MEASURED_TRAFFIC = {
    "dream7b_4bit": {
        "attn_source_sha256": "0293a1414c09087caaef9185cecc7f3c1f8d2e1b33f2a3a9fd6ab1641521c7ee",
        "kib": {"attn_kernel": {"fetch": 27232.25, "write": 15008},
                "combine_h16_kernel": {"fetch": 7536, "write": 1792}},
    },
}


def measured_traffic(workload):
    """Bytes per attention launch, or None if not measured for this source."""
    import hashlib
    m = MEASURED_TRAFFIC.get(workload)
    if m is None:
        return None
    with open(os.path.join(ROOT, "bit_kv_cache_kivi_amd", "csrc", "attn.hip"), "rb") as f:
        if hashlib.sha256(f.read()).hexdigest() != m["attn_source_sha256"]:
            return None
    return sum((k["fetch"] * _FETCH_SCALE + k["write"] * _WRITE_SCALE) * 1024.0 for k in m["kib"].values())


def attn_algorithmic(cfg, ntok_per_seq, nslots_per_seq, nprot_per_seq, record_bytes):
    """Bytes the method must move and flops it must do for one attention call."""
    B, Hq, Hkv, D = cfg.B, cfg.Hq, cfg.Hkv, cfg.D
    act = 2 if cfg.dtype == "bf16" else 4
    cache = sum(nslots_per_seq) * Hkv * record_bytes + sum(nslots_per_seq) * 16 \
        + sum(nprot_per_seq) * (Hkv * D * 2 + 4)
    io = B * 32 * Hq * D * act * 2 + B * 32 * Hkv * D * act * 2    # q, out, k_blk, v_blk
    flops = sum(4.0 * Hq * 32 * (n + 32) * D for n in ntok_per_seq)
    return cache + io, flops


def commit_algorithmic(cfg, ntok, nprot, record_bytes):
    Hkv, D = cfg.Hkv, cfg.D
    act = 2 if cfg.dtype == "bf16" else 4
    slots = sum(-(-n // 32) for n in ntok)
    return sum(ntok) * Hkv * D * act * 2 + slots * (Hkv * record_bytes + 16) + nprot * (Hkv * D * 2 + 4)


def cpu_baseline(cfg, w, steps_blocks, budget_s=20.0):
    """The oracle (NumPy, fp32 quantization + fp64 attention) on a bounded sample:
    sequence 0 only, all kv heads, full prefix: commit one block, then attention
    of its 32 query tokens for every query head."""
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        threads = 1
    c = cfg
    ora = O.OracleCache(1, c.Hkv, c.D, c.k_bits, c.v_bits, c.v_group)
    ora.commit(0, w.k_prefix[:1], w.v_prefix[:1], ntok=w.lengths[:1],
               prot=[w.prot_prefix[0]] if c.prot_frac else None)
    n_done, t_total = 0, 0.0
    while t_total < budget_s and n_done < 500:
        kb, vb, prot = steps_blocks[n_done % len(steps_blocks)]
        t0 = time.perf_counter()
        ora.commit(0, kb[:1], vb[:1], prot=[prot[0]] if c.step_protect else None)
        O.block_attention(ora, w.q[:1], w.k_blk[:1], w.v_blk[:1])
        t_total += time.perf_counter() - t0
        n_done += 1
    qtok = 32 * n_done
    # the oracle's prefill commit of sequence 0 (all kv heads), best of three,
    # with the thread pools as they are and limited to one thread
    def commit_rate():
        best = float("inf")
        for _ in range(3):
            o = O.OracleCache(1, c.Hkv, c.D, c.k_bits, c.v_bits, c.v_group)
            t0 = time.perf_counter()
            o.commit(0, w.k_prefix[:1], w.v_prefix[:1], ntok=w.lengths[:1],
                     prot=[w.prot_prefix[0]] if c.prot_frac else None)
            best = min(best, time.perf_counter() - t0)
        return float(w.lengths[0]) / best
    commit_tps = commit_rate()
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(1):
            commit_tps_1 = commit_rate()
    except Exception:
        commit_tps_1 = None
    return {"value": qtok / t_total, "unit": "query-tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{n_done} step(s) of sequence 0 of {c.B} (all {c.Hq} query heads, prefix "
                      f"{int(w.lengths[0])} tokens): oracle commit of one 32-token block + fp64 attention; "
                      f"{t_total:.1f} s",
            "commit_tokens_per_s": commit_tps, "commit_tokens_per_s_1thread": commit_tps_1,
            "commit_sample": f"oracle prefill commit of sequence 0 ({int(w.lengths[0])} tokens x {c.Hkv} kv heads), "
                             f"best of 3"}


def measured_peaks(lib, torch, num_cus):
    """Achievable HBM bandwidth (a streaming copy of 1 GiB, larger than the
    Infinity Cache) and dense fp16 MFMA rate (a loop of independent MFMAs with
    no memory traffic), timed with HIP events, from the library's calibration
    kernels."""
    import ctypes
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(3):
        lib.kvq_calib_copy(ctypes.c_void_p(dst.data_ptr()), ctypes.c_void_p(src.data_ptr()), n, sp)
    reps = 10
    e0.record(stream)
    for _ in range(reps):
        lib.kvq_calib_copy(ctypes.c_void_p(dst.data_ptr()), ctypes.c_void_p(src.data_ptr()), n, sp)
    e1.record(stream)
    torch.cuda.synchronize()
    copy_gbs = 2.0 * n * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    wgs, iters = 2 * num_cus, 4000
    out = torch.empty(wgs * 256, dtype=torch.float32, device="cuda")
    lib.kvq_calib_mfma(ctypes.c_void_p(out.data_ptr()), wgs, iters, sp)
    torch.cuda.synchronize()
    e0.record(stream)
    lib.kvq_calib_mfma(ctypes.c_void_p(out.data_ptr()), wgs, iters, sp)
    e1.record(stream)
    torch.cuda.synchronize()
    flops = float(wgs) * 4 * iters * 8 * 32 * 32 * 16 * 2
    mfma_tflops = flops / (e0.elapsed_time(e1) * 1e-3) / 1e12
    return {"hbm_gbs": copy_gbs, "mfma_f16_tflops": mfma_tflops,
            "how": "streaming copy of 1 GiB (2 x bytes moved per copy); 2 x CUs workgroups of 4 waves, each wave "
                   f"{iters} x 8 independent v_mfma_f32_32x32x16_f16"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="dream7b_4bit", choices=sorted(W.CONFIGS))
    ap.add_argument("--layers", type=int, default=28, help="per-layer caches the steps rotate over")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--select-budget", type=int, default=0, metavar="K",
                    help="also time mask-query selection of K entries per (sequence, kv head) and the "
                         "attention over the selection")
    ap.add_argument("--select-granularity", type=int, default=1, choices=(1, 32),
                    help="rank single entries (1) or whole 32-token units (32; the budget then counts units)")
    ap.add_argument("--kv-format", default="int", choices=("int", "int_h16", "mxfp4"),
                    help="cache format: asymmetric integer codes (fp32 or fp16 scales and zeros), or MX FP4 "
                         "(4-bit, 32-channel value groups)")
    ap.add_argument("--v-rotation", type=int, default=0, choices=(0, 16, 64),
                    help="store values K-RPBH rotated with this Hadamard block (0: plain values)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only copy a device buffer of MIB MiB five times (a reference kernel of known "
                         "traffic for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE), then exit")
    args = ap.parse_args()
    if args.calibrate_copy:
        import torch
        n = args.calibrate_copy << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n, "copies": 5}), flush=True)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(json.dumps({"error": "this build runs on one GPU only: there is no multi-GPU path; "
                                   "run with --gpus 1"}), flush=True)
        sys.exit(2)

    import torch
    from bit_kv_cache_kivi_amd import kvq

    cfg = W.CONFIGS[args.config]
    if args.kv_format == "mxfp4":
        import dataclasses
        cfg = dataclasses.replace(cfg, k_bits=4, v_bits=4, v_group=32)
    w = W.make(cfg)
    c = cfg
    L = args.layers
    # commits per layer cache: the warm-up loop, three timed loops of
    # consecutive steps (the step, the separate-calls step, commit alone) and
    # at most 2L single steps timed one by one, each spread round-robin over
    # the L caches
    commits_per_layer = -(-args.warmup // L) + 3 * -(-args.steps // L) + 2
    nblk = 4
    blocks = [W.step_block(c, s) for s in range(nblk)]

    dt = torch.bfloat16 if c.dtype == "bf16" else torch.float32
    to = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dt).cuda().contiguous()   # noqa: E731
    kp, vp = to(w.k_prefix), to(w.v_prefix)
    q, kblk, vblk = to(w.q), to(w.k_blk), to(w.v_blk)
    dblocks = [(to(k), to(v), p) for k, v, p in blocks]
    out = torch.empty(q.shape, dtype=torch.bfloat16, device="cuda")

    max_prefix = int(w.lengths.max())
    prot_cap = max(len(p) for p in w.prot_prefix) + c.step_protect * commits_per_layer + 8
    sprot_cap = max([len(p) for p in (w.prot_suffix or [])] + [0]) + 8
    caches = []
    for _ in range(L):
        caches.append(kvq.KVCache(c.B, c.Hkv, c.D, c.k_bits, c.v_bits, c.v_group,
                                  prefix_tokens=max_prefix + 32 * (commits_per_layer + 1),
                                  suffix_tokens=c.suffix, prefix_protected=prot_cap,
                                  suffix_protected=sprot_cap if c.suffix else 0, max_q_heads=c.Hq,
                                  v_rotation_block=args.v_rotation,
                                  kv_format={"int": kvq.KVQ_FMT_INT, "int_h16": kvq.KVQ_FMT_INT_H16,
                                             "mxfp4": kvq.KVQ_FMT_MXFP4}[args.kv_format]))
        if args.v_rotation:
            caches[-1].set_v_rotation(*W.krpbh_params(c.D, args.v_rotation))
    torch.cuda.synchronize()
    # Prefill: one commit of the whole prefix into each layer cache, through
    # prebuilt C-ABI arguments.  After an untimed first round (a handle's first
    # device call also sets up its host-side ring and events), every layer's
    # prefix is committed again with the segment reset, timed with events
    # around all L commits.
    stream0 = torch.cuda.current_stream()
    s0 = ctypes.c_void_p(stream0.cuda_stream)
    dt0 = kvq.KVQ_BF16 if c.dtype == "bf16" else kvq.KVQ_F32
    h_ntok = (ctypes.c_int32 * c.B)(*[int(n) for n in w.lengths])
    if c.prot_frac:
        offs = np.concatenate([[0], np.cumsum([len(p) for p in w.prot_prefix])]).astype(np.int32)
        h_off = (ctypes.c_int32 * (c.B + 1))(*[int(x) for x in offs])
        h_idx = (ctypes.c_int32 * max(int(offs[-1]), 1))(*[int(x) for p in w.prot_prefix for x in p])
    else:
        h_off = h_idx = None
    n_max = int(kp.shape[1])

    def prefill(cache, reset):
        kvq.check(kvq.lib.kvq_commit(cache.handle, 0, reset, ctypes.c_void_p(kp.data_ptr()),
                                     ctypes.c_void_p(vp.data_ptr()), dt0, n_max, h_ntok, h_off, h_idx, s0))
    for cache in caches:
        prefill(cache, 0)
    torch.cuda.synchronize()
    p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    p0.record(stream0)
    th0 = time.perf_counter()
    for cache in caches:
        prefill(cache, 1)
    prefill_host_ms = (time.perf_counter() - th0) * 1e3 / L    # host time to issue one call
    p1.record(stream0)
    torch.cuda.synchronize()
    prefill_ms = p0.elapsed_time(p1) / L
    if c.suffix:
        ks, vs = to(w.k_suffix), to(w.v_suffix)
        for cache in caches:
            cache.commit(ks, vs, protected=w.prot_suffix if c.prot_frac else None, segment=kvq.KVQ_SUFFIX)
        del ks, vs
    del kp, vp
    torch.cuda.synchronize()
    R = caches[0].layout["record_bytes"]
    stream = torch.cuda.current_stream()
    sptr = ctypes.c_void_p(stream.cuda_stream)
    lib = kvq.lib

    # Prebuilt C-ABI arguments: the timed loops are plain ctypes calls.
    dtc = kvq.KVQ_BF16 if c.dtype == "bf16" else kvq.KVQ_F32
    commit_args = []
    for kb, vb, prot in dblocks:
        if c.step_protect:
            off = (ctypes.c_int32 * (c.B + 1))(*[c.step_protect * i for i in range(c.B + 1)])
            idx = (ctypes.c_int32 * (c.step_protect * c.B))(*[int(x) for p in prot for x in p])
        else:
            off = idx = None
        commit_args.append((ctypes.c_void_p(kb.data_ptr()), ctypes.c_void_p(vb.data_ptr()), off, idx))
    attn_args = (ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(kblk.data_ptr()),
                 ctypes.c_void_p(vblk.data_ptr()), ctypes.c_void_p(out.data_ptr()))
    scale = 1.0 / math.sqrt(c.D)
    commits = [0] * L            # block commits made so far into each layer

    def do_commit(i):
        kp_, vp_, off, idx = commit_args[i % nblk]
        kvq.check(lib.kvq_commit(caches[i % L].handle, 0, 0, kp_, vp_, dtc, 32, None, off, idx, sptr))
        commits[i % L] += 1

    def do_attn(i):
        qp, kbp, vbp, op = attn_args
        kvq.check(lib.kvq_block_attn(caches[i % L].handle, 1 if c.suffix else 0, qp, c.Hq, dtc, kbp, vbp, dtc,
                                     32, scale, op, kvq.KVQ_BF16, sptr))

    def attn_counts(layer):
        """Algorithmic bytes/flops of one attention call on a layer's cache as it stands."""
        ntok = [int(n) + 32 * commits[layer] + c.suffix for n in w.lengths]
        nslots = [-(-int(n) // 32) + commits[layer] + -(-c.suffix // 32) for n in w.lengths]
        nprot = [len(p) + c.step_protect * commits[layer] for p in w.prot_prefix]
        if c.suffix and c.prot_frac:
            nprot = [n + len(p) for n, p in zip(nprot, w.prot_suffix)]
        return attn_algorithmic(c, ntok, nslots, nprot, R)

    def timed(fn, n, first):
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(first, first + n):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    # The same work as one kvq_attend_commit call: the attention of a block over
    # the cache as it is, then the commit of that block.
    def do_attend_commit(i):
        qp, _, _, op = attn_args
        kp_, vp_, off, idx = commit_args[i % nblk]
        kvq.check(lib.kvq_attend_commit(caches[i % L].handle, 1 if c.suffix else 0, qp, c.Hq, dtc, kp_, vp_, dtc,
                                        32, scale, op, kvq.KVQ_BF16, None, off, idx, sptr))
        commits[i % L] += 1

    def separate(i):
        do_commit(i)
        do_attn(i)
    # Untimed spin-up before the warmup steps: attention launches for about
    # 0.3 s, so that the device clocks have settled when the timed steps start
    # (the first timed loop otherwise runs a few percent slower).
    t_spin = time.perf_counter()
    i_spin = 0
    while time.perf_counter() - t_spin < 0.3:
        do_attn(i_spin)
        i_spin += 1
        if i_spin % 64 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    for i in range(args.warmup):
        do_attend_commit(i)
    torch.cuda.synchronize()

    # (1) the step: one kvq_attend_commit call (attention of the block over the
    # cache as it is, and the commit of the block, in one launch)
    t0 = time.perf_counter()
    ms_per_step = timed(do_attend_commit, args.steps, args.warmup)
    wall = time.perf_counter() - t0

    # (1a) the distribution of single-step times: each of min(steps, 2L)
    # further steps bracketed by its own pair of events (per-call GPU time,
    # taken after the timed loop so that the loop has no events inside it)
    n_dist = min(args.steps, 2 * L)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_dist)]
    torch.cuda.synchronize()
    for i, (ea, eb) in enumerate(ev):
        ea.record(stream)
        do_attend_commit(args.warmup + args.steps + i)
        eb.record(stream)
    torch.cuda.synchronize()
    step_dist = np.array([ea.elapsed_time(eb) for ea, eb in ev])

    # (1b) the same work as two calls: commit the finished block, then attend
    ms_per_step_separate = timed(separate, args.steps, 0)

    # (2) attention alone (one launch = attention kernel + split combine), same rotation
    a_bytes = a_flops = 0.0
    for i in range(args.steps):
        bts, fl = attn_counts(i % L)
        a_bytes += bts
        a_flops += fl
    a_bytes /= args.steps
    a_flops /= args.steps
    attn_ms = timed(do_attn, args.steps, 0)

    # (3) commit alone: 32-token blocks, same rotation
    commit_ms = timed(do_commit, args.steps, 0)
    commit_bytes = commit_algorithmic(c, [32] * c.B, c.step_protect * c.B, R)


    # (5) optional: selection of the top K entries per (sequence, kv head), then
    # attention over the selection (the block's mask queries = all 32 tokens)
    sel = None
    if args.select_budget:
        qp, kbp, vbp, op = attn_args
        use_suf = 1 if c.suffix else 0

        def do_select(i):
            kvq.check(lib.kvq_select(caches[i % L].handle, use_suf, qp, c.Hq, dtc, kbp, dtc, 32, scale, None,
                                     args.select_budget, args.select_granularity, sptr))

        def do_attn_sel(i):
            kvq.check(lib.kvq_block_attn_selected(caches[i % L].handle, use_suf, qp, c.Hq, dtc, kbp, vbp, dtc, 32,
                                                  scale, op, kvq.KVQ_BF16, sptr))
        def do_attend_select(i):
            kvq.check(lib.kvq_attend_select(caches[i % L].handle, use_suf, qp, c.Hq, dtc, kbp, vbp, dtc, 32, scale,
                                            op, kvq.KVQ_BF16, None, args.select_budget, args.select_granularity,
                                            sptr))
        # one untimed call of each first: a kernel's first launch in the
        # process loads its code
        for fn in (do_select, do_attend_select, do_attn_sel):
            fn(0)
        select_ms = timed(do_select, 2 * L, 0)
        attend_select_ms = timed(do_attend_select, 2 * L, 0)
        attn_sel_ms = timed(do_attn_sel, args.steps, 0)
        sel = {"budget": args.select_budget, "granularity": args.select_granularity, "select_ms": select_ms,
               "attend_select_ms": attend_select_ms, "attn_selected_ms": attn_sel_ms,
               "attn_full_ms": attn_ms,
               "attn_selected_query_tokens_per_s": c.B * 32 / (attn_sel_ms * 1e-3)}

    peaks = measured_peaks(lib, torch, torch.cuda.get_device_properties(0).multi_processor_count)

    qtok = c.B * 32
    attn_s = attn_ms * 1e-3
    achieved_tflops = a_flops / attn_s / 1e12
    achieved_gbs = a_bytes / attn_s / 1e9
    # the roofline that binds at this workload: MFMA time against HBM time of
    # the algorithmic flops and bytes
    if a_flops / (PEAK_F16_TFLOPS * 1e12) >= a_bytes / (PEAK_HBM_GBS * 1e9):
        roof = {"bound": "mfma", "achieved": achieved_tflops, "peak": PEAK_F16_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved_tflops / PEAK_F16_TFLOPS}
    else:
        roof = {"bound": "hbm", "achieved": achieved_gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": achieved_gbs / PEAK_HBM_GBS}
    prefill_bytes = commit_algorithmic(c, [int(n) for n in w.lengths], sum(len(p) for p in w.prot_prefix), R)
    res = {
        "metric": "block-attn query-tokens/s + achieved HBM GB/s, 4-bit KV, Dream-7B shape",
        "value": qtok / (ms_per_step * 1e-3),
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": c.name, "batch": c.B, "q_heads": c.Hq, "kv_heads": c.Hkv, "head_dim": c.D,
                   "prefix_tokens": int(max_prefix), "block": 32, "k_bits": c.k_bits, "v_bits": c.v_bits,
                   "v_group": c.v_group, "protected_frac": c.prot_frac, "layers_rotated": L,
                   "v_rotation_block": args.v_rotation, "kv_format": args.kv_format, "parallelism": "none"},
        "attn_ms": attn_ms,
        "commit_ms": commit_ms,
        "ms_per_step_attend_commit": ms_per_step,
        "ms_per_step_separate_calls": ms_per_step_separate,
        "step_ms_p10_p50_p90": [float(np.percentile(step_dist, p)) for p in (10, 50, 90)],
        "step_ms_samples": int(len(step_dist)),
        "attn_query_tokens_per_s": qtok / attn_s,
        "attn_hbm_gbs": achieved_gbs,
        "attn_tflops": achieved_tflops,
        "commit_tokens_per_s": c.B * 32 / (commit_ms * 1e-3),
        "commit_gbs": commit_bytes / (commit_ms * 1e-3) / 1e9,
        "prefill_commit_ms": prefill_ms,
        "prefill_commit_tokens_per_s": float(np.sum(w.lengths)) / (prefill_ms * 1e-3),
        "prefill_commit_gbs": prefill_bytes / (prefill_ms * 1e-3) / 1e9,
        "prefill_commit_hbm_frac": prefill_bytes / (prefill_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "prefill_commit_frac_of_measured_hbm": prefill_bytes / (prefill_ms * 1e-3) / 1e9 / peaks["hbm_gbs"],
        "prefill_commit_host_issue_ms": prefill_host_ms,
        "host_wall_ms_per_step": wall * 1e3 / args.steps,
        "roofline": {**roof, "traffic": None if (args.v_rotation or args.kv_format != "int") else measured_traffic(c.name),
                     "kernel": "attention launch (attn_kernel + combine_h16_kernel" +
                               (", with blk_prep_kernel and unrotate_kernel)" if args.v_rotation else ")"),
                     "mfma_frac": achieved_tflops / PEAK_F16_TFLOPS, "hbm_frac": achieved_gbs / PEAK_HBM_GBS,
                     "measured_peak": peaks,
                     "frac_of_measured_peak": (achieved_tflops / peaks["mfma_f16_tflops"]) if roof["bound"] == "mfma"
                                              else (achieved_gbs / peaks["hbm_gbs"])},
    }
    if sel is not None:
        res["selection"] = sel
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(c, w, blocks, args.cpu_budget)
    print(json.dumps(res), flush=True)
    for cache in caches:
        cache.close()


if __name__ == "__main__":
    main()
