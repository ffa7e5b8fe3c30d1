"""Helpers for the GPU parity tests: upload seeded inputs, run the C ABI, compare
with the oracle.  Imported only by tests marked ``gpu``."""
import sys

import numpy as np

import oracle as O
import workloads as W


def announce(*msg):
    print("[case]", *msg, flush=True)
    sys.stdout.flush()


def dev(x, dtype):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    t = t.to(torch.bfloat16) if dtype == "bf16" else t
    return t.cuda().contiguous()


def ulp_bf16(x):
    ax = np.abs(np.asarray(x, np.float64))
    e = np.floor(np.log2(np.maximum(ax, 2.0 ** -126)))
    return 2.0 ** (e - 7)


def compare_commit(cache, ora: O.OracleCache, segment: int, B: int):
    """Bytes of every record, header and protected row must be identical."""
    import torch
    torch.cuda.synchronize()
    D, kb, vb, gv = ora.D, ora.kb, ora.vb, ora.gv
    for b in range(B):
        ntok, nslots, nprot = (x[b] for x in cache.segment_info(segment))
        assert ntok == ora.ntok(segment, b) and nslots == ora.nslots(segment, b)
        if nslots == 0:
            continue
        got = cache.records(segment, b).cpu().numpy()
        want = ora.records(segment, b)
        assert got.shape == want.shape, (got.shape, want.shape)
        if not np.array_equal(got, want) and getattr(ora, "fmt", "int") != "int":
            bad = np.argwhere(got != want)
            raise AssertionError(f"segment {segment} seq {b}: {len(bad)} record bytes differ, first at "
                                 f"(slot, head, byte) {tuple(bad[0])}: gpu {got[tuple(bad[0])]} oracle {want[tuple(bad[0])]}")
        if not np.array_equal(got, want):
            gu = O.unpack_record(got, D, kb, vb, gv)
            wu = O.unpack_record(want, D, kb, vb, gv)
            report = []
            for k in gu:
                bad = np.argwhere(gu[k].view(np.uint32 if gu[k].dtype == np.float32 else gu[k].dtype)
                                  != wu[k].view(np.uint32 if wu[k].dtype == np.float32 else wu[k].dtype))
                if len(bad):
                    i = tuple(bad[0])
                    report.append(f"{k}: {len(bad)} differ, first {i}: gpu {gu[k][i]!r} oracle {wu[k][i]!r}")
            raise AssertionError(f"segment {segment} seq {b}: records differ; " + "; ".join(report))
        gh = cache.headers(segment, b).cpu().numpy()
        assert np.array_equal(gh, ora.headers(segment, b)), f"headers differ (seq {b})"
        pos, rows = cache.protected_rows(segment, b)
        opos, orows = ora.protected(segment, b)
        assert np.array_equal(pos.cpu().numpy(), opos), f"protected positions differ (seq {b})"
        assert len(opos) == nprot
        if nprot:
            obits = (orows.view(np.uint32) >> 16).astype(np.uint16).view(np.int16)
            assert np.array_equal(rows.cpu().numpy(), obits), f"protected rows differ (seq {b})"


def attention_error(out, ref, out_dtype="f32"):
    """(max abs error, max excess over the gate) for an output tensor vs fp64 oracle."""
    import torch
    o = out.float().cpu().numpy().astype(np.float64)
    mask = ~np.isnan(ref)
    err = np.abs(o - ref)[mask]
    gate = 2e-3 if out_dtype == "f32" else 2e-3 + 0.5 * ulp_bf16(ref[mask])
    return float(err.max()), float((err - gate).max())


def build_case(cfg, T=None, B=None, extra_slots=4, v_rot_block=0):
    """Seeded workload, a device cache and an oracle cache, both holding the
    committed prefix (and suffix).  Shared by the GPU parity tests.
    v_rot_block != 0: values are stored K-RPBH rotated (blocks of that size)."""
    from bit_kv_cache_kivi_amd import kvq
    w = W.make(cfg, T=T, B=B)
    c = w.cfg
    nprot_p = max([len(p) for p in w.prot_prefix] + [0]) + 64
    nprot_s = max([len(p) for p in (w.prot_suffix or [])] + [0]) + 64
    cache = kvq.KVCache(c.B, c.Hkv, c.D, c.k_bits, c.v_bits, c.v_group,
                        prefix_tokens=int(w.lengths.max()) + 32 * extra_slots,
                        suffix_tokens=c.suffix + (32 if c.suffix else 0),
                        prefix_protected=nprot_p, suffix_protected=nprot_s if c.suffix else 0,
                        max_q_heads=c.Hq, v_rotation_block=v_rot_block)
    v_rot = None
    if v_rot_block:
        perm, mix = W.krpbh_params(c.D, v_rot_block)
        cache.set_v_rotation(perm, mix)
        v_rot = (perm, mix, v_rot_block)
    ora = O.OracleCache(c.B, c.Hkv, c.D, c.k_bits, c.v_bits, c.v_group, v_rot=v_rot)
    prot = w.prot_prefix if c.prot_frac > 0 else None
    cache.commit(dev(w.k_prefix, c.dtype), dev(w.v_prefix, c.dtype), ntok=w.lengths, protected=prot)
    ora.commit(0, w.k_prefix, w.v_prefix, ntok=w.lengths, prot=prot)
    if c.suffix:
        sprot = w.prot_suffix if c.prot_frac > 0 else None
        cache.commit(dev(w.k_suffix, c.dtype), dev(w.v_suffix, c.dtype), protected=sprot, segment=kvq.KVQ_SUFFIX)
        ora.commit(1, w.k_suffix, w.v_suffix, prot=sprot)
    return w, cache, ora
