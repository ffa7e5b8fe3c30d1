"""GPU-vs-oracle parity of the cache variants at the full dream7b_4bit shape
(batch 8, 28/4 heads, D 128, prefix 8192 tokens, 10% protected key rows, bf16
inputs), in the launch configuration the benchmark times: MX FP4 records,
fp16 scales and zeros, K-RPBH rotated values, selection of whole 32-token
units, and the one-launch attend-and-commit step.  Every record, header and
protected row byte for byte; every attention output within the gate
(2e-3 with fp32 output, plus half a bf16 ulp with bf16 output)."""
import dataclasses

import numpy as np
import pytest

import oracle as O
import workloads as W
from oracle.selection import block_attention_selected

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from bit_kv_cache_kivi_amd import kvq  # noqa: E402
from gpu_util import announce, attention_error, build_case, compare_commit, dev  # noqa: E402
from test_gpu_selection import check_selection  # noqa: E402

CFG = W.CONFIGS["dream7b_4bit"]


def _attention_both(cache, w, ref, tag):
    c = w.cfg
    q, kb, vb = dev(w.q, c.dtype), dev(w.k_blk, c.dtype), dev(w.v_blk, c.dtype)
    for dt, gate in ((torch.float32, "f32"), (torch.bfloat16, "bf16")):
        out = cache.block_attn(q, kb, vb, out_dtype=dt)
        e, x = attention_error(out, ref, gate)
        print(f"{tag} {gate}-out err={e:.2e}", flush=True)
        assert x <= 0, (tag, gate, e)


@pytest.mark.parametrize("fmt", ["mxfp4", "int_h16"])
def test_full_size_record_formats(fmt):
    announce("full size format", fmt)
    cfg = dataclasses.replace(CFG, v_group=32) if fmt == "mxfp4" else CFG
    w = W.make(cfg)
    c = w.cfg
    kvf = kvq.KVQ_FMT_MXFP4 if fmt == "mxfp4" else kvq.KVQ_FMT_INT_H16
    cache = kvq.KVCache(c.B, c.Hkv, c.D, c.k_bits, c.v_bits, c.v_group, prefix_tokens=int(w.lengths.max()) + 64,
                        prefix_protected=max(len(p) for p in w.prot_prefix) + 64, max_q_heads=c.Hq, kv_format=kvf)
    ora = O.OracleCache(c.B, c.Hkv, c.D, c.k_bits, c.v_bits, c.v_group, fmt=fmt)
    cache.commit(dev(w.k_prefix, c.dtype), dev(w.v_prefix, c.dtype), ntok=w.lengths, protected=w.prot_prefix)
    ora.commit(0, w.k_prefix, w.v_prefix, ntok=w.lengths, prot=w.prot_prefix)
    compare_commit(cache, ora, 0, c.B)
    _attention_both(cache, w, O.block_attention(ora, w.q, w.k_blk, w.v_blk), fmt)
    cache.close()


def test_full_size_rotated_values():
    announce("full size rotated values")
    w, cache, ora = build_case(CFG, extra_slots=2, v_rot_block=64)
    c = w.cfg
    compare_commit(cache, ora, 0, c.B)
    _attention_both(cache, w, O.block_attention(ora, w.q, w.k_blk, w.v_blk), "rotated b=64")
    cache.close()


def test_full_size_unit_selection():
    announce("full size unit selection")
    w, cache, ora = build_case(CFG, extra_slots=2)
    c = w.cfg
    q, kb, vb = dev(w.q, c.dtype), dev(w.k_blk, c.dtype), dev(w.v_blk, c.dtype)
    budget = 32
    cache.select(q, kb, budget, granularity=32)
    selected = check_selection(cache, ora, w, budget, False, None, 32)
    ref = block_attention_selected(ora, w.q, w.k_blk, w.v_blk, selected)
    out = cache.block_attn_selected(q, kb, vb, out_dtype=torch.float32)
    e, x = attention_error(out, ref, "f32")
    print(f"unit selection of {budget} units: err={e:.2e}", flush=True)
    assert x <= 0, e
    cache.close()


@pytest.mark.parametrize("v_rot,odt", [(0, "f32"), (64, "bf16")])
def test_full_size_attend_commit_steps(v_rot, odt):
    """Two one-launch steps at full size: each output against the oracle's
    attention over the cache before its commit; records afterwards.  With
    rotated values and bf16 output (the rotated benchmark's configuration),
    the merge rotates the output back and the fused commit quantizes the
    rotated copy of the block."""
    announce("full size attend_commit", v_rot, odt)
    w, cache, ora = build_case(CFG, extra_slots=3, v_rot_block=v_rot)
    c = w.cfg
    out_dt = torch.float32 if odt == "f32" else torch.bfloat16
    for s in range(2):
        kb_, vb_, prot = W.step_block(c, s)
        ref = O.block_attention(ora, w.q, kb_, vb_)
        out = cache.attend_commit(dev(w.q, c.dtype), dev(kb_, c.dtype), dev(vb_, c.dtype), protected=prot,
                                  out_dtype=out_dt)
        ora.commit(0, kb_, vb_, prot=prot)
        e, x = attention_error(out, ref, odt)
        print(f"attend_commit step {s} (rotation {v_rot}, {odt}): err={e:.2e}", flush=True)
        assert x <= 0, (s, e)
    compare_commit(cache, ora, 0, c.B)
    cache.close()


def test_full_size_attend_select_entries():
    """kvq_attend_select at full size in the benchmark's launch configuration
    (bf16 output, split partials merged by the fp16 combine, which also writes
    the row statistics): the output within the bf16 gate of the oracle's
    attention, then a per-entry selection of 1024 of the 8224 entries of each
    (sequence, kv head) -- the radix path of the top-k -- checked as
    kvq_select's is."""
    announce("full size attend_select, entries")
    w, cache, ora = build_case(CFG, extra_slots=2)
    c = w.cfg
    q, kb, vb = dev(w.q, c.dtype), dev(w.k_blk, c.dtype), dev(w.v_blk, c.dtype)
    budget = 1024
    out = cache.attend_select(q, kb, vb, budget, out_dtype=torch.bfloat16)
    e, x = attention_error(out, O.block_attention(ora, w.q, w.k_blk, w.v_blk), "bf16")
    print(f"attend_select output: err={e:.2e}", flush=True)
    assert x <= 0, e
    check_selection(cache, ora, w, budget, False, None, 1)
    cache.close()
