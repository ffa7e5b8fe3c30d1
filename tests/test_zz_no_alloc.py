"""kvq_block_attn_noalloc (the attention entry point that allocates nothing:
its split partials and rotation staging live in the library's per-device
scratch array) against kvq_block_attn on the same cache (needs an MI355X):
outputs bit-identical, and within the attention gate of the fp64 oracle, over
calls in a row with shrinking inputs; a launch too large for the scratch array
is refused before any device work."""
import numpy as np
import pytest

import oracle as O
import workloads as W

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from bit_kv_cache_kivi_amd import kvq  # noqa: E402
from gpu_util import announce, attention_error, build_case, dev  # noqa: E402


def _check(name, T, B, v_rot=0, split_slots=0):
    announce("noalloc", name, T, B, v_rot, split_slots)
    w, cache, ora = build_case(W.CONFIGS[name], T, B, v_rot_block=v_rot)
    c = w.cfg
    if split_slots:
        cache.set_split_slots(split_slots)
    use_suffix = bool(c.suffix)
    q, kb, vb = dev(w.q, c.dtype), dev(w.k_blk, c.dtype), dev(w.v_blk, c.dtype)
    ref = O.block_attention(ora, w.q, w.k_blk, w.v_blk, use_suffix=use_suffix)
    for out_dtype, gate in ((torch.float32, "f32"), (torch.bfloat16, "bf16")):
        want = cache.block_attn(q, kb, vb, use_suffix=use_suffix, out_dtype=out_dtype)
        out = torch.full_like(want, float("nan"))
        got = cache.block_attn_noalloc(q, kb, vb, use_suffix=use_suffix, out=out)
        torch.cuda.synchronize()
        assert torch.equal(got, want), f"{name}: noalloc output differs from kvq_block_attn"
        e, x = attention_error(got, ref, gate)
        assert x <= 0, (name, gate, e)
    cache.close()


def test_noalloc_matches_block_attn_in_a_row():
    # large (several splits per (sequence, kv head), partials in the scratch
    # array), then a smaller cache (one split), then the dual cache, then
    # rotated values (rotation staging in the scratch array too)
    _check("dream7b_4bit", 2000, 4)
    _check("tiny", None, None)
    _check("dual_long", 640, 2, split_slots=3)
    _check("dream7b_4bit", 300, 2, v_rot=64, split_slots=4)


def test_noalloc_refuses_oversized_workspace():
    announce("noalloc capacity")
    cfg = W.CONFIGS["dream7b_4bit"]
    w = W.make(cfg, T=2048, B=8)
    c = w.cfg
    cache = kvq.KVCache(c.B, c.Hkv, c.D, c.k_bits, c.v_bits, c.v_group, prefix_tokens=2048 + 64,
                        prefix_protected=512, max_q_heads=c.Hq, max_splits=256)
    cache.commit(dev(w.k_prefix, c.dtype), dev(w.v_prefix, c.dtype), ntok=w.lengths, protected=w.prot_prefix)
    cache.set_split_slots(1)          # one unit per split: 65 splits x 32 pairs x 7 heads of partials
    q, kb, vb = dev(w.q, c.dtype), dev(w.k_blk, c.dtype), dev(w.v_blk, c.dtype)
    out = torch.zeros(q.shape, dtype=torch.float32, device="cuda")
    with pytest.raises(kvq.KvqError) as ei:
        cache.block_attn_noalloc(q, kb, vb, out=out)
    assert ei.value.status == kvq.KVQ_ECAPACITY
    torch.cuda.synchronize()
    assert torch.count_nonzero(out).item() == 0          # nothing ran
    # the regular call with its own workspace still serves this launch
    ref = O.OracleCache(c.B, c.Hkv, c.D, c.k_bits, c.v_bits, c.v_group)
    ref.commit(0, w.k_prefix, w.v_prefix, ntok=w.lengths, prot=w.prot_prefix)
    e, x = attention_error(cache.block_attn(q, kb, vb, out_dtype=torch.float32),
                           O.block_attention(ref, w.q, w.k_blk, w.v_blk), "f32")
    assert x <= 0, e
    cache.close()
