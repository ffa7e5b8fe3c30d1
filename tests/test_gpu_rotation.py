"""GPU parity of the K-RPBH rotated-value variant (SoloQ summary page, rotation
paragraphs; values follow the activation path, block-diffusion paragraph):
committed values are rotated before quantization, so the stored codes must
equal the oracle's bit for bit, and attention, which rotates the current
block's values alike and returns the transposed rotation of its output, must
meet the same gate as the plain path."""
import dataclasses

import numpy as np
import pytest

import oracle as O
import workloads as W

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from bit_kv_cache_kivi_amd import kvq  # noqa: E402
from gpu_util import announce, attention_error, build_case, compare_commit, dev  # noqa: E402


@pytest.mark.parametrize("name,T,B,block", [
    ("tiny", None, None, 16), ("tiny", None, None, 64),
    ("dream7b_4bit", 300, 2, 64), ("dream7b_2bit", 300, 2, 16), ("dual_long", 400, 2, 64)])
def test_rotated_commit_and_attention(name, T, B, block):
    announce("rotated", name, T, B, block)
    w, cache, ora = build_case(W.CONFIGS[name], T, B, v_rot_block=block)
    c = w.cfg
    compare_commit(cache, ora, 0, c.B)
    if c.suffix:
        compare_commit(cache, ora, 1, c.B)
    ref = O.block_attention(ora, w.q, w.k_blk, w.v_blk, use_suffix=bool(c.suffix))
    q, kb, vb = dev(w.q, c.dtype), dev(w.k_blk, c.dtype), dev(w.v_blk, c.dtype)
    out32 = cache.block_attn(q, kb, vb, use_suffix=bool(c.suffix), out_dtype=torch.float32)
    e32, x32 = attention_error(out32, ref, "f32")
    out16 = cache.block_attn(q, kb, vb, use_suffix=bool(c.suffix), out_dtype=torch.bfloat16)
    e16, x16 = attention_error(out16, ref, "bf16")
    print(f"{name} b={block}: fp32-out err={e32:.2e} bf16-out err={e16:.2e}")
    assert x32 <= 0, f"fp32 output error {e32}"
    assert x16 <= 0, f"bf16 output error {e16}"


@pytest.mark.parametrize("kb,vb,gv,block", [(2, 2, 32, 16), (4, 2, 128, 64), (2, 4, 64, 16)])
def test_rotated_value_groups_and_splits(kb, vb, gv, block):
    """Every value-group size under rotation, with forced split-K and with one
    split per pair.  fp32 output: the fp32 merge writes the rotated output,
    which is then rotated back; bf16 output: every pair's splits (one
    included) go to the fp16 merge, which also applies the transposed
    rotation."""
    announce("rotated groups", kb, vb, gv, block)
    cfg = dataclasses.replace(W.CONFIGS["dream7b_4bit"], k_bits=kb, v_bits=vb, v_group=gv)
    w, cache, ora = build_case(cfg, T=300, B=2, v_rot_block=block)
    c = w.cfg
    compare_commit(cache, ora, 0, c.B)
    ref = O.block_attention(ora, w.q, w.k_blk, w.v_blk)
    q, k_, v_ = dev(w.q, c.dtype), dev(w.k_blk, c.dtype), dev(w.v_blk, c.dtype)
    for split in (0, 3, 1000):
        cache.set_split_slots(split)
        out = cache.block_attn(q, k_, v_, out_dtype=torch.float32)
        e, x = attention_error(out, ref, "f32")
        out16 = cache.block_attn(q, k_, v_, out_dtype=torch.bfloat16)
        e16, x16 = attention_error(out16, ref, "bf16")
        print(f"kb={kb} vb={vb} gv={gv} b={block} split={split}: err={e:.2e} bf16-out err={e16:.2e}")
        assert x <= 0, f"fp32 output error {e}"
        assert x16 <= 0, f"bf16 output error {e16}"


def test_rotated_fp32_input_partial_slots():
    """fp32 inputs, ragged lengths, protected key rows (keys are not rotated),
    a second commit after partial slots, a suffix reset, then dual-cache
    attention with fp32 block operands."""
    B, H, D = 3, 2, 128
    g = np.random.default_rng(7)
    for block in (16, 64):
        announce("rotated fp32 ragged", block)
        perm, mix = W.krpbh_params(D, block, seed=3)
        cache = kvq.KVCache(B, H, D, 4, 2, 64, prefix_tokens=320, suffix_tokens=64, prefix_protected=64,
                            suffix_protected=8, max_q_heads=4, v_rotation_block=block)
        cache.set_v_rotation(perm, mix)
        ora = O.OracleCache(B, H, D, 4, 2, 64, v_rot=(perm, mix, block))
        # unit-scale keys and offset values (|x| < 4 or so: the fp16 operand
        # rounding then stays within the gate, as on the synthetic workloads)
        k = g.standard_normal((B, 100, H, D)).astype(np.float32)
        v = g.standard_normal((B, 100, H, D)).astype(np.float32) * np.float32(0.7) + np.float32(0.5)
        ntok = [100, 45, 1]
        prot = [np.array([0, 5, 64]), np.array([], np.int64), np.array([0])]
        cache.commit(dev(k, "f32"), dev(v, "f32"), ntok=ntok, protected=prot)
        ora.commit(0, k, v, ntok=ntok, prot=prot)
        cache.commit(dev(v[:, :40], "f32"), dev(k[:, :40], "f32"), ntok=[40, 33, 0])
        ora.commit(0, v[:, :40], k[:, :40], ntok=[40, 33, 0])
        cache.commit(dev(k[:, :64], "f32"), dev(v[:, :64], "f32"), segment=kvq.KVQ_SUFFIX)
        ora.commit(1, k[:, :64], v[:, :64])
        sk, sv = np.ascontiguousarray(v[:, 10:60]), np.ascontiguousarray(k[:, 10:60])
        cache.commit(dev(sk, "f32"), dev(sv, "f32"), ntok=[50, 20, 7], segment=kvq.KVQ_SUFFIX, reset=True)
        ora.commit(1, sk, sv, ntok=[50, 20, 7], reset=True)
        compare_commit(cache, ora, 0, B)
        compare_commit(cache, ora, 1, B)
        q = g.standard_normal((B, 32, 4, D)).astype(np.float32)
        kb = g.standard_normal((B, 32, H, D)).astype(np.float32)
        vb = g.standard_normal((B, 32, H, D)).astype(np.float32)
        ref = O.block_attention(ora, q, kb, vb, use_suffix=True)
        out = cache.block_attn(dev(q, "f32"), dev(kb, "f32"), dev(vb, "f32"), use_suffix=True,
                               out_dtype=torch.float32)
        e, x = attention_error(out, ref, "f32")
        print(f"fp32 ragged b={block}: err={e:.2e}")
        assert x <= 0, f"fp32 output error {e}"
