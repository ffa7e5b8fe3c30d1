"""GPU parity of the fp16-metadata variant of the integer format (scale and
zero stored in fp16, codes taken against the rounded pair): records, headers
and protected rows bit-exact against the oracle for every bit width, value
group and input dtype, including groups whose rounded zero lies above their
minimum and groups whose scale underflows fp16; attention within the gate."""
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
from gpu_util import announce, attention_error, compare_commit, dev  # noqa: E402


def _bf16(x):
    return torch.from_numpy(x).to(torch.bfloat16).float().numpy()


@pytest.mark.parametrize("D,kb,vb,gv,dtype", [
    (128, 4, 4, 128, "bf16"), (128, 2, 2, 32, "bf16"), (64, 4, 2, 64, "f32"), (128, 2, 4, 64, "f32"),
    (64, 2, 2, 32, "bf16")])
def test_h16_commit_and_attention(D, kb, vb, gv, dtype):
    announce("int_h16", D, kb, vb, gv, dtype)
    B, H, Hq = 3, 2, 8
    g = np.random.default_rng(31 + D + kb + 3 * vb + gv)
    n = 100
    k = g.standard_normal((B, n, H, D)).astype(np.float32)
    v = g.standard_normal((B, n, H, D)).astype(np.float32)
    # a key channel with an offset: fp16 rounding moves its zero by up to
    # half an fp16 ulp of 20 (2^-7), a sizeable part of its scale, so codes
    # near the minimum clamp at 0
    k[0, :32, 0, 5] = np.float32(20.0) + np.float32(0.05) * k[0, :32, 0, 5]
    k[1, 32:64, 1, 7] = np.float32(-20.0) + np.float32(0.05) * k[1, 32:64, 1, 7]
    k[0, :32, 1, 1] = np.float32(0.75)                      # constant channel: scale 0
    v[2, 5, 1, :] = np.float32(3.0) + np.float32(0.02) * v[2, 5, 1, :]
    v[2, 6, 0, :] = np.float32(-0.5)                        # constant token
    if dtype == "bf16":
        k, v = _bf16(k), _bf16(v)
    ntok = [100, 45, 33]
    prot = [np.array([0, 31, 32, 70]), np.array([], np.int64), np.array([5])]
    cache = kvq.KVCache(B, H, D, kb, vb, gv, prefix_tokens=256, suffix_tokens=64, prefix_protected=16,
                        suffix_protected=4, max_q_heads=Hq, kv_format=kvq.KVQ_FMT_INT_H16)
    ora = O.OracleCache(B, H, D, kb, vb, gv, fmt="int_h16")
    cache.commit(dev(k, dtype), dev(v, dtype), ntok=ntok, protected=prot)
    ora.commit(0, k, v, ntok=ntok, prot=prot)
    cache.commit(dev(v[:, :40], dtype), dev(k[:, :40], dtype), ntok=[40, 1, 0])
    ora.commit(0, v[:, :40], k[:, :40], ntok=[40, 1, 0])
    cache.commit(dev(k[:, :50], dtype), dev(v[:, :50], dtype), segment=kvq.KVQ_SUFFIX)
    ora.commit(1, k[:, :50], v[:, :50])
    compare_commit(cache, ora, 0, B)
    compare_commit(cache, ora, 1, B)
    q = g.standard_normal((B, 32, Hq, D)).astype(np.float32)
    kbk = g.standard_normal((B, 32, H, D)).astype(np.float32)
    vbk = g.standard_normal((B, 32, H, D)).astype(np.float32)
    if dtype == "bf16":
        q, kbk, vbk = _bf16(q), _bf16(kbk), _bf16(vbk)
    for use_suffix in (False, True):
        ref = O.block_attention(ora, q, kbk, vbk, use_suffix=use_suffix)
        out = cache.block_attn(dev(q, dtype), dev(kbk, dtype), dev(vbk, dtype), use_suffix=use_suffix,
                               out_dtype=torch.float32)
        e, x = attention_error(out, ref, "f32")
        print(f"D={D} K{kb}V{vb} G{gv} {dtype} suffix={use_suffix}: err={e:.2e}")
        assert x <= 0, e


def test_h16_extreme_groups():
    """Commit parity on groups at the edges of fp16: a scale that underflows to
    zero while the range is not zero, a scale in the fp16 subnormals, large
    offsets (zero rounded by up to 8), values up to 3e4."""
    announce("int_h16 extreme")
    B, H, D = 2, 2, 64
    g = np.random.default_rng(77)
    k = g.standard_normal((B, 64, H, D)).astype(np.float32)
    v = g.standard_normal((B, 64, H, D)).astype(np.float32)
    k[0, :32, 0, 0] = np.float32(1.0) + np.float32(1e-7) * k[0, :32, 0, 0]     # scale -> fp16 0
    k[0, :32, 0, 1] = np.float32(2e-5) * k[0, :32, 0, 1]                       # fp16 subnormal scale
    k[0, :32, 1, 2] = np.float32(3000.0) + k[0, :32, 1, 2]                     # zero moves by up to 1
    k[1, 32:, 0, 3] = np.float32(3e4) * k[1, 32:, 0, 3] / np.abs(k[1, 32:, 0, 3]).max()
    v[0, 3, 0, :] = np.float32(-1000.0) + np.float32(0.5) * v[0, 3, 0, :]
    v[1, 40, 1, :] = np.float32(1e-7) * v[1, 40, 1, :]
    for kb, vb, gv in ((4, 4, 64), (2, 2, 32)):
        cache = kvq.KVCache(B, H, D, kb, vb, gv, prefix_tokens=128, max_q_heads=H, kv_format=kvq.KVQ_FMT_INT_H16)
        ora = O.OracleCache(B, H, D, kb, vb, gv, fmt="int_h16")
        cache.commit(dev(k, "f32"), dev(v, "f32"), ntok=[64, 50])
        ora.commit(0, k, v, ntok=[64, 50])
        compare_commit(cache, ora, 0, B)


def test_h16_workload_shape():
    """The dream7b shape (Hq/Hkv = 28/4, D = 128, K4V4 G128) in the fp16-metadata
    format: the producer mapping of the headline kernel, with split-K."""
    announce("int_h16 workload")
    cfg = W.CONFIGS["dream7b_4bit"]
    w = W.make(cfg, T=300, B=2)
    c = w.cfg
    cache = kvq.KVCache(c.B, c.Hkv, c.D, c.k_bits, c.v_bits, c.v_group, prefix_tokens=int(w.lengths.max()) + 64,
                        prefix_protected=max(len(p) for p in w.prot_prefix) + 8, max_q_heads=c.Hq,
                        kv_format=kvq.KVQ_FMT_INT_H16)
    ora = O.OracleCache(c.B, c.Hkv, c.D, c.k_bits, c.v_bits, c.v_group, fmt="int_h16")
    cache.commit(dev(w.k_prefix, c.dtype), dev(w.v_prefix, c.dtype), ntok=w.lengths, protected=w.prot_prefix)
    ora.commit(0, w.k_prefix, w.v_prefix, ntok=w.lengths, prot=w.prot_prefix)
    compare_commit(cache, ora, 0, c.B)
    ref = O.block_attention(ora, w.q, w.k_blk, w.v_blk)
    for split in (0, 3):
        cache.set_split_slots(split)
        out = cache.block_attn(dev(w.q, c.dtype), dev(w.k_blk, c.dtype), dev(w.v_blk, c.dtype),
                               out_dtype=torch.float32)
        e, x = attention_error(out, ref, "f32")
        print(f"dream7b int_h16 split={split}: err={e:.2e}")
        assert x <= 0, e
    # selection reads integer records with fp32 metadata only: refused before any device work
    with pytest.raises(Exception):
        cache.select(dev(w.q, c.dtype), dev(w.k_blk, c.dtype), 64)
