"""GPU parity of the MX FP4 cache format (SoloQ abstract and summary page: a
hardware-native 4-bit floating-point format with per-block scales; here OCP
MX FP4): records, headers and protected rows bit-exact against the oracle,
attention within the gate."""
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


@pytest.mark.parametrize("D,dtype", [(128, "bf16"), (64, "f32"), (128, "f32")])
def test_mxfp4_commit_and_attention(D, dtype):
    announce("mxfp4", D, dtype)
    B, H, Hq = 3, 2, 8
    g = np.random.default_rng(21)
    n = 100
    # lognormal channel scales with bf16 inputs (queries exact in fp16); fp32
    # queries are rounded to the fp16 operand, so their keys stay unit-scale
    chan = np.exp(g.standard_normal((1, 1, H, D))) if dtype == "bf16" else np.ones((1, 1, H, D))
    k = (g.standard_normal((B, n, H, D)) * chan).astype(np.float32)
    v = g.standard_normal((B, n, H, D)).astype(np.float32)
    # edge groups: signed zeros next to nonzero values, an all-zero channel,
    # values on the grid, a huge and a tiny channel
    k[0, :32, 0, 0] = np.where(np.arange(32) % 3 == 0, -0.0, 1.5).astype(np.float32)
    k[0, :32, 0, 1] = 0.0
    k[0, :32, 1, 2] = np.tile(np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0], np.float32), 4)
    k[1, :32, 0, 3] *= np.float32(30.0)
    k[1, :32, 0, 4] *= np.float32(1e-4)
    v[2, 5, 1, :32] = -0.0
    v[2, 6, 1, :] = np.float32(0.75)
    if dtype == "bf16":
        k = torch.from_numpy(k).to(torch.bfloat16).float().numpy()
        v = torch.from_numpy(v).to(torch.bfloat16).float().numpy()
    ntok = [100, 45, 33]
    prot = [np.array([0, 31, 32, 70]), np.array([], np.int64), np.array([5])]
    cache = kvq.KVCache(B, H, D, 4, 4, 32, prefix_tokens=256, suffix_tokens=64, prefix_protected=16,
                        suffix_protected=4, max_q_heads=Hq, kv_format=kvq.KVQ_FMT_MXFP4)
    ora = O.OracleCache(B, H, D, 4, 4, 32, fmt="mxfp4")
    cache.commit(dev(k, dtype), dev(v, dtype), ntok=ntok, protected=prot)
    ora.commit(0, k, v, ntok=ntok, prot=prot)
    cache.commit(dev(v[:, :40], dtype), dev(k[:, :40], dtype), ntok=[40, 1, 0])
    ora.commit(0, v[:, :40], k[:, :40], ntok=[40, 1, 0])
    cache.commit(dev(k[:, :50], dtype), dev(v[:, :50], dtype), segment=kvq.KVQ_SUFFIX)
    ora.commit(1, k[:, :50], v[:, :50])
    compare_commit(cache, ora, 0, B)
    compare_commit(cache, ora, 1, B)
    q = g.standard_normal((B, 32, Hq, D)).astype(np.float32)
    kb = g.standard_normal((B, 32, H, D)).astype(np.float32)
    vb = g.standard_normal((B, 32, H, D)).astype(np.float32)
    if dtype == "bf16":
        q, kb, vb = (torch.from_numpy(x).to(torch.bfloat16).float().numpy() for x in (q, kb, vb))
    for use_suffix in (False, True):
        ref = O.block_attention(ora, q, kb, vb, use_suffix=use_suffix)
        out = cache.block_attn(dev(q, dtype), dev(kb, dtype), dev(vb, dtype), use_suffix=use_suffix,
                               out_dtype=torch.float32)
        e, x = attention_error(out, ref, "f32")
        print(f"D={D} {dtype} suffix={use_suffix}: err={e:.2e}")
        assert x <= 0, e


def test_mxfp4_workload_shape():
    """The dream7b shape (Hq/Hkv = 28/4, D = 128) with 32-channel value groups:
    the producer mapping of the headline kernel, with split-K."""
    announce("mxfp4 workload")
    cfg = dataclasses.replace(W.CONFIGS["dream7b_4bit"], v_group=32)
    w = W.make(cfg, T=300, B=2)
    c = w.cfg
    cache = kvq.KVCache(c.B, c.Hkv, c.D, 4, 4, 32, prefix_tokens=int(w.lengths.max()) + 64,
                        prefix_protected=max(len(p) for p in w.prot_prefix) + 8, max_q_heads=c.Hq,
                        kv_format=kvq.KVQ_FMT_MXFP4)
    ora = O.OracleCache(c.B, c.Hkv, c.D, 4, 4, 32, fmt="mxfp4")
    cache.commit(dev(w.k_prefix, c.dtype), dev(w.v_prefix, c.dtype), ntok=w.lengths, protected=w.prot_prefix)
    ora.commit(0, w.k_prefix, w.v_prefix, ntok=w.lengths, prot=w.prot_prefix)
    compare_commit(cache, ora, 0, c.B)
    ref = O.block_attention(ora, w.q, w.k_blk, w.v_blk)
    for split in (0, 3):
        cache.set_split_slots(split)
        out = cache.block_attn(dev(w.q, c.dtype), dev(w.k_blk, c.dtype), dev(w.v_blk, c.dtype), out_dtype=torch.float32)
        e, x = attention_error(out, ref, "f32")
        print(f"dream7b mxfp4 split={split}: err={e:.2e}")
        assert x <= 0, e
