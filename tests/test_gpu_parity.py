"""GPU-vs-oracle parity through the C ABI (needs an MI355X).

Commit: every byte of every slot record (codes, scales, zeros), slot header and
protected bf16 row must equal the oracle's.  Attention: max |gpu - oracle| <= 2e-3
with fp32 output; with bf16 output the bound adds half a bf16 ulp of the exact
value (the rounding of the output itself).
"""
import math

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


SMALL = [("tiny", None, None), ("llada8b", 512, None), ("dream7b_2bit", 384, 2), ("dream7b_4bit", 384, 2),
         ("serve_b32", 384, 6), ("dual_long", 640, 2)]


@pytest.mark.parametrize("name,T,B", SMALL)
def test_commit_and_attention_small(name, T, B):
    announce("small", name, T, B)
    cfg = W.CONFIGS[name]
    w, cache, ora = build_case(cfg, T, B)
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
    print(f"{name}: max|o|={np.abs(ref).max():.3f} fp32-out err={e32:.2e} bf16-out err={e16:.2e}")
    assert x32 <= 0, f"fp32 output error {e32}"
    assert x16 <= 0, f"bf16 output error {e16} exceeds 2e-3 + ulp/2"


def test_adversarial_groups():
    """Constant groups, exact rounding ties, signed zeros, subnormal ranges,
    partial slots, fully protected slots, fp32 input."""
    announce("adversarial")
    B, H, D = 3, 2, 64
    g = np.random.default_rng(123)
    n = 96
    k = g.standard_normal((B, n, H, D)).astype(np.float32)
    v = g.standard_normal((B, n, H, D)).astype(np.float32)
    k[0, :32, 0, 0] = 1.25                                   # constant K channel
    k[0, :32, 0, 1] = np.tile(np.array([0, 0.5, 1, 1.5, 2, 2.5, 3, 3], np.float32), 4)   # 2-bit ties
    k[0, :32, 0, 2] = np.tile(np.arange(16, dtype=np.float32) * 0.5 + 0.25, 2)
    k[0, :32, 1, 3] = np.where(np.arange(32) % 2, 0.0, -0.0).astype(np.float32)  # +-0
    k[1, :32, 0, 4] = (np.arange(32) % 4).astype(np.float32) * np.float32(2.0 ** -149)  # subnormal
    k[1, :32, 0, 5] = np.float32(3e38) * (np.arange(32) % 2) - np.float32(1e38)           # huge range
    v[0, 0, 0, :] = 0.75                                     # constant V group
    v[0, 1, 0, :] = np.tile(np.array([0, 1, 2, 3, 1.5, 0.5, 2.5, 3], np.float32), 8)     # V ties
    v[2, 5, 1, :32] = -0.0
    v[2, 5, 1, 32:] = np.float32(2.0 ** -140) * (np.arange(32) % 3)
    ntok = [96, 70, 33]
    prot = [np.arange(0, 32), np.array([0, 31, 32, 69]), np.array([], np.int64)]
    for kb, vb, gv in [(2, 2, 32), (4, 4, 64), (2, 4, 64), (4, 2, 32)]:
        announce("adversarial bits", kb, vb, gv)
        cache = kvq.KVCache(B, H, D, kb, vb, gv, prefix_tokens=256, prefix_protected=64, max_q_heads=H)
        ora = O.OracleCache(B, H, D, kb, vb, gv)
        cache.commit(dev(k, "f32"), dev(v, "f32"), ntok=ntok, protected=prot)
        ora.commit(0, k, v, ntok=ntok, prot=prot)
        # a second commit appends fresh slots after partial ones
        cache.commit(dev(v[:, :40], "f32"), dev(k[:, :40], "f32"), ntok=[40, 1, 0])
        ora.commit(0, v[:, :40], k[:, :40], ntok=[40, 1, 0])
        compare_commit(cache, ora, 0, B)


@pytest.mark.parametrize("kb,vb,gv", [(4, 4, 32), (2, 2, 32), (4, 2, 128), (2, 4, 128)])
def test_attention_value_groups_d128(kb, vb, gv):
    """Head dim 128 with every value-group size and bit width: the producer
    thread mapping differs between 32-channel groups and wider ones."""
    announce("value groups d128", kb, vb, gv)
    import dataclasses
    cfg = dataclasses.replace(W.CONFIGS["dream7b_4bit"], k_bits=kb, v_bits=vb, v_group=gv)
    w, cache, ora = build_case(cfg, T=300, B=2)
    c = w.cfg
    compare_commit(cache, ora, 0, c.B)
    ref = O.block_attention(ora, w.q, w.k_blk, w.v_blk)
    out = cache.block_attn(dev(w.q, c.dtype), dev(w.k_blk, c.dtype), dev(w.v_blk, c.dtype), out_dtype=torch.float32)
    e, x = attention_error(out, ref, "f32")
    print(f"kb={kb} vb={vb} gv={gv}: fp32-out err={e:.2e}")
    assert x <= 0, f"fp32 output error {e}"


def test_reset_suffix_and_dual():
    announce("suffix reset")
    cfg = W.CONFIGS["dual_long"]
    w, cache, ora = build_case(cfg, T=256, B=2)
    c = w.cfg
    # replace the suffix with a shorter one
    ks, vs = w.k_suffix[:, :100], w.v_suffix[:, :100]
    cache.commit(dev(ks, c.dtype), dev(vs, c.dtype), segment=kvq.KVQ_SUFFIX, reset=True,
                 protected=[np.array([3, 99]), np.array([])])
    ora.commit(1, ks, vs, prot=[np.array([3, 99]), np.array([])], reset=True)
    compare_commit(cache, ora, 1, c.B)
    ref = O.block_attention(ora, w.q, w.k_blk, w.v_blk, use_suffix=True)
    out = cache.block_attn(dev(w.q, c.dtype), dev(w.k_blk, c.dtype), dev(w.v_blk, c.dtype), use_suffix=True,
                           out_dtype=torch.float32)
    e, x = attention_error(out, ref)
    assert x <= 0, e
    ref0 = O.block_attention(ora, w.q, w.k_blk, w.v_blk, use_suffix=False)
    out0 = cache.block_attn(dev(w.q, c.dtype), dev(w.k_blk, c.dtype), dev(w.v_blk, c.dtype), use_suffix=False,
                            out_dtype=torch.float32)
    e0, x0 = attention_error(out0, ref0)
    assert x0 <= 0, e0


def test_split_invariance_and_determinism():
    """Any split of the cache into chunks gives a result within the oracle gate.

    Splits do not agree bit for bit: P is rounded to fp16 relative to each
    chunk's running maximum, so a key's rounding error (<= 2^-11 of its weight)
    differs between splits; the spread stays far below the gate."""
    announce("split invariance")
    cfg = W.CONFIGS["dream7b_4bit"]
    w, cache, ora = build_case(cfg, T=512, B=2)
    c = w.cfg
    q, kb, vb = dev(w.q, c.dtype), dev(w.k_blk, c.dtype), dev(w.v_blk, c.dtype)
    ref = O.block_attention(ora, w.q, w.k_blk, w.v_blk)
    outs = []
    for s in (1, 2, 3, 5, 17, 1000):
        cache.set_split_slots(s)
        out = cache.block_attn(q, kb, vb, out_dtype=torch.float32)
        e, x = attention_error(out, ref)
        assert x <= 0, (s, e)
        outs.append(out.cpu().numpy())
    spread = max(np.abs(o - outs[0]).max() for o in outs[1:])
    print(f"split spread {spread:.2e}")
    assert spread < 1e-3
    cache.set_split_slots(3)
    a = cache.block_attn(q, kb, vb, out_dtype=torch.float32).cpu().numpy()
    b = cache.block_attn(q, kb, vb, out_dtype=torch.float32).cpu().numpy()
    assert np.array_equal(a, b)


def test_empty_cache_attends_to_block_only():
    announce("empty cache")
    B, H, r, D = 2, 2, 3, 128
    g = np.random.default_rng(5)
    q = g.standard_normal((B, 32, H * r, D)).astype(np.float32)
    kb = g.standard_normal((B, 32, H, D)).astype(np.float32)
    vb = g.standard_normal((B, 32, H, D)).astype(np.float32)
    cache = kvq.KVCache(B, H, D, 4, 4, 128, prefix_tokens=64, max_q_heads=H * r)
    ora = O.OracleCache(B, H, D, 4, 4, 128)
    ref = O.block_attention(ora, q, kb, vb)
    out = cache.block_attn(dev(q, "f32"), dev(kb, "f32"), dev(vb, "f32"), out_dtype=torch.float32)
    e, x = attention_error(out, ref)
    assert x <= 0, e


def test_per_step_commit_then_attend():
    """Decode loop shape: commit the previous 32-token block, then attend."""
    announce("per-step loop")
    cfg = W.CONFIGS["dream7b_2bit"]
    w, cache, ora = build_case(cfg, T=256, B=2, extra_slots=4)
    c = w.cfg
    for step in range(3):
        k, v, prot = W.step_block(c, step)
        cache.commit(dev(k, c.dtype), dev(v, c.dtype), protected=prot)
        ora.commit(0, k, v, prot=prot)
        ref = O.block_attention(ora, w.q, w.k_blk, w.v_blk)
        out = cache.block_attn(dev(w.q, c.dtype), dev(w.k_blk, c.dtype), dev(w.v_blk, c.dtype),
                               out_dtype=torch.float32)
        e, x = attention_error(out, ref)
        assert x <= 0, (step, e)
    compare_commit(cache, ora, 0, c.B)


def test_many_pairs_grid_and_ragged_splits():
    """More (sequence, kv head) workgroups than the launch-argument list holds
    (the three-dimensional grid, whose idle splits exit at once), and a ragged
    batch on the listed grid; both against the oracle."""
    announce("grid shapes")
    import dataclasses
    g = np.random.default_rng(11)
    D, H, r = 64, 4, 2
    for B, lengths in [(140, None), (6, [40, 300, 700, 31, 256, 1]), (3, [0, 64, 96])]:
        T = 96 if lengths is None else max(max(lengths), 1)
        ntok = np.full(B, T) if lengths is None else np.array(lengths)
        k = g.standard_normal((B, T, H, D)).astype(np.float32)
        v = g.standard_normal((B, T, H, D)).astype(np.float32)
        q = g.standard_normal((B, 32, H * r, D)).astype(np.float32)
        kb = g.standard_normal((B, 32, H, D)).astype(np.float32)
        vb = g.standard_normal((B, 32, H, D)).astype(np.float32)
        cache = kvq.KVCache(B, H, D, 4, 4, 64, prefix_tokens=T + 32, max_q_heads=H * r)
        ora = O.OracleCache(B, H, D, 4, 4, 64)
        cache.commit(dev(k, "f32"), dev(v, "f32"), ntok=ntok)
        ora.commit(0, k, v, ntok=ntok)
        ref = O.block_attention(ora, q, kb, vb)
        for split in (0, 2):
            cache.set_split_slots(split)
            out = cache.block_attn(dev(q, "f32"), dev(kb, "f32"), dev(vb, "f32"), out_dtype=torch.float32)
            e, x = attention_error(out, ref)
            print(f"B={B} split={split}: err={e:.2e}")
            assert x <= 0, (B, split, e)
        cache.close()


def test_sink_protection():
    """protect_sink: the first token of each sequence's prefix is protected in
    addition to the caller's rows; records bit-exact, attention within the gate."""
    announce("sink protection")
    B, H, D = 3, 2, 128
    g = np.random.default_rng(11)
    k = g.standard_normal((B, 70, H, D)).astype(np.float32)
    v = g.standard_normal((B, 70, H, D)).astype(np.float32)
    cache = kvq.KVCache(B, H, D, 2, 2, 64, prefix_tokens=160, suffix_tokens=32, prefix_protected=8,
                        suffix_protected=4, max_q_heads=4, protect_sink=True)
    ora = O.OracleCache(B, H, D, 2, 2, 64, protect_sink=True)
    prot = [np.array([5, 40]), np.array([0, 3]), np.array([], np.int64)]
    cache.commit(dev(k, "f32"), dev(v, "f32"), ntok=[70, 33, 0], protected=prot)
    ora.commit(0, k, v, ntok=[70, 33, 0], prot=prot)
    cache.commit(dev(k[:, :10], "f32"), dev(v[:, :10], "f32"), ntok=[10, 10, 10])
    ora.commit(0, k[:, :10], v[:, :10], ntok=[10, 10, 10])
    cache.commit(dev(k[:, :20], "f32"), dev(v[:, :20], "f32"), segment=kvq.KVQ_SUFFIX)
    ora.commit(1, k[:, :20], v[:, :20])
    compare_commit(cache, ora, 0, B)
    compare_commit(cache, ora, 1, B)
    assert [cache.protected_rows(0, b)[0].cpu().tolist() for b in range(B)] == [[0, 5, 40], [0, 3], [0]]
    q = g.standard_normal((B, 32, 4, D)).astype(np.float32)
    kb = g.standard_normal((B, 32, H, D)).astype(np.float32)
    vb = g.standard_normal((B, 32, H, D)).astype(np.float32)
    ref = O.block_attention(ora, q, kb, vb, use_suffix=True)
    out = cache.block_attn(dev(q, "f32"), dev(kb, "f32"), dev(vb, "f32"), use_suffix=True, out_dtype=torch.float32)
    e, x = attention_error(out, ref, "f32")
    assert x <= 0, e


@pytest.mark.parametrize("vscale_log2", [0, 13, -10])
def test_bf16_output_split_partials_at_any_magnitude(vscale_log2):
    """With a 16-bit output the splits hand their normalised O to the combine
    in fp16, each row scaled by a power of two: values scaled by 2^13 (near
    the top of the fp16 operand range the inputs must keep to) and by 2^-10
    come out with the same relative error as unit values, over several split
    counts.  (Far smaller values keep the absolute bound only: the value
    operand itself is fp16, whose normal range ends at 2^-14.)"""
    announce("bf16 split partials, values x 2^", vscale_log2)
    g = np.random.default_rng(40 + vscale_log2)
    B, H, r, D, T = 2, 2, 4, 128, 700
    sc = np.float32(2.0 ** vscale_log2)
    k = g.standard_normal((B, T, H, D)).astype(np.float32)
    v = (g.standard_normal((B, T, H, D)) * sc).astype(np.float32)
    q = g.standard_normal((B, 32, H * r, D)).astype(np.float32)
    kb = g.standard_normal((B, 32, H, D)).astype(np.float32)
    vb = (g.standard_normal((B, 32, H, D)) * sc).astype(np.float32)
    # one query row with a peaked softmax: its O is one value row, the
    # largest |O| a split can hand over
    q[0, 5, 0] = 12.0 * k[0, 100, 0]
    k, v, q, kb, vb = (O.to_bf16_f32(x) for x in (k, v, q, kb, vb))
    cache = kvq.KVCache(B, H, D, 4, 4, 128, prefix_tokens=T + 32, max_q_heads=H * r)
    ora = O.OracleCache(B, H, D, 4, 4, 128)
    cache.commit(dev(k, "bf16"), dev(v, "bf16"))
    ora.commit(0, k, v)
    ref = O.block_attention(ora, q, kb, vb) / float(sc)
    for split in (1, 2, 3, 7, 0):
        cache.set_split_slots(split)
        out = cache.block_attn(dev(q, "bf16"), dev(kb, "bf16"), dev(vb, "bf16"), out_dtype=torch.bfloat16)
        assert torch.isfinite(out).all()
        e, x = attention_error(out.float() / float(sc), ref, "bf16")
        print(f"x2^{vscale_log2} split={split}: err/scale={e:.2e}")
        assert x <= 0, (split, e)
