"""GPU parity of kvq_attend_commit (attention of a block over the cache as it
is, then the commit of that block, in one call): over several steps, every output within the attention gate of the
oracle's attention before the commit, bit-identical to the output of separate
kvq_block_attn + kvq_commit calls on a twin cache, and records, headers and
protected rows bit-exact against the oracle afterwards."""
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


@pytest.mark.parametrize("name,T,B,nsteps,v_rot,odt", [
    ("tiny", None, None, 3, 0, "f32"), ("dream7b_4bit", 300, 2, 4, 0, "f32"), ("dual_long", 400, 2, 3, 0, "f32"),
    ("serve_b32", 200, 6, 2, 0, "f32"), ("dream7b_4bit", 300, 2, 2, 64, "f32"), ("dream7b_4bit", 300, 2, 2, 64, "bf16"),
    ("dream7b_4bit", 300, 2, 2, 0, "bf16")])
def test_attend_commit_steps(name, T, B, nsteps, v_rot, odt):
    """With rotated values and a bf16 output, the merge also rotates the output
    back and the fused commit quantizes the rotated copy of the block."""
    announce("attend_commit", name, T, B, nsteps, v_rot, odt)
    out_dt = torch.float32 if odt == "f32" else torch.bfloat16
    w, cache, ora = build_case(W.CONFIGS[name], T, B, extra_slots=nsteps + 1, v_rot_block=v_rot)
    _, twin, _ = build_case(W.CONFIGS[name], T, B, extra_slots=nsteps + 1, v_rot_block=v_rot)
    c = w.cfg
    use_suffix = bool(c.suffix)
    g = np.random.default_rng(5)
    for s in range(nsteps):
        kb, vb, prot = W.step_block(c, s)
        q = g.standard_normal(w.q.shape).astype(np.float32)
        if c.dtype == "bf16":
            q = torch.from_numpy(q).to(torch.bfloat16).float().numpy()
        ntok = [32] * c.B if s % 2 == 0 else [32 - (b % 3) * 7 for b in range(c.B)]   # ragged commits too
        prot_s = [p[p < n] for p, n in zip(prot, ntok)]
        ref = O.block_attention(ora, q, kb, vb, use_suffix=use_suffix)
        dq, dk, dv = dev(q, c.dtype), dev(kb, c.dtype), dev(vb, c.dtype)
        out = cache.attend_commit(dq, dk, dv, ntok=ntok, protected=prot_s, use_suffix=use_suffix,
                                  out_dtype=out_dt)
        out2 = twin.block_attn(dq, dk, dv, use_suffix=use_suffix, out_dtype=out_dt)
        twin.commit(dk, dv, ntok=ntok, protected=prot_s)
        ora.commit(0, kb, vb, ntok=ntok, prot=prot_s)
        e, x = attention_error(out, ref, odt)
        print(f"{name} step {s}: err={e:.2e}")
        assert x <= 0, (s, e)
        assert torch.equal(out, out2), f"step {s}: attend_commit output differs from block_attn"
    torch.cuda.synchronize()
    compare_commit(cache, ora, 0, c.B)
    compare_commit(twin, ora, 0, c.B)
    for b in range(c.B):
        assert torch.equal(cache.records(0, b), twin.records(0, b))


def test_attend_commit_errors_leave_cache_unchanged():
    """An attention argument error after the commit was checked: nothing runs,
    the cache is unchanged, and a later good call still works."""
    announce("attend_commit errors")
    w, cache, ora = build_case(W.CONFIGS["tiny"], extra_slots=2)
    c = w.cfg
    kb, vb, prot = W.step_block(c, 0)
    before = cache.segment_info(0)
    q = dev(w.q, c.dtype)
    bad_q = q[:, :, :c.Hkv + 1].contiguous() if c.Hq > c.Hkv else q[:, :, :1].contiguous()
    with pytest.raises(Exception):
        cache.attend_commit(bad_q, dev(kb, c.dtype), dev(vb, c.dtype), protected=prot)
    assert [list(x) for x in cache.segment_info(0)] == [list(x) for x in before]
    ref = O.block_attention(ora, w.q, kb, vb)
    out = cache.attend_commit(q, dev(kb, c.dtype), dev(vb, c.dtype), protected=prot, out_dtype=torch.float32)
    ora.commit(0, kb, vb, prot=prot)
    e, x = attention_error(out, ref, "f32")
    assert x <= 0, e
    compare_commit(cache, ora, 0, c.B)


@pytest.mark.parametrize("fmt", ["int", "int_h16", "mxfp4"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_attend_commit_fused_edges(fmt, dtype):
    """The one-launch attend-and-commit from an empty cache (the first slot has
    no previous header), with a sequence that commits nothing, partial blocks,
    attention-sink protection and caller rows at both ends of the block, in
    every record format; outputs equal separate calls on a twin cache, records
    equal the oracle's."""
    announce("attend_commit fused edges", fmt, dtype)
    B, H, D, r = 3, 2, 64, 3
    kb_, vb_, gv = (4, 4, 32) if fmt == "mxfp4" else (4, 2, 32)
    kvf = {"int": kvq.KVQ_FMT_INT, "int_h16": kvq.KVQ_FMT_INT_H16, "mxfp4": kvq.KVQ_FMT_MXFP4}[fmt]
    mk = lambda: kvq.KVCache(B, H, D, kb_, vb_, gv, prefix_tokens=6 * 32, prefix_protected=64,   # noqa: E731
                             max_q_heads=H * r, protect_sink=True, kv_format=kvf)
    cache, twin = mk(), mk()
    ora = O.OracleCache(B, H, D, kb_, vb_, gv, protect_sink=True, fmt=fmt)
    g = np.random.default_rng(11)
    counts = [[32, 0, 17], [5, 32, 32], [32, 1, 0], [32, 32, 32]]
    for s, ntok in enumerate(counts):
        q = g.standard_normal((B, 32, H * r, D)).astype(np.float32)
        k = g.standard_normal((B, 32, H, D)).astype(np.float32)
        v = g.standard_normal((B, 32, H, D)).astype(np.float32)
        if dtype == "bf16":
            q, k, v = O.to_bf16_f32(q), O.to_bf16_f32(k), O.to_bf16_f32(v)
        prot = [np.array([p for p in (0, 2, 31) if p < n], np.int64) if (b + s) % 2 else np.array([], np.int64)
                for b, n in enumerate(ntok)]
        ref = O.block_attention(ora, q, k, v)
        dq, dk, dv = dev(q, dtype), dev(k, dtype), dev(v, dtype)
        out = cache.attend_commit(dq, dk, dv, ntok=ntok, protected=prot, out_dtype=torch.float32)
        out2 = twin.block_attn(dq, dk, dv, out_dtype=torch.float32)
        twin.commit(dk, dv, ntok=ntok, protected=prot)
        ora.commit(0, k, v, ntok=ntok, prot=prot)
        e, x = attention_error(out, ref, "f32")
        assert x <= 0, (s, e)
        assert torch.equal(out, out2), f"step {s}: one-launch output differs from block_attn"
        torch.cuda.synchronize()
        compare_commit(cache, ora, 0, B)
    compare_commit(twin, ora, 0, B)
