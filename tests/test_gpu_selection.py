"""GPU parity of the mask-query selection (MaskAhead / Q-MaskAhead abstract):
contributions against the fp64 oracle (within 2e-3 relative: the scores use
the attention kernel's hi + lo key operands), the top-k selection exact on the
GPU's own contributions (integer work: masks, unit lists and counts bit-exact
against a NumPy top-k with ties to the lower entry), the selection equal to the
oracle's exact top-k wherever the k-th and (k+1)-th oracle values are further
apart than twice the measured contribution error (and valid within that error
elsewhere), and attention over the selection within the attention gate of the
oracle's attention over the same entries."""
import dataclasses

import numpy as np
import pytest

import oracle as O
import workloads as W
from oracle.selection import block_attention_selected, contributions, select_topk

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from gpu_util import announce, attention_error, build_case, dev  # noqa: E402

SLOT = 32


def check_selection(cache, ora, w, budget, use_suffix, qmask, granularity=1):
    """Returns {(b, h): selected entry numbers} after checking contributions,
    the GPU top-k and the validity of the selection."""
    c = w.cfg
    ref = contributions(ora, w.q, w.k_blk, use_suffix=use_suffix, qmask=qmask)
    torch.cuda.synchronize()
    selected = {}
    for b in range(c.B):
        nu = ora.nslots(0, b) + (ora.nslots(1, b) if use_suffix else 0)
        for h in range(c.Hkv):
            ids, cref = ref[(b, h)]
            contrib, masks, units, usums = (x.cpu().numpy() for x in cache.selection(b, h, nu))
            # slot positions past the valid tokens carry -1
            valid = np.zeros(nu * SLOT, bool)
            valid[ids] = True
            assert np.all(contrib[~valid] == -1.0), (b, h)
            got = contrib[ids].astype(np.float64)
            scale = max(cref.max(), 1e-30)
            err = np.abs(got - cref)
            assert np.all(err <= 2e-3 * cref + 1e-5 * scale), (b, h, float((err - 2e-3 * cref).max() / scale))
            eabs = float(err.max())
            # unit sums against the oracle's sums of its entry contributions
            uref = np.bincount(ids // SLOT, weights=cref, minlength=nu)
            uerr = np.abs(usums.astype(np.float64) - uref)
            assert np.all(uerr <= 2e-3 * uref + 1e-5 * uref.max()), (b, h)
            ueabs = float(uerr.max())
            sel = np.flatnonzero(np.unpackbits(masks.view(np.uint8), bitorder="little"))
            nz = np.flatnonzero(masks != 0)
            assert np.array_equal(units, nz), (b, h)
            if granularity == 1:
                # the GPU's top-k of its own contributions: bit-exact
                want = select_topk(ids, got, budget)
                assert np.array_equal(sel, want), (b, h, len(sel), len(want))
                # against the oracle's exact top-k: equal where the cut is wider
                # than the contribution error, and otherwise nothing left out
                # beats what was kept by more than that error
                if 0 < len(sel) < len(ids):
                    srt = np.sort(cref)[::-1]
                    k = len(sel)
                    if srt[k - 1] - srt[k] > 2 * eabs:
                        assert np.array_equal(sel, select_topk(ids, cref, budget)), (b, h, "oracle top-k")
                    kept = cref[np.isin(ids, sel)]
                    left = cref[~np.isin(ids, sel)]
                    assert kept.min() >= left.max() - 2 * eabs, (b, h, kept.min(), left.max())
            else:
                # top units of the GPU's own unit sums (ties to the lower unit), all their valid entries
                order = np.lexsort((np.arange(nu), -usums.astype(np.float64)))
                keep = np.sort(order[:min(budget, nu)])
                want = np.sort(ids[np.isin(ids // SLOT, keep)])
                assert np.array_equal(sel, want), (b, h, len(sel), len(want))
                if 0 < len(keep) < nu:
                    srt = np.sort(uref)[::-1]
                    k = len(keep)
                    if srt[k - 1] - srt[k] > 2 * ueabs:
                        ok = np.sort(np.lexsort((np.arange(nu), -uref))[:k])
                        assert np.array_equal(keep, ok), (b, h, "oracle top units")
                    kept = uref[keep]
                    left = np.delete(uref, keep)
                    assert kept.min() >= left.max() - 2 * ueabs, (b, h)
            selected[(b, h)] = sel
    return selected


@pytest.mark.parametrize("name,T,B,budget,use_suffix,qmask,gran", [
    ("tiny", None, None, 40, False, None, 1),
    ("dream7b_4bit", 300, 2, 64, False, [0xFFFF0000, 0x0F0F0F0F], 1),
    ("dream7b_2bit", 300, 2, 0, False, None, 1),
    ("dual_long", 400, 2, 150, True, None, 1),
    ("serve_b32", 384, 6, 10_000, False, None, 1),
    ("dream7b_4bit", 300, 2, 3, False, None, 32),
    ("dual_long", 400, 2, 5, True, [0x0000FFFF, 0xFFFFFFFF], 32),
    ("tiny", None, None, 100, False, None, 32),
])
def test_select_then_attend(name, T, B, budget, use_suffix, qmask, gran):
    announce("selection", name, T, B, budget, use_suffix, gran)
    w, cache, ora = build_case(W.CONFIGS[name], T, B)
    c = w.cfg
    q, kb, vb = dev(w.q, c.dtype), dev(w.k_blk, c.dtype), dev(w.v_blk, c.dtype)
    cache.select(q, kb, budget, use_suffix=use_suffix, query_mask=qmask, granularity=gran)
    selected = check_selection(cache, ora, w, budget, use_suffix, qmask, gran)
    ref = block_attention_selected(ora, w.q, w.k_blk, w.v_blk, selected, use_suffix=use_suffix)
    out = cache.block_attn_selected(q, kb, vb, use_suffix=use_suffix, out_dtype=torch.float32)
    e, x = attention_error(out, ref, "f32")
    n_sel = sum(len(v) for v in selected.values())
    print(f"{name} budget={budget}: {n_sel} entries selected, attention err={e:.2e}")
    assert x <= 0, f"attention over the selection: error {e}"
    # a commit ends the selection
    cache.commit(dev(w.k_blk, c.dtype), dev(w.v_blk, c.dtype))
    with pytest.raises(Exception):
        cache.block_attn_selected(q, kb, vb, use_suffix=use_suffix)


def test_selection_splits_and_rotation():
    """Forced split-K on the selected attention, and a cache with rotated
    values (the contributions use the norms of the stored rotated rows)."""
    announce("selection rotated")
    cfg = dataclasses.replace(W.CONFIGS["dream7b_4bit"], v_bits=2, v_group=128)
    w, cache, ora = build_case(cfg, T=300, B=2, v_rot_block=64)
    c = w.cfg
    q, kb, vb = dev(w.q, c.dtype), dev(w.k_blk, c.dtype), dev(w.v_blk, c.dtype)
    cache.select(q, kb, 100)
    selected = check_selection(cache, ora, w, 100, False, None)
    ref = block_attention_selected(ora, w.q, w.k_blk, w.v_blk, selected)
    for split in (0, 2):
        cache.set_split_slots(split)
        out = cache.block_attn_selected(q, kb, vb, out_dtype=torch.float32)
        e, x = attention_error(out, ref, "f32")
        print(f"rotated, split={split}: err={e:.2e}")
        assert x <= 0, e


@pytest.mark.parametrize("name,T,B,budget,use_suffix,qmask,gran,split,odt", [
    ("dream7b_4bit", 300, 2, 64, False, [0xFFFF0000, 0x0F0F0F0F], 1, 64, "bf16"),   # one split per row
    ("dream7b_4bit", 300, 2, 64, False, None, 1, 2, "bf16"),       # split partials, fp16 combine
    ("dual_long", 400, 2, 150, True, None, 1, 3, "f32"),           # split partials, fp32 combine
    ("serve_b32", 384, 6, 10_000, False, None, 1, 0, "bf16"),
    ("dual_long", 400, 2, 5, True, [0x0000FFFF, 0xFFFFFFFF], 32, 0, "f32"),
    ("tiny", None, None, 40, False, None, 1, 0, "f32"),
])
def test_attend_select(name, T, B, budget, use_suffix, qmask, gran, split, odt):
    """One pass of full attention whose softmax statistics feed the selection:
    the output bit-identical to kvq_block_attn's, the selection checked as
    kvq_select's against the oracle.  A first call with other queries leaves
    statistics that the second must replace."""
    announce("attend+select", name, T, B, budget, use_suffix, gran, split, odt)
    w, cache, ora = build_case(W.CONFIGS[name], T, B)
    c = w.cfg
    q, kb, vb = dev(w.q, c.dtype), dev(w.k_blk, c.dtype), dev(w.v_blk, c.dtype)
    out_dt = torch.float32 if odt == "f32" else torch.bfloat16
    cache.set_split_slots(split)
    cache.attend_select((q.float() * 1.7 - 0.3).to(q.dtype), kb, vb, budget, use_suffix=use_suffix, out_dtype=out_dt)
    out = cache.attend_select(q, kb, vb, budget, use_suffix=use_suffix, query_mask=qmask, granularity=gran,
                              out_dtype=out_dt)
    ref = cache.block_attn(q, kb, vb, use_suffix=use_suffix, out_dtype=out_dt)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16) if odt == "bf16" else out.view(torch.int32),
                       ref.view(torch.int16) if odt == "bf16" else ref.view(torch.int32))
    selected = check_selection(cache, ora, w, budget, use_suffix, qmask, gran)
    oref = block_attention_selected(ora, w.q, w.k_blk, w.v_blk, selected, use_suffix=use_suffix)
    att = cache.block_attn_selected(q, kb, vb, use_suffix=use_suffix, out_dtype=torch.float32)
    e, x = attention_error(att, oref, "f32")
    print(f"{name} split={split} {odt}: {sum(len(v) for v in selected.values())} selected, attention err={e:.2e}")
    assert x <= 0, e


def test_attend_select_rotated():
    """Rotated values: the statistics come from the attention over the rotated
    basis (scores are unaffected) and the norms from the stored rotated rows."""
    announce("attend+select rotated")
    cfg = dataclasses.replace(W.CONFIGS["dream7b_4bit"], v_bits=2, v_group=128)
    w, cache, ora = build_case(cfg, T=300, B=2, v_rot_block=64)
    c = w.cfg
    q, kb, vb = dev(w.q, c.dtype), dev(w.k_blk, c.dtype), dev(w.v_blk, c.dtype)
    out = cache.attend_select(q, kb, vb, 100, out_dtype=torch.float32)
    ref = cache.block_attn(q, kb, vb, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int32), ref.view(torch.int32))
    check_selection(cache, ora, w, 100, False, None)


def test_attend_select_empty_cache_and_zero_budget():
    """An empty cache: the attention covers the block alone, nothing is
    selected, and attention over the (empty) selection equals it.  Then a
    budget of 0 on a filled cache: no unit listed, no token kept."""
    announce("attend+select empty cache, budget 0")
    from bit_kv_cache_kivi_amd import kvq
    B, H, Hq, D = 2, 2, 4, 64
    g = np.random.default_rng(41)
    cache = kvq.KVCache(B, H, D, 4, 4, 64, prefix_tokens=320, prefix_protected=8, max_q_heads=Hq)
    q = dev(g.standard_normal((B, SLOT, Hq, D)), "bf16")
    kb = dev(g.standard_normal((B, SLOT, H, D)), "bf16")
    vb = dev(g.standard_normal((B, SLOT, H, D)), "bf16")
    out = cache.attend_select(q, kb, vb, 5, out_dtype=torch.float32)
    ref = cache.block_attn(q, kb, vb, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    for b in range(B):
        for h in range(H):
            _, _, units, _ = cache.selection(b, h, 0)
            assert units.numel() == 0
    sel = cache.block_attn_selected(q, kb, vb, out_dtype=torch.float32)
    assert torch.allclose(sel, ref, rtol=0, atol=1e-6)
    k = g.standard_normal((B, 200, H, D)).astype(np.float32)
    v = g.standard_normal((B, 200, H, D)).astype(np.float32)
    cache.commit(dev(k, "bf16"), dev(v, "bf16"), ntok=[200, 137])
    out = cache.attend_select(q, kb, vb, 0, out_dtype=torch.float32)
    ref = cache.block_attn(q, kb, vb, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    for b, n in enumerate([200, 137]):
        nu = -(-n // SLOT)
        for h in range(H):
            contrib, masks, units, _ = cache.selection(b, h, nu)
            assert units.numel() == 0 and int((masks != 0).sum()) == 0
            c = contrib.cpu().numpy()
            assert np.all(c[:n] >= 0) and np.all(c[n:] == -1.0)
