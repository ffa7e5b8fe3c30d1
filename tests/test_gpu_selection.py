"""GPU parity of the mask-query selection (MaskAhead / Q-MaskAhead abstract):
contributions against the fp64 oracle, the top-k selection exact on the GPU's
own contributions (integer work: masks, unit lists and counts bit-exact against
a NumPy top-k with ties to the lower entry), the selection valid against the
oracle's ranking up to the contribution tolerance, and attention over the
selection within the attention gate of the oracle's attention over the same
entries."""
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
            assert np.all(err <= 1e-2 * cref + 1e-4 * scale), (b, h, float((err - 1e-2 * cref).max() / scale))
            # unit sums against the oracle's sums of its entry contributions
            uref = np.bincount(ids // SLOT, weights=cref, minlength=nu)
            assert np.all(np.abs(usums.astype(np.float64) - uref) <= 1e-2 * uref + 1e-4 * uref.max()), (b, h)
            sel = np.flatnonzero(np.unpackbits(masks.view(np.uint8), bitorder="little"))
            nz = np.flatnonzero(masks != 0)
            assert np.array_equal(units, nz), (b, h)
            if granularity == 1:
                # the GPU's top-k of its own contributions: bit-exact
                want = select_topk(ids, got, budget)
                assert np.array_equal(sel, want), (b, h, len(sel), len(want))
                # valid against the oracle: nothing left out is clearly better than what was kept
                if 0 < len(sel) < len(ids):
                    kept = cref[np.isin(ids, sel)]
                    left = cref[~np.isin(ids, sel)]
                    assert kept.min() >= left.max() - 2e-2 * scale, (b, h, kept.min(), left.max())
            else:
                # top units of the GPU's own unit sums (ties to the lower unit), all their valid entries
                order = np.lexsort((np.arange(nu), -usums.astype(np.float64)))
                keep = np.sort(order[:min(budget, nu)])
                want = np.sort(ids[np.isin(ids // SLOT, keep)])
                assert np.array_equal(sel, want), (b, h, len(sel), len(want))
                if 0 < len(keep) < nu:
                    kept = uref[keep]
                    left = np.delete(uref, keep)
                    assert kept.min() >= left.max() - 2e-2 * uref.max(), (b, h)
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
