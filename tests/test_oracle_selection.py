"""Pins of the selection oracle (oracle/selection.py) to things other than
itself: pure-Python brute force, conservation of softmax mass, additivity over
mask queries, hand-built rankings with ties, and the limits of a selection that
keeps every entry or none."""
import math

import numpy as np
import pytest

import oracle as O
from oracle.selection import block_attention_selected, contributions, select_topk


def _cache(B=2, H=2, D=64, seed=0, ntok=(70, 40), suffix=None, bits=4):
    g = np.random.default_rng(seed)
    n = max(ntok)
    k = g.standard_normal((B, n, H, D)).astype(np.float32)
    v = g.standard_normal((B, n, H, D)).astype(np.float32)
    c = O.OracleCache(B, H, D, bits, bits, 32)
    c.commit(0, k, v, ntok=list(ntok), prot=[np.array([1, 33]), np.array([], np.int64)][:B])
    if suffix:
        ks = g.standard_normal((B, suffix, H, D)).astype(np.float32)
        vs = g.standard_normal((B, suffix, H, D)).astype(np.float32)
        c.commit(1, ks, vs)
    return c, g


def test_entry_numbering_by_hand():
    c, _ = _cache(ntok=(70, 40), suffix=20)
    ids, _, _ = O.selection.cached_entries(c, 0, 0, True)
    # prefix: slots of 32, 32, 6 tokens (units 0..2); suffix: one slot of 20 (unit 3)
    want = list(range(0, 32)) + list(range(32, 64)) + list(range(64, 70)) + list(range(96, 116))
    assert ids.tolist() == want
    ids1, _, _ = O.selection.cached_entries(c, 1, 0, True)
    assert ids1.tolist() == list(range(0, 32)) + list(range(32, 40)) + list(range(64, 84))


def test_contributions_brute_force():
    """Pure-Python softmax per query and head (math.exp, math.fsum)."""
    c, g = _cache(B=1, H=1, D=64, ntok=(45,))
    q = g.standard_normal((1, 32, 2, 64)).astype(np.float32)
    kb = g.standard_normal((1, 32, 1, 64)).astype(np.float32)
    qmask = [0x8000_0011]
    got = contributions(c, q, kb, qmask=qmask, scale=0.11)[(0, 0)]
    ids, kc, vc = O.selection.cached_entries(c, 0, 0, False)
    keys = [list(map(float, r)) for r in kc] + [list(map(float, r)) for r in kb[0, :, 0]]
    want = [0.0] * len(ids)
    for hq in range(2):
        for t in (0, 4, 31):
            qr = list(map(float, q[0, t, hq]))
            s = [0.11 * math.fsum(a * b for a, b in zip(qr, kr)) for kr in keys]
            m = max(s)
            e = [math.exp(x - m) for x in s]
            z = math.fsum(e)
            for j in range(len(ids)):
                want[j] += e[j] / z
    norms = [math.sqrt(math.fsum(float(x) ** 2 for x in row)) for row in vc]
    want = [w * n for w, n in zip(want, norms)]
    assert np.array_equal(got[0], ids)
    np.testing.assert_allclose(got[1], want, rtol=1e-12, atol=1e-15)


def test_mass_conservation():
    """Block keys far below every cached score: the softmax mass of each query
    sits on the cache, so contribution / ||v|| sums to heads x mask queries."""
    c, g = _cache(B=2, H=2, D=64, suffix=40)
    q = np.abs(g.standard_normal((2, 32, 6, 64))).astype(np.float32)
    kb = np.full((2, 32, 2, 64), -50.0, np.float32)
    qmask = [0xFFFFFFFF, 0x0000F0F0]
    res = contributions(c, q, kb, use_suffix=True, qmask=qmask)
    for b in range(2):
        nq = bin(qmask[b]).count("1")
        for h in range(2):
            ids, _, vc = O.selection.cached_entries(c, b, h, True)
            cj = res[(b, h)][1]
            w = cj / np.linalg.norm(vc, axis=1)
            assert abs(w.sum() - 3 * nq) < 1e-9 * 3 * nq


def test_additive_over_mask_queries():
    c, g = _cache(suffix=33)
    q = g.standard_normal((2, 32, 4, 64)).astype(np.float32)
    kb = g.standard_normal((2, 32, 2, 64)).astype(np.float32)
    a = contributions(c, q, kb, True, qmask=[0x0000FFFF, 0x1])
    b_ = contributions(c, q, kb, True, qmask=[0xFFFF0000, 0x6])
    ab = contributions(c, q, kb, True, qmask=[0xFFFFFFFF, 0x7])
    for key in ab:
        np.testing.assert_allclose(a[key][1] + b_[key][1], ab[key][1], rtol=1e-12, atol=1e-15)


def test_topk_ties_and_limits():
    ids = np.array([10, 11, 12, 13, 14, 40])
    cj = np.array([3.0, 1.0, 3.0, 2.0, 3.0, 0.0])
    assert select_topk(ids, cj, 2).tolist() == [10, 12]
    assert select_topk(ids, cj, 4).tolist() == [10, 12, 13, 14]
    assert select_topk(ids, cj, 99).tolist() == ids.tolist()
    assert select_topk(ids, cj, 0).tolist() == []
    # a dominant key is the one kept at budget 1
    c, g = _cache(B=1, H=1, ntok=(64,))
    ids, kc, _ = O.selection.cached_entries(c, 0, 0, False)
    q = np.zeros((1, 32, 1, 64), np.float32)
    q[0, :, 0] = (kc[37] / np.linalg.norm(kc[37]) * 40).astype(np.float32)
    kb = np.zeros((1, 32, 1, 64), np.float32)
    res = contributions(c, q, kb)[(0, 0)]
    assert select_topk(*res, 1).tolist() == [37]


@pytest.mark.parametrize("rot", [False, True])
def test_selected_attention_limits(rot):
    c, g = _cache(suffix=30)
    if rot:
        from workloads import krpbh_params
        perm, mix = krpbh_params(64, 16)
        c2 = O.OracleCache(2, 2, 64, 4, 4, 32, v_rot=(perm, mix, 16))
        g2 = np.random.default_rng(5)
        kk = g2.standard_normal((2, 50, 2, 64)).astype(np.float32)
        vv = g2.standard_normal((2, 50, 2, 64)).astype(np.float32)
        c2.commit(0, kk, vv)
        c2.commit(1, kk[:, :30], vv[:, :30])
        c = c2
    q = g.standard_normal((2, 32, 4, 64)).astype(np.float32)
    kb = g.standard_normal((2, 32, 2, 64)).astype(np.float32)
    vb = g.standard_normal((2, 32, 2, 64)).astype(np.float32)
    every = {(b, h): O.selection.cached_entries(c, b, h, True)[0] for b in range(2) for h in range(2)}
    full = O.block_attention(c, q, kb, vb, use_suffix=True)
    np.testing.assert_allclose(block_attention_selected(c, q, kb, vb, every, True), full, rtol=0, atol=1e-12)
    none = {key: np.zeros(0, np.int64) for key in every}
    got = block_attention_selected(c, q, kb, vb, none, True)
    for b in range(2):
        for hq in range(4):
            vbb = vb[b, :, hq // 2]
            if rot:
                vbb = O.unrotate(O.rotate_f32(vbb, *c.v_rot), *c.v_rot)
            want = O.attention_rows(q[b, :, hq], kb[b, :, hq // 2], vbb, 1 / 8)
            np.testing.assert_allclose(got[b, :, hq], want, rtol=0, atol=1e-6 if rot else 1e-12)


def test_unit_granular_selection_by_hand():
    """Units ranked by summed contributions; ties to the lower unit; every
    valid token of a kept unit is kept."""
    from oracle.selection import select_topk_units
    ids = np.array([0, 1, 2, 32, 33, 64, 96, 97, 98, 99])
    cj = np.array([1.0, 1.0, 1.0, 2.0, 1.0, 3.0, 0.5, 0.5, 0.5, 1.5])
    # unit sums: u0 = 3, u1 = 3, u2 = 3, u3 = 3 -> all tie: lower units first
    assert select_topk_units(ids, cj, 1).tolist() == [0, 1, 2]
    assert select_topk_units(ids, cj, 2).tolist() == [0, 1, 2, 32, 33]
    cj2 = cj.copy()
    cj2[6] = 5.0                                   # u3 = 7.5 now leads
    assert select_topk_units(ids, cj2, 1).tolist() == [96, 97, 98, 99]
    assert select_topk_units(ids, cj2, 0).tolist() == []
    assert select_topk_units(ids, cj2, 9).tolist() == ids.tolist()
