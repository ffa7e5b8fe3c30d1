"""Mask-query selection of cached KV entries (oracle).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Method (MaskAhead / Q-MaskAhead abstract): the current block's mask queries
rank the cached KV entries by their estimated contribution to the attention
output, the block then attends only to the top-ranked entries, and the
quantized variant computes both the ranking and the attention directly from
the low-bit cache.

Readings where the abstract is silent (each listed in the design notes):
  * selection is made per (sequence, kv head): the query heads of a kv head's
    group share its entries, so their evidence is summed;
  * the mask queries are the block positions flagged in a caller-given 32-bit
    mask per sequence (bit t = block token t is still masked);
  * the contribution of cached entry j is the size of its term in the
    attention output, summed over the group's heads and the mask queries:
        c_j = ||v_j|| * sum_{heads h} sum_{mask queries t} p_{h,t}(j),
    where p_{h,t} is the softmax over everything the query attends to (all
    valid cached tokens and the 32 block tokens) and v_j the dequantized value
    row as stored;
  * an entry is a token; entry j of a (sequence, kv head) is numbered
    32 * u + t, u the unit (prefix slots first, then suffix slots) and t the
    position in the slot; only valid tokens take part;
  * the top k = min(budget, number of valid entries) entries are selected,
    ties broken by the lower number;
  * the block always attends to itself; with a selection it attends to the
    selected cached entries only;
  * a coarser variant ranks whole 32-token slots by the sum of their entries'
    contributions and keeps every valid entry of the top slots (ties to the
    lower unit).
"""
from __future__ import annotations

import numpy as np

from .layout import SLOT


def _entries(cache, segment: int, b: int, unit0: int):
    """Entry numbers of the valid tokens of a segment, in storage order."""
    ids = []
    for s, hd in enumerate(cache.seg[segment][b].headers):
        ids.extend(SLOT * (unit0 + s) + t for t in range(hd[0]))
    return np.asarray(ids, np.int64)


def cached_entries(cache, b: int, h: int, use_suffix: bool):
    """(entry numbers, K rows, V rows) of every valid cached token of (b, h), fp64."""
    kp, vp = cache.dequantized(0, b, h)
    ids = [_entries(cache, 0, b, 0)]
    ks, vs = [kp], [vp]
    if use_suffix:
        ksu, vsu = cache.dequantized(1, b, h)
        ids.append(_entries(cache, 1, b, cache.nslots(0, b)))
        ks.append(ksu)
        vs.append(vsu)
    return np.concatenate(ids), np.concatenate(ks), np.concatenate(vs)


def contributions(cache, q: np.ndarray, k_blk: np.ndarray, use_suffix: bool = False,
                  scale: float | None = None, qmask=None):
    """{(b, h): (entry numbers, contributions fp64)} for every sequence and kv head.

    q [B, 32, Hq, D]; k_blk [B, 32, Hkv, D]; qmask: per-sequence 32-bit masks of
    the mask queries (None = all 32 block tokens)."""
    B, L, Hq, D = q.shape
    Hkv = k_blk.shape[2]
    r = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    out = {}
    for b in range(B):
        m = 0xFFFFFFFF if qmask is None else int(qmask[b])
        rows = [t for t in range(L) if (m >> t) & 1]
        for h in range(Hkv):
            ids, kc, vc = cached_entries(cache, b, h, use_suffix)
            keys = np.concatenate([kc, np.asarray(k_blk[b, :, h], np.float64)])
            weight = np.zeros(len(ids))
            for hq in range(h * r, (h + 1) * r):
                qq = np.asarray(q[b, rows, hq], np.float64)
                s = (qq @ keys.T) * scale
                s -= s.max(axis=1, keepdims=True)
                p = np.exp(s)
                p /= p.sum(axis=1, keepdims=True)
                weight += p[:, :len(ids)].sum(axis=0)
            out[(b, h)] = (ids, np.linalg.norm(vc, axis=1) * weight)
    return out


def select_topk(ids: np.ndarray, contrib: np.ndarray, budget: int) -> np.ndarray:
    """The min(budget, n) entry numbers with the largest contributions, ties to
    the lower number; returned in ascending entry order."""
    order = np.lexsort((ids, -np.asarray(contrib, np.float64)))
    k = min(int(budget), len(ids))
    return np.sort(np.asarray(ids)[order[:k]])


def select_topk_units(ids: np.ndarray, contrib: np.ndarray, budget: int) -> np.ndarray:
    """Slot-granular selection: the min(budget, units) units with the largest
    summed contributions (ties to the lower unit); returns the entry numbers
    of all their valid tokens, ascending."""
    ids = np.asarray(ids, np.int64)
    units = ids // SLOT
    uniq = np.unique(units)
    sums = np.array([np.asarray(contrib, np.float64)[units == u].sum() for u in uniq])
    order = np.lexsort((uniq, -sums))
    keep = uniq[order[:min(int(budget), len(uniq))]]
    return np.sort(ids[np.isin(units, keep)])


def block_attention_selected(cache, q: np.ndarray, k_blk: np.ndarray, v_blk: np.ndarray,
                             selected: dict, use_suffix: bool = False,
                             scale: float | None = None) -> np.ndarray:
    """Attention output fp64 [B, L, Hq, D] of the block over itself and the
    selected cached entries; selected[(b, h)] = entry numbers."""
    from .attention import attention_rows
    from .rotation import rotate_f32, unrotate
    B, L, Hq, D = q.shape
    Hkv = k_blk.shape[2]
    r = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    rot = getattr(cache, "v_rot", None)
    if rot is not None:
        v_blk = rotate_f32(v_blk, *rot)
    out = np.empty((B, L, Hq, D))
    for b in range(B):
        for h in range(Hkv):
            ids, kc, vc = cached_entries(cache, b, h, use_suffix)
            keep = np.isin(ids, np.asarray(selected[(b, h)], np.int64))
            keys = np.concatenate([kc[keep], np.asarray(k_blk[b, :, h], np.float64)])
            vals = np.concatenate([vc[keep], np.asarray(v_blk[b, :, h], np.float64)])
            for hq in range(h * r, (h + 1) * r):
                o = attention_rows(q[b, :, hq], keys, vals, scale)
                out[b, :, hq] = o if rot is None else unrotate(o, *rot)
    return out
