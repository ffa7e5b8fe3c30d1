"""Block attention over the dequantized cache, in fp64 (oracle).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Method (pages): the block being denoised stays in full precision and attends to
the cache at every denoising step (MaskAhead abstract; SoloQ summary page,
block-diffusion paragraph); attention is bidirectional (SoloQ summary page,
opening paragraph), so every query token of the block sees every block token
and every cached token; the cache is the prefix, or prefix plus suffix for the
dual cache (Tai et al., abstract).  Attention over low-bit KV uses the
dequantized values (Q-MaskAhead: attention directly from low-bit KV).

Readings: scores are q.k times a softmax scale (1/sqrt(D) unless given); no
causal or positional mask (keys arrive already position-encoded); grouped-query
heads map query head hq to kv head hq // (Hq / Hkv).

With a value rotation R on the cache (oracle/rotation.py; SoloQ summary page:
values follow the rotated activation path), the cached values are R v: the
block's own values are rotated the same way (fp32, as at commit), attention
yields R o, and the output is R^T (R o).
"""
from __future__ import annotations

import numpy as np

from .rotation import rotate_f32, unrotate


def attention_rows(q: np.ndarray, keys: np.ndarray, vals: np.ndarray, scale: float) -> np.ndarray:
    """softmax(q keys^T * scale) vals for q [M, D], keys/vals [N, D]; fp64."""
    q = np.asarray(q, np.float64)
    s = (q @ np.asarray(keys, np.float64).T) * float(scale)
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    p /= p.sum(axis=1, keepdims=True)
    return p @ np.asarray(vals, np.float64)


def block_attention(cache, q: np.ndarray, k_blk: np.ndarray, v_blk: np.ndarray,
                    use_suffix: bool = False, scale: float | None = None,
                    pairs=None) -> np.ndarray:
    """Attention output fp64 [B, L, Hq, D].

    q [B, L, Hq, D]; k_blk, v_blk [B, L, Hkv, D] (the full-precision block).
    pairs: optional iterable of (b, hq) to compute (others left as NaN)."""
    B, L, Hq, D = q.shape
    Hkv = k_blk.shape[2]
    assert Hq % Hkv == 0
    r = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    out = np.full((B, L, Hq, D), np.nan)
    want = None if pairs is None else set(pairs)
    rot = getattr(cache, "v_rot", None)
    if rot is not None:
        v_blk = rotate_f32(v_blk, *rot)
    for b in range(B):
        for h in range(Hkv):
            heads = [hq for hq in range(h * r, (h + 1) * r) if want is None or (b, hq) in want]
            if not heads:
                continue
            kp, vp = cache.dequantized(0, b, h)
            ks = [kp, np.asarray(k_blk[b, :, h], np.float64)]
            vs = [vp, np.asarray(v_blk[b, :, h], np.float64)]
            if use_suffix:
                ksu, vsu = cache.dequantized(1, b, h)
                ks.append(ksu)
                vs.append(vsu)
            keys = np.concatenate(ks)
            vals = np.concatenate(vs)
            for hq in heads:
                o = attention_rows(q[b, :, hq], keys, vals, scale)
                out[b, :, hq] = o if rot is None else unrotate(o, *rot)
    return out
