"""Asymmetric min/max quantization of one group, in IEEE fp32 (oracle).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Method: KIVI-style asymmetric quantization (Tai et al., "KV Cache Quantization
for Diffusion Language Models", abstract; SoloQ summary page, block-diffusion
paragraph: keys per channel, asymmetric).  The pages print no formula; this is
the plain reading of an asymmetric b-bit quantizer:

    mn = min over the group, mx = max over the group
    scale = (mx - mn) / (2^b - 1)            fp32 subtract, fp32 division
    zero  = mn
    code  = 0 if scale == 0 else clamp(rint((x - mn) / scale), 0, 2^b - 1)
            fp32 subtract, fp32 division, rint = round half to even
    x_hat = code * scale + zero

Scale and zero are stored as canonical +0 when they are zero (x + 0.0 in IEEE
arithmetic turns -0 into +0 and leaves every other value unchanged).
"""
from __future__ import annotations

import numpy as np

F32 = np.float32


def asym_quantize(x: np.ndarray, bits: int, member: np.ndarray | None = None):
    """Quantize groups laid out along the LAST axis of ``x``.

    x      : float32 array [..., n]; each [..., :] row is one group.
    bits   : code width b (1..16).
    member : optional bool array like x; only True entries form the group's
             statistics and get codes; other entries get code 0.  A group with
             no member has scale = zero = 0.

    Returns (codes uint16 [..., n], scale float32 [...], zero float32 [...]).
    """
    x = np.asarray(x)
    assert x.dtype == np.float32, "the quantizer works on fp32 inputs"
    assert np.all(np.isfinite(x)), "non-finite inputs are outside the contract"
    if member is None:
        member = np.ones(x.shape, dtype=bool)
    member = np.asarray(member, dtype=bool)
    levels = F32(2 ** bits - 1)

    any_member = member.any(axis=-1)
    mn = np.where(member, x, F32(np.inf)).min(axis=-1)
    mx = np.where(member, x, F32(-np.inf)).max(axis=-1)
    mn = np.where(any_member, mn, F32(0)).astype(F32)
    mx = np.where(any_member, mx, F32(0)).astype(F32)

    rng = (mx - mn).astype(F32)                  # fp32 subtract
    scale = (rng / levels).astype(F32) + F32(0)  # fp32 division, canonical +0
    zero = mn + F32(0)

    safe = np.where(scale == 0, F32(1), scale)[..., None]
    q = ((x - mn[..., None]).astype(F32) / safe).astype(F32)   # fp32 subtract, fp32 division
    code = np.clip(np.rint(q), F32(0), levels)                  # half to even
    code = np.where(member & (scale[..., None] != 0), code, F32(0))
    return code.astype(np.uint16), scale.astype(F32), zero.astype(F32)


def asym_quantize_h16(x: np.ndarray, bits: int, member: np.ndarray | None = None):
    """asym_quantize with fp16 metadata: the fp32 scale and zero above are
    rounded to fp16 (nearest, ties to even), and the codes are taken against the
    rounded pair, so that code * scale16 + zero16 is the stored reconstruction:
        code = scale16 == 0 ? 0 : clamp(rint(fl(fl(x - zero16) / scale16)), 0, 2^b - 1)
    Returns (codes uint16, scale16, zero16) with the fp16 values as float32."""
    x = np.asarray(x, F32)
    if member is None:
        member = np.ones(x.shape, dtype=bool)
    member = np.asarray(member, dtype=bool)
    _, s32, z32 = asym_quantize(x, bits, member)
    s16 = s32.astype(np.float16).astype(F32) + F32(0)
    z16 = z32.astype(np.float16).astype(F32) + F32(0)
    levels = F32(2 ** bits - 1)
    safe = np.where(s16 == 0, F32(1), s16)[..., None]
    q = ((x - z16[..., None]).astype(F32) / safe).astype(F32)
    code = np.clip(np.rint(q), F32(0), levels)
    code = np.where(member & (s16[..., None] != 0), code, F32(0))
    return code.astype(np.uint16), s16.astype(F32), z16.astype(F32)


def dequantize(code: np.ndarray, scale: np.ndarray, zero: np.ndarray) -> np.ndarray:
    """x_hat = code * scale + zero, evaluated exactly in fp64.

    scale/zero broadcast against the group axis (the last axis of ``code``)."""
    return code.astype(np.float64) * np.asarray(scale, np.float64)[..., None] + \
        np.asarray(zero, np.float64)[..., None]


def to_bf16_f32(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 (ties to even); returned as fp32.

    Protected key rows are stored in bf16; bf16 inputs pass through unchanged."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    lsb = (bits >> 16) & 1
    bits = ((bits + 0x7FFF + lsb) >> 16) << 16
    return bits.astype(np.uint32).view(np.float32).reshape(x.shape)
