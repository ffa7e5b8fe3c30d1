"""MX FP4 cache format (oracle): E2M1 codes with one power-of-two scale per group.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Source: the SoloQ abstract (The Latest in AI card page) and the SoloQ summary
page (opening summary): a hardware-native 4-bit floating-point format with
per-block scales (NVFP4) is one of the method's targets.  Here the format is
the OCP microscaling FP4 that gfx950 converts natively (it is not NVFP4, which
scales blocks of 16 with fp8 factors):
  * an element is E2M1: sign, 2 exponent bits, 1 mantissa bit, magnitudes
    {0, 0.5, 1, 1.5, 2, 3, 4, 6}; code = sign << 3 | index into that list;
  * a group of 32 elements shares an E8M0 scale byte s, X = 2^(s - 127);
  * keys keep the KIVI-style groups (one channel over the 32 tokens of a slot,
    protected and invalid tokens left out), values take groups of 32 channels
    of one token.

Readings (listed in the design notes):
  * s = max(E(amax) - 2, 0), E(amax) the biased exponent field of the group's
    largest magnitude in fp32 (0 for zero or subnormal maxima), i.e. the shared
    exponent floor(log2(amax)) - 2 of the OCP scale rule, 2 being the largest
    exponent of E2M1, clamped at the bottom of the E8M0 range;
  * code = E2M1 round-to-nearest-even of x / X with saturation at 6 (x / X is
    exact: X is a power of two), the sign taken from the sign bit of x;
  * members only: other elements get code 0; a group without members, or with
    amax = 0, gets s = 0 and codes 0;
  * dequantized value: e2m1(code) * X, exact.
"""
from __future__ import annotations

import numpy as np

E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
_MID = (E2M1[:-1] + E2M1[1:]) / 2          # 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5


def e2m1_code(v: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even onto E2M1 with saturation; v exact (fp64)."""
    v = np.asarray(v, np.float64)
    a = np.abs(v)
    idx = np.searchsorted(_MID, a, side="left")            # number of midpoints below a
    tie = (idx < len(_MID)) & (a == _MID[np.minimum(idx, len(_MID) - 1)])
    idx = np.where(tie & (idx % 2 == 1), idx + 1, idx)     # a tie goes to the even index
    idx = np.minimum(idx, 7)                               # saturation
    return (np.signbit(v).astype(np.uint16) << 3) | idx.astype(np.uint16)


def e2m1_value(code: np.ndarray) -> np.ndarray:
    code = np.asarray(code).astype(np.int64)
    return np.where(code & 8, -1.0, 1.0) * E2M1[code & 7]


def scale_byte(amax: np.ndarray) -> np.ndarray:
    """E8M0 byte of groups with largest magnitude amax (fp32)."""
    bits = np.asarray(amax, np.float32).view(np.uint32)
    e = ((bits >> np.uint32(23)) & np.uint32(0xFF)).astype(np.int64)
    return np.maximum(e - 2, 0).astype(np.uint8)


def mx_quantize(x: np.ndarray, member: np.ndarray | None = None):
    """Groups along the LAST axis of fp32 x; returns (codes uint16, scale bytes uint8)."""
    x = np.asarray(x, np.float32)
    assert np.all(np.isfinite(x))
    if member is None:
        member = np.ones(x.shape, bool)
    member = np.asarray(member, bool)
    amax = np.where(member, np.abs(x), np.float32(0)).max(axis=-1).astype(np.float32)
    s = scale_byte(amax)
    X = np.ldexp(1.0, s.astype(np.int64) - 127)[..., None]
    code = e2m1_code(x.astype(np.float64) / X)
    code = np.where(member & (amax[..., None] > 0), code, 0).astype(np.uint16)
    return code, s


def mx_dequantize(code: np.ndarray, s: np.ndarray) -> np.ndarray:
    """e2m1(code) * 2^(s - 127), fp64; s broadcasts against the last axis."""
    return e2m1_value(code) * np.ldexp(1.0, np.asarray(s).astype(np.int64) - 127)[..., None]


def record_layout_mx(D: int) -> dict:
    """Record of the MX FP4 format: codes as the 4-bit integer layout, then one
    scale byte per key channel, then per 32-channel value group one byte per token."""
    kc = 32 * D * 4 // 8
    vc = D * 4 * 4
    km = D
    vm = (D // 32) * 32
    return dict(kc_offset=0, vc_offset=kc, kmeta_offset=kc + vc, vmeta_offset=kc + vc + km,
                record_bytes=(kc + vc + km + vm + 255) // 256 * 256)
