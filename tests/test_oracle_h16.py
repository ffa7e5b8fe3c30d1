"""Pins of the fp16-metadata quantizer and record (oracle/quant.py
asym_quantize_h16, oracle/layout.py record_layout_h16): agreement with the fp32
quantizer where scale and zero are fp16 values, clamping when the rounded zero
lies above the group minimum, the reconstruction bound, and record bytes."""
import numpy as np

import oracle as O
from oracle.layout import record_layout_h16
from oracle.quant import asym_quantize, asym_quantize_h16


def test_agrees_where_metadata_is_fp16_exact():
    x = np.arange(16, dtype=np.float32)[None, :] * np.float32(0.5) + np.float32(-3.0)   # scale 0.5, zero -3
    a = asym_quantize(x, 4)
    h = asym_quantize_h16(x, 4)
    assert np.array_equal(a[0], h[0]) and a[1][0] == h[1][0] == 0.5 and a[2][0] == h[2][0] == -3.0


def test_rounded_zero_above_minimum_clamps():
    mn = np.float32(1.0 + 3 * 2.0 ** -12)                 # fp16 neighbours 1 and 1 + 2^-10: rounds up
    x = np.array([[mn, np.float32(2.0), np.float32(1.5), np.float32(3.0)]], np.float32)
    code, s16, z16 = asym_quantize_h16(x, 2)
    assert z16[0] == np.float32(1.0 + 2.0 ** -10) and z16[0] > mn
    assert code[0, 0] == 0 and code.max() <= 3
    assert code[0, 3] == 3                                # the maximum still reaches the top code


def test_reconstruction_bound():
    g = np.random.default_rng(4)
    x = (g.standard_normal((300, 32)) * 2 + 0.5).astype(np.float32)
    for bits in (2, 4):
        code, s16, z16 = asym_quantize_h16(x, bits)
        rec = code * s16[:, None].astype(np.float64) + z16[:, None]
        # half a step, plus what rounding the pair to fp16 moved the grid by
        lev = 2 ** bits - 1
        _, s32, z32 = asym_quantize(x, bits)
        bound = s16 / 2 + np.abs(z16 - z32) + lev * np.abs(s16 - s32)
        assert np.all(np.abs(rec - x).max(axis=1) <= bound * (1 + 1e-6) + 1e-7)


def test_record_bytes_h16():
    g = np.random.default_rng(5)
    B, H, D = 1, 1, 64
    k = g.standard_normal((B, 32, H, D)).astype(np.float32)
    v = g.standard_normal((B, 32, H, D)).astype(np.float32)
    c = O.OracleCache(B, H, D, 4, 2, 32, fmt="int_h16")
    c.commit(0, k, v)
    rec = c.records(0, 0)[0, 0]
    L = record_layout_h16(D, 4, 2, 32)
    assert rec.shape[0] == L["record_bytes"] == 2048          # 2560 with fp32 metadata
    for ch in (0, 17, 63):
        _, s16, z16 = asym_quantize_h16(k[0, :, 0, ch][None, :].copy(), 4)
        got_s = rec[L["kmeta_offset"] + 2 * ch:L["kmeta_offset"] + 2 * ch + 2].view("<f2")[0]
        got_z = rec[L["kmeta_offset"] + 2 * D + 2 * ch:L["kmeta_offset"] + 2 * D + 2 * ch + 2].view("<f2")[0]
        assert np.float32(got_s) == s16[0] and np.float32(got_z) == z16[0]
    for grp, t in ((0, 0), (1, 31)):
        _, s16, z16 = asym_quantize_h16(v[0, t, 0, 32 * grp:32 * grp + 32][None, :].copy(), 2)
        off = L["vmeta_offset"] + grp * 128
        assert np.float32(rec[off + 2 * t:off + 2 * t + 2].view("<f2")[0]) == s16[0]
        assert np.float32(rec[off + 64 + 2 * t:off + 64 + 2 * t + 2].view("<f2")[0]) == z16[0]


def test_codes_against_the_rounded_pair():
    # Group {0, 0.5 - 2^-13, 1} at 2 bits: the fp32 scale is fl(1/3) =
    # 0.3333333432..., which rounds to the fp16 scale 1365/4096 = 0.333251953125,
    # and the zero 0 is exact in both.  Against the rounded pair the middle
    # element is (0.5 - 2^-13) / (1365/4096) = 1.5 exactly (1.5 * 1365/4096 =
    # 0.4998779296875), a tie that rounds to even: code 2.  Against the fp32
    # pair it is 1.49963 and would give code 1.
    x = np.array([[0.0, 0.5 - 2.0 ** -13, 1.0]], np.float32)
    code, s16, z16 = asym_quantize_h16(x, 2)
    assert s16[0] == np.float32(1365 / 4096) and z16[0] == 0.0
    assert list(code[0]) == [0, 2, 3]
    # the fp32 quantizer on the same group gives the other code for the middle
    c32, s32, _ = asym_quantize(x, 2)
    assert s32[0] == np.float32(1.0) / np.float32(3.0) and list(c32[0]) == [0, 1, 3]
