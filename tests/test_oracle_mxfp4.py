"""Pins of the MX FP4 oracle (oracle/mxfp4.py): the E2M1 grid and its ties by
hand, saturation, the scale rule against log2, exact reconstruction of values
on the grid, members, and the record layout sizes."""
import math

import numpy as np

from oracle.mxfp4 import e2m1_code, e2m1_value, mx_dequantize, mx_quantize, record_layout_mx, scale_byte


def test_e2m1_grid_and_ties_by_hand():
    vals = [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    assert e2m1_code(np.array(vals)).tolist() == list(range(8))
    # midpoints go to the even code: 0.25->0, 0.75->1.0, 1.25->1.0, 1.75->2.0, 2.5->2, 3.5->4, 5->4
    assert e2m1_code(np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])).tolist() == [0, 2, 2, 4, 4, 6, 6]
    assert e2m1_code(np.array([0.26, 0.74, 2.51, 5.01, 6.5, 1e9])).tolist() == [1, 1, 5, 7, 7, 7]
    assert e2m1_code(np.array([-0.5, -6.0, -100.0, -0.1, -0.0])).tolist() == [9, 15, 15, 8, 8]
    assert np.array_equal(e2m1_value(np.arange(16)), [0, .5, 1, 1.5, 2, 3, 4, 6, 0, -.5, -1, -1.5, -2, -3, -4, -6])


def test_scale_rule_against_log2():
    for a in [1.0, 1.5, 5.99, 6.0, 7.9, 8.0, 0.3, 3e-20, 1e30]:
        want = math.floor(math.log2(np.float32(a))) - 2 + 127
        assert int(scale_byte(np.float32(a))) == want, a
    assert int(scale_byte(np.float32(0.0))) == 0
    assert int(scale_byte(np.float32(1e-40))) == 0          # subnormal maximum: smallest scale


def test_grid_values_reconstruct_exactly():
    g = np.random.default_rng(0)
    for e in (-20, -3, 0, 5, 13):
        codes = g.integers(0, 16, (64, 32))
        codes[:, 0] = 7                                      # amax = 6 * 2^e in every group
        x = (e2m1_value(codes) * 2.0 ** e).astype(np.float32)
        c, s = mx_quantize(x)
        assert np.all(s == e + 127)
        np.testing.assert_array_equal(mx_dequantize(c, s), x.astype(np.float64))


def test_members_and_empty_groups():
    x = np.array([[1.0, -3.0, 100.0, 0.5], [0.0, 0.0, 0.0, 0.0]], np.float32)
    member = np.array([[True, True, False, True], [True, True, True, True]])
    c, s = mx_quantize(x, member)
    # amax over members is 3: scale 2^(1 - 2) = 0.5; 1 -> 2 (code 4), -3 -> -6 (code 15), 0.5 -> 1 (code 2)
    assert s.tolist() == [126, 0] and c.tolist() == [[4, 15, 0, 2], [0, 0, 0, 0]]
    err = np.abs(mx_dequantize(c, s) - x)[0, [0, 1, 3]]
    assert np.all(err == 0)


def test_quantization_error_bound():
    """On the grid (|x| <= 6X) the error is at most half the largest step, X;
    above it the scale rule (amax < 8X) saturates at 6X, an error below 2X."""
    g = np.random.default_rng(1)
    x = (g.standard_normal((200, 32)) * 3).astype(np.float32)
    c, s = mx_quantize(x)
    X = np.ldexp(1.0, s.astype(np.int64) - 127)[:, None]
    err = np.abs(mx_dequantize(c, s) - x)
    on = np.abs(x) <= 6 * X
    assert np.all(err[on] <= np.broadcast_to(X, x.shape)[on])
    assert np.all(err < 2 * X) and np.any(~on)


def test_record_layout_sizes():
    for D, want in ((128, 4352), (64, 2304)):
        L = record_layout_mx(D)
        assert L["record_bytes"] == want
        assert L["vc_offset"] == 16 * D and L["kmeta_offset"] == 32 * D and L["vmeta_offset"] == 33 * D


def test_cache_records_by_hand():
    """MX FP4 records of the oracle cache, read back byte by byte: key scale
    bytes per channel over the slot's member tokens, key nibbles at the
    integer layout's positions, value scale bytes per (32-channel group, token)."""
    import oracle as O
    g = np.random.default_rng(2)
    B, H, D = 1, 1, 64
    k = (g.standard_normal((B, 40, H, D)) * 2).astype(np.float32)
    v = g.standard_normal((B, 40, H, D)).astype(np.float32)
    c = O.OracleCache(B, H, D, 4, 4, 32, fmt="mxfp4")
    c.commit(0, k, v, prot=[np.array([3])])
    rec = c.records(0, 0)[0, 0]                                  # first slot: tokens 0..31
    L = record_layout_mx(D)
    for ch in (0, 7, 33, 63):
        members = [t for t in range(32) if t != 3]
        amax = max(abs(float(k[0, t, 0, ch])) for t in members)
        e = math.floor(math.log2(np.float32(amax))) - 2
        assert rec[L["kmeta_offset"] + ch] == e + 127
        for t in (0, 3, 17, 31):
            word = int.from_bytes(bytes(rec[(ch // 8 * 32 + t) * 4:(ch // 8 * 32 + t) * 4 + 4]), "little")
            nib = (word >> (4 * (ch % 8))) & 15
            want = 0 if t == 3 else int(e2m1_code(np.array([float(k[0, t, 0, ch]) / 2.0 ** e]))[0])
            assert nib == want, (ch, t, nib, want)
    for grp in (0, 1):
        for t in (0, 9, 31):
            amax = max(abs(float(x)) for x in v[0, t, 0, 32 * grp:32 * grp + 32])
            e = math.floor(math.log2(np.float32(amax))) - 2
            assert rec[L["vmeta_offset"] + 32 * grp + t] == e + 127
