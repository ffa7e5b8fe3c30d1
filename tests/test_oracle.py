"""Pins for the CPU oracle: closed forms, invariants, special cases and brute force.

The pages print no worked example for this path, so every pin here comes from
mathematics: values the quantizer formula fixes by hand, bounds it must obey,
cases that reduce to a textbook routine, and pure-Python brute force.
"""
import math

import numpy as np
import pytest

import oracle as O
from oracle.layout import pack_k_words, pack_v_words, record_layout

F32 = np.float32


def q1(vals, bits, member=None):
    x = np.asarray(vals, dtype=F32)[None, :]
    m = None if member is None else np.asarray(member, bool)[None, :]
    c, s, z = O.asym_quantize(x, bits, m)
    return c[0], s[0], z[0]


# --------------------------------------------------------------- quantizer
def test_constant_group_is_exact():
    for v in [0.0, 1.5, -3.25, 1e-30]:
        c, s, z = q1([v] * 32, 4)
        assert s == 0 and z == F32(v) and np.all(c == 0)
        assert np.all(O.dequantize(c[None], s[None], z[None])[0] == F32(v))


def test_negative_zero_is_canonical():
    c, s, z = q1([-0.0] * 8, 2)
    assert np.signbit(z) == False and np.signbit(s) == False  # noqa: E712
    c, s, z = q1([-0.0, 0.0, -0.0], 4)
    assert s == 0 and not np.signbit(s) and not np.signbit(z)


def test_identity_group():
    # {0..15} at 4 bits: scale = 15/15 = 1, zero = 0, codes = values
    c, s, z = q1(np.arange(16), 4)
    assert s == F32(1) and z == F32(0) and np.array_equal(c, np.arange(16))
    c, s, z = q1([3, 0, 1, 2], 2)
    assert s == F32(1) and np.array_equal(c, [3, 0, 1, 2])


def test_round_half_to_even():
    # scale = (3 - 0)/3 = 1; 2.5 is a tie -> 2 (half up would give 3)
    c, s, _ = q1([0, 2.5, 3], 2)
    assert s == 1 and list(c) == [0, 2, 3]
    c, _, _ = q1([0, 0.5, 1, 1.5, 3], 2)
    assert list(c) == [0, 0, 1, 2, 3]
    c, _, _ = q1([0, 3.5, 4.5, 15], 4)
    assert list(c) == [0, 4, 4, 15]


def test_division_not_reciprocal():
    # The code takes an IEEE fp32 division (x - mn) / scale.  Hand values, all
    # exact in bf16: {-2.109375, 0.7265625, 3.5625} at 2 bits has range
    # 5.671875 and scale 5.671875 / 3 = 1.890625 exactly; the middle element
    # sits at 2.8359375 / 1.890625 = 1.5 exactly, a tie that rounds to even (2).
    # Multiplying by the rounded reciprocal 1/1.890625 instead gives
    # 1.4999999 and code 1, so a reciprocal-multiply quantizer fails here.
    c, s, z = q1([-2.109375, 0.7265625, 3.5625], 2)
    assert s == F32(1.890625) and z == F32(-2.109375)
    assert list(c) == [0, 2, 3]
    # the same group one octave up: scale 3.78125, the same tie
    c, s, z = q1([-4.21875, 1.453125, 7.125], 2)
    assert s == F32(3.78125) and list(c) == [0, 2, 3]


def test_subnormal_group():
    # values k * 2^-149 (fp32 subnormals): range 3 * 2^-149, scale 2^-149 exactly
    tiny = np.float32(2.0 ** -149)
    c, s, z = q1(np.array([0, 1, 2, 3], F32) * tiny, 2)
    assert s == tiny and z == 0 and list(c) == [0, 1, 2, 3]


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_power_of_two_scaling(bits):
    g = np.random.default_rng(7)
    x = g.standard_normal((200, 32)).astype(F32)
    c0, s0, z0 = O.asym_quantize(x, bits)
    for k in (-3, 5):
        c1, s1, z1 = O.asym_quantize((x * F32(2.0 ** k)).astype(F32), bits)
        assert np.array_equal(c0, c1)
        assert np.array_equal(s1, s0 * F32(2.0 ** k)) and np.array_equal(z1, z0 * F32(2.0 ** k))


@pytest.mark.parametrize("bits", [2, 4, 8, 16])
def test_invariants_and_error_bound(bits):
    g = np.random.default_rng(bits)
    x = (g.standard_normal((4000, 32)) * g.lognormal(0, 2, (4000, 1))).astype(F32)
    c, s, z = O.asym_quantize(x, bits)
    n = 2 ** bits - 1
    assert c.max() <= n
    rows = np.arange(x.shape[0])
    assert np.all(c[rows, x.argmin(1)] == 0)
    assert np.all(c[rows, x.argmax(1)] == n)
    err = np.abs(O.dequantize(c, s, z) - x.astype(np.float64))
    bound = s.astype(np.float64)[:, None] * (0.5 + n * 2.0 ** -23 * (1 + 1e-6))
    assert np.all(err <= bound)


def test_sixteen_bit_limit():
    g = np.random.default_rng(3)
    x = g.standard_normal((500, 32)).astype(F32)
    c, s, z = O.asym_quantize(x, 16)
    rng = (x.max(1) - x.min(1)).astype(np.float64)
    err = np.abs(O.dequantize(c, s, z) - x).max(1)
    assert np.all(err <= rng * (0.5 + 65535 * 2.0 ** -23) / 65535 * 1.0001)


def test_member_mask_excludes_entries():
    g = np.random.default_rng(11)
    x = g.standard_normal((50, 32)).astype(F32)
    m = g.random((50, 32)) < 0.7
    m[:, 0] = True
    c, s, z = O.asym_quantize(x, 4, m)
    for i in range(50):
        ci, si, zi = q1(x[i][m[i]], 4)
        assert si == s[i] and zi == z[i]
        assert np.array_equal(c[i][m[i]], ci) and np.all(c[i][~m[i]] == 0)
    c, s, z = q1([1.0, 2.0], 4, member=[False, False])
    assert s == 0 and z == 0 and list(c) == [0, 0]


def test_bf16_rounding():
    vals = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5, 3.0e38], F32)
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7 -> even (1.0); 1 + 3*2^-8 -> 1 + 2^-6
    out = O.to_bf16_f32(vals)
    assert list(out[:3]) == [1.0, 1.0, 1.0 + 2 ** -6]
    assert out[3] == 1.0 and out[4] == -2.5


# --------------------------------------------------------------- layout
def test_record_sizes():
    assert record_layout(128, 4, 4, 64)["record_bytes"] == 5632
    assert record_layout(128, 2, 2, 64)["record_bytes"] == 3584
    assert record_layout(128, 4, 4, 128)["record_bytes"] == 5376
    assert record_layout(64, 4, 4, 64)["record_bytes"] == 2816
    lay = record_layout(128, 4, 4, 64)
    assert (lay["vc_offset"], lay["kmeta_offset"], lay["vmeta_offset"]) == (2048, 4096, 5120)


def test_k_words_by_hand():
    # channel c of a 4-bit row sits at bits 4*(c % 8) of word c // 8.
    # row codes (t + 3c) % 16 for t = 0: channels 0..7 -> 0,3,6,9,12,15,2,5
    # -> nibbles (high..low) 5 2 F C 9 6 3 0 = 0x52FC9630
    codes = (np.arange(32)[:, None] + 3 * np.arange(64)[None, :]) % 16
    w = pack_k_words(codes, 4)
    assert w[0, 0] == 0x52FC9630
    # t = 1, channels 8..15: (1 + 24 + 3e) % 16 = 9,12,15,2,5,8,11,14 -> 0xEB852FC9
    assert w[1, 1] == 0xEB852FC9
    # 2-bit: 16 channels per word; codes (c % 4) -> 0,1,2,3 repeating -> 0xE4E4E4E4
    w2 = pack_k_words(np.tile(np.arange(64) % 4, (32, 1)), 2)
    assert np.all(w2 == 0xE4E4E4E4)


def test_v_token_positions_by_hand():
    P = O.v_token_position
    assert [P(t, 4) for t in (0, 3, 4, 8, 11, 12, 16, 20, 24, 31)] == [
        (0, 0), (0, 12), (1, 0), (0, 16), (0, 28), (1, 16), (2, 0), (3, 0), (2, 16), (3, 28)]
    assert [P(t, 2) for t in (0, 4, 8, 16, 24, 31)] == [(0, 0), (1, 0), (0, 8), (0, 16), (0, 24), (1, 30)]
    for vb in (2, 4):
        seen = {P(t, vb) for t in range(32)}
        assert len(seen) == 32 and all(0 <= w < vb and b % vb == 0 for w, b in seen)
    # one channel whose token codes are t % 16 at 4 bits: word 0 holds tokens
    # 0..3 then 8..11 -> nibbles (high..low) B A 9 8 3 2 1 0
    w = pack_v_words((np.arange(32) % 16)[None, :], 4)
    assert w[0, 0] == 0xBA983210 and w[0, 1] == 0xFEDC7654


def test_record_words_are_word_major():
    # Kc: word w of token t at byte (w*32 + t)*4; Vc: word j of channel c at
    # byte kc_bytes + (j*D + c)*4 (ABI header, packed cache layout).
    D = 64
    kcodes = (np.arange(32)[:, None] + 3 * np.arange(D)[None, :]) % 16
    vcodes = np.tile(np.arange(32) % 16, (D, 1))
    z = np.zeros
    rec = O.pack_record(kcodes, vcodes, z(D, F32), z(D, F32), z((1, 32), F32), z((1, 32), F32), 4, 4, 64)
    u32 = lambda off: int(rec[off:off + 4].view("<u4")[0])
    assert u32((0 * 32 + 0) * 4) == 0x52FC9630
    assert u32((1 * 32 + 1) * 4) == 0xEB852FC9
    kc = 32 * D * 4 // 8
    assert u32(kc + (0 * D + 0) * 4) == 0xBA983210
    assert u32(kc + (1 * D + 5) * 4) == 0xFEDC7654


def test_pack_unpack_round_trip():
    g = np.random.default_rng(5)
    for (D, kb, vb, gv) in [(128, 4, 4, 64), (128, 2, 2, 64), (64, 4, 2, 32), (128, 2, 4, 128)]:
        G = D // gv
        a = dict(kcodes=g.integers(0, 2 ** kb, (3, 32, D)), vcodes=g.integers(0, 2 ** vb, (3, D, 32)),
                 kscale=g.random((3, D), F32), kzero=g.standard_normal((3, D), F32),
                 vscale=g.random((3, G, 32), F32), vzero=g.standard_normal((3, G, 32), F32))
        rec = O.pack_record(**a, kb=kb, vb=vb, gv=gv)
        assert rec.shape == (3, record_layout(D, kb, vb, gv)["record_bytes"])
        u = O.unpack_record(rec, D, kb, vb, gv)
        for k, v in a.items():
            assert np.array_equal(u[k], v), k


# --------------------------------------------------------------- cache model
def _kv(B, n, H, D, seed=0):
    g = np.random.default_rng(seed)
    return g.standard_normal((B, n, H, D), dtype=F32), g.standard_normal((B, n, H, D), dtype=F32)


def test_slots_start_at_each_commit():
    c = O.OracleCache(1, 2, 64, 4, 4, 32)
    k, v = _kv(1, 40, 2, 64)
    c.commit(0, k, v)
    k2, v2 = _kv(1, 24, 2, 64, 1)
    c.commit(0, k2, v2)
    hd = c.headers(0, 0).view("<i4").reshape(-1, 4)
    assert hd[:, 0].tolist() == [32, 8, 24] and hd[:, 3].tolist() == [0, 32, 40]
    # the second slot's group statistics use only its 8 tokens
    cc = c.codes(0, 0)
    ks, kz = cc["kscale"][1, 0], cc["kzero"][1, 0]
    ref_c, ref_s, ref_z = O.asym_quantize(np.ascontiguousarray(k[0, 32:40, 0].T), 4)
    assert np.array_equal(ks, ref_s) and np.array_equal(kz, ref_z)
    assert np.all(cc["kcodes"][1, 0, 8:] == 0) and np.all(cc["vcodes"][1, 0, :, 8:] == 0)
    assert np.all(cc["vscale"][1, 0, :, 8:] == 0) and np.all(cc["vzero"][1, 0, :, 8:] == 0)
    kh, vh = c.dequantized(0, 0, 1)
    assert kh.shape == (64, 64) and vh.shape == (64, 64)


def test_protected_rows():
    B, n, H, D = 2, 64, 2, 64
    k, v = _kv(B, n, H, D, 3)
    # all tokens protected: K is exact (bf16 of the input); K codes/meta are 0
    c = O.OracleCache(B, H, D, 2, 2, 64)
    c.commit(0, k, v, prot=[np.arange(n)] * B)
    cc = c.codes(0, 1)
    assert np.all(cc["kcodes"] == 0) and np.all(cc["kscale"] == 0) and np.all(cc["kzero"] == 0)
    kh, vh = c.dequantized(0, 1, 1)
    assert np.array_equal(kh, O.to_bf16_f32(k[1, :, 1]).astype(np.float64))
    c0 = O.OracleCache(B, H, D, 2, 2, 64)
    c0.commit(0, k, v)
    assert np.array_equal(vh, c0.dequantized(0, 1, 1)[1])       # V does not change
    # some protected: excluded from the statistics, rank bases count them in order
    prot = [np.array([0, 5, 33, 63]), np.array([31])]
    c1 = O.OracleCache(B, H, D, 4, 4, 64)
    c1.commit(0, k, v, prot=prot)
    hd = c1.headers(0, 0).view("<i4").reshape(-1, 4)
    assert hd[:, 1].view("<u4").tolist() == [(1 << 0) | (1 << 5), (1 << 1) | (1 << 31)]
    assert hd[:, 2].tolist() == [0, 2]
    pos, rows = c1.protected(0, 0)
    assert pos.tolist() == [0, 5, 33, 63] and np.array_equal(rows[2], O.to_bf16_f32(k[0, 33]))
    keep = np.ones(32, bool)
    keep[[0, 5]] = False
    ref_c, ref_s, ref_z = O.asym_quantize(np.ascontiguousarray(k[0, :32, 1][keep].T), 4)
    assert np.array_equal(c1.codes(0, 0)["kscale"][0, 1], ref_s)
    kh1, _ = c1.dequantized(0, 0, 1)
    assert np.array_equal(kh1[5], O.to_bf16_f32(k[0, 5, 1]).astype(np.float64))


def test_reset_segment():
    c = O.OracleCache(1, 1, 64, 4, 4, 64)
    k, v = _kv(1, 64, 1, 64)
    c.commit(1, k, v, prot=[np.array([3])])
    c.commit(1, k[:, :32], v[:, :32], reset=True)
    assert c.ntok(1, 0) == 32 and c.nslots(1, 0) == 1 and len(c.protected(1, 0)[0]) == 0


# --------------------------------------------------------------- attention
def _brute(q, keys, vals, scale):
    out = []
    for qi in q:
        s = [math.fsum(float(a) * float(b) for a, b in zip(qi, k)) * scale for k in keys]
        m = max(s)
        e = [math.exp(x - m) for x in s]
        tot = math.fsum(e)
        out.append([math.fsum(e[j] * float(vals[j][d]) for j in range(len(keys))) / tot
                    for d in range(len(vals[0]))])
    return np.array(out)


def test_attention_matches_brute_force():
    g = np.random.default_rng(9)
    q, k, v = g.standard_normal((4, 16)), g.standard_normal((40, 16)) * 2, g.standard_normal((40, 16))
    ref = _brute(q, k, v, 0.25)
    assert np.abs(O.attention_rows(q, k, v, 0.25) - ref).max() < 1e-12


def test_attention_special_cases():
    g = np.random.default_rng(2)
    k, v = g.standard_normal((50, 8)), g.standard_normal((50, 8))
    # rows of P sum to one: all-ones values give all-ones output
    assert np.abs(O.attention_rows(g.standard_normal((3, 8)), k, np.ones((50, 8)), 0.3) - 1).max() < 1e-14
    # Q = 0: uniform weights -> mean of the values
    assert np.abs(O.attention_rows(np.zeros((2, 8)), k, v, 0.3) - v.mean(0)).max() < 1e-14
    # equal value rows -> that row
    vv = np.tile(v[:1], (50, 1))
    assert np.abs(O.attention_rows(g.standard_normal((2, 8)), k, vv, 0.3) - v[0]).max() < 1e-14
    # one key scoring 50 above all others -> its value row (others weigh e^-50)
    q = np.zeros((1, 8)); q[0, 0] = 1.0
    kk = np.zeros((50, 8)); kk[17, 0] = 50.0
    assert np.abs(O.attention_rows(q, kk, v, 1.0) - v[17]).max() < 1e-19 * 50 + 1e-20


def test_block_attention_sixteen_bits_matches_sdpa():
    torch = pytest.importorskip("torch")
    B, H, r, D, n = 2, 2, 3, 64, 96
    k, v = _kv(B, n, H, D, 4)
    g = np.random.default_rng(8)
    q = g.standard_normal((B, 32, H * r, D), dtype=F32)
    kb, vb = _kv(B, 32, H, D, 5)
    errs = []
    for bits in (8, 12, 16):
        c = O.OracleCache(B, H, D, bits, bits, 64)
        c.commit(0, k, v)
        out = O.block_attention(c, q, kb, vb)
        K = np.concatenate([k, kb], 1).astype(np.float64)     # [B, n+32, H, D]
        V = np.concatenate([v, vb], 1).astype(np.float64)
        Kt = torch.from_numpy(K).permute(0, 2, 1, 3).repeat_interleave(r, dim=1)
        Vt = torch.from_numpy(V).permute(0, 2, 1, 3).repeat_interleave(r, dim=1)
        Qt = torch.from_numpy(q.astype(np.float64)).permute(0, 2, 1, 3)
        ref = torch.nn.functional.scaled_dot_product_attention(Qt, Kt, Vt).permute(0, 2, 1, 3).numpy()
        errs.append(np.abs(out - ref).max())
    assert errs[2] < 1e-3 and errs[0] > errs[1] > errs[2]
    # error shrinks roughly 16x per 4 extra bits
    assert errs[0] / errs[2] > 100


def test_gqa_head_mapping_and_dual_cache():
    B, H, r, D = 1, 2, 3, 64
    c = O.OracleCache(B, H, D, 4, 4, 64)
    # prefix values: head h holds the constant 10 + h; suffix: 100 + h; block: 0
    n, ns = 64, 32
    k = np.random.default_rng(1).standard_normal((B, n, H, D), dtype=F32)
    v = np.broadcast_to((10 + np.arange(H, dtype=F32))[None, None, :, None], (B, n, H, D)).copy()
    c.commit(0, k, v)
    ksu = np.random.default_rng(2).standard_normal((B, ns, H, D), dtype=F32)
    vsu = np.broadcast_to((100 + np.arange(H, dtype=F32))[None, None, :, None], (B, ns, H, D)).copy()
    c.commit(1, ksu, vsu)
    q = np.zeros((B, 32, H * r, D), F32)                     # uniform weights
    kb = np.zeros((B, 32, H, D), F32)
    vb = np.zeros((B, 32, H, D), F32)
    out = O.block_attention(c, q, kb, vb)
    for hq in range(H * r):
        assert np.allclose(out[0, :, hq], (10 + hq // r) * n / (n + 32), rtol=0, atol=1e-12)
    out = O.block_attention(c, q, kb, vb, use_suffix=True)
    for hq in range(H * r):
        h = hq // r
        assert np.allclose(out[0, :, hq], ((10 + h) * n + (100 + h) * ns) / (n + ns + 32), atol=1e-12)
