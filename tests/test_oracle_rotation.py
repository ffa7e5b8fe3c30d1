"""Pins of the oracle's K-RPBH value rotation (oracle/rotation.py) against
closed forms and invariants, and of rotated-value attention against exact
attention; CPU only."""
import numpy as np
import pytest

import oracle as O
import workloads as W


def sylvester(n):
    """Unnormalised Hadamard matrix by the doubling recursion."""
    h = np.ones((1, 1))
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


@pytest.mark.parametrize("b", [16, 64])
def test_hadamard_closed_form(b):
    h = O.hadamard(b)
    assert np.array_equal(h * np.sqrt(b), sylvester(b))
    assert np.allclose(h @ h.T, np.eye(b), atol=1e-12)


@pytest.mark.parametrize("b", [16, 64])
def test_fwht_of_unit_vectors_is_exact(b):
    # identity permutation, one block, mix [[1]]: the rotation is H_b, and every
    # output is exactly +-1/sqrt(b) (a power of two), so fp32 is exact
    perm = np.arange(b)
    mix = np.ones((1, 1), np.float32)
    e = np.eye(b, dtype=np.float32)
    y = O.rotate_f32(e, perm, mix, b)
    assert np.array_equal(y.astype(np.float64), O.hadamard(b).T)


@pytest.mark.parametrize("D,b", [(64, 16), (64, 64), (128, 16), (128, 64)])
def test_rotation_matches_matrix_and_is_orthogonal(D, b):
    perm, mix = W.krpbh_params(D, b, seed=3)
    g = np.random.default_rng(7)
    x = (g.standard_normal((40, D)) * np.exp(g.standard_normal((40, 1)))).astype(np.float32)
    R = O.rotation_matrix(perm, mix, b)
    y = O.rotate_f32(x, perm, mix, b)
    ref = x.astype(np.float64) @ R.T
    scale = np.linalg.norm(x, axis=1, keepdims=True)
    assert np.all(np.abs(y - ref) <= 4e-7 * scale * np.sqrt(D / b))
    assert np.allclose(R @ R.T, np.eye(D), atol=1e-6)            # mix is fp32-rounded orthogonal
    assert np.allclose(np.linalg.norm(y, axis=1), scale[:, 0], rtol=1e-5)
    assert np.allclose(O.unrotate(y, perm, mix, b), x, atol=2e-6 * scale.max())


def test_rotation_structure():
    # the permutation alone (k = 1, Hadamard undone): R = H P, so H^T R = P
    D = 64
    perm = np.random.default_rng(1).permutation(D)
    R = O.rotation_matrix(perm, np.ones((1, 1), np.float32), D)
    P = O.hadamard(D).T @ R
    assert np.allclose(P, np.eye(D)[perm], atol=1e-12)
    # the mix acts on the same coordinate of every block: a vector that is one
    # Hadamard column per block is moved only between blocks
    D, b = 128, 16
    perm, mix = np.arange(D), W.krpbh_params(D, b, seed=5)[1]
    x = np.zeros(D, np.float32)
    x[3], x[16 + 3] = 1.0, -2.0                                    # coordinate 3 of blocks 0 and 1
    y = O.rotate_f32(x, perm, mix, b).reshape(D // b, b)
    hcol = O.hadamard(b)[:, 3]
    coef = mix[:, 0].astype(np.float64) * 1.0 + mix[:, 1] * -2.0
    assert np.allclose(y, coef[:, None] * hcol[None, :], atol=1e-6)


def test_attention_is_rotation_invariant():
    # softmax(q K^T) (V R^T) R = softmax(q K^T) V exactly (fp64 closed form)
    g = np.random.default_rng(2)
    D = 128
    perm, mix = W.krpbh_params(D, 64, seed=1)
    R = O.rotation_matrix(perm, mix, 64)
    Rq, _ = np.linalg.qr(R)                                        # exactly orthogonal copy
    q, k, v = g.standard_normal((32, D)), g.standard_normal((90, D)), g.standard_normal((90, D))
    o = O.attention_rows(q, k, v, 0.1)
    o_rot = O.attention_rows(q, k, v @ Rq.T, 0.1) @ Rq
    assert np.allclose(o, o_rot, atol=1e-12)


def test_rotated_cache_high_precision_limit():
    # with 16-bit codes the quantization error vanishes, so the rotated cache's
    # attention must approach the exact attention over the unquantized inputs
    g = np.random.default_rng(4)
    B, H, D, r, n = 2, 2, 64, 2, 96
    perm, mix = W.krpbh_params(D, 16, seed=2)
    k = g.standard_normal((B, n, H, D)).astype(np.float32)
    v = g.standard_normal((B, n, H, D)).astype(np.float32)
    q = g.standard_normal((B, 32, H * r, D)).astype(np.float32)
    kb = g.standard_normal((B, 32, H, D)).astype(np.float32)
    vb = g.standard_normal((B, 32, H, D)).astype(np.float32)
    ora = O.OracleCache(B, H, D, 16, 16, 16, v_rot=(perm, mix, 16))
    ora.commit(0, k, v)
    out = O.block_attention(ora, q, kb, vb)
    for bb in range(B):
        for hq in range(H * r):
            h = hq // r
            keys = np.concatenate([k[bb, :, h], kb[bb, :, h]])
            vals = np.concatenate([v[bb, :, h], vb[bb, :, h]])
            exact = O.attention_rows(q[bb, :, hq], keys, vals, 1 / np.sqrt(D))
            assert np.abs(out[bb, :, hq] - exact).max() < 2e-4


# ---- the fp32 operation order of the forward rotation decides value codes;
# these hand-computed rows fail for any other order, for a fused multiply-add
# in the mix, and for a rotation computed in higher precision and rounded once.

def test_hadamard_stage_order_by_hand():
    # One block of 16, identity permutation, mix [[1]].  x = (1, 2^-24, 2^-24, 0, ...).
    # Stage h=1: (1 + 2^-24 -> 1 (tie to even), 1 - 2^-24, 2^-24, 2^-24).
    # Stage h=2: y0 = 1 + 2^-24 -> 1, y2 = 1 - 2^-24, y1 = (1 - 2^-24) + 2^-24 = 1,
    #            y3 = (1 - 2^-24) - 2^-24 = 1 - 2^-23.
    # Stages h=4, 8 pair these with zeros, so they are copied.  Then /4.
    # Stages in the reverse order would give y1 = 1 - 2^-24, and the exact
    # transform gives y0 = 1 + 2^-23.
    x = np.zeros((1, 16), np.float32)
    x[0, 0], x[0, 1], x[0, 2] = 1.0, 2.0 ** -24, 2.0 ** -24
    y = O.rotate_f32(x, np.arange(16), np.ones((1, 1), np.float32), 16)[0]
    quad = np.array([1.0, 1.0, 1.0 - 2.0 ** -24, 1.0 - 2.0 ** -23], np.float64) / 4
    assert np.array_equal(y.astype(np.float64), np.tile(quad, 4))


def test_mix_products_rounded_before_the_sum():
    # D = 128, b = 64 (k = 2).  x = 8 (1 + 2^-23) at the first coordinate of each
    # block, so every Hadamard output is 1 + 2^-23 (exact).  Mix row 0 =
    # (1 + 2^-23, -(1 + 2^-22)):
    #   p0 = (1 + 2^-23)^2 = 1 + 2^-22 + 2^-46 -> 1 + 2^-22
    #   p1 = -(1 + 2^-23)(1 + 2^-22) = -(1 + 3*2^-23 + 2^-45) -> -(1 + 3*2^-23)
    #   p0 + p1 = -2^-23 exactly.
    # A fused multiply-add gives -(2^-23 + 2^-45); exact products summed and
    # rounded once give -(2^-23 + 2^-46).  Mix row 1 = (1, 0): 1 + 2^-23.
    D, b = 128, 64
    x = np.zeros((1, D), np.float32)
    x[0, 0] = x[0, 64] = np.float32(8 * (1 + 2.0 ** -23))
    mix = np.array([[1 + 2.0 ** -23, -(1 + 2.0 ** -22)], [1.0, 0.0]], np.float32)
    z = O.rotate_f32(x, np.arange(D), mix, b)[0]
    assert np.all(z[:64] == np.float32(-(2.0 ** -23)))
    assert np.all(z[64:] == np.float32(1 + 2.0 ** -23))


def test_mix_summed_in_block_order():
    # D = 64, b = 16 (k = 4).  x = 4 at the first coordinate of each block, so
    # every Hadamard output is 1.  Mix row 0 = (2^-24, 1, 2^-24, 2^-24):
    # in block order ((2^-24 + 1) + 2^-24) + 2^-24 rounds to 1 at every step
    # (each a tie to even).  The reverse order gives 1 + 2^-22, pairs summed
    # first give 1 + 2^-23, and one rounding of the exact sum 1 + 3*2^-24
    # gives 1 + 2^-22.
    D, b = 64, 16
    x = np.zeros((1, D), np.float32)
    x[0, [0, 16, 32, 48]] = 4.0
    mix = np.eye(4, dtype=np.float32)
    mix[0] = [2.0 ** -24, 1.0, 2.0 ** -24, 2.0 ** -24]
    z = O.rotate_f32(x, np.arange(D), mix, b)[0].reshape(4, 16)
    assert np.all(z[0] == 1.0)
    assert np.all(z[1:] == 1.0)
