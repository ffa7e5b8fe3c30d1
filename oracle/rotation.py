"""K-RPBH rotation of value rows (oracle).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Method (SoloQ summary page, rotation paragraphs): a random permutation of the
coordinates, a Hadamard transform on each block of b consecutive coordinates,
then a k x k random orthogonal mix of the same coordinate across the k = D / b
blocks (k = 1 leaves plain RPBH).  For block diffusion the values of a committed
block follow this activation path before they are quantized (same page,
block-diffusion paragraph), so attention over the cache yields R times the
output, and the output comes back through the transpose of R.

Readings where the pages are silent (each listed in the design notes):
  * the permutation and the k x k mix are inputs (the caller draws them);
  * the Hadamard block is normalised by 1/sqrt(b), with b in {16, 64} so that
    this factor is a power of two;
  * the forward rotation is computed in fp32 in this order, so that every
    implementation rounds identically (the quantized codes depend on it):
      y = x[perm];
      Hadamard stages h = 1, 2, 4, ..., b/2 on each block: for every pair
      (i, i + h) with i & h == 0, (y_i, y_{i+h}) <- (y_i + y_{i+h}, y_i - y_{i+h});
      y <- y / sqrt(b) (exact: a power of two);
      z[i*b + j] = sum over l = 0..k-1, in that order, of mix[i, l] * y[l*b + j],
      each product rounded to fp32, then added (no fused multiply-add);
  * the length correction that rescales the quantized vector is not applied.
"""
from __future__ import annotations

import numpy as np

BLOCKS = (16, 64)


def check_params(D: int, perm, mix, block: int):
    perm = np.asarray(perm)
    mix = np.asarray(mix, np.float32)
    assert block in BLOCKS and D % block == 0, (D, block)
    k = D // block
    assert perm.shape == (D,) and np.array_equal(np.sort(perm), np.arange(D)), "perm must permute 0..D-1"
    assert mix.shape == (k, k), (mix.shape, k)
    return perm.astype(np.int64), mix, k


def rotate_f32(x: np.ndarray, perm, mix, block: int) -> np.ndarray:
    """Forward K-RPBH rotation of the last axis of x, in fp32 (order above)."""
    x = np.asarray(x, np.float32)
    D = x.shape[-1]
    perm, mix, k = check_params(D, perm, mix, block)
    y = x[..., perm].reshape(x.shape[:-1] + (k, block)).copy()
    h = 1
    while h < block:
        y = y.reshape(x.shape[:-1] + (k, block // (2 * h), 2, h))
        a = y[..., 0, :].copy()
        c = y[..., 1, :].copy()
        y[..., 0, :] = a + c          # fp32 arrays: each op rounds once
        y[..., 1, :] = a - c
        h *= 2
    y = y.reshape(x.shape[:-1] + (k, block)) * np.float32(1.0 / np.sqrt(block))
    z = np.empty_like(y)
    for i in range(k):
        acc = mix[i, 0] * y[..., 0, :]
        for l in range(1, k):
            acc = acc + mix[i, l] * y[..., l, :]
        z[..., i, :] = acc
    return z.reshape(x.shape)


def hadamard(block: int) -> np.ndarray:
    """Sylvester Hadamard matrix / sqrt(b), fp64: entry (i, j) = (-1)^popcount(i & j) / sqrt(b)."""
    i = np.arange(block)
    bits = np.bitwise_and.outer(i, i)
    par = np.zeros_like(bits)
    while bits.any():
        par ^= bits & 1
        bits >>= 1
    return np.where(par, -1.0, 1.0) / np.sqrt(block)


def rotation_matrix(perm, mix, block: int) -> np.ndarray:
    """R (fp64 [D, D]) with rotate(x) = R x in exact arithmetic:
    R = (mix kron I_b) (I_k kron H_b) P, P the permutation (P x = x[perm])."""
    perm = np.asarray(perm, np.int64)
    D = perm.shape[0]
    _, mix, k = check_params(D, perm, mix, block)
    P = np.zeros((D, D))
    P[np.arange(D), perm] = 1.0
    Hb = np.kron(np.eye(k), hadamard(block))
    M = np.kron(np.asarray(mix, np.float64), np.eye(block))
    return M @ Hb @ P


def unrotate(y: np.ndarray, perm, mix, block: int) -> np.ndarray:
    """R^T y over the last axis, fp64 (the inverse when mix is orthogonal)."""
    R = rotation_matrix(perm, mix, block)
    return np.asarray(y, np.float64) @ R
