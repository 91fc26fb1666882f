"""Random-sign + Walsh-Hadamard rotation.

[T "Highlights"]: quantisation after a random Hadamard rotation; the
workloads fix the rotation as seeded +-1 signs followed by a Walsh-Hadamard
transform scaled by 1/sqrt(d).

Reading of an open point: signs first, then the Sylvester (natural-order) Hadamard matrix
H_d with H[i][j] = (-1)^popcount(i & j), then 1/sqrt(d):

    R = H_d diag(s) / sqrt(d),      R^-1 = R^T = diag(s) H_d / sqrt(d).

The transform is computed by the radix-2 butterfly in a fixed order
(stage h = 1, 2, 4, ..., d/2; each pair (j, j+h) with j & h == 0 becomes
(a + b, a - b)).  With that order pinned, every output is a fixed sequence of
correctly rounded float64 additions, so any implementation that performs the
same additions gets the same bits.
"""
from __future__ import annotations

import numpy as np


def fwht(x: np.ndarray) -> np.ndarray:
    """Unnormalised Walsh-Hadamard transform along the last axis, in float64,
    by butterflies h = 1, 2, ..., d/2 (natural order)."""
    y = np.array(x, dtype=np.float64, copy=True)
    d = y.shape[-1]
    if d & (d - 1):
        raise ValueError("length must be a power of two")
    lead = y.shape[:-1]
    h = 1
    while h < d:
        v = y.reshape(lead + (d // (2 * h), 2, h))
        a = v[..., 0, :].copy()
        b = v[..., 1, :].copy()
        v[..., 0, :] = a + b
        v[..., 1, :] = a - b
        y = v.reshape(lead + (d,))
        h *= 2
    return y


def sylvester_hadamard(d: int) -> np.ndarray:
    """Dense Sylvester Hadamard matrix from its entry formula (used as a pin
    for the butterfly, never by the butterfly itself)."""
    i = np.arange(d)[:, None]
    j = np.arange(d)[None, :]
    bits = np.bitwise_and(i, j)
    pop = np.zeros_like(bits)
    while np.any(bits):
        pop += bits & 1
        bits >>= 1
    return np.where(pop % 2 == 0, 1.0, -1.0)


def rotate(x: np.ndarray, signs: np.ndarray) -> np.ndarray:
    """w = H (s * x): the unnormalised rotated row.  The orthonormal rotated
    row is y = w / sqrt(d)."""
    return fwht(np.asarray(x, dtype=np.float64) * np.asarray(signs, dtype=np.float64))


def inverse_rotate(y: np.ndarray, signs: np.ndarray) -> np.ndarray:
    """x = R^T y = s * (H y) / sqrt(d) (H is symmetric)."""
    d = y.shape[-1]
    return np.asarray(signs, dtype=np.float64) * fwht(y) / np.sqrt(d)
