"""Lloyd-Max scalar codebook for a unit Gaussian, rounded to fp16.

[S "Architecture notes", Codebook caching]: the codebooks are Lloyd-Max
quantisers computed once on the CPU.  The workloads fix them as 2^b-level
Lloyd-Max quantisers of a Gaussian; the unit-variance codebook is used and
the row's norm carries the scale (a reading: the pages name Lloyd-Max
codebooks, not their scale).

Lloyd-Max optimality (Lloyd 1957 / Max 1960) is the pair of conditions

  * every decision threshold is the midpoint of its two neighbouring levels;
  * every level is the conditional mean of the density over its cell,
        c_i = (phi(t_i) - phi(t_{i+1})) / (Phi(t_{i+1}) - Phi(t_i)).

The oracle reaches the fixed point by Lloyd's alternation from
equal-probability cells and then polishes it with a library root finder
(scipy.optimize.root) on the same equations, because plain Lloyd steps
converge very slowly for 16 levels.
"""
from __future__ import annotations

import struct

import numpy as np
from scipy import optimize, special


def _phi(x):
    return np.exp(-0.5 * x * x) / np.sqrt(2.0 * np.pi)


def _cell_prob(a, b):
    """P(a < X < b) for X ~ N(0,1), taking the tail complement where it is
    more accurate."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    upper = special.ndtr(-a) - special.ndtr(-b)
    lower = special.ndtr(b) - special.ndtr(a)
    return np.where(a >= 0, upper, lower)


def centroids_of(thresh_inner: np.ndarray) -> np.ndarray:
    """Conditional means of N(0,1) over the cells cut by the inner thresholds."""
    t = np.concatenate([[-np.inf], thresh_inner, [np.inf]])
    a, b = t[:-1], t[1:]
    pa = np.where(np.isinf(a), 0.0, _phi(np.where(np.isinf(a), 0.0, a)))
    pb = np.where(np.isinf(b), 0.0, _phi(np.where(np.isinf(b), 0.0, b)))
    return (pa - pb) / _cell_prob(a, b)


def midpoints(c: np.ndarray) -> np.ndarray:
    return 0.5 * (c[:-1] + c[1:])


def lloyd_max_gaussian(levels: int, lloyd_iters: int = 500) -> np.ndarray:
    """fp64 Lloyd-Max levels for N(0,1), ascending and exactly symmetric."""
    if levels < 2 or levels & (levels - 1):
        raise ValueError("levels must be a power of two >= 2")
    # equal-probability starting cells
    t = special.ndtri(np.arange(1, levels) / levels)
    c = centroids_of(t)
    for _ in range(lloyd_iters):
        c = centroids_of(midpoints(c))
    # polish: solve c = centroids(midpoints(c)) on the positive half
    half = levels // 2

    def full(pos):
        return np.concatenate([-pos[::-1], pos])

    def resid(pos):
        cc = full(pos)
        return (centroids_of(midpoints(cc)) - cc)[half:]

    sol = optimize.root(resid, c[half:], method="hybr", tol=1e-15)
    pos = sol.x if np.max(np.abs(resid(sol.x))) <= np.max(np.abs(resid(c[half:]))) else c[half:]
    return full(pos)


def fixed_point_residual(c: np.ndarray) -> float:
    return float(np.max(np.abs(centroids_of(midpoints(c)) - c)))


def f64_to_f16_bits(x) -> np.ndarray:
    """IEEE binary16 bit patterns of float64 values, rounded directly from
    float64 to nearest, ties to even (numpy's conversion; the tests pin it
    against Python's struct 'e' packing and hand-made tie cases)."""
    with np.errstate(over="ignore"):
        return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)


def f16_bits_to_f64(b) -> np.ndarray:
    return np.asarray(b, dtype=np.uint16).view(np.float16).astype(np.float64)


def codebook_f16(bits: int) -> np.ndarray:
    """The codebook itself: 2^bits fp16 levels (ascending), as float16.

    The fp64 Lloyd-Max levels are symmetrised and rounded to fp16; these fp16
    values are the codebook both the encoder and the decoder use, so the
    codebook contributes no rounding of its own (a reading: the pages do not
    say at which precision the levels are stored)."""
    c = lloyd_max_gaussian(1 << bits)
    c = 0.5 * (c - c[::-1])          # exact symmetry c_i = -c_{L-1-i}
    return c.astype(np.float16)


def codebook_f16_bits(bits: int) -> np.ndarray:
    return codebook_f16(bits).view(np.uint16)


def thresholds_f64(cb16: np.ndarray) -> np.ndarray:
    """Decision thresholds: exact fp64 midpoints of consecutive fp16 levels
    (the midpoint condition of Lloyd-Max applied to the stored codebook)."""
    c = np.asarray(cb16, dtype=np.float16).astype(np.float64)
    return (c[:-1] + c[1:]) * 0.5


def struct_f16_bits(x: float) -> int:
    """Python's own binary16 packing (correctly rounded), used as a pin."""
    return struct.unpack("<H", struct.pack("<e", x))[0]
