"""Pins for the oracle's Lloyd-Max codebook and fp64 -> fp16 rounding."""
import json
import math
import os
import struct

import numpy as np
import pytest
from scipy import integrate

from oracle import codebook as cbm

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _pdf(x):
    return math.exp(-0.5 * x * x) / math.sqrt(2 * math.pi)


@pytest.mark.parametrize("levels", [2, 4, 8, 16])
def test_fixed_point_by_independent_quadrature(levels):
    """Each level is the conditional mean of N(0,1) over its cell, checked by
    adaptive quadrature (not the closed form the solver uses)."""
    c = cbm.lloyd_max_gaussian(levels)
    t = np.concatenate([[-np.inf], 0.5 * (c[:-1] + c[1:]), [np.inf]])
    for i in range(levels):
        mass, _ = integrate.quad(_pdf, t[i], t[i + 1], epsabs=1e-14, epsrel=1e-13)
        first, _ = integrate.quad(lambda x: x * _pdf(x), t[i], t[i + 1], epsabs=1e-14, epsrel=1e-13)
        assert abs(first / mass - c[i]) < 1e-9


@pytest.mark.parametrize("levels", [2, 4, 8, 16])
def test_fixed_point_residual_and_symmetry(levels):
    c = cbm.lloyd_max_gaussian(levels)
    assert cbm.fixed_point_residual(c) < 1e-12
    assert np.all(np.diff(c) > 0)
    np.testing.assert_array_equal(c, -c[::-1])


def test_two_level_closed_form():
    """Two levels: +-E|X| = +-sqrt(2/pi), distortion 1 - 2/pi."""
    c = cbm.lloyd_max_gaussian(2)
    assert abs(c[1] - math.sqrt(2 / math.pi)) < 1e-14
    mse = 1.0 - c[1] ** 2  # D = E[X^2] - sum p_i c_i^2 with p = 1/2 each
    assert abs(mse - (1 - 2 / math.pi)) < 1e-14


@pytest.mark.parametrize("levels", ["2", "4", "8", "16"])
def test_against_published_table(levels):
    g = json.load(open(os.path.join(GOLDEN, "lloyd_max_published.json")))
    ref = g["levels"][levels]
    tol = g["tolerance"]
    L = int(levels)
    c = cbm.lloyd_max_gaussian(L)
    pos = c[L // 2:]
    np.testing.assert_allclose(pos, ref["outputs"], atol=tol)
    th = 0.5 * (c[:-1] + c[1:])[L // 2:]
    np.testing.assert_allclose(th, ref["thresholds"], atol=tol)
    # distortion by quadrature over the cells
    t = np.concatenate([[-np.inf], 0.5 * (c[:-1] + c[1:]), [np.inf]])
    mse = sum(integrate.quad(lambda x, ci=c[i]: (x - ci) ** 2 * _pdf(x), t[i], t[i + 1])[0]
              for i in range(L))
    assert abs(mse - ref["mse"]) < max(2e-4, 0.01 * ref["mse"])


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_fp16_codebook_is_far_from_rounding_ties(bits):
    """The fp16 codebook must not depend on the solver's last digits: every
    fp64 level sits well away from an fp16 rounding boundary."""
    c = cbm.lloyd_max_gaussian(1 << bits)
    for v in c:
        f = np.float16(v)
        up = np.nextafter(f, np.float16(np.inf))
        dn = np.nextafter(f, np.float16(-np.inf))
        ulp = float(up) - float(f) if abs(v) >= abs(float(f)) else float(f) - float(dn)
        frac = abs(v - float(f)) / abs(ulp)
        assert frac < 0.5 - 1e-6


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_codebook_f16_properties(bits):
    cb = cbm.codebook_f16(bits)
    assert cb.dtype == np.float16 and cb.shape == (1 << bits,)
    assert np.all(np.diff(cb.astype(np.float64)) > 0)
    np.testing.assert_array_equal(cb, -cb[::-1])
    t = cbm.thresholds_f64(cb)
    assert t[(1 << bits) // 2 - 1] == 0.0
    # midpoints of two fp16 values are exact in fp64
    c = cb.astype(np.float64)
    for i in range(len(t)):
        assert t[i] * 2 == c[i] + c[i + 1]


def test_f16_rounding_pins():
    """numpy's float64 -> float16 conversion rounds to nearest even directly
    from float64; pinned against Python's struct packing and hand cases."""
    rng = np.random.default_rng(7)
    vals = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-8, 5, 20000),
                           rng.uniform(0, 70000, 2000)])
    got = cbm.f64_to_f16_bits(vals)
    for v, b in zip(vals[:5000], got[:5000]):
        assert cbm.struct_f16_bits(float(v)) == int(b)
    # ties to even: 1 + 2^-11 is halfway between 1 and 1 + 2^-10
    assert cbm.f64_to_f16_bits(1.0 + 2.0 ** -11) == 0x3C00
    assert cbm.f64_to_f16_bits(1.0 + 3 * 2.0 ** -11) == 0x3C02
    # just above a tie rounds up: no double rounding through float32
    x = 1.0 + 2.0 ** -11 + 2.0 ** -40
    assert float(np.float32(x)) == 1.0 + 2.0 ** -11       # fp32 would lose the sticky bit
    assert cbm.f64_to_f16_bits(x) == 0x3C01
    assert cbm.f64_to_f16_bits(65504.0) == 0x7BFF
    assert cbm.f64_to_f16_bits(65520.0) == 0x7C00          # overflow rounds to +inf
    assert cbm.f64_to_f16_bits(2.0 ** -24) == 0x0001       # smallest subnormal
    assert cbm.f64_to_f16_bits(2.0 ** -25) == 0x0000       # tie to even -> 0
    assert cbm.f64_to_f16_bits(0.0) == 0x0000
