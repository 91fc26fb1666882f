"""Device self-test of the write path's fp64 arithmetic: sqrt, division,
multiplication and the direct binary64 -> binary16 rounding, computed by a
kernel built like the write kernel, against the host's IEEE results.  The
bit-exact encoding (signs, Walsh-Hadamard transform, group norms, midpoint
thresholds) rests on these operations being correctly rounded on both
sides.

Host reference: numpy's binary64 sqrt, / and * (correctly rounded on x86),
and numpy's float64 -> float16 conversion, itself pinned against an exact
rational rounding (round to nearest, ties to even) in
test_selftest_reference.py on the cases where a wrong method would differ:
exact midpoints between binary16 neighbours, their binary64 neighbours,
subnormal binary16 results and the overflow boundary.
"""
from fractions import Fraction

import numpy as np
import pytest

from tests.conftest import gpu_available

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def random_doubles(seed, n, lo_exp=1, hi_exp=2046):
    """Finite binary64 values: uniform random exponent field in [lo_exp,
    hi_exp], random mantissa and sign."""
    g = np.random.default_rng(seed)
    e = g.integers(lo_exp, hi_exp + 1, size=n, dtype=np.uint64)
    m = g.integers(0, 1 << 52, size=n, dtype=np.uint64)
    s = g.integers(0, 2, size=n, dtype=np.uint64)
    return ((s << np.uint64(63)) | (e << np.uint64(52)) | m).view(np.float64)


def f16_edge_cases():
    """Midpoints between consecutive binary16 values (positive, finite,
    subnormal included), one binary64 ulp either side of each, the overflow
    boundary, and binary64 subnormals."""
    h = np.arange(0, 0x7BFF, dtype=np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).view(np.float16).astype(np.float64)
    mid = (lo + hi) / 2   # exact in binary64
    cases = [mid, np.nextafter(mid, np.inf), np.nextafter(mid, -np.inf)]
    big = np.array([65504.0, 65519.0, 65519.99999999999, 65520.0, 65520.00000000001, 1e300, 2.0 ** -24,
                    2.0 ** -25, np.nextafter(2.0 ** -25, 1.0), 2.0 ** -26, 5e-324, 2.2250738585072014e-308, 0.0])
    x = np.concatenate(cases + [big])
    return np.concatenate([x, -x])


def exact_f16_bits(x: float) -> int:
    """binary16 bits of x rounded to nearest, ties to even, by exact
    rational arithmetic."""
    sign = 0x8000 if np.signbit(x) else 0
    a = Fraction(abs(float(x)))
    if a == 0:
        return sign
    lo_bits, hi_bits = 0, 0x7BFF
    while lo_bits < hi_bits:   # largest finite magnitude <= a
        midb = (lo_bits + hi_bits + 1) // 2
        if Fraction(float(np.uint16(midb).view(np.float16))) <= a:
            lo_bits = midb
        else:
            hi_bits = midb - 1
    v0 = Fraction(float(np.uint16(lo_bits).view(np.float16)))
    if lo_bits == 0x7BFF:
        # beyond the largest finite value: infinity from 65520 on
        return sign | (0x7C00 if a >= 65520 else 0x7BFF)
    v1 = Fraction(float(np.uint16(lo_bits + 1).view(np.float16)))
    if a - v0 < v1 - a or (a - v0 == v1 - a and lo_bits % 2 == 0):
        return sign | lo_bits
    return sign | (lo_bits + 1)


def test_device_fp64_ops_match_host_bit_for_bit():
    import torch
    import quantized_paged_kv_amd as tq
    n = 1 << 20
    a = np.concatenate([random_doubles(11, n), f16_edge_cases(), random_doubles(12, 4096, 900, 1100)])
    b = np.concatenate([random_doubles(13, n), random_doubles(14, len(a) - n)])
    b[b == 0] = 1.0
    print(f"case fp64 self-test, {len(a)} values", flush=True)
    ad, bd = torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda()
    sq, dv, ml, f16 = (t.cpu().numpy() for t in tq.selftest_fp64(ad, bd))
    with np.errstate(all="ignore"):
        ref_sq = np.sqrt(a)   # NaN below zero; sqrt(-0) = -0
        ref_dv = a / b
        ref_ml = a * b
        ref_f16 = a.astype(np.float16).view(np.uint16)

    def same(got, ref, what, bits):
        g, r = got.view(bits), ref.view(bits)
        nan = np.isnan(ref) if ref.dtype.kind == "f" else np.zeros(len(ref), bool)
        bad = np.flatnonzero((g != r) & ~(nan & np.isnan(got)))
        for i in bad[:5]:
            print(f"{what}: a={a[i]!r} b={b[i]!r} device={got[i]!r} host={ref[i]!r}", flush=True)
        assert len(bad) == 0, f"{what} differs in {len(bad)} of {len(ref)} values"

    same(sq, ref_sq, "sqrt", np.uint64)
    same(dv, ref_dv, "division", np.uint64)
    same(ml, ref_ml, "multiplication", np.uint64)
    same(f16.view(np.uint16), ref_f16, "binary16 rounding", np.uint16)
