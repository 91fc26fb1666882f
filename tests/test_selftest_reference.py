"""The host reference of the device fp64 self-test, pinned on the CPU:
numpy's float64 -> float16 conversion equals exact rational rounding (to
nearest, ties to even, directly from binary64) on the edge cases, so it can
judge the device's binary16 bits; a conversion through binary32 would fail
on the midpoints' binary64 neighbours."""
import numpy as np

from tests.test_gpu_selftest import exact_f16_bits, f16_edge_cases


def test_numpy_binary16_rounding_is_exact_on_edge_cases():
    x = f16_edge_cases()
    sel = np.random.default_rng(3).choice(len(x), 3000, replace=False)
    with np.errstate(over="ignore"):   # values past 65520 round to infinity, as they should
        got = x[sel].astype(np.float16).view(np.uint16)
    ref = np.array([exact_f16_bits(v) for v in x[sel]], dtype=np.uint16)
    assert np.array_equal(got, ref)


def test_exact_rounding_catches_double_rounding():
    """A binary64 value one ulp above a binary16 midpoint rounds up exactly,
    while rounding through binary32 first lands on the midpoint and then on
    the even neighbour: the pin can tell the two methods apart."""
    lo = float(np.float16(1.0))
    hi = float(np.nextafter(np.float16(1.0), np.float16(2.0)))
    mid = (lo + hi) / 2
    x = np.nextafter(mid, 2.0)
    assert exact_f16_bits(x) == int(np.float16(hi).view(np.uint16))
    via32 = np.float32(x).astype(np.float16).view(np.uint16)
    assert int(via32) == int(np.float16(lo).view(np.uint16))
