"""Pins for norms, indices and packing in the oracle's encoder."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import encode as enc
from oracle.codebook import thresholds_f64
from oracle.rotation import rotate, inverse_rotate
from workloads import bf16_round, signs, channel_subset

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def fmt1(d=128, bits=4, seed=0):
    return enc.Format.make(d, [bits], signs(seed, 1, d))


def fmt2(d=128, bits=(4, 3), seed=0):
    hi = channel_subset(seed, 3, d, d // 2)
    lo = np.array(sorted(set(range(d)) - set(hi.tolist())))
    return enc.Format.make(d, list(bits), signs(seed, 1, d), np.concatenate([hi, lo]))


def test_tree_sum_order_is_pinned():
    """Adjacent pairs first: (1e16 + 1) + (-1e16 + 1) = 0 in fp64, whereas a
    left-to-right sum gives 1 and the exact sum is 2."""
    v = np.array([1e16, 1.0, -1e16, 1.0])
    assert enc.tree_sum(v) == 0.0
    assert ((v[0] + v[1]) + v[2]) + v[3] == 1.0
    v8 = np.array([1e16, 1.0, 1.0, 1.0, -1e16, 1.0, 1.0, 1.0])
    # ((1e16+1)+(1+1)) + ((-1e16+1)+(1+1)) = (1e16+2) + (-1e16+2) = 4
    assert enc.tree_sum(v8) == 4.0


@pytest.mark.parametrize("case", json.load(open(os.path.join(GOLDEN, "pack_examples.json")))["cases"])
def test_pack_hand_examples(case):
    got = enc.pack_group(np.array(case["indices"]), case["bits"])
    assert [int(b) for b in got] == [int(h, 16) for h in case["bytes"]]
    back = enc.unpack_group(got, case["bits"], len(case["indices"]))
    assert back.tolist() == case["indices"]


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("m", [32, 64, 128])
def test_pack_roundtrip(bits, m):
    rng = np.random.default_rng(bits * m)
    idx = rng.integers(0, 1 << bits, size=(50, m))
    data = enc.pack_group(idx, bits)
    assert data.shape == (50, m * bits // 8)
    np.testing.assert_array_equal(enc.unpack_group(data, bits, m), idx)


def test_norm_matches_vector_norm():
    rng = np.random.default_rng(2)
    f = fmt1()
    x = bf16_round(rng.standard_normal((500, 128)).astype(np.float32)).astype(np.float64)
    _, n16 = enc.encode_rows(x, f)
    norms = n16[:, 0].view(np.float16).astype(np.float64)
    ref = np.linalg.norm(x, axis=1)
    # the stored value is fp16(|y|) with |y| = |x| (orthogonal rotation)
    np.testing.assert_array_equal(norms, ref.astype(np.float16).astype(np.float64))
    w = rotate(x, f.signs)
    ss = enc.tree_sum(w * w)
    np.testing.assert_allclose(np.sqrt(ss / 128), ref, rtol=1e-12)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_indices_are_nearest_level(bits):
    """Away from thresholds the index is the brute-force nearest level of the
    unit-variance coordinate g = w / sqrt(ss / m)."""
    rng = np.random.default_rng(bits)
    f = fmt1(bits=bits)
    x = rng.standard_normal((300, 128))
    (idx,), _ = enc.encode_rows(x, f)
    w = rotate(x, f.signs)
    g = w / np.sqrt(np.sum(w * w, axis=1, keepdims=True) / 128)
    c = f.codebooks[0].astype(np.float64)
    dist = np.abs(g[..., None] - c)
    brute = np.argmin(dist, axis=-1)
    t = thresholds_f64(f.codebooks[0])
    near = np.min(np.abs(g[..., None] - t), axis=-1) < 1e-9
    assert np.all(brute[~near] == idx[~near])
    assert near.sum() < 5


def _four_squares(n):
    r = int(math.isqrt(n))
    for a in range(r, -1, -1):
        ra = n - a * a
        for b in range(int(math.isqrt(ra)), -1, -1):
            rb = ra - b * b
            for c in range(int(math.isqrt(rb)), -1, -1):
                rc = rb - c * c
                e = int(math.isqrt(rc))
                if e * e == rc:
                    return a, b, c, e
    raise AssertionError


@pytest.mark.parametrize("i", [8, 10, 13, 3])
def test_exact_threshold_tie_goes_to_lower_index(i):
    """Build a rotated row with ss/m == 1 exactly, so T_i == t_i, and place
    one coordinate exactly on threshold t_i: the index is i (T_i < w fails)."""
    f = fmt1(bits=4)
    t = thresholds_f64(f.codebooks[0])
    ti = Fraction(float(t[i]))
    scale = max(4096, ti.denominator)          # a power of two: k/scale squares exactly
    A = ti * scale
    assert A.denominator == 1
    A = int(A)
    # t_i^2 + rest = 5 with rest a sum of four squares of k/4096
    rest = 5 * scale * scale - A * A
    a, b, c, e = _four_squares(rest)
    w = np.array([float(ti), a / scale, b / scale, c / scale, e / scale] + [1.0] * 123)
    assert enc.tree_sum(w * w) == 128.0
    (idx,), norms = enc.quantize_rotated(w[None, :], f)
    assert idx[0, 0] == i
    # nudging up by one ulp crosses the threshold
    w2 = w.copy()
    w2[0] = np.nextafter(w2[0], np.inf)
    (idx2,), _ = enc.quantize_rotated(w2[None, :], f)
    assert idx2[0, 0] == i + 1
    assert norms[0, 0] == np.float16(1.0).view(np.uint16)


def test_zero_coordinate_and_zero_row():
    f = fmt1(bits=4)
    w = np.ones((2, 128))
    w[0, 5] = 0.0
    w[0, 6] = -0.0
    w[1, :] = 0.0
    (idx,), norms = enc.quantize_rotated(w, f)
    assert idx[0, 5] == 7 and idx[0, 6] == 7      # T_7 = 0 is not < 0
    assert np.all(idx[1] == 7) and norms[1, 0] == 0
    # zero row through encode_rows (rotation of zeros is zeros)
    (idx0,), n0 = enc.encode_rows(np.zeros((1, 128)), f)
    assert np.all(idx0 == 7) and n0[0, 0] == 0
    # dequantised zero row is zero
    y = enc.dequantize_rotated([idx0], n0, f)
    assert np.all(y == 0)


def test_two_groups_match_per_group_encoding():
    """Each group is normalised by its own norm and quantised with its own
    codebook, in listed channel order."""
    f = fmt2()
    rng = np.random.default_rng(5)
    x = rng.standard_normal((40, 128))
    (i_hi, i_lo), n = enc.encode_rows(x, f)
    w = rotate(x, f.signs)
    for g, (ch, idx, b) in enumerate(zip(f.groups(), (i_hi, i_lo), (4, 3))):
        wg = w[:, ch]
        ss = enc.tree_sum(wg * wg)
        r = np.sqrt(ss / 64)
        c = f.codebooks[g].astype(np.float64)
        brute = np.argmin(np.abs((wg / r[:, None])[..., None] - c), axis=-1)
        assert np.mean(brute == idx) > 0.999
        np.testing.assert_array_equal(n[:, g], np.sqrt(ss / 128).astype(np.float16).view(np.uint16))
    rb = enc.row_bytes(f)
    assert rb == 32 + 24


@pytest.mark.parametrize("bits,expect", [(4, 0.009497), (3, 0.03454), (2, 0.1175)])
def test_reconstruction_error_matches_lloyd_max_distortion(bits, expect):
    """[D "Diagnostic Route Design"]: vector reconstruction error.  On Gaussian
    rows the mean relative squared error is close to the scalar Lloyd-Max
    distortion (a large-d approximation; fp16 levels and norms shift it a
    little)."""
    rng = np.random.default_rng(11)
    f = fmt1(bits=bits)
    x = rng.standard_normal((4000, 128))
    idx, n = enc.encode_rows(x, f)
    xh = inverse_rotate(enc.dequantize_rotated(idx, n, f), f.signs)
    rel = np.sum((x - xh) ** 2, axis=1) / np.sum(x * x, axis=1)
    assert abs(np.mean(rel) - expect) / expect < 0.05
    assert np.all(np.isfinite(xh))


def test_format_validation_errors():
    s = signs(0, 1, 128)
    with pytest.raises(ValueError):
        enc.Format.make(128, [5], s)
    with pytest.raises(ValueError):
        enc.Format.make(96, [4], s[:96])
    with pytest.raises(ValueError):
        enc.Format.make(128, [4, 3], s)             # two groups need a channel list
    bad = s.copy()
    bad[3] = 0
    with pytest.raises(ValueError):
        enc.Format.make(128, [4], bad)
    ch = np.arange(128)
    ch[0], ch[1] = 1, 0                              # not ascending within group
    with pytest.raises(ValueError):
        enc.Format.make(128, [4, 3], s, ch)
