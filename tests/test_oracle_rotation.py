"""Pins for the oracle's rotation (signs + Walsh-Hadamard)."""
from fractions import Fraction

import numpy as np
import pytest

from oracle import rotation as rot
from workloads import bf16_round, signs


@pytest.mark.parametrize("d", [2, 4, 8, 16, 32, 64, 128])
def test_sylvester_square_is_d_identity(d):
    H = rot.sylvester_hadamard(d)
    np.testing.assert_array_equal(H @ H, d * np.eye(d))
    np.testing.assert_array_equal(H, H.T)


@pytest.mark.parametrize("d", [2, 8, 64, 128])
def test_butterfly_equals_dense_matrix(d):
    rng = np.random.default_rng(d)
    X = rng.integers(-1000, 1000, size=(20, d)).astype(np.float64)   # exact in fp64
    H = rot.sylvester_hadamard(d)
    np.testing.assert_array_equal(rot.fwht(X), X @ H.T)
    Xf = rng.standard_normal((20, d))
    np.testing.assert_allclose(rot.fwht(Xf), Xf @ H.T, rtol=0, atol=1e-12)


def test_natural_order_first_rows():
    """Natural (Sylvester) order, not sequency order: the second output is the
    alternating-sign sum, the third pairs signs (+,+,-,-,...)."""
    d = 8
    e = np.eye(d)
    out = rot.fwht(e)  # column j = H e_j
    np.testing.assert_array_equal(out[:, 1], [1, -1, 1, -1, 1, -1, 1, -1])
    np.testing.assert_array_equal(out[:, 2], [1, 1, -1, -1, 1, 1, -1, -1])


@pytest.mark.parametrize("d", [64, 128])
def test_rotation_is_orthogonal(d):
    rng = np.random.default_rng(1)
    s = signs(0, 1, d)
    x = rng.standard_normal((200, d))
    y = rot.rotate(x, s) / np.sqrt(d)
    np.testing.assert_allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-12)
    back = rot.inverse_rotate(y, s)
    np.testing.assert_allclose(back, x, rtol=0, atol=1e-12)
    # R = H diag(s)/sqrt(d) as a dense matrix
    R = rot.sylvester_hadamard(d) * s[None, :] / np.sqrt(d)
    np.testing.assert_allclose(R @ R.T, np.eye(d), atol=1e-14)
    np.testing.assert_allclose(y, x @ R.T, atol=1e-12)


def test_bf16_rows_transform_exactly():
    """For bf16 inputs the float64 butterfly equals exact rational arithmetic
    (so the result does not depend on the order of additions there)."""
    rng = np.random.default_rng(3)
    d = 128
    s = signs(0, 1, d)
    x = bf16_round(rng.standard_normal((4, d)).astype(np.float32)).astype(np.float64)
    w = rot.rotate(x, s)
    H = rot.sylvester_hadamard(d).astype(int)
    for r in range(4):
        xs = [Fraction(float(v)) * int(si) for v, si in zip(x[r], s)]
        for i in range(0, d, 7):
            exact = sum((xs[j] if H[i, j] > 0 else -xs[j]) for j in range(d))
            assert Fraction(float(w[r, i])) == exact
