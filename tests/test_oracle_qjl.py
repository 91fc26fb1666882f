"""Pins of the oracle's QJL residual stage (oracle/qjl.py).

The pages only name the fields ([D "Recipe Strategy"]: [MSE indices][QJL
signs][vector norm][residual norm]); these tests pin the reading to what
the mathematics fixes:
  * for a Gaussian projection the sketch's term has mean gamma (q.e)/|e|
    and variance (pi/2) gamma^2 (|q|^2 - (2/pi)(q.e)^2/|e|^2) / m over the
    draws of S (checked by sampling many projections);
  * with S = I the signs are those of the residual y - y_hat itself, with
    S = -I they flip, with a permutation matrix they permute; the residual
    norm is |y - y_hat| rounded to fp16;
  * the effective key's score equals the decoder's projected-query form;
  * pages round-trip the fields (layout), and QJL is rejected on V."""
import math

import numpy as np
import pytest

from oracle import encode as enc, qjl, pages as pg
from oracle.rotation import rotate
from oracle.codebook import f64_to_f16_bits
import workloads as wl


def fmt_with(S, d=64, bits=(2,), seed=1):
    signs = wl.signs(seed, 1, d)
    ch = None
    if len(bits) == 2:
        ch = np.concatenate([np.arange(0, d, 2), np.arange(1, d, 2)])
    return enc.Format.make(d, list(bits), signs, ch, qjl_proj=S)


def fields(x, f):
    w = rotate(np.asarray(x, dtype=np.float64), f.signs)
    idx, nb = enc.quantize_rotated(w, f)
    sb, gb = qjl.residual_fields(w, idx, nb, f)
    return w, idx, nb, sb, gb


def residual_y(x, f):
    """y - y_hat in the normalised rotated domain from the (separately
    pinned) rotation and MSE dequantisation."""
    w, idx, nb, _, _ = fields(x, f)
    y = w / math.sqrt(f.head_dim)
    return y - enc.dequantize_rotated(idx, nb, f)


@pytest.mark.parametrize("bits", [(2,), (4,), (3, 2)])
def test_identity_projection_gives_residual_signs_and_norm(bits):
    d = 64
    m = d // len(bits)
    rng = np.random.default_rng(5)
    x = rng.standard_normal((20, d))
    f = fmt_with(np.stack([np.eye(m, dtype=np.float32)] * len(bits)), d, bits)
    _, _, _, sb, gb = fields(x, f)
    e = residual_y(x, f)
    for g, ch in enumerate(f.groups()):
        assert np.array_equal(sb[:, g, :], (e[:, ch] < 0).astype(np.uint8))
        ref = f64_to_f16_bits(np.linalg.norm(e[:, ch], axis=-1))
        got = gb[:, g].astype(np.int64)
        assert np.max(np.abs(got - ref.astype(np.int64))) <= 1   # fp16 of the same value (1 ulp at a tie)
        assert np.mean(got == ref) > 0.9
    fn = fmt_with(-np.stack([np.eye(m, dtype=np.float32)] * len(bits)), d, bits)
    _, _, _, sbn, gbn = fields(x, fn)
    nz = np.abs(e[:, f.groups()[0]]) > 0
    assert np.array_equal(sbn[:, 0, :][nz], 1 - sb[:, 0, :][nz]) and np.array_equal(gbn, gb)


def test_permutation_projection_permutes_the_signs():
    d = m = 64
    rng = np.random.default_rng(6)
    x = rng.standard_normal((10, d))
    perm = rng.permutation(m)
    P = np.zeros((m, m), np.float32)
    P[np.arange(m), perm] = 1.0              # z_i = r_perm[i]
    _, _, _, s_id, _ = fields(x, fmt_with(np.eye(m, dtype=np.float32)[None]))
    _, _, _, s_p, _ = fields(x, fmt_with(P[None]))
    assert np.array_equal(s_p[:, 0, :], s_id[:, 0, perm])


@pytest.mark.parametrize("bits", [(2,), (3, 2)])
def test_gaussian_sketch_mean_and_variance(bits):
    """Over many draws of S the sketch term has the published estimator's
    mean and variance (a wrong constant, a transposed S, or flipped signs
    fail this)."""
    d = 64
    m = d // len(bits)
    rng = np.random.default_rng(7)
    x = rng.standard_normal(d)
    q = rng.standard_normal(d)
    f0 = fmt_with(np.zeros((len(bits), m, m), np.float32), d, bits)
    qr = rotate(q, f0.signs) / math.sqrt(d)
    e = residual_y(x, f0)                      # independent of S
    N = 4000
    terms = np.empty((N, len(bits)))
    gam = None
    f = fmt_with(np.zeros((len(bits), m, m), np.float32), d, bits)
    for k in range(N):
        f.qjl_proj = rng.standard_normal((len(bits), m, m)).astype(np.float32)   # a fresh draw
        _, idx, nb, sb, gb = fields(x, f)
        _, sk = qjl.score_terms(qr, idx, nb, sb, gb, f)
        terms[k] = sk
        gam = gb.view(np.float16).astype(np.float64)
    for g, ch in enumerate(f0.groups()):
        en = np.linalg.norm(e[ch])
        qe = qr[ch] @ e[ch]
        mean = gam[g] * qe / en
        var = (math.pi / 2) * gam[g] ** 2 * (qr[ch] @ qr[ch] - (2 / math.pi) * qe ** 2 / en ** 2) / m
        se = math.sqrt(var / N)
        assert abs(terms[:, g].mean() - mean) < 4.5 * se, (g, terms[:, g].mean(), mean, se)
        assert abs(terms[:, g].var() / var - 1) < 0.12, (g, terms[:, g].var(), var)
        assert abs(gam[g] / en - 1) < 2 ** -10


def test_effective_key_matches_projected_query_form():
    d = 128
    rng = np.random.default_rng(8)
    S = rng.standard_normal((2, 64, 64)).astype(np.float32)
    f = fmt_with(S, d, (3, 2))
    x = rng.standard_normal((30, d))
    q = rng.standard_normal(d)
    w, idx, nb, sb, gb = fields(x, f)
    qr = rotate(q, f.signs) / math.sqrt(d)
    k_eff = enc.dequantize_rotated(idx, nb, f) + qjl.correction_rotated(sb, gb, f)
    mse, sk = qjl.score_terms(qr, idx, nb, sb, gb, f)
    assert np.allclose(k_eff @ qr, mse.sum(-1) + sk.sum(-1), rtol=1e-12, atol=1e-12)


def test_qjl_pages_round_trip_and_v_rejected():
    d = 128
    rng = np.random.default_rng(9)
    S = rng.standard_normal((2, 64, 64)).astype(np.float32)
    f = fmt_with(S, d, (3, 2))
    rb, noff, tile = pg.tile_layout(f, 16)
    assert rb == 40 + 16 and noff == 16 * 56 and tile == 1024
    x = rng.standard_normal((40, 2, d))
    slots = rng.permutation(64)[:40]
    pages = np.zeros((4, 2, tile), np.uint8)
    pg.write_pages(x, slots, pages, f, 16)
    for h in range(2):
        idx, nb, sb, gb = pg.read_rows(pages, slots // 16, slots % 16, h, f, 16)
        _, idx0, nb0, sb0, gb0 = fields(x[:, h], f)
        assert all(np.array_equal(a, b) for a, b in zip(idx, idx0))
        assert np.array_equal(nb, nb0) and np.array_equal(sb, sb0) and np.array_equal(gb, gb0)
    with pytest.raises(ValueError):
        pg.write_pages(x, slots, np.zeros((4, 2, tile), np.uint8), f, 16, "v")
    with pytest.raises(ValueError):
        enc.Format.make(d, [3, 2], f.signs, f.group_channels, qjl_proj=S[:, :32])


# ---------------------------------------------------------------- projection order
def test_projection_equals_plain_python_loop():
    """The vectorised projection equals the defined order written as a plain
    Python loop over IEEE doubles (brute force, element by element)."""
    from tests import qjl_cases as qc
    rng = np.random.default_rng(11)
    r = rng.standard_normal((6, 32)) * np.exp(rng.uniform(-20, 20, (6, 32)))
    S = rng.standard_normal((32, 32)).astype(np.float32)
    z = qjl.project(r, S)
    for t in range(6):
        for i in range(32):
            assert z[t, i] == qc.python_chain(S[i], r[t])


def test_projection_order_decides_a_cancelling_sum():
    """Hand-worked: r = (0.1, -1e-30, -0.1), S row (1, 1, 1).  In the defined
    order 0.1 + (-1e-30) rounds to 0.1 and 0.1 - 0.1 = +0, so the bit is 0,
    although the exact sum is -1e-30 (an order adding the first and last
    terms first would give bit 1).  r = (x, -x), S row (sigma, sigma) with
    sigma * x inexact: unfused products cancel to +0."""
    from fractions import Fraction
    r = np.array([[0.1, -1e-30, -0.1]])
    S = np.ones((1, 3), np.float32)
    z = qjl.project(r, S)
    assert z[0, 0] == 0.0 and not np.signbit(z[0, 0])
    assert sum(Fraction(v) for v in r[0]) < 0
    x = 0.1
    sig = np.float32(1 / 3)
    assert Fraction(float(sig) * x) != Fraction(float(sig)) * Fraction(x)   # inexact product
    z2 = qjl.project(np.array([[x, -x]]), np.array([[sig, sig]], np.float32))
    assert z2[0, 0] == 0.0


@pytest.mark.parametrize("bits,d", [((4,), 128), ((2,), 128), ((3, 2), 128), ((4, 3), 128), ((4,), 64),
                                    ((3, 2), 64)])
def test_sign_bits_of_cancelling_sums_follow_the_defined_order(bits, d):
    """Rows and projections built so that some projection sums cancel
    exactly (tests/qjl_cases.py): the stage's order gives +0 (bit 0) for
    every such sum, while exact arithmetic ("order" rows) or a fused
    multiply-add ("fusion" rows) would give a negative z (bit 1).  The
    oracle's bits for those rows are 0, its z equals the plain Python loop,
    and each built case is really sensitive to the order."""
    from tests import qjl_cases as qc
    x, S, f, cases = qc.build(d, bits)
    assert any(c[0] == "order" for c in cases) and any(c[0] == "fusion" for c in cases)
    w = rotate(x[:, 0].astype(np.float64), f.signs)
    idx, nb = enc.quantize_rotated(w, f)
    res = qjl.residuals(w, idx, nb, f)
    sb, _ = qjl.residual_fields(w, idx, nb, f)
    for kind, g, i, tok, (a, c) in cases:
        r = res[g][tok]
        assert r[a] == -r[c] != 0
        assert qc.python_chain(S[g, i], r) == 0.0
        assert sb[tok, g, i] == 0, (kind, g, i, tok)
        if kind == "order":
            assert qc.exact_sum(S[g, i], r) < 0
        else:
            assert qc.fused_chain(S[g, i], r) < 0
