"""Rows and projections for which the QJL projection sums cancel exactly, so
that only the order and rounding the stage defines decide the sign bits.

Row t is x = c_t * (s * e_{k_t}) + c_t 2^-30 (s * e_{k'_t}) (signs s, unit
vectors e_k, all values exact in bf16), so its rotated row is
w = c_t (H[:, k_t] + 2^-30 H[:, k'_t]): every channel is +-c_t (1 + 2^-30)
or +-c_t (1 - 2^-30), values with more than 30 significant bits.  The
codebook and its thresholds are symmetric, so within a group two positions
a, c with w_a = -w_c have residuals r_a = -r_c exactly.

Projection rows built on that (all other entries of such a row are 0):
  * "order" rows: S[i, a] = 1, S[i, b] = +-2^-60, S[i, c] = 1 with
    a < b < c.  Summed in the defined order (j ascending, each step
    rounded) the tiny middle term is absorbed by r_a and the last term
    cancels it: z_i = +0, sign bit 0.  The exact sum is the tiny term,
    chosen negative for the row the pair was placed on: exact arithmetic,
    or an order that adds r_a and r_c first, gives bit 1.
  * "fusion" rows: S[i, a] = S[i, c] = sigma (an fp32 value for which
    sigma * r_c is not exact in fp64).  Unfused products round
    symmetrically, so z_i = +0 (bit 0); a fused multiply-add for the last
    term leaves -(fl(sigma r_c) - sigma r_c), and sigma is chosen so that
    this is negative (bit 1).
Every other projection row holds the usual N(0, 1) draws.

The helper uses the oracle's rotation, MSE stage and residual to place the
cancelling pairs; the expected bits of the built rows are derived in the
tests from the definition, not read from the oracle.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

from oracle import encode as enc, qjl
from oracle.rotation import rotate
import workloads as wl

TINY = 2.0 ** -60


def _rounded_product_error(s: float, r: float) -> Fraction:
    """fl(s * r) - s * r, exactly."""
    return Fraction(float(s) * float(r)) - Fraction(float(s)) * Fraction(float(r))


def build(d: int = 128, bits=(4,), seed: int = 7, rows_per_kind: int = 3, extra_tokens: int = 13):
    """-> (x [T, 1, d] float32, S [G, m, m] float32, fmt (oracle), cases)

    cases: list of (kind, group, i, token, positions) for the built
    projection rows; token is the row whose residuals place the pair."""
    ng = len(bits)
    m = d // ng
    signs = wl.signs(seed, 1, d)
    ch = None
    if ng == 2:
        ch = np.sort(wl.channel_subset(seed, 3, d, d // 2))
        ch = np.concatenate([ch, np.setdiff1d(np.arange(d), ch)])
    g = np.random.default_rng(seed)
    S = g.standard_normal((ng, m, m)).astype(np.float32)
    # base rows: c s_k e_k + c 2^-30 s_k' e_k' for a few (k, k', c)
    ks = [1, 2, 3, 5, 6, 7, 9, 10, 12, 17, 33, 45][: 3 + extra_tokens // 4]
    cs = [1.0, 3.0, 0.375, 11.5, 0.0703125]
    base = []
    for i, k in enumerate(ks):
        row = np.zeros(d, np.float32)
        k2 = (k + 7 + 3 * i) % d
        row[k] = cs[i % len(cs)] * signs[k]
        row[k2] = np.float32(cs[i % len(cs)] * 2.0 ** -30) * signs[k2]
        base.append(row)
    # a few Gaussian rows as well (their signs are robust)
    gauss = wl.bf16_round(g.standard_normal((max(extra_tokens - len(ks), 1), d)).astype(np.float32))
    x = np.concatenate([np.stack(base), gauss]).astype(np.float32)
    fmt = enc.Format.make(d, list(bits), signs, ch, qjl_proj=S)
    w = rotate(x.astype(np.float64), fmt.signs)
    idx, nb = enc.quantize_rotated(w, fmt)
    res = qjl.residuals(w, idx, nb, fmt)
    cases = []
    sigmas = np.float32([1 / 3, 0.1, 0.7, 1.3, 2.2, 0.37, 5.1, 0.013, 1 / 7, 0.9, 3.3, 1 / 11, 0.29, 7.7])
    for grp in range(ng):
        r = res[grp]
        for kind in ("order", "fusion"):
            made = 0
            for tok in range(len(ks)):
                if made == rows_per_kind:
                    break
                rt = r[tok]
                pos = [j for j in range(m) if rt[j] != 0]
                plus = [j for j in pos if rt[j] > 0]
                minus = [j for j in pos if rt[j] < 0]
                if not plus or not minus:
                    continue
                a = min(plus[0], minus[0])
                cpos = next((j for j in range(a + 2, m) if rt[j] == -rt[a]), None)
                if cpos is None or rt[a + 1] == 0:
                    continue
                assert rt[a] == -rt[cpos]
                i = (7 * made + 3 + 29 * grp + (0 if kind == "order" else 31)) % m
                row = np.zeros(m, np.float32)
                if kind == "order":
                    b = a + 1
                    row[a] = row[cpos] = 1.0
                    row[b] = np.float32(-TINY if rt[b] > 0 else TINY)   # tiny * r_b < 0
                else:
                    # fused last step: fl(fl(sigma r_a) + sigma r_c) with
                    # fl(sigma r_a) = -fl(sigma r_c), i.e. -(fl(sigma r_c) -
                    # sigma r_c): negative when that product rounds up
                    sig = next((s for s in sigmas if _rounded_product_error(s, rt[cpos]) > 0), None)
                    if sig is None:
                        continue
                    row[a] = row[cpos] = sig
                S[grp, i] = row
                cases.append((kind, grp, i, tok, (a, cpos)))
                made += 1
    fmt = enc.Format.make(d, list(bits), signs, ch, qjl_proj=S)
    return x[:, None, :], S, fmt, cases


def exact_sum(S_row: np.ndarray, r: np.ndarray) -> Fraction:
    return sum((Fraction(float(s)) * Fraction(float(v)) for s, v in zip(S_row, r)), Fraction(0))


def fused_chain(S_row: np.ndarray, r: np.ndarray) -> float:
    """z from +0 by j ascending with one rounding per step (a fused
    multiply-add), emulated exactly."""
    z = 0.0
    for s, v in zip(S_row, r):
        z = float(Fraction(z) + Fraction(float(s)) * Fraction(float(v)))
    return z


def python_chain(S_row: np.ndarray, r: np.ndarray) -> float:
    """The defined order in plain Python floats (IEEE binary64, no fusion)."""
    z = 0.0
    for s, v in zip(S_row, r):
        z = z + float(s) * float(v)
    return z
