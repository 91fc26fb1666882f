"""QJL residual stage of a channel group (a reading).  Test infrastructure.

[D "Recipe Strategy"]: each group of a recipe row stores
[MSE indices][QJL signs][vector norm][residual norm].  The pages name the
fields and nothing more.  The reading taken here is the quantised
Johnson-Lindenstrauss transform as published with TurboQuant's
inner-product quantiser: after the MSE stage, the group's residual is
projected by an m x m matrix of i.i.d. standard normal entries (passed in,
seeded by the caller), the signs of the projection are kept (one bit per
output) together with the residual's norm, and the score of a query adds
the sketch's unbiased estimate of <q, residual>.

Per row, group G of m channels (ascending), after the MSE stage of
oracle/encode.py (rotated row w = H (s * x), stored fp16 norm n_G, indices
idx_j), all in float64:

  a_G   = n_G * sqrt(d / m)                  the level scale in w units
  r_j   = w_j - a_G * c[idx_j]               residual in w units (j in G)
  ssr   = tree_sum(r_j^2)                    same pinned tree as the norm
  gamma = fp16_rne(sqrt(ssr / d))            = |e|, e = r / sqrt(d) (y units)
  z_i   = sum_j S_G[i, j] r_j                (S_G float32 entries, exact in fp64),
          evaluated in one fixed order: z = +0, then for j = 0, 1, ..., m-1
          (ascending position in the group) z = z + S_G[i, j] * r_j with the
          product rounded to fp64 and then the sum rounded (no fused
          multiply-add).  The order fixes the sign of a sum whose exact value
          lies within rounding of zero.
  bit_i = 1 if z_i < 0 else 0                (bit 1 stands for sign -1)

Decoding (rotated, normalised domain, q~ = H (s * q) / sqrt(d)):
  q~ . k  ~  sum_G [ n_G / sqrt(m) * sum_j q~_j c[idx_j]
                     + sqrt(pi / 2) / m * gamma_G * sum_i (S_G q~_G)_i (1 - 2 bit_i) ]
which is q~ . k_eff with the effective key
  k_eff_G = y_hat_G + sqrt(pi / 2) / m * gamma_G * S_G^T sigma_G.
For s ~ N(0, I): E[(s . q) sign(s . e)] = sqrt(2 / pi) (q . e) / |e|, so
the second term has mean gamma (q . e) / |e| (= q . e up to the fp16
rounding of gamma) and variance (pi / 2) gamma^2 (|q|^2 - (2 / pi)(q . e)^2 / |e|^2) / m.
"""
from __future__ import annotations

import math

import numpy as np

from .codebook import f64_to_f16_bits
from .encode import Format, tree_sum


def project(r: np.ndarray, S: np.ndarray) -> np.ndarray:
    """z[..., i] = sum_j S[i, j] r[..., j] in the order the stage defines:
    start from +0 and add the terms for j = 0, 1, ... in turn, each product
    rounded to fp64, then each sum rounded (numpy's elementwise multiply and
    add, never fused)."""
    r = np.asarray(r, dtype=np.float64)
    S = np.asarray(S, dtype=np.float64)          # float32 entries: exact
    z = np.zeros(r.shape[:-1] + (S.shape[0],))
    for j in range(S.shape[1]):
        z = z + r[..., j:j + 1] * S[:, j]
    return z


def residuals(w: np.ndarray, idx_groups, norm_bits: np.ndarray, fmt: Format):
    """Per group, the MSE residual r_j = w_j - a_G c[idx_j] of rotated rows
    w[..., d] in w units, [..., m] in the group's listed channel order."""
    w = np.asarray(w, dtype=np.float64)
    d, m = fmt.head_dim, fmt.group_size
    kappa = math.sqrt(d / m)
    norms = np.asarray(norm_bits, dtype=np.uint16).view(np.float16).astype(np.float64)
    out = []
    for g, ch in enumerate(fmt.groups()):
        c = fmt.codebooks[g].astype(np.float64)
        a = norms[..., g] * kappa
        out.append(w[..., ch] - a[..., None] * c[idx_groups[g]])
    return out


def residual_fields(w: np.ndarray, idx_groups, norm_bits: np.ndarray, fmt: Format):
    """QJL fields of rotated rows w[..., d] whose MSE stage gave idx_groups
    (list of [..., m]) and norm_bits [..., G] -> (sign bits uint8
    [..., G, m], residual-norm fp16 bits uint16 [..., G])."""
    if not fmt.qjl:
        raise ValueError("format has no QJL stage")
    d = fmt.head_dim
    bits, gam = [], []
    for g, r in enumerate(residuals(w, idx_groups, norm_bits, fmt)):
        ssr = tree_sum(r * r)
        gam.append(f64_to_f16_bits(np.sqrt(ssr / d)).astype(np.uint16))
        z = project(r, fmt.qjl_proj[g])
        bits.append((z < 0).astype(np.uint8))
    return np.stack(bits, axis=-2), np.stack(gam, axis=-1)


def pack_signs(bits: np.ndarray) -> np.ndarray:
    """Sign bits [..., G, m] -> bytes [..., G*m/8]: group 0 first, output i
    of a group at bit i of the group's string (LSB-first)."""
    bits = np.asarray(bits, dtype=np.uint8)
    flat = bits.reshape(bits.shape[:-2] + (bits.shape[-2] * bits.shape[-1],))
    return np.packbits(flat, axis=-1, bitorder="little")


def unpack_signs(data: np.ndarray, num_groups: int, m: int) -> np.ndarray:
    bits = np.unpackbits(np.asarray(data, dtype=np.uint8), axis=-1, bitorder="little")[..., :num_groups * m]
    return bits.reshape(bits.shape[:-1] + (num_groups, m))


def correction_rotated(bits: np.ndarray, gamma_bits: np.ndarray, fmt: Format) -> np.ndarray:
    """The sketch's part of the effective rotated key, [..., d]:
    sqrt(pi / 2) / m * gamma_G * S_G^T sigma_G on the channels of G."""
    gam = np.asarray(gamma_bits, dtype=np.uint16).view(np.float16).astype(np.float64)
    m = fmt.group_size
    out = np.zeros(gam.shape[:-1] + (fmt.head_dim,))
    for g, ch in enumerate(fmt.groups()):
        sigma = 1.0 - 2.0 * np.asarray(bits[..., g, :], dtype=np.float64)
        S = fmt.qjl_proj[g].astype(np.float64)
        out[..., ch] = (math.sqrt(math.pi / 2) / m) * gam[..., g:g + 1] * (sigma @ S)   # (S^T sigma)_j
    return out


def score_terms(q_rot: np.ndarray, idx_groups, norm_bits, bits, gamma_bits, fmt: Format):
    """Per-group score terms of a normalised rotated query q~[d] against
    encoded rows: (MSE part [..., G], sketch part [..., G]).  The estimator
    in the form a decoder evaluates: the query is projected once per group
    (u = S_G q~_G) and dotted with the signs."""
    q_rot = np.asarray(q_rot, dtype=np.float64)
    norms = np.asarray(norm_bits, dtype=np.uint16).view(np.float16).astype(np.float64)
    gam = np.asarray(gamma_bits, dtype=np.uint16).view(np.float16).astype(np.float64)
    m = fmt.group_size
    mse, sk = [], []
    for g, ch in enumerate(fmt.groups()):
        c = fmt.codebooks[g].astype(np.float64)
        mse.append(norms[..., g] / math.sqrt(m) * (c[idx_groups[g]] @ q_rot[ch]))
        u = fmt.qjl_proj[g].astype(np.float64) @ q_rot[ch]
        sigma = 1.0 - 2.0 * np.asarray(bits[..., g, :], dtype=np.float64)
        sk.append(math.sqrt(math.pi / 2) / m * gam[..., g] * (sigma @ u))
    return np.stack(mse, axis=-1), np.stack(sk, axis=-1)
