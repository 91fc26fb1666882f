"""Quantise-on-write of one row: rotate, group norms, nearest level, pack.

[D "Recipe Strategy"]: a row stores, per channel group, its quantiser
indices and a vector norm ("[MSE indices] ... [vector norm]"); the
high/low channel groups come from metadata, never from a runtime guess
[D "System Invariants"].  [D "Format Strategy"]: K and V formats are
independent.  The QJL sign and residual-norm fields of the recipe row are
an option of a K format (oracle/qjl.py); the steps below are
the MSE stage every format has.

Per row x (length d) and per group G of m channels (listed ascending):

  1. w = H (s * x)                                  (rotation, float64)
  2. ss_G = tree sum of w_j^2 over G                (pinned pairwise tree)
  3. stored norm n_G = fp16_rne(sqrt(ss_G / d))     (= |y_G|, y = w / sqrt d)
  4. r_G = sqrt(ss_G / m);  T_i = fl(t_i * r_G)     (thresholds in w units)
     idx_j = #{ i : T_i < w_j }                      (nearest level of w_j / r_G)
  5. pack idx LSB-first, groups concatenated.

A group with ss_G == 0 stores norm +0 and every index L/2 - 1 (a reading:
the pages do not cover an all-zero group).
Reconstruction of channel j in G: y_j = n_G * c[idx_j] / sqrt(m).
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence

import numpy as np

from .codebook import codebook_f16, thresholds_f64, f64_to_f16_bits
from .rotation import rotate


@dataclasses.dataclass
class Format:
    """One tensor's format (K and V each have their own)."""
    head_dim: int
    group_bits: List[int]
    group_channels: np.ndarray          # int [d]: group 0 ascending, then group 1 ascending
    codebooks: List[np.ndarray]         # float16 [2^bits] per group, ascending
    signs: np.ndarray                   # int8 [d] of +-1
    qjl_proj: Optional[np.ndarray] = None   # float32 [num_groups, m, m]: QJL projection per group

    @staticmethod
    def make(head_dim: int, group_bits: Sequence[int], signs: np.ndarray,
             group_channels: Optional[np.ndarray] = None, qjl_proj: Optional[np.ndarray] = None) -> "Format":
        ng = len(group_bits)
        if group_channels is None:
            if ng != 1:
                raise ValueError("two groups need a channel list")
            group_channels = np.arange(head_dim)
        f = Format(head_dim, list(group_bits), np.asarray(group_channels, dtype=np.int64),
                   [codebook_f16(b) for b in group_bits], np.asarray(signs, dtype=np.int8),
                   None if qjl_proj is None else np.asarray(qjl_proj, dtype=np.float32))
        f.validate()
        return f

    @property
    def qjl(self) -> bool:
        return self.qjl_proj is not None

    @property
    def num_groups(self) -> int:
        return len(self.group_bits)

    @property
    def group_size(self) -> int:
        return self.head_dim // self.num_groups

    def groups(self):
        m = self.group_size
        return [self.group_channels[g * m:(g + 1) * m] for g in range(self.num_groups)]

    def validate(self):
        """[D "Error Model"]: bad shapes, bit widths and malformed metadata
        are ValueErrors."""
        d = self.head_dim
        if d not in (64, 128):
            raise ValueError(f"head_dim {d} not in (64, 128)")
        if self.num_groups not in (1, 2):
            raise ValueError("one or two channel groups")
        for b in self.group_bits:
            if b not in (2, 3, 4):
                raise ValueError(f"unsupported bit width {b}")
        ch = np.asarray(self.group_channels)
        if ch.shape != (d,) or sorted(ch.tolist()) != list(range(d)):
            raise ValueError("channel list must be a permutation of 0..d-1")
        for grp in self.groups():
            if np.any(np.diff(grp) <= 0):
                raise ValueError("channels must ascend within a group")
        if self.num_groups == 1 and not np.array_equal(ch, np.arange(d)):
            raise ValueError("a single group lists channels in natural order")
        s = np.asarray(self.signs)
        if s.shape != (d,) or not np.all(np.abs(s) == 1):
            raise ValueError("signs must be +-1 of length d")
        for cb, b in zip(self.codebooks, self.group_bits):
            c = np.asarray(cb, dtype=np.float16).astype(np.float64)
            if c.shape != (1 << b,) or not np.all(np.isfinite(c)) or np.any(np.diff(c) <= 0):
                raise ValueError("codebook must be 2^bits finite, strictly ascending levels")
        if self.qjl_proj is not None:
            S = np.asarray(self.qjl_proj)
            m = self.group_size
            if S.dtype != np.float32 or S.shape != (self.num_groups, m, m) or not np.all(np.isfinite(S)):
                raise ValueError("QJL projection must be finite float32 [num_groups, m, m]")


def tree_sum(v: np.ndarray) -> np.ndarray:
    """Pairwise sum along the last axis (length a power of two): level h adds
    element k+h into element k for k = 0 mod 2h.  Adjacent pairs first."""
    v = np.asarray(v, dtype=np.float64)
    while v.shape[-1] > 1:
        v = v[..., 0::2] + v[..., 1::2]
    return v[..., 0]


def mse_row_bytes(fmt: Format) -> int:
    """Bytes of a row's packed MSE indices (all groups)."""
    return sum(fmt.group_size * b for b in fmt.group_bits) // 8


def row_bytes(fmt: Format) -> int:
    """Index-plane bytes of a row: MSE indices, then (QJL formats) one sign
    bit per channel of every group."""
    return mse_row_bytes(fmt) + (fmt.head_dim // 8 if fmt.qjl else 0)


def encode_rows(x: np.ndarray, fmt: Format):
    """Encode rows x[..., d] -> (list of index arrays [..., m] per group,
    uint16 fp16 norm bits [..., num_groups])."""
    x = np.asarray(x, dtype=np.float64)
    if x.shape[-1] != fmt.head_dim:
        raise ValueError("row length differs from head_dim")
    return quantize_rotated(rotate(x, fmt.signs), fmt)


def quantize_rotated(w: np.ndarray, fmt: Format):
    """Steps 2-4 on an already rotated (unnormalised) row w[..., d]."""
    d = fmt.head_dim
    idx_out, norms = [], []
    for g, ch in enumerate(fmt.groups()):
        m = len(ch)
        wg = w[..., ch]
        ss = tree_sum(wg * wg)
        n16 = f64_to_f16_bits(np.sqrt(ss / d))
        r = np.sqrt(ss / m)
        t = thresholds_f64(fmt.codebooks[g])
        T = t * r[..., None]                                   # fl(t_i * r)
        idx = np.sum(T[..., None, :] < wg[..., :, None], axis=-1)
        L = 1 << fmt.group_bits[g]
        zero = ss == 0
        idx = np.where(zero[..., None], L // 2 - 1, idx)
        n16 = np.where(zero, np.uint16(0), n16)
        idx_out.append(idx.astype(np.int64))
        norms.append(n16.astype(np.uint16))
    return idx_out, np.stack(norms, axis=-1)


def pack_group(idx: np.ndarray, bits: int) -> np.ndarray:
    """Pack indices [..., m] LSB-first into a little-endian bit string of
    m*bits/8 bytes: index p occupies bits [p*bits, p*bits + bits)."""
    idx = np.asarray(idx, dtype=np.int64)
    if np.any(idx < 0) or np.any(idx >= (1 << bits)):
        raise ValueError("index out of range for bit width")
    bitarr = ((idx[..., :, None] >> np.arange(bits)) & 1).astype(np.uint8)
    flat = bitarr.reshape(idx.shape[:-1] + (idx.shape[-1] * bits,))
    return np.packbits(flat, axis=-1, bitorder="little")


def unpack_group(data: np.ndarray, bits: int, m: int) -> np.ndarray:
    data = np.asarray(data, dtype=np.uint8)
    bitarr = np.unpackbits(data, axis=-1, bitorder="little")[..., :m * bits]
    bitarr = bitarr.reshape(data.shape[:-1] + (m, bits)).astype(np.int64)
    return np.sum(bitarr << np.arange(bits), axis=-1)


def pack_row(idx_groups, fmt: Format) -> np.ndarray:
    """Row bytes: groups' bit strings concatenated, group 0 first (a reading:
    the pages give the field order of a group, not the bit order)."""
    return np.concatenate([pack_group(i, b) for i, b in zip(idx_groups, fmt.group_bits)], axis=-1)


def unpack_row(data: np.ndarray, fmt: Format):
    out, off = [], 0
    m = fmt.group_size
    for b in fmt.group_bits:
        nb = m * b // 8
        out.append(unpack_group(data[..., off:off + nb], b, m))
        off += nb
    return out


def dequantize_rotated(idx_groups, norm_bits: np.ndarray, fmt: Format) -> np.ndarray:
    """Rotated-domain reconstruction y_hat[..., d] (float64):
    y_j = n_G * c[idx_j] / sqrt(m) for channel j in group G."""
    norms = np.asarray(norm_bits, dtype=np.uint16).view(np.float16).astype(np.float64)
    lead = norms.shape[:-1]
    y = np.zeros(lead + (fmt.head_dim,), dtype=np.float64)
    m = fmt.group_size
    for g, ch in enumerate(fmt.groups()):
        c = fmt.codebooks[g].astype(np.float64)
        y[..., ch] = norms[..., g:g + 1] * c[idx_groups[g]] / np.sqrt(m)
    return y
