"""Persistent uint8 pages: slot mapping, block tables, tile layout.

[D "Serving Route Design"]: a token slot maps to a physical block and an
offset, block = slot // block_size and offset = slot % block_size, then to
the packed row bytes; packed rows are written into persistent pages and
read back through block tables.  [D "Data Ownership"]: the page cache owns
vLLM-style uint8 pages.  [D "Error Model"]: slots outside the allocated
pages are IndexErrors.

Layout (the pages fix slot -> block -> offset -> row only; the arrangement
inside a tile is this implementation's reading): pages are [num_blocks][num_kv_heads][tile].
A tile holds the index plane of block_size packed rows followed by the norm
plane, fp16 little-endian, group-major, with the 16 rows of a block in
interleaved slots: the norm of group g for the row at in-block offset t sits
at block_size*row_bytes + (g*block_size + norm_slot(t))*2, where
norm_slot(t) = 4*(t % 4) + t // 4.  The tile is padded to a multiple of 16
bytes.  Only block_size 16 is defined.

Index plane: in K pages ("k" role) row t occupies bytes
[t*row_bytes, (t+1)*row_bytes).  In V pages ("v" role), when row_bytes is a
multiple of 16, the plane is lane-major: with c = row_bytes / 16, byte b of
row t sits at ((16*(t % 4) + b // c)*4 + t // 4)*c + b % c, i.e. 64 runs of
4*c bytes, run 16*q + j holding bytes [c*j, c*(j+1)) of rows q, q+4, q+8,
q+12 in that order.  Two-group V formats (the recipe row applied to V)
store each group's bytes in a sub-plane of its own, group g's at 16 times
the group's byte offset in a row: a row's m * b_g bits of group g fall into
m / 8 octets of b_g bytes (8 indices each), and octet o of row t sits in
run (m / 8) * (t % 4) + o of 4 * b_g bytes, at place t // 4.  Other V
formats use the K layout.

QJL K formats (oracle/qjl.py): each row's index bytes are its MSE indices
followed by its sign string (oracle/qjl.py), and the norm plane holds the
vector norms as above followed by the residual norms in the same
arrangement: residual norm of group g at block_size*row_bytes +
((G + g)*block_size + norm_slot(t))*2.  QJL is a K stage only.
"""
from __future__ import annotations

import numpy as np

from .encode import Format, quantize_rotated, pack_row, unpack_row, dequantize_rotated, row_bytes, mse_row_bytes
from .rotation import rotate, inverse_rotate
from . import qjl as _qjl


def norm_slot(t):
    """Slot of in-block offset t (0..15) in a norm plane."""
    return 4 * (np.asarray(t) % 4) + np.asarray(t) // 4


def lane_chunk(fmt: Format, role: str) -> int:
    """Bytes per lane run of the V index plane (0: rows are contiguous)."""
    if role not in ("k", "v"):
        raise ValueError("role must be 'k' or 'v'")
    rb = row_bytes(fmt)
    return rb // 16 if role == "v" and rb % 16 == 0 else 0


def octet_run_positions(fmt: Format, t) -> np.ndarray:
    """Tile byte offsets of the index bytes of rows at in-block offsets t in
    a two-group V page (octet runs per group, see the module docstring):
    array [len(t), row_bytes]."""
    t = np.asarray(t, dtype=np.int64).reshape(-1, 1)
    m = fmt.group_size
    cols, base = [], 0
    for b in fmt.group_bits:
        nbytes = m * b // 8
        j = np.arange(nbytes, dtype=np.int64)[None, :]
        o, q = j // b, j % b
        cols.append(16 * base + ((m // 8) * (t % 4) + o) * 4 * b + (t // 4) * b + q)
        base += nbytes
    return np.concatenate(cols, axis=1)


def index_positions(fmt: Format, role: str, t) -> np.ndarray:
    """Tile byte offsets of index bytes 0..row_bytes-1 of the rows at in-block
    offsets t for the page role ("k" or "v"): array [len(t), row_bytes]."""
    if role == "v" and fmt.num_groups == 2 and not fmt.qjl:
        return octet_run_positions(fmt, t)
    return row_positions(row_bytes(fmt), t, lane_chunk(fmt, role))


def row_positions(rb: int, t, chunk: int) -> np.ndarray:
    """Tile byte offsets of bytes 0..rb-1 of the rows at in-block offsets t:
    array [len(t), rb]."""
    t = np.asarray(t, dtype=np.int64).reshape(-1, 1)
    b = np.arange(rb, dtype=np.int64)[None, :]
    if chunk == 0:
        return t * rb + b
    return ((16 * (t % 4) + b // chunk) * 4 + t // 4) * chunk + b % chunk


def tile_layout(fmt: Format, block_size: int):
    """(row_idx_bytes, norm_plane_offset, tile_bytes)."""
    if block_size != 16:
        raise ValueError("block_size must be 16")
    rb = row_bytes(fmt)
    norm_off = block_size * rb
    raw = norm_off + block_size * fmt.num_groups * 2 * (2 if fmt.qjl else 1)
    tile = (raw + 15) // 16 * 16
    return rb, norm_off, tile


def write_pages(x: np.ndarray, slot_mapping: np.ndarray, pages: np.ndarray, fmt: Format,
                block_size: int, role: str = "k") -> None:
    """Quantise rows x[T, H, d] and store them in pages[num_blocks, H, tile]
    at the rows named by slot_mapping[T] (role "k" or "v" picks the index
    plane layout).  Bytes outside the written rows and norm slots are left
    untouched."""
    x = np.asarray(x)
    slots = np.asarray(slot_mapping, dtype=np.int64)
    T, H, d = x.shape
    nb = pages.shape[0]
    rb, norm_off, tile = tile_layout(fmt, block_size)
    if role not in ("k", "v"):
        raise ValueError("role must be 'k' or 'v'")
    if pages.dtype != np.uint8 or pages.shape[1:] != (H, tile):
        raise ValueError("page pool shape does not match the format")
    if fmt.qjl and role != "k":
        raise ValueError("the QJL stage is defined for K formats only")
    if slots.shape != (T,):
        raise ValueError("slot_mapping length differs from the number of tokens")
    bad = (slots < 0) | (slots >= nb * block_size)
    if np.any(bad):
        i = int(np.nonzero(bad)[0][0])
        raise IndexError(f"slot {int(slots[i])} of token {i} outside [0, {nb * block_size})")
    if len(np.unique(slots)) != T:
        raise ValueError("duplicate slots in one write")
    blk = slots // block_size
    off = slots % block_size
    if x.shape[-1] != fmt.head_dim:
        raise ValueError("row length differs from head_dim")
    w = rotate(np.asarray(x, dtype=np.float64), fmt.signs)
    idx_groups, norms = quantize_rotated(w, fmt)          # [T, H, m] per group, [T, H, G]
    data = pack_row(idx_groups, fmt)                      # [T, H, mse bytes]
    if fmt.qjl:
        sbits, gam = _qjl.residual_fields(w, idx_groups, norms, fmt)
        data = np.concatenate([data, _qjl.pack_signs(sbits)], axis=-1)
        norms = np.concatenate([norms, gam], axis=-1)     # [T, H, 2G]: vector norms, residual norms
    pos_rows = index_positions(fmt, role, off)            # [T, rb]
    for h in range(H):
        for b in range(rb):
            pages[blk, h, pos_rows[:, b]] = data[:, h, b]
        for g in range(norms.shape[-1]):
            pos = norm_off + (g * block_size + norm_slot(off)) * 2
            pages[blk, h, pos] = (norms[:, h, g] & 0xFF).astype(np.uint8)
            pages[blk, h, pos + 1] = (norms[:, h, g] >> 8).astype(np.uint8)


def read_rows(pages: np.ndarray, blocks: np.ndarray, offsets: np.ndarray, head: int, fmt: Format,
              block_size: int, role: str = "k"):
    """Unpack the rows at (blocks[i], offsets[i]) of one kv head ->
    (index arrays per group, fp16 norm bits [n, G]); QJL formats also give
    (sign bits [n, G, m], residual-norm bits [n, G])."""
    rb, norm_off, tile = tile_layout(fmt, block_size)
    blocks = np.asarray(blocks, dtype=np.int64)
    offsets = np.asarray(offsets, dtype=np.int64)
    t = pages[blocks, head]                                          # [n, tile]
    cols = index_positions(fmt, role, offsets)
    data = np.take_along_axis(t, cols, axis=1)
    idx = unpack_row(data, fmt)
    G = fmt.num_groups
    nn = 2 * G if fmt.qjl else G
    norms = np.empty((len(blocks), nn), dtype=np.uint16)
    for g in range(nn):
        pos = norm_off + (g * block_size + norm_slot(offsets)) * 2
        lo = t[np.arange(len(blocks)), pos].astype(np.uint16)
        hi = t[np.arange(len(blocks)), pos + 1].astype(np.uint16)
        norms[:, g] = lo | (hi << 8)
    if not fmt.qjl:
        return idx, norms
    sbits = _qjl.unpack_signs(data[:, mse_row_bytes(fmt):], G, fmt.group_size)
    return idx, norms[:, :G], sbits, norms[:, G:]


def reconstruct_sequence(pages: np.ndarray, block_table_row: np.ndarray, ctx: int, head: int,
                         fmt: Format, block_size: int, rotated: bool = False, role: str = "k") -> np.ndarray:
    """Dense float64 K or V rows [ctx, d] of one sequence and kv head, walked
    through its block table ([D "Diagnostic Route Design"]: dense
    reconstruction is a diagnostic, allowed for validation only).  With
    rotated=True the rows stay in the rotated domain."""
    t = np.arange(ctx)
    bt = np.asarray(block_table_row, dtype=np.int64)
    blocks = bt[t // block_size]
    if np.any(blocks < 0) or np.any(blocks >= pages.shape[0]):
        raise IndexError("block table entry outside the page pool")
    fields = read_rows(pages, blocks, t % block_size, head, fmt, block_size, role)
    y = dequantize_rotated(fields[0], fields[1], fmt)
    if fmt.qjl:   # the effective key: MSE reconstruction plus the sketch's term
        y = y + _qjl.correction_rotated(fields[2], fields[3], fmt)
    return y if rotated else inverse_rotate(y, fmt.signs)
