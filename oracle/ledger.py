"""Byte ledger.

[D "System Invariants"]: storage bytes and metadata bytes are reported
separately, and a compression ratio must include norms, scales, zeros,
codebooks, transforms, recent windows and workspace.  [S "What it does"]
prints bits-only ratios (16/3.5 and 16/2.5); the ledger reports both the
bits-only ratio and the all-inclusive one.
"""
from __future__ import annotations

from .encode import Format, row_bytes
from .pages import tile_layout


def ledger(kfmt: Format, vfmt: Format, num_tokens: int, num_kv_heads: int, block_size: int,
           num_blocks: int, num_seqs: int = 0, max_blocks_per_seq: int = 0,
           workspace_bytes: int = 0, dense_bytes_per_value: int = 2, window_tokens: int = 0,
           window_capacity_tokens: int = 0):
    """Storage / metadata accounting for a K+V cache of num_tokens packed
    tokens held in a pool of num_blocks blocks, plus window_tokens tokens kept
    unquantised (boundary and recent tokens, dense_bytes_per_value bytes per
    value) in buffers with room for window_capacity_tokens tokens (default:
    exactly window_tokens)."""
    out = {}
    for name, f in (("k", kfmt), ("v", vfmt)):
        rb, _, tile = tile_layout(f, block_size)
        out[f"{name}_row_index_bytes"] = rb
        nn = 2 * f.num_groups * (2 if f.qjl else 1)   # vector norms (and residual norms)
        out[f"{name}_row_norm_bytes"] = nn
        out[f"{name}_row_bytes"] = rb + nn
        out[f"{name}_tile_bytes"] = tile
        out[f"{name}_pool_bytes"] = num_blocks * num_kv_heads * tile
        out[f"{name}_bits_per_channel"] = (sum(b * (f.head_dim // f.num_groups) for b in f.group_bits) / f.head_dim
                                           + (1 if f.qjl else 0))   # QJL: one sign bit per channel
        out[f"{name}_projection_bytes"] = 4 * f.num_groups * f.group_size ** 2 if f.qjl else 0
        out[f"{name}_codebook_bytes"] = sum(2 * (1 << b) for b in f.group_bits)
        out[f"{name}_signs_bytes"] = f.head_dim
        out[f"{name}_channel_list_bytes"] = f.head_dim if f.num_groups > 1 else 0
    d = kfmt.head_dim
    dense = 2 * (num_tokens + window_tokens) * num_kv_heads * d * dense_bytes_per_value
    packed_rows = num_tokens * num_kv_heads * (out["k_row_bytes"] + out["v_row_bytes"])
    cap = max(window_capacity_tokens, window_tokens)
    out["window_bytes"] = 2 * cap * num_kv_heads * d * dense_bytes_per_value
    storage = out["k_pool_bytes"] + out["v_pool_bytes"] + out["window_bytes"]
    meta = (out["k_codebook_bytes"] + out["v_codebook_bytes"] + out["k_signs_bytes"]
            + out["v_signs_bytes"] + out["k_channel_list_bytes"] + out["v_channel_list_bytes"]
            + out["k_projection_bytes"] + out["v_projection_bytes"]
            + 4 * num_seqs * max_blocks_per_seq + workspace_bytes)
    out.update(dense_bytes=dense, packed_row_bytes=packed_rows, storage_bytes=storage,
               metadata_bytes=meta,
               ratio_bits_only=16.0 / ((out["k_bits_per_channel"] + out["v_bits_per_channel"]) / 2),
               ratio_rows_with_norms=(dense / (packed_rows + out["window_bytes"])
                                      if packed_rows + out["window_bytes"] else float("nan")),
               ratio_all_inclusive=dense / (storage + meta) if storage else float("nan"))
    return out
