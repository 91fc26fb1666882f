"""Pins for the byte ledger: closed forms and the server README's table."""
import json
import os

import numpy as np
import pytest

from oracle import encode as enc
from oracle.ledger import ledger
from workloads import signs, channel_subset

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _f(bits, d=128):
    s = signs(0, 1, d)
    if len(bits) == 2:
        hi = channel_subset(0, 3, d, d // 2)
        lo = np.array(sorted(set(range(d)) - set(hi.tolist())))
        return enc.Format.make(d, bits, s, np.concatenate([hi, lo]))
    return enc.Format.make(d, bits, s)


def test_row_and_tile_bytes():
    L = ledger(_f([4]), _f([2]), 100, 8, 16, 10)
    assert L["k_row_bytes"] == 66 and L["v_row_bytes"] == 34
    assert L["k_tile_bytes"] == 1056 and L["v_tile_bytes"] == 544
    L = ledger(_f([4, 3]), _f([2]), 100, 8, 16, 10)
    assert L["k_row_bytes"] == 60 and L["k_tile_bytes"] == 960
    assert L["k_bits_per_channel"] == 3.5
    L = ledger(_f([4], 64), _f([4], 64), 100, 1, 16, 10)
    assert L["k_row_bytes"] == 34 and L["k_tile_bytes"] == 544


def test_bits_only_ratio_reproduces_server_table():
    """The README's ratios are 16 / bits (index bits only)."""
    g = json.load(open(os.path.join(GOLDEN, "server_table.json")))
    for key in ("tq35", "tq25"):
        bits = g["bits_per_channel"][key]
        ratio = 16.0 / bits
        assert round(ratio, g["ratio_print_digits"]) == pytest.approx(g["compression_ratio"][key])
        # equivalent context scales with the ratio from the fp16 figure
        assert abs(g["equivalent_context_k"]["full"] * ratio - g["equivalent_context_k"][key]) < 1.0
    L = ledger(_f([4, 3]), _f([4, 3]), 1000, 8, 16, 63)
    assert L["ratio_bits_only"] == pytest.approx(16 / 3.5)


def test_norm_inclusive_ratios_are_lower():
    """Counting norms, the per-token ratio vs bf16 drops below the bits-only
    figure: 512/132 (K4/V4), 512/100 (K4/V2), 512/94 (K3.5/V2), 512/120
    (K3.5/V3.5)."""
    cases = [([4], [4], 512 / 132), ([4], [2], 512 / 100), ([4, 3], [2], 512 / 94),
             ([4, 3], [4, 3], 512 / 120)]
    for kb, vb, ratio in cases:
        T, H = 4096, 8
        L = ledger(_f(kb), _f(vb), T, H, 16, T // 16, num_seqs=1, max_blocks_per_seq=T // 16)
        assert L["ratio_rows_with_norms"] == pytest.approx(ratio)
        assert L["ratio_all_inclusive"] < L["ratio_rows_with_norms"] < L["ratio_bits_only"] + 1e-12
        # metadata lowers it only a little
        assert L["ratio_all_inclusive"] > 0.999 * L["dense_bytes"] / L["storage_bytes"] - 1e-9


def test_dense_window_counts_in_storage():
    """Tokens kept unquantised (boundary + recent window) cost their full
    bf16 bytes in storage and count in the dense baseline: with a window of
    W tokens next to T packed ones (K4/V4, 132 B per packed token-head), the
    rows-with-norms ratio is 512 (T + W) / (132 T + 512 W)."""
    T, H, W = 4096, 8, 132
    L0 = ledger(_f([4]), _f([4]), T, H, 16, T // 16)
    L = ledger(_f([4]), _f([4]), T, H, 16, T // 16, window_tokens=W)
    assert L["window_bytes"] == 2 * W * H * 128 * 2
    assert L["storage_bytes"] == L0["storage_bytes"] + L["window_bytes"]
    assert L["dense_bytes"] == 2 * (T + W) * H * 128 * 2
    assert L["ratio_rows_with_norms"] == pytest.approx(512 * (T + W) / (132 * T + 512 * W))
    assert L["ratio_rows_with_norms"] < L0["ratio_rows_with_norms"]
    # a ring buffer with spare room is charged for its capacity
    Lc = ledger(_f([4]), _f([4]), T, H, 16, T // 16, window_tokens=W, window_capacity_tokens=256)
    assert Lc["window_bytes"] == 2 * 256 * H * 128 * 2


def test_qjl_row_bytes_and_bits():
    """The QJL reading of the 3.5-bit recipe: 3 + 2 MSE bits and one sign bit
    per channel; per row 40 + 16 index bytes, 2 vector + 2 residual norms."""
    import numpy as np
    from oracle import encode as enc
    from oracle.ledger import ledger
    s = np.ones(128, np.int8)
    ch = np.concatenate([np.arange(0, 128, 2), np.arange(1, 128, 2)])
    k = enc.Format.make(128, [3, 2], s, ch, qjl_proj=np.zeros((2, 64, 64), np.float32))
    v = enc.Format.make(128, [2], s)
    L = ledger(k, v, num_tokens=16, num_kv_heads=1, block_size=16, num_blocks=1)
    assert L["k_row_bytes"] == 56 + 8 and L["k_tile_bytes"] == 1024
    assert L["k_bits_per_channel"] == 3.5
    assert L["k_projection_bytes"] == 2 * 64 * 64 * 4
