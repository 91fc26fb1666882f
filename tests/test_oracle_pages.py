"""Pins for the oracle's page writer and reader (slot -> block -> offset -> row)."""
import numpy as np
import pytest

from oracle import encode as enc
from oracle import pages as pg
from workloads import signs, channel_subset


def fmts():
    s = signs(0, 1, 128)
    k = enc.Format.make(128, [4], s)
    v = enc.Format.make(128, [2], s)
    hi = channel_subset(0, 3, 128, 64)
    lo = np.array(sorted(set(range(128)) - set(hi.tolist())))
    km = enc.Format.make(128, [4, 3], s, np.concatenate([hi, lo]))
    k64 = enc.Format.make(64, [4], signs(0, 1, 64))
    return k, v, km, k64


def test_tile_layout_closed_forms():
    k, v, km, k64 = fmts()
    assert pg.tile_layout(k, 16) == (64, 1024, 1056)
    assert pg.tile_layout(v, 16) == (32, 512, 544)
    assert pg.tile_layout(km, 16) == (56, 896, 960)
    assert pg.tile_layout(k64, 16) == (32, 512, 544)


def test_write_places_rows_at_slot_block_offset():
    """A hand-built slot list: each row lands at block = slot // 16,
    offset = slot % 16 and nothing else in the pool changes."""
    k, _, _, _ = fmts()
    bs, H, nb = 16, 2, 5
    rb, noff, tile = pg.tile_layout(k, bs)
    pages = np.full((nb, H, tile), 0xA5, dtype=np.uint8)
    rng = np.random.default_rng(0)
    x = rng.standard_normal((4, H, 128))
    slots = np.array([0, 17, 79, 35])
    pg.write_pages(x, slots, pages, k, bs)
    idx, norms = enc.encode_rows(x, k)
    data = enc.pack_row(idx, k)
    touched = np.zeros_like(pages, dtype=bool)
    for i, s in enumerate(slots):
        b, o = divmod(int(s), bs)
        for h in range(H):
            np.testing.assert_array_equal(pages[b, h, o * rb:(o + 1) * rb], data[i, h])
            touched[b, h, o * rb:(o + 1) * rb] = True
            slot = 4 * (o % 4) + o // 4
            lo, hi = pages[b, h, noff + 2 * slot], pages[b, h, noff + 2 * slot + 1]
            assert int(lo) | (int(hi) << 8) == int(norms[i, h, 0])
            touched[b, h, noff + 2 * slot:noff + 2 * slot + 2] = True
    assert np.all(pages[~touched] == 0xA5)


def test_norm_slots_are_interleaved():
    """Slot of offset t is 4*(t%4) + t//4: a permutation of 0..15 in which
    offsets q, q+4, q+8, q+12 occupy four consecutive slots."""
    t = np.arange(16)
    sl = pg.norm_slot(t)
    assert sorted(sl.tolist()) == list(range(16))
    for q in range(4):
        assert sl[[q, q + 4, q + 8, q + 12]].tolist() == [4 * q, 4 * q + 1, 4 * q + 2, 4 * q + 3]
    assert sl.tolist()[:6] == [0, 4, 8, 12, 1, 5]


def test_two_group_norm_plane_is_group_major():
    _, _, km, _ = fmts()
    bs = 16
    rb, noff, tile = pg.tile_layout(km, bs)
    pages = np.zeros((2, 1, tile), dtype=np.uint8)
    x = np.random.default_rng(1).standard_normal((1, 1, 128))
    pg.write_pages(x, np.array([16 + 5]), pages, km, bs)
    _, norms = enc.encode_rows(x, km)
    for g in range(2):
        pos = noff + (g * bs + 4 * 1 + 1) * 2      # offset 5 -> slot 4*(5%4) + 5//4 = 5
        assert int(pages[1, 0, pos]) | (int(pages[1, 0, pos + 1]) << 8) == int(norms[0, 0, g])


def test_read_back_and_reconstruct():
    k, v, km, _ = fmts()
    bs, H = 16, 3
    rng = np.random.default_rng(2)
    n = 53
    bt = np.array([4, 0, 6, 2], dtype=np.int32)        # 4 blocks cover 53 tokens
    slots = bt[np.arange(n) // bs].astype(np.int64) * bs + np.arange(n) % bs
    for f in (k, v, km):
        rb, noff, tile = pg.tile_layout(f, bs)
        pages = np.zeros((7, H, tile), dtype=np.uint8)
        x = rng.standard_normal((n, H, 128))
        pg.write_pages(x, slots, pages, f, bs)
        idx, norms = enc.encode_rows(x, f)
        for h in range(H):
            ridx, rn = pg.read_rows(pages, bt[np.arange(n) // bs], np.arange(n) % bs, h, f, bs)
            for g in range(f.num_groups):
                np.testing.assert_array_equal(ridx[g], idx[g][:, h])
            np.testing.assert_array_equal(rn, norms[:, h])
            K = pg.reconstruct_sequence(pages, bt, n, h, f, bs)
            ref = enc.dequantize_rotated([i[:, h] for i in idx], norms[:, h], f)
            from oracle.rotation import inverse_rotate
            np.testing.assert_allclose(K, inverse_rotate(ref, f.signs), atol=1e-15)
            # reconstruction is close to the input (4-bit: ~10% relative)
            rel = np.linalg.norm(K - x[:, h], axis=1) / np.linalg.norm(x[:, h], axis=1)
            assert np.all(rel < {4: 0.2, 2: 0.55}[max(f.group_bits)])


def test_write_errors():
    k, _, _, _ = fmts()
    bs = 16
    _, _, tile = pg.tile_layout(k, bs)
    pages = np.zeros((2, 1, tile), dtype=np.uint8)
    x = np.zeros((2, 1, 128))
    with pytest.raises(IndexError):
        pg.write_pages(x, np.array([0, 32]), pages, k, bs)
    with pytest.raises(IndexError):
        pg.write_pages(x, np.array([-1, 3]), pages, k, bs)
    with pytest.raises(ValueError):
        pg.write_pages(x, np.array([3, 3]), pages, k, bs)
    with pytest.raises(ValueError):
        pg.write_pages(np.zeros((2, 1, 64)), np.array([0, 1]), pages, k, bs)
    with pytest.raises(IndexError):
        pg.reconstruct_sequence(pages, np.array([0, 5]), 20, 0, k, bs)


def test_v_lane_major_closed_form():
    """V pages with row bytes a multiple of 16 are lane-major: with
    c = row_bytes / 16, byte b of row t is at ((16*(t%4) + b//c)*4 + t//4)*c + b%c.
    Hand-computed spots for the 2-bit d=128 format (c = 2)."""
    _, v, _, _ = fmts()
    assert pg.lane_chunk(v, "v") == 2 and pg.lane_chunk(v, "k") == 0
    rb = 32
    pos = pg.row_positions(rb, [0, 5, 15], 2)
    assert pos[0, 0] == 0 and pos[0, 1] == 1 and pos[0, 2] == 8     # row 0: run 0, then run 1
    assert pos[1, 7] == 155                                         # run 19 at 152, row 1 of it, byte 1
    assert pos[2, 31] == ((16 * 3 + 15) * 4 + 3) * 2 + 1            # last byte of the plane
    assert pos[2, 31] == 16 * rb - 1


@pytest.mark.parametrize("rb", [16, 32, 48, 64])
def test_v_lane_major_is_a_permutation_with_runs(rb):
    """Every byte of the index plane is used once, and run 16q+j holds bytes
    [c*j, c*(j+1)) of rows q, q+4, q+8, q+12 in order."""
    c = rb // 16
    pos = pg.row_positions(rb, np.arange(16), c)
    assert sorted(pos.ravel().tolist()) == list(range(16 * rb))
    for q in range(4):
        for j in range(16):
            run = pos[[q, q + 4, q + 8, q + 12]][:, c * j:c * (j + 1)].ravel()
            assert run.tolist() == list(range((16 * q + j) * 4 * c, (16 * q + j + 1) * 4 * c))


def test_v_two_group_octet_runs_closed_form():
    """Two-group V pages: group g's bytes in a sub-plane at 16 x its byte
    offset in a row; octet o (b_g bytes, 8 indices) of row t in run
    (m/8)(t%4) + o of 4 b_g bytes, at place t//4.  Hand-computed spots for
    the 4+3-bit d=128 format (m = 64: group 0 bytes 0-31, group 1 bytes
    32-55)."""
    _, _, km, _ = fmts()
    pos = pg.index_positions(km, "v", [0, 5, 15])
    assert pos[0, 0] == 0 and pos[0, 3] == 3 and pos[0, 4] == 16      # row 0: octet 0 in run 0, octet 1 in run 1
    assert pos[1, 9] == (8 * 1 + 2) * 16 + 1 * 4 + 1 == 165            # row 5, group 0 octet 2 byte 1
    assert pos[0, 32] == 16 * 32                                       # group 1 sub-plane starts at 512
    assert pos[1, 32 + 7] == 512 + (8 * 1 + 2) * 12 + 1 * 3 + 1        # row 5, group 1 octet 2 byte 1
    assert pos[2, 55] == 895 == 16 * 56 - 1                            # last byte of the plane
    # K pages of the same format keep whole rows
    assert pg.index_positions(km, "k", [5])[0].tolist() == list(range(5 * 56, 6 * 56))


@pytest.mark.parametrize("bits,d", [([4, 3], 128), ([3, 2], 128), ([4, 3], 64), ([3, 2], 64), ([4, 2], 128)])
def test_v_two_group_octet_runs_permutation(bits, d):
    """Every byte of the index plane is used once, and each run holds one
    octet of rows q, q+4, q+8, q+12 in that order."""
    f = enc.Format.make(d, bits, np.ones(d, dtype=np.int8), np.arange(d))
    m = d // 2
    pos = pg.index_positions(f, "v", np.arange(16))
    rb = enc.row_bytes(f)
    assert sorted(pos.ravel().tolist()) == list(range(16 * rb))
    base = 0
    for b in bits:
        for q in range(4):
            for o in range(m // 8):
                cols = [base + o * b + k for k in range(b)]
                run = pos[[q, q + 4, q + 8, q + 12]][:, cols].ravel()
                start = 16 * base + ((m // 8) * q + o) * 4 * b
                assert run.tolist() == list(range(start, start + 4 * b))
        base += m * b // 8


def test_v_pages_roundtrip_and_other_formats_stay_row_major():
    """Rows written with role v read back with role v; a V format whose row
    bytes are not a multiple of 16 keeps the row-major plane."""
    _, v, km, _ = fmts()
    bs, H, nb = 16, 2, 3
    rng = np.random.default_rng(3)
    x = rng.standard_normal((20, H, 128))
    slots = rng.permutation(nb * bs)[:20]
    for f in (v, km):
        _, _, tile = pg.tile_layout(f, bs)
        pages = np.full((nb, H, tile), 0xA5, dtype=np.uint8)
        pg.write_pages(x, slots, pages, f, bs, "v")
        idx, norms = enc.encode_rows(x, f)
        for h in range(H):
            ridx, rn = pg.read_rows(pages, slots // bs, slots % bs, h, f, bs, "v")
            for g in range(f.num_groups):
                np.testing.assert_array_equal(ridx[g], idx[g][:, h])
            np.testing.assert_array_equal(rn, norms[:, h])
    assert pg.lane_chunk(km, "v") == 0   # 56-byte rows: two groups, octet runs
    # the row-major reader sees a lane-major plane as different bytes
    _, _, tile = pg.tile_layout(v, bs)
    pages = np.zeros((nb, H, tile), dtype=np.uint8)
    pg.write_pages(x, slots, pages, v, bs, "v")
    k_view, _ = pg.read_rows(pages, slots // bs, slots % bs, 0, v, bs, "k")
    assert not np.array_equal(k_view[0], enc.encode_rows(x, v)[0][0][:, 0])
