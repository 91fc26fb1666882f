"""CPU model of tq_decode_paged's balanced split of work over workgroups.

The decode kernel lays the work out as (sequence, kv-head group) segments,
sequence-major; a segment of nb > 0 blocks spans seg_cost + nb work
positions (a fixed charge for starting a piece, then one position per
block), and workgroup w takes the positions [w*R, (w+1)*R).  The blocks of
a segment that fall in a range form one piece.  With num_splits == 1 the
range ends are moved to segment starts so that no segment is ever split
(there is no workspace then).  This test re-derives that index arithmetic
in Python and checks the invariants the kernel relies on: every block
processed exactly once, at most P pieces per segment with piece indices in
[0, P) and equal to the kernel's piece count, no partial written when
P == 1.
"""
import math

import numpy as np
import pytest


def plan(ctx, NG, max_blocks, P, n_wg, seg_cost):
    cap = max_blocks * 16
    nb = [(min(max(int(c), 0), cap) + 15) // 16 for c in ctx]
    span = [n + seg_cost if n > 0 else 0 for n in nb]
    seg_start = {}
    pos = 0
    for s, n in enumerate(nb):
        for g in range(NG):
            if n:
                seg_start[(s, g)] = pos
            pos += span[s]
    W = pos
    R = max(1, -(-W // n_wg))
    if P > 1:
        R = max(R, -(-max_blocks // (P - 1)))

    def locate(x):
        for (s, g), st in seg_start.items():
            if st <= x < st + span[s]:
                return s, g, x - st
        raise AssertionError

    def snap(x):
        if x >= W:
            return W
        s, g, off = locate(x)
        return x if off == 0 else x - off + span[s]

    pieces = []   # (wg, s, grp, b0, b1, whole, piece_index)
    for w in range(n_wg):
        r0, r1 = w * R, min(W, w * R + R)
        if P == 1:
            r0, r1 = snap(r0), snap(r1)
        x = r0
        while x < r1:
            s, g, off = locate(x)
            vb0 = x - off + seg_cost
            b0 = max(off - seg_cost, 0)
            b1 = min(nb[s], r1 - vb0)
            if b1 > b0:
                whole = P == 1 or vb0 // R == (vb0 + nb[s] - 1) // R
                pieces.append((w, s, g, b0, b1, whole, w - vb0 // R))
            x = vb0 + nb[s]
    return nb, seg_start, R, pieces


def piece_count(nb, seg_start, R, s, g, seg_cost):
    vb0 = seg_start[(s, g)] + seg_cost
    return (vb0 + nb[s] - 1) // R - vb0 // R + 1


CASES = [
    ([1, 17, 300, 1000], 2, 65, 1),
    ([1, 17, 300, 1000], 2, 65, 3),
    ([33, 0, 517], 2, 35, 4),
    ([700, 64], 2, 46, 5),
    ([5, 400], 3, 27, 2),
    ([1000, 16], 1, 65, 7),
    ([256], 1, 16, 1),
    ([131072], 8, 8192, 64),
    ([32768] * 8, 8, 2048, 16),
]


@pytest.mark.parametrize("ctx,NG,max_blocks,P", CASES)
@pytest.mark.parametrize("n_wg", [512, 7, 1])
@pytest.mark.parametrize("seg_cost", [0, 16, 128])
def test_plan_invariants(ctx, NG, max_blocks, P, n_wg, seg_cost):
    n_wg = min(n_wg, len(ctx) * NG * max_blocks)
    nb, seg_start, R, pieces = plan(ctx, NG, max_blocks, P, n_wg, seg_cost)
    seen = {}
    per_seg = {}
    for (w, s, g, b0, b1, whole, k) in pieces:
        assert 0 <= b0 < b1 <= nb[s]
        for b in range(b0, b1):
            assert (s, g, b) not in seen
            seen[(s, g, b)] = w
        per_seg.setdefault((s, g), []).append((k, whole))
        if P == 1:
            assert whole and b0 == 0 and b1 == nb[s]
        else:
            assert 0 <= k < P
    assert len(seen) == sum(nb) * NG
    for (s, g), lst in per_seg.items():
        ks = [k for k, _ in lst]
        if P > 1:
            assert sorted(ks) == list(range(len(ks)))
            assert len(lst) == piece_count(nb, seg_start, R, s, g, seg_cost) <= P
            assert all(wh == (len(lst) == 1) for _, wh in lst)


def test_piece_charge_moves_blocks_off_segment_starts():
    """A workgroup whose range starts a segment gets seg_cost fewer blocks."""
    nb, seg_start, R, pieces = plan([16 * 100, 16 * 100], 1, 100, 8, 4, 20)
    per_wg = {}
    for (w, s, g, b0, b1, whole, k) in pieces:
        per_wg[w] = per_wg.get(w, 0) + b1 - b0
    assert R == 60 and per_wg == {0: 40, 1: 60, 2: 40, 3: 60}


def test_plan_random_shapes():
    rng = np.random.default_rng(0)
    for _ in range(40):
        S = int(rng.integers(1, 12))
        NG = int(rng.integers(1, 5))
        ctx = rng.integers(0, 700, size=S)
        max_blocks = int(math.ceil(max(ctx.max(), 1) / 16)) + int(rng.integers(0, 3))
        P = int(rng.integers(1, 9))
        n_wg = int(rng.integers(1, 40))
        test_plan_invariants(list(ctx), NG, max_blocks, P, n_wg, int(rng.integers(0, 40)))
