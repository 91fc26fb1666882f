"""CPU model of tq_decode_paged's balanced split of work over workgroups.

The decode kernel flattens the work into (sequence, kv head, block) triples,
sequence-major, and gives workgroup w the contiguous range [w*R, (w+1)*R);
with num_splits == 1 the range ends are moved to segment starts so that no
(sequence, kv head) segment is ever split (there is no workspace then).
This test re-derives that index arithmetic in Python and checks the
invariants the kernel relies on: every block processed exactly once, at
most P pieces per segment with piece indices in [0, P), no partial written
when P == 1, and the merge kernel's piece count equal to the real one.
"""
import math

import numpy as np
import pytest


def plan(ctx, Hkv, max_blocks, P, n_wg):
    cap = max_blocks * 16
    nb = [(min(max(int(c), 0), cap) + 15) // 16 for c in ctx]
    seg_start = {}
    pos = 0
    for s, n in enumerate(nb):
        for h in range(Hkv):
            seg_start[(s, h)] = pos
            pos += n
    W = pos
    R = max(1, -(-W // n_wg))
    if P > 1:
        R = max(R, -(-max_blocks // (P - 1)))

    def locate(x):
        for (s, h), st in seg_start.items():
            if st <= x < st + nb[s]:
                return s, h, x - st
        raise AssertionError

    def snap(x):
        if x >= W:
            return W
        s, h, blk = locate(x)
        return x if blk == 0 else x - blk + nb[s]

    pieces = []   # (wg, s, kvh, b0, b1, whole, piece_index)
    for w in range(n_wg):
        r0, r1 = w * R, min(W, w * R + R)
        if P == 1:
            r0, r1 = snap(r0), snap(r1)
        x = r0
        while x < r1:
            s, h, blk = locate(x)
            st = seg_start[(s, h)]
            b1 = nb[s] if nb[s] - blk < r1 - x else blk + (r1 - x)
            whole = P == 1 or st // R == (st + nb[s] - 1) // R
            pieces.append((w, s, h, blk, b1, whole, w - st // R))
            x += b1 - blk
    return nb, seg_start, R, pieces


def merge_count(nb, seg_start, R, s, h):
    st = seg_start[(s, h)]
    return (st + nb[s] - 1) // R - st // R + 1


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


@pytest.mark.parametrize("ctx,Hkv,max_blocks,P", CASES)
@pytest.mark.parametrize("n_wg", [512, 7, 1])
def test_plan_invariants(ctx, Hkv, max_blocks, P, n_wg):
    n_wg = min(n_wg, len(ctx) * Hkv * max_blocks)
    nb, seg_start, R, pieces = plan(ctx, Hkv, max_blocks, P, n_wg)
    seen = {}
    per_seg = {}
    for (w, s, h, b0, b1, whole, k) in pieces:
        assert 0 <= b0 < b1 <= nb[s]
        for b in range(b0, b1):
            assert (s, h, b) not in seen
            seen[(s, h, b)] = w
        per_seg.setdefault((s, h), []).append((k, whole))
        if P == 1:
            assert whole and b0 == 0 and b1 == nb[s]
        else:
            assert 0 <= k < P
    assert len(seen) == sum(nb) * Hkv
    for (s, h), lst in per_seg.items():
        ks = [k for k, _ in lst]
        assert len(set(ks)) == len(ks)
        if P > 1:
            assert len(lst) == merge_count(nb, seg_start, R, s, h) <= P
            assert all(wh == (len(lst) == 1) for _, wh in lst)


def test_plan_random_shapes():
    rng = np.random.default_rng(0)
    for _ in range(40):
        S = int(rng.integers(1, 12))
        Hkv = int(rng.integers(1, 5))
        ctx = rng.integers(0, 700, size=S)
        max_blocks = int(math.ceil(max(ctx.max(), 1) / 16)) + int(rng.integers(0, 3))
        P = int(rng.integers(1, 9))
        n_wg = int(rng.integers(1, 40))
        test_plan_invariants(list(ctx), Hkv, max_blocks, P, n_wg)
