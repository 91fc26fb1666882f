"""Pins for the oracle's attention, split partials and merge."""
import math
from decimal import Decimal, getcontext

import numpy as np
import pytest

from oracle import attn as att
from oracle import encode as enc
from oracle import pages as pg
from oracle.rotation import rotate
from workloads import signs


def _brute(q, K, V, scale, digits=50):
    """Attention in 50-digit decimal arithmetic, straight from the definition."""
    getcontext().prec = digits
    qd = [Decimal(float(v)) for v in q]
    sc = Decimal(float(scale))
    s = [sc * sum(qd[j] * Decimal(float(K[t, j])) for j in range(len(q))) for t in range(K.shape[0])]
    mx = max(s)
    e = [(si - mx).exp() for si in s]
    tot = sum(e)
    lse = mx + tot.ln()
    o = [sum(e[t] * Decimal(float(V[t, j])) for t in range(K.shape[0])) / tot for j in range(V.shape[1])]
    return np.array([float(v) for v in o]), float(lse)


@pytest.mark.parametrize("n,d", [(1, 8), (5, 8), (37, 16)])
def test_attention_against_high_precision(n, d):
    rng = np.random.default_rng(n)
    q = rng.standard_normal(d)
    K = rng.standard_normal((n, d)) * 3
    V = rng.standard_normal((n, d))
    o, lse = att.attention(q, K, V, 0.7)
    ob, lb = _brute(q, K, V, 0.7)
    np.testing.assert_allclose(o, ob, rtol=0, atol=1e-13)
    assert abs(lse - lb) < 1e-12


def test_special_cases():
    rng = np.random.default_rng(0)
    q = rng.standard_normal(16)
    K = rng.standard_normal((1, 16))
    V = rng.standard_normal((1, 16))
    o, lse = att.attention(q, K, V, 0.25)
    np.testing.assert_array_equal(o, V[0])
    assert lse == pytest.approx(0.25 * float(q @ K[0]), abs=1e-15)
    # identical keys: uniform weights, lse = s + ln n
    Kr = np.repeat(K, 9, axis=0)
    Vr = rng.standard_normal((9, 16))
    o, lse = att.attention(q, Kr, Vr, 0.25)
    np.testing.assert_allclose(o, Vr.mean(axis=0), atol=1e-15)
    assert lse == pytest.approx(0.25 * float(q @ K[0]) + math.log(9), abs=1e-14)
    # empty context
    o, lse = att.attention(q, np.zeros((0, 16)), np.zeros((0, 16)), 1.0)
    assert np.all(o == 0) and lse == -math.inf


@pytest.mark.parametrize("P", [1, 2, 3, 7, 64])
def test_split_merge_identity(P):
    rng = np.random.default_rng(P)
    n, d, bs = 301, 32, 16
    q = rng.standard_normal(d)
    K = rng.standard_normal((n, d))
    V = rng.standard_normal((n, d))
    nb = -(-n // bs)
    chunk = -(-nb // P)
    o_p, l_p = att.split_partials(q, K, V, 0.3, bs, chunk, P)
    if P == 64:
        assert np.sum(np.isinf(l_p)) > 0          # empty chunks present
    o, lse = att.merge_partials(o_p, l_p)
    o_ref, l_ref = att.attention(q, K, V, 0.3)
    np.testing.assert_allclose(o, o_ref, atol=1e-12)
    assert abs(lse - l_ref) < 1e-12


def test_merge_all_empty():
    o, lse = att.merge_partials(np.zeros((3, 4)), np.full(3, -math.inf))
    assert np.all(o == 0) and lse == -math.inf


def test_rotated_domain_equals_original_domain():
    """Scores and outputs computed against the rotated-domain cache (q rotated
    once, output inverse-rotated once) equal the original-domain ones."""
    d, bs, n = 128, 16, 70
    s = signs(4, 1, d)
    f = enc.Format.make(d, [4], s)
    rng = np.random.default_rng(9)
    x = rng.standard_normal((n, 1, d))
    _, _, tile = pg.tile_layout(f, bs)
    pages = np.zeros((5, 1, tile), dtype=np.uint8)
    bt = np.array([3, 1, 4, 0, 2])
    slots = bt[np.arange(n) // bs] * bs + np.arange(n) % bs
    pg.write_pages(x, slots, pages, f, bs)
    K = pg.reconstruct_sequence(pages, bt, n, 0, f, bs)
    Y = pg.reconstruct_sequence(pages, bt, n, 0, f, bs, rotated=True)
    q = rng.standard_normal(d)
    q_rot = rotate(q, s) / np.sqrt(d)
    np.testing.assert_allclose(Y @ q_rot, K @ q, atol=1e-12)
    o, lse = att.attention(q, K, K, 0.1)
    o_r, lse_r = att.attention(q_rot, Y, Y, 0.1)
    from oracle.rotation import inverse_rotate
    np.testing.assert_allclose(inverse_rotate(o_r, s), o, atol=1e-12)
    assert abs(lse - lse_r) < 1e-12


def _paged_history(rng, B, Hkv, d, ctx, f, bs=16):
    """A small packed history: per-sequence consecutive physical blocks in a
    shuffled pool, written by the oracle's own encoder."""
    nb_s = [-(-int(c) // bs) for c in ctx]
    nb = max(1, sum(nb_s))
    perm = rng.permutation(nb)
    mb = max(1, max(nb_s))
    bt = np.zeros((B, mb), dtype=np.int64)
    _, _, tile = pg.tile_layout(f, bs)
    kp = np.zeros((nb, Hkv, tile), dtype=np.uint8)
    vp = np.zeros((nb, Hkv, tile), dtype=np.uint8)
    used = 0
    for s in range(B):
        bt[s, :nb_s[s]] = perm[used:used + nb_s[s]]
        used += nb_s[s]
        n = int(ctx[s])
        if n:
            sl = bt[s, np.arange(n) // bs] * bs + np.arange(n) % bs
            pg.write_pages(rng.standard_normal((n, Hkv, d)), sl, kp, f, bs)
            pg.write_pages(rng.standard_normal((n, Hkv, d)), sl, vp, f, bs, "v")
    return kp, vp, bt


def _window_case(seed=3, B=3, Hq=4, Hkv=2, d=64, ctx=(40, 0, 17), wl=(5, 9, 0), cap=9):
    rng = np.random.default_rng(seed)
    f = enc.Format.make(d, [4], signs(seed, 1, d))
    kp, vp, bt = _paged_history(rng, B, Hkv, d, ctx, f)
    kw = rng.standard_normal((B, cap, Hkv, d))
    vw = rng.standard_normal((B, cap, Hkv, d))
    q = rng.standard_normal((B, Hq, d))
    return q, kw, vw, np.array(wl), kp, vp, bt, np.array(ctx), f


def test_window_equals_merge_of_history_and_window():
    """Attention over the union equals the log-sum-exp merge of the history's
    and the window's own attention (the merge identity), for every mix of
    empty and non-empty parts."""
    q, kw, vw, wl, kp, vp, bt, ctx, f = _window_case()
    sc = 0.4
    o, lse = att.decode_window_reference(q, kw, vw, wl, sc, kp, vp, bt, ctx, f, f)
    oh, lh = att.decode_reference(q, kp, vp, bt, ctx, f, f, sc, 16)
    G = q.shape[1] // kw.shape[2]
    for s in range(q.shape[0]):
        for h in range(q.shape[1]):
            ow, lw = att.attention(q[s, h], kw[s, :wl[s], h // G], vw[s, :wl[s], h // G], sc)
            om, lm = att.merge_partials(np.stack([oh[s, h], ow]), np.array([lh[s, h], lw]))
            np.testing.assert_allclose(o[s, h], om, atol=1e-12)
            assert lse[s, h] == lm or abs(lse[s, h] - lm) < 1e-12
    # sequence 1: no history -> the window alone; sequence 2: no window -> the history alone
    np.testing.assert_allclose(o[2], oh[2], atol=1e-13)
    np.testing.assert_allclose(lse[2], lh[2], atol=1e-13)


def test_window_holding_a_copy_of_the_history():
    """A window that repeats every history token (their decoded values)
    leaves the output unchanged and adds ln 2 to the lse."""
    q, kw, vw, wl, kp, vp, bt, ctx, f = _window_case(seed=5, ctx=(33, 20, 1), wl=(0, 0, 0), cap=33)
    B, Hkv, d = q.shape[0], kw.shape[2], q.shape[2]
    for s in range(B):
        n = int(ctx[s])
        for kvh in range(Hkv):
            kw[s, :n, kvh] = pg.reconstruct_sequence(kp, bt[s], n, kvh, f, 16)
            vw[s, :n, kvh] = pg.reconstruct_sequence(vp, bt[s], n, kvh, f, 16, role="v")
    o, lse = att.decode_window_reference(q, kw, vw, ctx, 0.3, kp, vp, bt, ctx, f, f)
    oh, lh = att.decode_reference(q, kp, vp, bt, ctx, f, f, 0.3, 16)
    np.testing.assert_allclose(o, oh, atol=1e-13)
    np.testing.assert_allclose(lse, lh + math.log(2.0), atol=1e-13)


def test_window_alone_and_all_empty():
    """Without pages the result is plain attention over the window rows; a
    sequence with neither history nor window gives o = 0, lse = -inf; a
    one-token window returns that token's V row and lse = scale q.k."""
    q, kw, vw, wl, *_ = _window_case(seed=7, wl=(1, 9, 0))
    o, lse = att.decode_window_reference(q, kw, vw, wl, 0.5)
    G = q.shape[1] // kw.shape[2]
    for h in range(q.shape[1]):
        np.testing.assert_array_equal(o[0, h], vw[0, 0, h // G])
        assert lse[0, h] == pytest.approx(0.5 * float(q[0, h] @ kw[0, 0, h // G]), abs=1e-14)
        ob, lb = _brute(q[1, h], kw[1, :9, h // G], vw[1, :9, h // G], 0.5)
        np.testing.assert_allclose(o[1, h], ob, atol=1e-13)
        assert abs(lse[1, h] - lb) < 1e-12
    assert np.all(o[2] == 0) and np.all(lse[2] == -math.inf)


def test_multi_query_is_single_query_at_each_causal_length():
    """Query i of NQ sees the first ctx - (NQ - 1 - i) tokens: it equals the
    single-query reference run with that context length; queries left with
    no token give o = 0, lse = -inf."""
    rng = np.random.default_rng(11)
    B, Hq, Hkv, d, NQ = 3, 4, 2, 64, 3
    ctx = np.array([40, 2, 17])
    f = enc.Format.make(d, [4], signs(11, 1, d))
    kp, vp, bt = _paged_history(rng, B, Hkv, d, ctx, f)
    q = rng.standard_normal((B, NQ, Hq, d))
    o, lse = att.decode_multi_reference(q, kp, vp, bt, ctx, f, f, 0.3, 16)
    for i in range(NQ):
        ci = np.maximum(ctx - (NQ - 1 - i), 0)
        oi, li = att.decode_reference(q[:, i], kp, vp, bt, ci, f, f, 0.3, 16)
        np.testing.assert_allclose(o[:, i], oi, atol=1e-13)
        np.testing.assert_array_equal(np.isinf(lse[:, i]), np.isinf(li))
        fin = np.isfinite(li)
        np.testing.assert_allclose(lse[:, i][fin], li[fin], atol=1e-13)
    # sequence 1 has 2 tokens: query 0 sees none, query 1 one, query 2 both
    assert np.all(o[1, 0] == 0) and np.all(lse[1, 0] == -math.inf)
    assert np.all(np.isfinite(lse[1, 1:]))
    # one query is the plain decode
    o1, l1 = att.decode_multi_reference(q[:, -1:], kp, vp, bt, ctx, f, f, 0.3, 16)
    ob, lb = att.decode_reference(q[:, -1], kp, vp, bt, ctx, f, f, 0.3, 16)
    np.testing.assert_allclose(o1[:, 0], ob, atol=1e-13)
    np.testing.assert_allclose(l1[:, 0], lb, atol=1e-13)
