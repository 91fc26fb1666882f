"""GPU parity of the QJL residual stage (K formats with qjl = 1).

Write: whole pools bit-exact against the oracle (MSE indices, sign bits,
vector and residual norms; bytes a write must not touch unchanged).  The
sign bits come from fp64 projection sums taken in one defined order (j
ascending, each product and partial sum rounded, no fused multiply-add),
which both sides follow; rows whose sums cancel exactly check that order.

Decode: out and lse against the oracle's fp64 attention over the effective
keys (MSE reconstruction plus the sketch's term, reconstructed from the
oracle's own pages), with the decode's tolerances (lse 1e-4; out 2e-3
normwise and elementwise, bf16 output net of its own rounding)."""
import math

import numpy as np
import pytest

from oracle import attn as oatt
from oracle import pages as opg
from tests.conftest import gpu_available
from tests.helpers import oracle_format, product_format, to_device, oracle_pages, slots_of, out_error, elem_error
import workloads as wl

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

LSE_TOL = 1e-4
OUT_TOL = 2e-3


def _assert_pool_equal(got, ref, what):
    if not np.array_equal(got, ref):
        bad = np.argwhere(got != ref)
        raise AssertionError(f"{what}: {len(bad)} bytes differ, first at {bad[:5].tolist()}")


@pytest.mark.parametrize("kbits,d,dtype,dist", [
    ([3, 2], 128, "bf16", "t3"),
    ([4], 128, "bf16", "normal"),
    ([2], 128, "f32", "t5u"),
    ([4, 3], 128, "f32", "normal"),
    ([2], 64, "bf16", "normal"),
    ([3, 2], 64, "f32", "t3"),
])
def test_qjl_write_bit_exact(kbits, d, dtype, dist):
    import torch
    import quantized_paged_kv_amd as tq
    seed = 300 + d + 5 * sum(kbits) + len(kbits)
    print(f"case write K{kbits}+QJL d{d} {dtype} {dist}", flush=True)
    w = wl.write_workload(seed=seed, num_seqs=3, new_tokens=150, num_kv_heads=3, head_dim=d, kbits=kbits,
                          vbits=[4], kv_dist=dist, in_dtype=dtype, qjl=True)
    xk = wl.write_values(w, "k")
    slots = w.slot_mapping.copy()
    slots[7] = -1                                  # an invalid slot: that row is not written
    kf = product_format(w.kfmt)
    kp = torch.full((w.num_blocks, 3, kf.tile_bytes()[1]), 0xA5, dtype=torch.uint8, device="cuda")
    err = tq.new_error_word()
    tq.write_kv(to_device(xk, dtype), None, torch.from_numpy(slots).cuda(), kp, None, kf, None, dev_err=err)
    torch.cuda.synchronize()
    e = err.cpu().numpy()
    assert e[0] == tq.TQ_ERR_INDEX and e[1] == 7
    keep = np.ones(len(slots), bool)
    keep[7] = False
    ref = oracle_pages(xk[keep], slots[keep], w.num_blocks, oracle_format(w.kfmt), "k")
    _assert_pool_equal(kp.cpu().numpy(), ref, "K (QJL)")


@pytest.mark.parametrize("bits,d,dtype", [((4,), 128, "bf16"), ((2,), 128, "f32"), ((3, 2), 128, "bf16"),
                                          ((4, 3), 128, "f32"), ((4,), 64, "f32"), ((3, 2), 64, "bf16")])
def test_qjl_write_cancelling_projection_sums(bits, d, dtype):
    """Rows and projections whose projection sums cancel exactly
    (tests/qjl_cases.py): the defined order (j ascending, product and sum
    each rounded, no fused multiply-add) gives bit 0 where exact arithmetic
    or a fused multiply-add would give 1.  The pool written on the GPU equals
    the oracle's byte for byte."""
    import torch
    import quantized_paged_kv_amd as tq
    from tests import qjl_cases as qc
    print(f"case cancelling sums K{list(bits)}+QJL d{d} {dtype}", flush=True)
    x, S, f, cases = qc.build(d, bits)
    T = x.shape[0]
    nb = (T + 15) // 16 + 1
    slots = np.arange(T, dtype=np.int64) + 16   # blocks 1.. (block 0 untouched)
    kf = tq.Format(d, list(bits), f.signs, f.group_channels, qjl_proj=torch.from_numpy(S.copy()).cuda())
    kp = torch.full((nb, 1, kf.tile_bytes()[1]), 0xA5, dtype=torch.uint8, device="cuda")
    tq.write_kv(to_device(x, dtype), None, torch.from_numpy(slots).cuda(), kp, None, kf, None, check=True)
    torch.cuda.synchronize()
    ref = oracle_pages(x, slots, nb, f, "k")
    _assert_pool_equal(kp.cpu().numpy(), ref, "K (QJL, cancelling sums)")


def test_qjl_rejected_on_v_and_past_64_columns():
    import torch
    import quantized_paged_kv_amd as tq
    w = wl.small_decode_workload(41, 1, 4, 2, 128, [40], [3, 2], [4], qjl=True)
    kf = product_format(w.kfmt)
    vf = product_format(w.vfmt)
    x = torch.zeros((1, 2, 128), dtype=torch.bfloat16, device="cuda")
    pool = torch.zeros((4, 2, kf.tile_bytes()[1]), dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError):   # the QJL format used for V
        tq.write_kv(None, x, torch.zeros(1, dtype=torch.int64, device="cuda"), None, pool, vf, kf)
    kp, vp = build_cache(w)
    bt = torch.from_numpy(w.block_tables).cuda()
    cl = torch.from_numpy(w.context_lens).cuda()
    q2 = torch.zeros((1, 33, 4, 128), dtype=torch.bfloat16, device="cuda")   # 66 columns per kv head
    with pytest.raises(tq.UnsupportedFormatError):
        tq.decode_paged(q2, kp, vp, bt, cl, kf, vf, w.scale)


def build_cache(w):
    import torch
    import quantized_paged_kv_amd as tq
    kf, vf = product_format(w.kfmt), product_format(w.vfmt)
    kp = torch.full((w.num_blocks, w.num_kv_heads, kf.tile_bytes()[1]), 0xA5, dtype=torch.uint8, device="cuda")
    vp = torch.full((w.num_blocks, w.num_kv_heads, vf.tile_bytes()[1]), 0xA5, dtype=torch.uint8, device="cuda")
    err = tq.new_error_word()
    for s, sl in enumerate(slots_of(w.block_tables, w.context_lens)):
        if len(sl):
            tq.write_kv(to_device(wl.kv_values(w, "k", s), w.in_dtype), to_device(wl.kv_values(w, "v", s), w.in_dtype),
                        torch.from_numpy(sl).cuda(), kp, vp, kf, vf, dev_err=err)
    tq.raise_device_error(err, "cache build")
    w._gpu_formats = (kf, vf)
    return kp, vp


def run_decode(w, kp, vp, P, out_dtype):
    import torch
    import quantized_paged_kv_amd as tq
    kf, vf = w._gpu_formats
    q = wl.q_values(w)
    od = torch.float32 if out_dtype == "f32" else torch.bfloat16
    o, l = tq.decode_paged(to_device(q, w.q_dtype), kp, vp, torch.from_numpy(w.block_tables).cuda(),
                           torch.from_numpy(w.context_lens).cuda(), kf, vf, w.scale, num_splits=P, out_dtype=od,
                           check=True)
    torch.cuda.synchronize()
    return q, o.float().cpu().numpy(), l.cpu().numpy()


def check(o, l, o_ref, l_ref, cells, out_dtype):
    worst_o = worst_l = worst_e = 0.0
    for c in cells:
        if l_ref[c] == -math.inf:
            assert l[c] == -math.inf and np.all(o[c] == 0), c
            continue
        worst_o = max(worst_o, out_error(o[c][None], o_ref[c][None], out_dtype == "bf16")[0])
        worst_l = max(worst_l, abs(float(l[c]) - float(l_ref[c])))
        if out_dtype == "f32":
            worst_e = max(worst_e, float(np.max(elem_error(o[c][None], o_ref[c][None]))))
    print(f"[{out_dtype}] worst out {worst_o:.2e}  lse {worst_l:.2e}  elem {worst_e:.2e}", flush=True)
    assert worst_l <= LSE_TOL and worst_o <= OUT_TOL and worst_e <= OUT_TOL


CASES = [
    # d, kbits, vbits, Hq, Hkv, ctx, splits, in dtype, out dtype, dist
    (128, [3, 2], [2], 16, 2, [1, 17, 300, 1000], 1, "bf16", "f32", "t3"),
    (128, [3, 2], [2], 16, 2, [1, 17, 300, 1000], 5, "bf16", "bf16", "t3"),
    (128, [4], [4], 8, 2, [0, 333, 64], 3, "f32", "f32", "normal"),
    (128, [2], [4], 4, 4, [95, 257], 1, "bf16", "bf16", "t5u"),
    (128, [4, 3], [2], 8, 8, [700], 20, "bf16", "f32", "normal"),
    (64, [2], [2], 8, 1, [1000, 16], 7, "bf16", "f32", "normal"),
    (64, [3, 2], [4], 6, 3, [5, 400, 129], 2, "f32", "f32", "t3"),
    (64, [4], [2], 4, 1, [77, 300], 2, "bf16", "f32", "normal"),
    (64, [4, 3], [4], 2, 2, [129], 1, "f32", "f32", "t3"),
    # a K layout the main kernel does not read (one 3-bit group): the
    # separate QJL kernel
    (128, [3], [4], 8, 2, [200, 33], 2, "bf16", "f32", "normal"),
]


@pytest.mark.parametrize("case", CASES, ids=[f"d{c[0]}K{c[1]}V{c[2]}G{c[3]//c[4]}P{c[6]}{c[8]}" for c in CASES])
def test_qjl_decode_small(case):
    d, kb, vb, hq, hkv, ctx, P, idt, odt, dist = case
    seed = 600 + d + 7 * len(ctx) + P
    print(f"case {case}", flush=True)
    w = wl.small_decode_workload(seed, len(ctx), hq, hkv, d, ctx, kb, vb, kv_dist=dist, in_dtype=idt,
                                 out_dtype=odt, num_splits=P, max_blocks_per_seq=(max(ctx) + 15) // 16 + 1, qjl=True)
    kp, vp = build_cache(w)
    q, o, l = run_decode(w, kp, vp, P, odt)
    kof, vof = oracle_format(w.kfmt), oracle_format(w.vfmt)
    sl = slots_of(w.block_tables, w.context_lens)
    nonempty = [s for s in range(w.num_seqs) if len(sl[s])]
    allsl = np.concatenate([sl[s] for s in nonempty])
    okp = oracle_pages(np.concatenate([wl.kv_values(w, "k", s) for s in nonempty]), allsl, w.num_blocks, kof, "k")
    ovp = oracle_pages(np.concatenate([wl.kv_values(w, "v", s) for s in nonempty]), allsl, w.num_blocks, vof, "v")
    assert np.array_equal(kp.cpu().numpy(), okp), "K pool differs from the oracle's"
    o_ref, l_ref = oatt.decode_reference(q.astype(np.float64), okp, ovp, w.block_tables, w.context_lens,
                                         kof, vof, w.scale, 16)
    check(o, l, o_ref, l_ref, [(s, h) for s in range(w.num_seqs) for h in range(hq)], odt)


def test_qjl_decode_full_size_long_context():
    """The 131072-token context with the 3+2-bit K recipe plus the QJL stage
    (64 splits, the benchmark's launch); two kv heads' q heads against the
    oracle, each kv head's history reconstructed from oracle pages."""
    w = wl.decode_workload(7)
    print("case workload 7 (QJL long context), splits 64", flush=True)
    kp, vp = build_cache(w)
    q, o, l = run_decode(w, kp, vp, w.num_splits, w.out_dtype)
    kof, vof = oracle_format(w.kfmt), oracle_format(w.vfmt)
    n = int(w.context_lens[0])
    xk, xv = wl.kv_values(w, "k", 0), wl.kv_values(w, "v", 0)
    bt = np.arange((n + 15) // 16)
    slots = bt[np.arange(n) // 16] * 16 + np.arange(n) % 16
    G = w.num_q_heads // w.num_kv_heads
    o_ref = np.zeros(o.shape)
    l_ref = np.full(l.shape, -math.inf)
    cells = []
    for kvh in (0, 5):
        Kp = np.zeros((len(bt), 1, opg.tile_layout(kof, 16)[2]), np.uint8)
        Vp = np.zeros((len(bt), 1, opg.tile_layout(vof, 16)[2]), np.uint8)
        opg.write_pages(xk[:, kvh:kvh + 1], slots, Kp, kof, 16)
        opg.write_pages(xv[:, kvh:kvh + 1], slots, Vp, vof, 16, "v")
        K = opg.reconstruct_sequence(Kp, bt, n, 0, kof, 16)
        V = opg.reconstruct_sequence(Vp, bt, n, 0, vof, 16, role="v")
        for h in range(kvh * G, (kvh + 1) * G):
            o_ref[0, h], l_ref[0, h] = oatt.attention(q[0, h].astype(np.float64), K, V, w.scale)
            cells.append((0, h))
    check(o, l, o_ref, l_ref, cells, w.out_dtype)


def test_qjl_bad_block_entry_and_context_length():
    """A block-table entry outside the pool is reported as (INDEX, s * max_blocks
    + b) and its block skipped: the output equals the oracle's attention over
    the other blocks.  A context length past the capacity is reported as
    (INDEX, -1 - s)."""
    import torch
    import quantized_paged_kv_amd as tq
    w = wl.small_decode_workload(71, 2, 8, 2, 128, [64, 100], [3, 2], [2], out_dtype="f32", num_splits=3,
                                 qjl=True)
    print("case QJL bad entry", flush=True)
    kp, vp = build_cache(w)
    kf, vf = w._gpu_formats
    q = wl.q_values(w)
    bt = w.block_tables.copy()
    bt[1, 2] = w.num_blocks + 5
    err = tq.new_error_word()
    o, l = tq.decode_paged(to_device(q, w.q_dtype), kp, vp, torch.from_numpy(bt).cuda(),
                           torch.from_numpy(w.context_lens).cuda(), kf, vf, w.scale, num_splits=3,
                           out_dtype=torch.float32, dev_err=err)
    torch.cuda.synchronize()
    e = err.cpu().numpy()
    assert e[0] == tq.TQ_ERR_INDEX and e[1] == 1 * bt.shape[1] + 2
    kof, vof = oracle_format(w.kfmt), oracle_format(w.vfmt)
    n = int(w.context_lens[1])
    xk, xv = wl.kv_values(w, "k", 1), wl.kv_values(w, "v", 1)
    keep = np.array([t for t in range(n) if t // 16 != 2])
    nbk = (n + 15) // 16
    sl = np.arange(nbk)[np.arange(n) // 16] * 16 + np.arange(n) % 16
    o_ref = np.zeros((2, 8, 128))
    l_ref = np.full((2, 8), -math.inf)
    for kvh in range(2):
        Kp = np.zeros((nbk, 1, opg.tile_layout(kof, 16)[2]), np.uint8)
        Vp = np.zeros((nbk, 1, opg.tile_layout(vof, 16)[2]), np.uint8)
        opg.write_pages(xk[:, kvh:kvh + 1], sl, Kp, kof, 16)
        opg.write_pages(xv[:, kvh:kvh + 1], sl, Vp, vof, 16, "v")
        K = opg.reconstruct_sequence(Kp, np.arange(nbk), n, 0, kof, 16)[keep]
        V = opg.reconstruct_sequence(Vp, np.arange(nbk), n, 0, vof, 16, role="v")[keep]
        for h in range(kvh * 4, kvh * 4 + 4):
            o_ref[1, h], l_ref[1, h] = oatt.attention(q[1, h].astype(np.float64), K, V, w.scale)
    check(o.cpu().numpy(), l.cpu().numpy(), o_ref, l_ref, [(1, h) for h in range(8)], "f32")
    # a context length past the capacity; every entry of that row is in the
    # pool, so the length is the only error (with two, which one the error
    # word records is unspecified)
    cl = w.context_lens.copy()
    cl[0] = 16 * bt.shape[1] + 1
    bt_full = w.block_tables.copy()
    bt_full[0][bt_full[0] < 0] = 0
    with pytest.raises(IndexError, match="position -1"):
        tq.decode_paged(to_device(q, w.q_dtype), kp, vp, torch.from_numpy(bt_full).cuda(),
                        torch.from_numpy(cl).cuda(), kf, vf, w.scale, check=True)


MULTI = [
    # d, kbits, vbits, Hq, Hkv, ctx, queries, splits, out dtype
    (128, [3, 2], [2], 16, 2, [1, 40, 300, 700], 2, 3, "f32"),
    (128, [4], [4], 8, 2, [20, 500], 8, 1, "bf16"),
    (128, [4, 3], [2], 8, 1, [64, 1000], 8, 4, "f32"),      # 64 columns
    (64, [2], [4], 4, 2, [17, 257], 5, 2, "f32"),
]


@pytest.mark.parametrize("case", MULTI, ids=[f"d{c[0]}K{c[1]}V{c[2]}G{c[3]//c[4]}NQ{c[6]}P{c[7]}" for c in MULTI])
def test_qjl_multi_query(case):
    """QJL K formats with several queries per sequence (up to 64 (query, q
    head) columns per kv head) against the oracle's multi-query reference,
    whose keys include the sketch term."""
    import torch
    import quantized_paged_kv_amd as tq
    d, kb, vb, hq, hkv, ctx, NQ, P, odt = case
    print(f"case {case}", flush=True)
    w = wl.small_decode_workload(650 + d + NQ + P, len(ctx), hq, hkv, d, ctx, kb, vb, out_dtype=odt, num_splits=P,
                                 max_blocks_per_seq=(max(ctx) + 15) // 16 + 1, qjl=True)
    kp, vp = build_cache(w)
    kf, vf = w._gpu_formats
    g = wl.rng(w.seed, 41)
    q = wl.bf16_round(g.standard_normal((w.num_seqs, NQ, hq, d), dtype=np.float32))
    od = torch.float32 if odt == "f32" else torch.bfloat16
    o, l = tq.decode_paged(to_device(q, "bf16"), kp, vp, torch.from_numpy(w.block_tables).cuda(),
                           torch.from_numpy(w.context_lens).cuda(), kf, vf, w.scale, num_splits=P, out_dtype=od,
                           check=True)
    torch.cuda.synchronize()
    o, l = o.float().cpu().numpy(), l.cpu().numpy()
    kof, vof = oracle_format(w.kfmt), oracle_format(w.vfmt)
    sl = slots_of(w.block_tables, w.context_lens)
    allsl = np.concatenate(sl)
    okp = oracle_pages(np.concatenate([wl.kv_values(w, "k", s) for s in range(w.num_seqs)]), allsl, w.num_blocks, kof, "k")
    ovp = oracle_pages(np.concatenate([wl.kv_values(w, "v", s) for s in range(w.num_seqs)]), allsl, w.num_blocks, vof, "v")
    o_ref, l_ref = oatt.decode_multi_reference(q.astype(np.float64), okp, ovp, w.block_tables, w.context_lens,
                                               kof, vof, w.scale, 16)
    check(o, l, o_ref, l_ref, [(s, i, h) for s in range(w.num_seqs) for i in range(NQ) for h in range(hq)], odt)
