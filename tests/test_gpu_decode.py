"""GPU parity of tq_decode_paged (and the split merge inside it) against the
oracle's fp64 attention over the dense reconstruction of the same pages.

Tolerances (from the target: max relative error 2e-3 with fp32 accumulation
and bf16 q/out; LSE within 1e-4 absolute):
  * lse: max |lse - lse_ref| <= 1e-4;
  * fp32 out: per (sequence, head) normwise relative error <= 2e-3 and every
    element within 2e-3 of the vector's largest |value|;
  * bf16 out: the normwise distance from the fp64 reference rounded to bf16,
    ||o - bf16(ref)|| / ||ref|| <= 2e-3 (bf16 rounding of the exact result
    alone is ~1.7e-3 RMS normwise, so it cannot be charged to the kernel);
    the raw normwise error against fp64 is printed beside it.
Full-size cases check every (sequence, q head) output with both output
dtypes.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import attn as oatt
from oracle import pages as opg
from tests.conftest import gpu_available
from tests.helpers import oracle_format, product_format, to_device, out_error, elem_error, slots_of
from tests.oracle_refs import decode_refs, cpu_procs
import workloads as wl

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

LSE_TOL = 1e-4
OUT_TOL = 2e-3


def build_gpu_cache(w, fill=0xA5):
    """Write every sequence's K/V through tq_write_kv (one call per sequence)
    into pools whose other bytes hold `fill`."""
    import torch
    import quantized_paged_kv_amd as tq
    kf, vf = product_format(w.kfmt), product_format(w.vfmt)
    kp = torch.full((w.num_blocks, w.num_kv_heads, kf.tile_bytes()[1]), fill, dtype=torch.uint8, device="cuda")
    vp = torch.full((w.num_blocks, w.num_kv_heads, vf.tile_bytes()[1]), fill, dtype=torch.uint8, device="cuda")
    err = tq.new_error_word()
    for s, sl in enumerate(slots_of(w.block_tables, w.context_lens)):
        if len(sl) == 0:
            continue
        xk, xv = wl.kv_values(w, "k", s), wl.kv_values(w, "v", s)
        tq.write_kv(to_device(xk, w.in_dtype), to_device(xv, w.in_dtype), torch.from_numpy(sl).cuda(),
                    kp, vp, kf, vf, dev_err=err)
    tq.raise_device_error(err, "cache build")
    return kp, vp, kf, vf


def oracle_decode(w, q, pairs, procs=0):
    """fp64 reference for the (seq, q head) pairs: the oracle encodes each
    (sequence, kv head)'s rows itself into a pool of its own and attends over
    the dense reconstruction (procs > 1: spread over CPU worker processes)."""
    return decode_refs(w, q, pairs, procs)


def run_decode(w, kp, vp, kf, vf, num_splits, out_dtype, q=None):
    import torch
    import quantized_paged_kv_amd as tq
    q = wl.q_values(w) if q is None else q
    qd = to_device(q, w.q_dtype)
    bt = torch.from_numpy(w.block_tables.astype(np.int32)).cuda()
    cl = torch.from_numpy(w.context_lens.astype(np.int32)).cuda()
    od = torch.float32 if out_dtype == "f32" else torch.bfloat16
    o, l = tq.decode_paged(qd, kp, vp, bt, cl, kf, vf, w.scale, num_splits=num_splits, out_dtype=od, check=True)
    torch.cuda.synchronize()
    return q, o.float().cpu().numpy(), l.cpu().numpy()


def check(w, q, o, l, pairs, out_dtype, ref=None):
    ref = ref if ref is not None else oracle_decode(w, q, pairs)
    worst_o = worst_l = worst_e = worst_raw = 0.0
    for (s, h) in pairs:
        o_ref, l_ref = ref[(s, h)]
        if l_ref == -math.inf:
            assert l[s, h] == -math.inf and np.all(o[s, h] == 0), (s, h)
            continue
        eo = out_error(o[s, h][None], o_ref[None], out_dtype == "bf16")[0]
        worst_raw = max(worst_raw, out_error(o[s, h][None], o_ref[None])[0])
        el = abs(float(l[s, h]) - l_ref)
        worst_o, worst_l = max(worst_o, eo), max(worst_l, el)
        if out_dtype == "f32":
            worst_e = max(worst_e, float(np.max(elem_error(o[s, h][None], o_ref[None]))))
    print(f"[{out_dtype}] worst out {worst_o:.2e} (raw normwise {worst_raw:.2e})  lse {worst_l:.2e}  "
          f"elem {worst_e:.2e}", flush=True)
    assert worst_l <= LSE_TOL
    assert worst_o <= OUT_TOL
    assert worst_e <= OUT_TOL


SMALL = [
    # d, kbits, vbits, Hq, Hkv, ctx, splits, in/out dtype, dist
    (128, [4], [4], 8, 2, [1, 17, 300, 1000], 1, "bf16", "bf16", "normal"),
    (128, [4], [4], 8, 2, [1, 17, 300, 1000], 3, "bf16", "f32", "normal"),
    (128, [4], [2], 16, 2, [33, 0, 517], 4, "bf16", "bf16", "normal"),
    (128, [4, 3], [2], 16, 2, [700, 64], 5, "bf16", "f32", "t3"),
    (128, [2], [4], 4, 4, [95, 257], 2, "f32", "f32", "normal"),
    (128, [2], [2], 3, 1, [150], 1, "bf16", "bf16", "t5u"),
    (64, [4], [4], 1, 1, [256], 1, "f32", "f32", "normal"),
    (64, [4], [2], 6, 3, [5, 400], 2, "bf16", "bf16", "normal"),
    (64, [4, 3], [4], 2, 2, [129], 1, "f32", "f32", "t3"),
    (64, [2], [2], 8, 1, [1000, 16], 7, "bf16", "f32", "normal"),
    # the 2.5-bit K recipe (3-bit high + 2-bit low channel groups)
    (128, [3, 2], [2], 16, 2, [700, 64, 0], 5, "bf16", "bf16", "t3"),
    (128, [3, 2], [4], 8, 2, [33, 300], 1, "f32", "f32", "normal"),
    (64, [3, 2], [2], 6, 3, [5, 400, 129], 3, "bf16", "f32", "t5u"),
    (64, [3, 2], [4], 1, 1, [256], 1, "f32", "f32", "normal"),
    # two-group (recipe) V formats, with every K kind
    (128, [4], [4, 3], 8, 2, [1, 17, 300, 1000], 3, "bf16", "f32", "normal"),
    (128, [4, 3], [4, 3], 16, 2, [700, 64], 5, "bf16", "bf16", "t3"),
    (128, [3, 2], [3, 2], 16, 2, [700, 64, 0], 4, "bf16", "f32", "t3"),
    (128, [2], [3, 2], 4, 4, [95, 257], 1, "f32", "f32", "normal"),
    (128, [4, 3], [3, 2], 8, 2, [33, 300], 2, "bf16", "f32", "t5u"),
    (64, [4], [3, 2], 6, 3, [5, 400, 129], 3, "bf16", "f32", "normal"),
    (64, [3, 2], [4, 3], 2, 2, [129, 1000], 2, "f32", "f32", "t3"),
    # many splits: the merge spreads each row's partials over 2 and 4 waves,
    # and past 64 slots
    (128, [4], [4], 8, 2, [1, 17, 300, 5000], 24, "bf16", "f32", "normal"),
    (64, [4], [2], 4, 1, [3000, 40, 1700], 80, "f32", "f32", "normal"),
]


@pytest.mark.parametrize("case", SMALL, ids=[f"d{c[0]}K{c[1]}V{c[2]}G{c[3]//c[4]}P{c[6]}{c[8]}" for c in SMALL])
def test_small_cases(case):
    d, kb, vb, hq, hkv, ctx, P, idt, odt, dist = case
    seed = 100 + d + len(ctx) * 7 + P
    w = wl.small_decode_workload(seed, len(ctx), hq, hkv, d, ctx, kb, vb, kv_dist=dist, in_dtype=idt,
                                 out_dtype=odt, num_splits=P, max_blocks_per_seq=(max(ctx) + 15) // 16 + 2)
    print(f"case {case}", flush=True)
    kp, vp, kf, vf = build_gpu_cache(w)
    q, o, l = run_decode(w, kp, vp, kf, vf, P, odt)
    pairs = [(s, h) for s in range(w.num_seqs) for h in range(hq)]
    check(w, q, o, l, pairs, odt)


def test_pages_written_on_gpu_match_oracle_for_decode_cache():
    """The decode tests consume pages written by tq_write_kv; they equal the
    oracle's pages byte for byte (so decode parity is not masking a write bug)."""
    w = wl.small_decode_workload(11, 2, 8, 2, 128, [70, 33], [4, 3], [2], kv_dist="t3")
    kp, vp, _, _ = build_gpu_cache(w)
    kof, vof = oracle_format(w.kfmt), oracle_format(w.vfmt)
    for pool, of, which in ((kp, kof, "k"), (vp, vof, "v")):
        ref = np.full(tuple(pool.shape), 0xA5, np.uint8)
        for s, sl in enumerate(slots_of(w.block_tables, w.context_lens)):
            opg.write_pages(wl.kv_values(w, which, s), sl, ref, of, 16, which)
        assert np.array_equal(pool.cpu().numpy(), ref)


def test_identical_keys_uniform_attention():
    """All cached keys equal -> softmax is uniform: out = mean of V rows,
    lse = s + ln n (checked against the oracle's same special case)."""
    import torch
    import quantized_paged_kv_amd as tq
    d, n = 128, 333
    s = wl.signs(1, 1, d)
    kf = tq.Format(d, [4], s)
    rng = np.random.default_rng(0)
    krow = wl.bf16_round(rng.standard_normal(d).astype(np.float32))
    xk = np.repeat(krow[None, None, :], n, axis=0)
    xv = wl.bf16_round(rng.standard_normal((n, 1, d)).astype(np.float32))
    nb = (n + 15) // 16
    kp = tq.alloc_pages(nb, 1, kf)
    vp = tq.alloc_pages(nb, 1, kf)
    slots = np.arange(n, dtype=np.int64)
    tq.write_kv(to_device(xk, "bf16"), to_device(xv, "bf16"), torch.from_numpy(slots).cuda(), kp, vp, kf, kf,
                check=True)
    q = wl.bf16_round(rng.standard_normal((1, 4, d)).astype(np.float32))
    bt = torch.arange(nb, dtype=torch.int32).view(1, -1).cuda()
    cl = torch.tensor([n], dtype=torch.int32).cuda()
    o, l = tq.decode_paged(to_device(q, "bf16"), kp, vp, bt, cl, kf, kf, 0.1, out_dtype=torch.float32, check=True)
    of = oracle.Format.make(d, [4], s)
    Kp = np.zeros((nb, 1, opg.tile_layout(of, 16)[2]), np.uint8)
    Vp = Kp.copy()
    opg.write_pages(xk, slots, Kp, of, 16)
    opg.write_pages(xv, slots, Vp, of, 16, "v")
    K = opg.reconstruct_sequence(Kp, np.arange(nb), n, 0, of, 16)
    V = opg.reconstruct_sequence(Vp, np.arange(nb), n, 0, of, 16, role="v")
    for h in range(4):
        sc = 0.1 * float(q[0, h].astype(np.float64) @ K[0])
        assert abs(float(l[0, h]) - (sc + math.log(n))) < LSE_TOL
        np.testing.assert_allclose(o[0, h].cpu().numpy(), V.mean(axis=0), atol=2e-3 * np.abs(V).max())


def test_bad_block_table_entry_reports_and_skips():
    import torch
    import quantized_paged_kv_amd as tq
    w = wl.small_decode_workload(5, 2, 4, 1, 128, [64, 64], [4], [4])
    kp, vp, kf, vf = build_gpu_cache(w)
    bt = w.block_tables.copy()
    bt[1, 2] = w.num_blocks + 5
    q = to_device(wl.q_values(w), "bf16")
    with pytest.raises(IndexError, match=f"position {1 * bt.shape[1] + 2}"):
        tq.decode_paged(q, kp, vp, torch.from_numpy(bt).cuda(), torch.from_numpy(w.context_lens).cuda(), kf, vf,
                        w.scale, check=True)
    # a context length past the capacity; every entry of that row is in the
    # pool, so the length is the only error (with two, which one the error
    # word records is unspecified)
    cl = w.context_lens.copy()
    cl[0] = 16 * bt.shape[1] + 1
    bt_full = w.block_tables.copy()
    bt_full[0][bt_full[0] < 0] = 0
    with pytest.raises(IndexError, match="position -1"):
        tq.decode_paged(q, kp, vp, torch.from_numpy(bt_full).cuda(), torch.from_numpy(cl).cuda(), kf, vf,
                        w.scale, check=True)


@pytest.mark.parametrize("P,d", [(7, 128), (16, 64), (17, 128), (40, 64), (64, 128), (100, 128)])
def test_split_merge_against_oracle_partials(P, d):
    """tq_split_merge on partials the oracle computed (ragged chunks, empty
    chunks at -inf) equals the oracle's merge; split counts on both sides of
    each 16-slot wave boundary and past 64 slots."""
    import torch
    import quantized_paged_kv_amd as tq
    print(f"case P={P} d={d}", flush=True)
    rng = np.random.default_rng(3 + P)
    S, H = 3, 5
    po = np.zeros((S, H, P, d))
    pl = np.full((S, H, P), -math.inf)
    ref_o = np.zeros((S, H, d))
    ref_l = np.zeros((S, H))
    for s in range(S):
        n = [300, 17, 1600][s]
        K = rng.standard_normal((n, d))
        V = rng.standard_normal((n, d))
        for h in range(H):
            qv = rng.standard_normal(d)
            nb = (n + 15) // 16
            po[s, h], pl[s, h] = oatt.split_partials(qv, K, V, 0.09, 16, -(-nb // P), P)
            ref_o[s, h], ref_l[s, h] = oatt.merge_partials(po[s, h], pl[s, h])
    o, l = tq.split_merge(torch.from_numpy(po.astype(np.float32)).cuda(),
                          torch.from_numpy(pl.astype(np.float32)).cuda())
    o, l = o.cpu().numpy(), l.cpu().numpy()
    assert np.max(np.abs(l - ref_l)) < 1e-5
    assert np.max(out_error(o, ref_o, False)) < 1e-5
    # all partials empty
    o, l = tq.split_merge(torch.zeros((1, 1, 3, 64)).cuda(), torch.full((1, 1, 3), -math.inf).cuda())
    assert np.all(o.cpu().numpy() == 0) and l.item() == -math.inf


def test_split_workspace_contents_do_not_matter():
    """The workspace is read only where the same call wrote it: a NaN-filled
    workspace, and one left over from a call with other context lengths,
    give the same outputs as a zeroed one."""
    import torch
    import quantized_paged_kv_amd as tq
    P = 4
    w = wl.small_decode_workload(21, 3, 8, 2, 128, [1000, 0, 300], [4], [4], num_splits=P,
                                 max_blocks_per_seq=70)
    kp, vp, kf, vf = build_gpu_cache(w)
    q = to_device(wl.q_values(w), "bf16")
    bt = torch.from_numpy(w.block_tables.astype(np.int32)).cuda()
    nbytes = tq.workspace_bytes(w.num_seqs, w.num_q_heads, w.head_dim, P)

    def run(cl, ws):
        o, l = tq.decode_paged(q, kp, vp, bt, torch.tensor(cl, dtype=torch.int32).cuda(), kf, vf, w.scale,
                               num_splits=P, workspace=ws, out_dtype=torch.float32, check=True)
        torch.cuda.synchronize()
        return o.cpu().numpy(), l.cpu().numpy()

    cl = [int(c) for c in w.context_lens]
    o0, l0 = run(cl, torch.zeros(nbytes, dtype=torch.uint8, device="cuda"))
    o1, l1 = run(cl, torch.full((nbytes // 4,), math.nan, dtype=torch.float32, device="cuda"))
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    run([500, 0, 100], ws)   # leaves partials of other segment cuts behind
    o2, l2 = run(cl, ws)
    for o, l in ((o1, l1), (o2, l2)):
        assert np.all(np.isfinite(o))
        # same cuts, same pieces: only the accumulation order inside a piece may differ
        assert np.max(np.abs(l - l0)[np.isfinite(l0)]) <= 1e-5 and np.array_equal(np.isinf(l), np.isinf(l0))
        assert np.max(np.abs(o - o0)) <= 1e-5
    q_np = wl.q_values(w)
    pairs = [(s, h) for s in range(w.num_seqs) for h in range(w.num_q_heads)]
    check(w, q_np, o1, l1, pairs, "f32")


# ------------------------------------------------------------------ full size
BENCH_SPLITS = {2: 16, 4: 16, 5: 64, 6: 64}


@pytest.mark.parametrize("index", [1, 2, 4, 5, 6])
def test_full_size_workloads_every_output(index):
    """The decode workloads at full size, in the launch configuration the
    benchmark times (same num_splits): every (sequence, q head) output
    against the oracle, with the workload's output dtype and with fp32
    output (the references are computed on the host's cores in parallel)."""
    w = wl.decode_workload(index)
    P = BENCH_SPLITS.get(index, 1)
    print(f"case workload {index} {w.name} splits {P}", flush=True)
    kp, vp, kf, vf = build_gpu_cache(w)
    pairs = [(s, h) for s in range(w.num_seqs) for h in range(w.num_q_heads)]
    ref = oracle_decode(w, wl.q_values(w), pairs, procs=cpu_procs())
    for odt in sorted({w.out_dtype, "f32"}):
        q, o, l = run_decode(w, kp, vp, kf, vf, P, odt)
        check(w, q, o, l, pairs, odt, ref=ref)
        assert np.all(np.isfinite(o)) and np.all(np.isfinite(l))


# ------------------------------------------------------------------ norm scale
TINY = [
    # d, kbits, vbits, Hq, Hkv, ctx, splits, in dtype
    (128, [4], [4], 8, 2, [300, 40], 1, "bf16"),
    (128, [4], [2], 16, 2, [700, 1], 3, "bf16"),
    (128, [4, 3], [2], 16, 2, [500, 17], 4, "bf16"),
    (128, [3, 2], [4], 8, 2, [129], 1, "f32"),
    (64, [2], [2], 4, 1, [1000], 2, "f32"),
    (128, [4, 3], [4, 3], 8, 2, [300, 40], 2, "bf16"),
    (128, [4], [3, 2], 8, 2, [129, 500], 1, "f32"),
]


@pytest.mark.parametrize("qmul", [1.0, 2.0 ** 17])
@pytest.mark.parametrize("case", TINY, ids=[f"d{c[0]}K{c[1]}V{c[2]}P{c[6]}" for c in TINY])
def test_tiny_row_norms(case, qmul):
    """Every K and V row with its L2 norm log-uniform in [1e-7, 5e-5]: the
    stored fp16 norms are subnormal or just above.  fp32 output against the
    oracle (which uses the stored norms as they are).  With q scaled by 2^17
    the scores are of order one, so K norms read as zero would show as a
    large error; with q as drawn, tiny V norms must not underflow in the
    products of the weights and norms."""
    d, kb, vb, hq, hkv, ctx, P, idt = case
    seed = 700 + d + P + len(kb)
    w = wl.small_decode_workload(seed, len(ctx), hq, hkv, d, ctx, kb, vb, kv_dist="tiny", in_dtype=idt,
                                 out_dtype="f32", num_splits=P, max_blocks_per_seq=(max(ctx) + 15) // 16 + 1)
    print(f"case tiny norms {case} q x {qmul}", flush=True)
    kp, vp, kf, vf = build_gpu_cache(w)
    q = (wl.q_values(w) * np.float32(qmul)).astype(np.float32)
    q, o, l = run_decode(w, kp, vp, kf, vf, P, "f32", q=q)
    pairs = [(s, h) for s in range(w.num_seqs) for h in range(hq)]
    check(w, q, o, l, pairs, "f32")


def test_tiny_and_normal_rows_in_one_call():
    """Sequences of tiny rows next to sequences of ordinary rows, in one
    call and in one split segment's neighbourhood."""
    d, hq, hkv = 128, 8, 2
    w_t = wl.small_decode_workload(731, 2, hq, hkv, d, [200, 513], [4], [2], kv_dist="tiny", out_dtype="f32",
                                   num_splits=3, max_blocks_per_seq=40)
    w_n = wl.small_decode_workload(731, 2, hq, hkv, d, [200, 513], [4], [2], kv_dist="normal", out_dtype="f32",
                                   num_splits=3, max_blocks_per_seq=40)
    print("case tiny + normal rows", flush=True)
    import torch
    import quantized_paged_kv_amd as tq
    kf, vf = product_format(w_t.kfmt), product_format(w_t.vfmt)
    kp = torch.full((w_t.num_blocks, hkv, kf.tile_bytes()[1]), 0xA5, dtype=torch.uint8, device="cuda")
    vp = torch.full((w_t.num_blocks, hkv, vf.tile_bytes()[1]), 0xA5, dtype=torch.uint8, device="cuda")
    sls = slots_of(w_t.block_tables, w_t.context_lens)
    for s, ww in ((0, w_t), (1, w_n)):   # sequence 0 tiny, sequence 1 ordinary
        tq.write_kv(to_device(wl.kv_values(ww, "k", s), "bf16"), to_device(wl.kv_values(ww, "v", s), "bf16"),
                    torch.from_numpy(sls[s]).cuda(), kp, vp, kf, vf, check=True)
    q, o, l = run_decode(w_t, kp, vp, kf, vf, 3, "f32")
    ref = {}
    ref.update(oracle_decode(w_t, q, [(0, h) for h in range(hq)]))
    ref.update(oracle_decode(w_n, q, [(1, h) for h in range(hq)]))
    check(w_t, q, o, l, [(s, h) for s in range(2) for h in range(hq)], "f32", ref=ref)


@pytest.mark.parametrize("kb,vb", [([4], [4]), ([4], [2]), ([4, 3], [2]), ([3, 2], [4]), ([4, 3], [4, 3]),
                                   ([3, 2], [3, 2])])
def test_unwritten_rows_holding_nan_bytes(kb, vb):
    """Pools whose unwritten bytes are all 0xFF (NaN as fp16): the rows past
    each context length in a sequence's last block, and a block-table entry
    outside the pool (skipped, read as another block), must not leak NaN
    into the outputs."""
    import torch
    import quantized_paged_kv_amd as tq
    w = wl.small_decode_workload(741 + len(kb), 3, 8, 2, 128, [37, 250, 16 * 9 + 5], kb, vb, out_dtype="f32",
                                 num_splits=3, max_blocks_per_seq=17)
    print(f"case NaN-filled pools K{kb} V{vb}", flush=True)
    kp, vp, kf, vf = build_gpu_cache(w, fill=0xFF)
    q, o, l = run_decode(w, kp, vp, kf, vf, 3, "f32")
    pairs = [(s, h) for s in range(w.num_seqs) for h in range(w.num_q_heads)]
    check(w, q, o, l, pairs, "f32")
    bt = w.block_tables.copy()
    bt[1, 3] = w.num_blocks + 2
    err = tq.new_error_word()
    o2, l2 = tq.decode_paged(to_device(q, w.q_dtype), kp, vp, torch.from_numpy(bt).cuda(),
                             torch.from_numpy(w.context_lens).cuda(), kf, vf, w.scale, num_splits=3,
                             out_dtype=torch.float32, dev_err=err)
    torch.cuda.synchronize()
    assert err.cpu().tolist()[0] == tq.TQ_ERR_INDEX
    assert np.all(np.isfinite(o2.cpu().numpy())) and np.all(np.isfinite(l2.cpu().numpy()))


@pytest.mark.parametrize("S,P", [(64, 1), (65, 3), (130, 4)])
def test_sequences_beyond_the_first_64(S, P):
    """The work split holds the first 64 context lengths in registers and
    reads later ones from memory: 64, 65 and 130 ragged sequences (some
    empty), every output against the oracle."""
    g = wl.rng(900 + S, 1)
    ctx = g.integers(0, 200, size=S)
    ctx[::9] = 0
    w = wl.small_decode_workload(900 + S, S, 4, 2, 64, list(ctx), [4], [2], out_dtype="f32", num_splits=P,
                                 max_blocks_per_seq=(int(ctx.max()) + 15) // 16 + 1)
    print(f"case S={S} P={P}", flush=True)
    kp, vp, kf, vf = build_gpu_cache(w)
    q, o, l = run_decode(w, kp, vp, kf, vf, P, "f32")
    pairs = [(s, h) for s in range(S) for h in range(4)]
    check(w, q, o, l, pairs, "f32")


def test_context_length_out_of_range_past_the_first_64():
    """A context length past the capacity, for a sequence beyond the first
    64, is reported as (INDEX, -1 - s) and clamped to the capacity."""
    import torch
    import quantized_paged_kv_amd as tq
    S = 70
    ctx = np.full(S, 40)
    w = wl.small_decode_workload(950, S, 4, 2, 64, list(ctx), [4], [4], out_dtype="f32", num_splits=2,
                                 max_blocks_per_seq=3)
    print("case bad context length at s=66", flush=True)
    kp, vp, kf, vf = build_gpu_cache(w)
    q = wl.q_values(w)
    bt = torch.from_numpy(w.block_tables.astype(np.int32)).cuda()
    cl_host = w.context_lens.astype(np.int32).copy()
    cl_host[66] = 3 * 16 + 7   # capacity is 3 blocks = 48 tokens
    cl = torch.from_numpy(cl_host).cuda()
    err = tq.new_error_word()
    o, l = tq.decode_paged(to_device(q, w.q_dtype), kp, vp, bt, cl, kf, vf, w.scale, num_splits=2,
                           out_dtype=torch.float32, dev_err=err)
    torch.cuda.synchronize()
    code, pos = err.cpu().tolist()
    assert code == tq.TQ_ERR_INDEX and pos == -1 - 66
    # sequence 66 was written with 40 tokens; the clamped length (48) reads 8
    # more slots of its third block, which hold the sentinel bytes of a
    # never-written row: only the finiteness of the other sequences is checked
    o, l = o.cpu().numpy(), l.cpu().numpy()
    pairs = [(s, h) for s in range(S) if s != 66 for h in range(4)]
    check(w, q, o, l, pairs, "f32")


def test_blocks_at_the_top_of_a_4_gib_pool():
    """Page pools just under 4 GiB (the largest the 32-bit tile offsets
    serve): one sequence whose blocks are the last ones of the pool, written
    and decoded, against the oracle."""
    import torch
    import quantized_paged_kv_amd as tq
    w = wl.small_decode_workload(960, 1, 8, 8, 128, [100], [4], [4], out_dtype="f32", num_splits=2)
    kf, vf = product_format(w.kfmt), product_format(w.vfmt)
    tile = kf.tile_bytes()[1]
    nb = (2 ** 32 - 1) // (8 * tile)          # 8 kv heads per block
    assert nb * 8 * tile < 2 ** 32 and (nb + 1) * 8 * tile >= 2 ** 32
    print(f"case 4 GiB pool: {nb} blocks of {8 * tile} B", flush=True)
    kp = torch.full((nb, 8, tile), 0xA5, dtype=torch.uint8, device="cuda")
    vp = torch.full((nb, 8, tile), 0xA5, dtype=torch.uint8, device="cuda")
    bt = np.array([[nb - 1, nb - 3, nb - 7, nb - 2, nb - 5, nb - 4, nb - 6]], dtype=np.int64)
    n = int(w.context_lens[0])
    slots = bt[0, np.arange(n) // 16] * 16 + np.arange(n) % 16
    err = tq.new_error_word()
    tq.write_kv(to_device(wl.kv_values(w, "k", 0), w.in_dtype), to_device(wl.kv_values(w, "v", 0), w.in_dtype),
                torch.from_numpy(slots).cuda(), kp, vp, kf, vf, dev_err=err)
    tq.raise_device_error(err, "write")
    q = wl.q_values(w)
    o, l = tq.decode_paged(to_device(q, w.q_dtype), kp, vp, torch.from_numpy(bt.astype(np.int32)).cuda(),
                           torch.tensor([n], dtype=torch.int32, device="cuda"), kf, vf, w.scale, num_splits=2,
                           out_dtype=torch.float32, check=True)
    torch.cuda.synchronize()
    pairs = [(0, h) for h in range(8)]
    check(w, q, o.cpu().numpy(), l.cpu().numpy(), pairs, "f32")
    del kp, vp
    torch.cuda.empty_cache()
