"""GPU parity of tq_decode_dense: exact attention over a dense window of
boundary and recent tokens, alone and merged with tq_decode_paged's result
over the packed history, against the oracle's fp64 attention over the union
of the decoded history and the window rows.

Tolerances are the decode's (lse within 1e-4; out normwise and elementwise
2e-3, bf16 output judged net of bf16's own rounding).
"""
import math

import numpy as np
import pytest

from oracle import attn as oatt
from tests.conftest import gpu_available
from tests.helpers import oracle_format, oracle_pages, slots_of, to_device
from tests.test_gpu_decode import build_gpu_cache, check, oracle_decode, BENCH_SPLITS
import workloads as wl

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def window(seed, B, cap, Hkv, d, dtype):
    return (wl.window_values(seed, B, cap, Hkv, d, "k", dtype), wl.window_values(seed, B, cap, Hkv, d, "v", dtype))


def oracle_union(w, q, kw, vw, wlens):
    """fp64 attention over (decoded packed history) + (window rows), the
    oracle writing its own pages for the history."""
    kof, vof = oracle_format(w.kfmt), oracle_format(w.vfmt)
    sl = slots_of(w.block_tables, w.context_lens)
    slots = np.concatenate(sl) if sum(len(x) for x in sl) else np.zeros(0, np.int64)
    xs = {c: [wl.kv_values(w, c, s) for s in range(w.num_seqs)] for c in ("k", "v")}
    kp = oracle_pages(np.concatenate(xs["k"]), slots, w.num_blocks, kof, "k")
    vp = oracle_pages(np.concatenate(xs["v"]), slots, w.num_blocks, vof, "v")
    o, l = oatt.decode_window_reference(q, kw, vw, wlens, w.scale, kp, vp, w.block_tables, w.context_lens,
                                        kof, vof, 16)
    return {(s, h): (o[s, h], l[s, h]) for s in range(w.num_seqs) for h in range(w.num_q_heads)}


def run(w, kp, vp, kf, vf, kw, vw, wlens, kv_dtype, out_dtype, num_splits=1, history=True, in_place=False):
    import torch
    import quantized_paged_kv_amd as tq
    q = wl.q_values(w)
    qd = to_device(q, w.q_dtype)
    ho = hl = None
    if history:
        bt = torch.from_numpy(w.block_tables.astype(np.int32)).cuda()
        cl = torch.from_numpy(w.context_lens.astype(np.int32)).cuda()
        ho, hl = tq.decode_paged(qd, kp, vp, bt, cl, kf, vf, w.scale, num_splits=num_splits,
                                 out_dtype=torch.float32, check=True)
    kwd, vwd = to_device(kw, kv_dtype), to_device(vw, kv_dtype)
    lens = torch.from_numpy(np.asarray(wlens, dtype=np.int32)).cuda()
    od = torch.float32 if out_dtype == "f32" else torch.bfloat16
    if in_place:
        o, l = tq.decode_dense(qd, kwd, vwd, lens, w.scale, hist_out=ho, hist_lse=hl, out=ho, lse=hl, check=True)
    else:
        o, l = tq.decode_dense(qd, kwd, vwd, lens, w.scale, hist_out=ho, hist_lse=hl, out_dtype=od, check=True)
    torch.cuda.synchronize()
    return q, o.float().cpu().numpy(), l.cpu().numpy()


CASES = [
    # d, kbits, vbits, Hq, Hkv, ctx, splits, window capacity, window lengths, q/kv dtype, window dtype, out
    (128, [4], [4], 8, 2, [37, 0, 200, 16], 1, 40, [5, 40, 0, 23], "bf16", "bf16", "f32"),
    (128, [4], [4], 8, 2, [37, 0, 200, 16], 3, 40, [5, 40, 0, 23], "bf16", "bf16", "bf16"),
    (128, [4, 3], [2], 16, 2, [700, 64], 4, 300, [300, 257], "bf16", "bf16", "bf16"),
    (128, [4], [2], 4, 4, [95, 1], 2, 513, [1, 513], "f32", "f32", "f32"),
    (64, [4], [4], 8, 1, [129, 0, 3], 1, 260, [256, 257, 0], "f32", "bf16", "f32"),
    (64, [2], [2], 6, 3, [5, 400], 2, 8, [8, 7], "bf16", "f32", "bf16"),
]


@pytest.mark.parametrize("case", CASES, ids=[f"d{c[0]}G{c[3]//c[4]}cap{c[7]}{c[10]}{c[11]}" for c in CASES])
def test_window_merged_with_history(case):
    d, kb, vb, hq, hkv, ctx, P, cap, wlens, idt, wdt, odt = case
    seed = 300 + d + cap + P
    print(f"case {case}", flush=True)
    w = wl.small_decode_workload(seed, len(ctx), hq, hkv, d, ctx, kb, vb, in_dtype=idt, out_dtype=odt,
                                 num_splits=P, max_blocks_per_seq=(max(ctx) + 15) // 16 + 1)
    kp, vp, kf, vf = build_gpu_cache(w)
    kw, vw = window(seed, len(ctx), cap, hkv, d, wdt)
    q, o, l = run(w, kp, vp, kf, vf, kw, vw, wlens, wdt, odt, num_splits=P)
    pairs = [(s, h) for s in range(w.num_seqs) for h in range(hq)]
    check(w, q, o, l, pairs, odt, ref=oracle_union(w, q, kw, vw, wlens))


def test_window_alone_and_in_place():
    """No history: plain attention over the window; then the in-place merge
    (out = hist_out, lse = hist_lse) equals the out-of-place one."""
    import torch
    import quantized_paged_kv_amd as tq
    w = wl.small_decode_workload(41, 3, 8, 2, 128, [300, 17, 0], [4], [2], out_dtype="f32")
    kp, vp, kf, vf = build_gpu_cache(w)
    kw, vw = window(41, 3, 33, 2, 128, "bf16")
    wlens = [33, 0, 9]
    print("case window alone", flush=True)
    q, o, l = run(w, kp, vp, kf, vf, kw, vw, wlens, "bf16", "f32", history=False)
    ref = {}
    G = 4
    for s in range(3):
        for h in range(8):
            ref[(s, h)] = oatt.attention(q[s, h].astype(np.float64), kw[s, :wlens[s], h // G].astype(np.float64),
                                         vw[s, :wlens[s], h // G].astype(np.float64), w.scale)
    check(w, q, o, l, list(ref), "f32", ref=ref)
    print("case in place", flush=True)
    _, o1, l1 = run(w, kp, vp, kf, vf, kw, vw, wlens, "bf16", "f32")
    _, o2, l2 = run(w, kp, vp, kf, vf, kw, vw, wlens, "bf16", "f32", in_place=True)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    check(w, q, o1, l1, list(ref), "f32", ref=oracle_union(w, q, kw, vw, wlens))


@pytest.mark.parametrize("d", [64, 128])
def test_window_sixteen_q_heads_per_kv_head(d):
    """G = 16 (more than the paged decode serves): window alone, f32 rows,
    lengths around the 256-token chunk boundary."""
    w = wl.small_decode_workload(45 + d, 3, 32, 2, d, [1, 1, 1], [4], [4], in_dtype="f32", out_dtype="f32")
    kw, vw = window(45 + d, 3, 300, 2, d, "f32")
    wlens = [256, 257, 300]
    print(f"case G16 d{d}", flush=True)
    q, o, l = run(w, None, None, None, None, kw, vw, wlens, "f32", "f32", history=False)
    ref = {}
    for s in range(3):
        for h in range(32):
            ref[(s, h)] = oatt.attention(q[s, h].astype(np.float64), kw[s, :wlens[s], h // 16].astype(np.float64),
                                         vw[s, :wlens[s], h // 16].astype(np.float64), w.scale)
    check(w, q, o, l, list(ref), "f32", ref=ref)


def test_window_lengths_out_of_range_are_reported_and_clamped():
    import torch
    import quantized_paged_kv_amd as tq
    w = wl.small_decode_workload(43, 2, 4, 1, 64, [20, 20], [4], [4], out_dtype="f32")
    kw, vw = window(43, 2, 12, 1, 64, "bf16")
    q = wl.q_values(w)
    print("case bad window lengths", flush=True)
    err = tq.new_error_word()
    lens = torch.tensor([-3, 50], dtype=torch.int32, device="cuda")
    o, l = tq.decode_dense(to_device(q, w.q_dtype), to_device(kw, "bf16"), to_device(vw, "bf16"), lens, w.scale,
                           out_dtype=torch.float32, dev_err=err)
    torch.cuda.synchronize()
    code, pos = err.cpu().tolist()
    assert code == tq.TQ_ERR_INDEX and pos in (-1, -2)
    o, l = o.cpu().numpy(), l.cpu().numpy()
    assert np.all(o[0] == 0) and np.all(l[0] == -math.inf)       # clamped to 0 tokens
    ref = {(1, h): oatt.attention(q[1, h].astype(np.float64), kw[1, :, 0].astype(np.float64),
                                  vw[1, :, 0].astype(np.float64), w.scale) for h in range(4)}
    check(w, q, o, l, list(ref), "f32", ref=ref)                  # clamped to the capacity
    with pytest.raises(IndexError):
        tq.decode_dense(to_device(q, w.q_dtype), to_device(kw, "bf16"), to_device(vw, "bf16"), lens, w.scale,
                        out_dtype=torch.float32, check=True)


def test_full_size_8b_shape_with_window():
    """The 8B-shaped packed cache at full size (the benchmark's split count)
    plus a 132-token dense window per sequence (4 boundary + 128 recent
    tokens, bf16); sampled outputs against the oracle, whose union result is
    the merge of its history and window attention (the merge identity)."""
    w = wl.decode_workload(2)
    P = BENCH_SPLITS.get(2, 1)
    print(f"case workload 2 + window, splits {P}", flush=True)
    kp, vp, kf, vf = build_gpu_cache(w)
    cap = 132
    kw, vw = window(2, w.num_seqs, cap, w.num_kv_heads, w.head_dim, "bf16")
    wlens = [cap] * w.num_seqs
    q, o, l = run(w, kp, vp, kf, vf, kw, vw, wlens, "bf16", w.out_dtype, num_splits=P)
    pairs = [(s, h) for s in (0, 13, 31) for h in range(w.num_q_heads)]
    hist = oracle_decode(w, q, pairs)
    G = w.num_q_heads // w.num_kv_heads
    ref = {}
    for s, h in pairs:
        ow, lw = oatt.attention(q[s, h].astype(np.float64), kw[s, :, h // G].astype(np.float64),
                                vw[s, :, h // G].astype(np.float64), w.scale)
        ref[(s, h)] = oatt.merge_partials(np.stack([hist[(s, h)][0], ow]), np.array([hist[(s, h)][1], lw]))
    check(w, q, o, l, pairs, w.out_dtype, ref=ref)


# ---------------------------------------------------------------- one call
# tq_decode_paged_window: the packed history and the bf16 window in one call
# (window items in the persistent decode workgroups, one more merge slot).

def run_fused(w, kp, vp, kf, vf, kw, vw, wlens, num_splits, out_dtype, q=None):
    import torch
    import quantized_paged_kv_amd as tq
    q = wl.q_values(w) if q is None else q
    bt = torch.from_numpy(w.block_tables.astype(np.int32)).cuda()
    cl = torch.from_numpy(w.context_lens.astype(np.int32)).cuda()
    lens = torch.from_numpy(np.asarray(wlens, dtype=np.int32)).cuda()
    od = torch.float32 if out_dtype == "f32" else torch.bfloat16
    o, l = tq.decode_paged_window(to_device(q, w.q_dtype), kp, vp, bt, cl, kf, vf, to_device(kw, "bf16"),
                                  to_device(vw, "bf16"), lens, w.scale, num_splits=num_splits, out_dtype=od,
                                  check=True)
    torch.cuda.synchronize()
    return q, o.float().cpu().numpy(), l.cpu().numpy()


FUSED = [
    # d, kbits, vbits, Hq, Hkv, ctx, splits, window capacity, window lengths, q dtype, out
    (128, [4], [4], 8, 2, [37, 0, 200, 16], 1, 40, [5, 40, 0, 23], "bf16", "f32"),
    (128, [4], [4], 8, 2, [37, 0, 200, 16], 3, 40, [5, 40, 0, 23], "bf16", "bf16"),
    # history and window both empty, each alone
    (128, [4], [2], 8, 2, [0, 0, 33, 1], 2, 12, [0, 12, 0, 1], "bf16", "f32"),
    # the 128-token chunks of the item: lengths across two boundaries
    (128, [4, 3], [2], 16, 2, [700, 64], 4, 300, [300, 257], "bf16", "bf16"),
    (128, [3, 2], [4, 3], 16, 2, [700, 64, 0], 5, 129, [128, 129, 127], "bf16", "f32"),
    (128, [2], [3, 2], 4, 4, [95, 257], 1, 129, [1, 129], "f32", "f32"),
    (128, [4], [4], 32, 2, [300, 17], 2, 200, [200, 31], "bf16", "f32"),   # 16 q heads per kv head
    (64, [4], [4], 32, 2, [129, 0, 3], 1, 260, [256, 257, 0], "f32", "f32"),
    (64, [4], [2], 6, 3, [5, 400], 2, 8, [8, 7], "bf16", "bf16"),
    (64, [4, 3], [4, 3], 2, 2, [129, 1000], 3, 70, [70, 64], "f32", "f32"),
    (64, [3, 2], [2], 8, 1, [1000, 16], 7, 150, [150, 149], "bf16", "f32"),
]


@pytest.mark.parametrize("case", FUSED, ids=[f"d{c[0]}K{c[1]}V{c[2]}G{c[3]//c[4]}P{c[6]}cap{c[7]}{c[10]}"
                                             for c in FUSED])
def test_fused_window_against_oracle(case):
    d, kb, vb, hq, hkv, ctx, P, cap, wlens, idt, odt = case
    seed = 800 + d + cap + P
    print(f"case fused {case}", flush=True)
    w = wl.small_decode_workload(seed, len(ctx), hq, hkv, d, ctx, kb, vb, in_dtype=idt, out_dtype=odt,
                                 num_splits=P, max_blocks_per_seq=(max(ctx) + 15) // 16 + 1)
    kp, vp, kf, vf = build_gpu_cache(w)
    kw, vw = window(seed, len(ctx), cap, hkv, d, "bf16")
    q, o, l = run_fused(w, kp, vp, kf, vf, kw, vw, wlens, P, odt)
    pairs = [(s, h) for s in range(w.num_seqs) for h in range(hq)]
    check(w, q, o, l, pairs, odt, ref=oracle_union(w, q, kw, vw, wlens))


def test_fused_window_matches_the_two_call_path():
    """Same inputs through tq_decode_paged + tq_decode_dense and through the
    one call: both within the decode tolerance of each other (different
    merge orders, so not bit-equal), and of the oracle."""
    w = wl.small_decode_workload(77, 4, 16, 2, 128, [513, 0, 40, 1100], [4], [4], out_dtype="f32", num_splits=3,
                                 max_blocks_per_seq=70)
    kp, vp, kf, vf = build_gpu_cache(w)
    kw, vw = window(77, 4, 132, 2, 128, "bf16")
    wlens = [132, 100, 0, 17]
    print("case fused vs two calls", flush=True)
    q, o1, l1 = run_fused(w, kp, vp, kf, vf, kw, vw, wlens, 3, "f32")
    _, o2, l2 = run(w, kp, vp, kf, vf, kw, vw, wlens, "bf16", "f32", num_splits=3)
    ref = oracle_union(w, q, kw, vw, wlens)
    pairs = list(ref)
    check(w, q, o1, l1, pairs, "f32", ref=ref)
    assert np.max(np.abs(l1 - l2)[np.isfinite(l2)]) <= 1e-4
    assert np.array_equal(np.isfinite(l1), np.isfinite(l2))
    assert np.max(np.abs(o1 - o2)) <= 2e-3


def test_fused_window_with_qjl_history():
    """A K format with the QJL stage (matrix-core sketch term, 8 q heads per
    kv head): the history's reference is the oracle's QJL estimator, merged
    with the window's exact attention by the merge identity."""
    from tests.test_gpu_qjl import build_cache
    w = wl.small_decode_workload(81, 3, 16, 2, 128, [300, 0, 77], [3, 2], [2], out_dtype="f32", num_splits=2,
                                 max_blocks_per_seq=20, qjl=True)
    kp, vp = build_cache(w)
    kf, vf = w._gpu_formats
    kw, vw = window(81, 3, 64, 2, 128, "bf16")
    wlens = [64, 5, 0]
    print("case fused window + QJL", flush=True)
    q, o, l = run_fused(w, kp, vp, kf, vf, kw, vw, wlens, 2, "f32")
    kof, vof = oracle_format(w.kfmt), oracle_format(w.vfmt)
    sl = slots_of(w.block_tables, w.context_lens)
    nonempty = [s for s in range(w.num_seqs) if len(sl[s])]
    allsl = np.concatenate([sl[s] for s in nonempty])
    okp = oracle_pages(np.concatenate([wl.kv_values(w, "k", s) for s in nonempty]), allsl, w.num_blocks, kof, "k")
    ovp = oracle_pages(np.concatenate([wl.kv_values(w, "v", s) for s in nonempty]), allsl, w.num_blocks, vof, "v")
    oh, lh = oatt.decode_reference(q.astype(np.float64), okp, ovp, w.block_tables, w.context_lens, kof, vof,
                                   w.scale, 16)
    G = 8
    ref = {}
    for s in range(3):
        for h in range(16):
            ow, lw = oatt.attention(q[s, h].astype(np.float64), kw[s, :wlens[s], h // G].astype(np.float64),
                                    vw[s, :wlens[s], h // G].astype(np.float64), w.scale)
            ref[(s, h)] = oatt.merge_partials(np.stack([np.nan_to_num(oh[s, h]), ow]), np.array([lh[s, h], lw]))
    check(w, q, o, l, list(ref), "f32", ref=ref)


def test_fused_window_lengths_out_of_range_and_empty_capacity():
    import torch
    import quantized_paged_kv_amd as tq
    w = wl.small_decode_workload(83, 2, 4, 1, 64, [20, 40], [4], [4], out_dtype="f32")
    kp, vp, kf, vf = build_gpu_cache(w)
    kw, vw = window(83, 2, 12, 1, 64, "bf16")
    q = wl.q_values(w)
    bt = torch.from_numpy(w.block_tables.astype(np.int32)).cuda()
    cl = torch.from_numpy(w.context_lens.astype(np.int32)).cuda()
    print("case fused bad window lengths", flush=True)
    err = tq.new_error_word()
    lens = torch.tensor([-3, 50], dtype=torch.int32, device="cuda")
    o, l = tq.decode_paged_window(to_device(q, w.q_dtype), kp, vp, bt, cl, kf, vf, to_device(kw, "bf16"),
                                  to_device(vw, "bf16"), lens, w.scale, out_dtype=torch.float32, dev_err=err)
    torch.cuda.synchronize()
    code, pos = err.cpu().tolist()
    assert code == tq.TQ_ERR_INDEX and pos in (-1, -2)
    o, l = o.cpu().numpy(), l.cpu().numpy()
    check(w, q, o, l, [(s, h) for s in range(2) for h in range(4)], "f32",
          ref=oracle_union(w, q, kw, vw, [0, 12]))   # clamped to 0 and to the capacity
    print("case fused zero capacity", flush=True)
    e = torch.empty((2, 0, 1, 64), dtype=torch.bfloat16, device="cuda")
    zl = torch.zeros(2, dtype=torch.int32, device="cuda")
    o, l = tq.decode_paged_window(to_device(q, w.q_dtype), kp, vp, bt, cl, kf, vf, e, e, zl, w.scale,
                                  out_dtype=torch.float32, check=True)
    torch.cuda.synchronize()
    check(w, q, o.cpu().numpy(), l.cpu().numpy(), [(s, h) for s in range(2) for h in range(4)], "f32")


def test_fused_window_full_size_8b_shape():
    """The 8B-shaped packed cache at full size with the benchmark's split
    count and a 132-token bf16 window per sequence, in one call; sampled
    outputs against the oracle's history merged with its window attention."""
    w = wl.decode_workload(2)
    P = BENCH_SPLITS.get(2, 1)
    print(f"case fused workload 2 + window, splits {P}", flush=True)
    kp, vp, kf, vf = build_gpu_cache(w)
    cap = 132
    kw, vw = window(2, w.num_seqs, cap, w.num_kv_heads, w.head_dim, "bf16")
    wlens = [cap] * w.num_seqs
    q, o, l = run_fused(w, kp, vp, kf, vf, kw, vw, wlens, P, w.out_dtype)
    pairs = [(s, h) for s in (0, 13, 31) for h in range(w.num_q_heads)]
    hist = oracle_decode(w, q, pairs)
    G = w.num_q_heads // w.num_kv_heads
    ref = {}
    for s, h in pairs:
        ow, lw = oatt.attention(q[s, h].astype(np.float64), kw[s, :, h // G].astype(np.float64),
                                vw[s, :, h // G].astype(np.float64), w.scale)
        ref[(s, h)] = oatt.merge_partials(np.stack([hist[(s, h)][0], ow]), np.array([hist[(s, h)][1], lw]))
    check(w, q, o, l, pairs, w.out_dtype, ref=ref)
