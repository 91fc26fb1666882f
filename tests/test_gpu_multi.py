"""GPU parity of tq_decode_paged_multi: several queries per sequence attend
the packed pages causally (query i sees the first ctx - (NQ - 1 - i)
tokens), against the oracle's fp64 multi-query reference over the oracle's
own pages.  Tolerances are the decode's (lse 1e-4; out 2e-3 normwise and
elementwise, bf16 output net of bf16's own rounding)."""
import math

import numpy as np
import pytest

from oracle import attn as oatt
from oracle import pages as opg
from tests.conftest import gpu_available
from tests.helpers import oracle_format, oracle_pages, slots_of, to_device, out_error, elem_error
from tests.test_gpu_decode import build_gpu_cache, BENCH_SPLITS, LSE_TOL, OUT_TOL
import workloads as wl

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def multi_q(w, NQ):
    """q [B, NQ, H_q, d] (exact in the workload's q dtype)."""
    g = wl.rng(w.seed, 41)
    q = g.standard_normal((w.num_seqs, NQ, w.num_q_heads, w.head_dim), dtype=np.float32)
    return wl.bf16_round(q) if w.q_dtype == "bf16" else q


def run_multi(w, kp, vp, kf, vf, q, num_splits, out_dtype):
    import torch
    import quantized_paged_kv_amd as tq
    bt = torch.from_numpy(w.block_tables.astype(np.int32)).cuda()
    cl = torch.from_numpy(w.context_lens.astype(np.int32)).cuda()
    od = torch.float32 if out_dtype == "f32" else torch.bfloat16
    o, l = tq.decode_paged(to_device(q, w.q_dtype), kp, vp, bt, cl, kf, vf, w.scale, num_splits=num_splits,
                           out_dtype=od, check=True)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), l.cpu().numpy()


def check_multi(o, l, o_ref, l_ref, out_dtype, cells):
    worst_o = worst_l = worst_e = 0.0
    for (s, i, h) in cells:
        if l_ref[s, i, h] == -math.inf:
            assert l[s, i, h] == -math.inf and np.all(o[s, i, h] == 0), (s, i, h)
            continue
        worst_o = max(worst_o, out_error(o[s, i, h][None], o_ref[s, i, h][None], out_dtype == "bf16")[0])
        worst_l = max(worst_l, abs(float(l[s, i, h]) - float(l_ref[s, i, h])))
        if out_dtype == "f32":
            worst_e = max(worst_e, float(np.max(elem_error(o[s, i, h][None], o_ref[s, i, h][None]))))
    print(f"[{out_dtype}] worst out {worst_o:.2e}  lse {worst_l:.2e}  elem {worst_e:.2e}", flush=True)
    assert worst_l <= LSE_TOL and worst_o <= OUT_TOL and worst_e <= OUT_TOL


CASES = [
    # d, kbits, vbits, Hq, Hkv, ctx, queries, splits, in dtype, out dtype
    (128, [4], [4], 8, 2, [1, 17, 300, 1000], 2, 1, "bf16", "f32"),
    (128, [4], [4], 8, 2, [1, 17, 300, 1000], 2, 5, "bf16", "bf16"),
    (128, [4], [2], 4, 4, [5, 700, 8], 8, 4, "bf16", "bf16"),
    (128, [3, 2], [2], 16, 8, [33, 100], 3, 2, "f32", "f32"),
    (64, [4, 3], [4], 2, 1, [129, 64, 2], 4, 3, "bf16", "f32"),
    (64, [2], [2], 8, 2, [3, 1000], 2, 7, "f32", "bf16"),
    # more than 8 (query, q head) columns per kv head: several column groups
    (128, [4], [4], 16, 2, [1, 17, 300, 1000], 2, 1, "bf16", "f32"),       # 16 columns
    (128, [4], [2], 16, 2, [5, 700, 40], 16, 3, "bf16", "bf16"),           # 128 columns
    (128, [4], [2], 16, 2, [2000, 37], 16, 1, "bf16", "f32"),              # 128 columns, whole segments
    (128, [4, 3], [2], 8, 2, [33, 100, 260], 5, 2, "f32", "f32"),          # 20 columns (one dead group)
    (128, [3, 2], [4], 24, 8, [48, 3, 500], 7, 1, "bf16", "bf16"),         # 21 columns, 3 q heads per kv head
    (128, [2], [4], 32, 8, [300, 1], 16, 2, "bf16", "f32"),                # 64 columns (8B-shaped heads)
    (64, [4], [4], 8, 1, [129, 64, 2000], 16, 4, "bf16", "f32"),           # 128 columns, d 64
    (64, [4, 3], [2], 4, 2, [20, 300], 32, 2, "f32", "bf16"),              # 64 columns, mixed K, d 64
]


@pytest.mark.parametrize("case", CASES, ids=[f"d{c[0]}K{c[1]}V{c[2]}G{c[3]//c[4]}NQ{c[6]}P{c[7]}{c[9]}" for c in CASES])
def test_multi_query_small(case):
    d, kb, vb, hq, hkv, ctx, NQ, P, idt, odt = case
    seed = 500 + d + NQ * 3 + P
    print(f"case {case}", flush=True)
    w = wl.small_decode_workload(seed, len(ctx), hq, hkv, d, ctx, kb, vb, in_dtype=idt, out_dtype=odt,
                                 num_splits=P, max_blocks_per_seq=(max(ctx) + 15) // 16 + 1)
    kp, vp, kf, vf = build_gpu_cache(w)
    q = multi_q(w, NQ)
    o, l = run_multi(w, kp, vp, kf, vf, q, P, odt)
    kof, vof = oracle_format(w.kfmt), oracle_format(w.vfmt)
    sl = slots_of(w.block_tables, w.context_lens)
    slots = np.concatenate(sl)
    okp = oracle_pages(np.concatenate([wl.kv_values(w, "k", s) for s in range(w.num_seqs)]), slots,
                       w.num_blocks, kof, "k")
    ovp = oracle_pages(np.concatenate([wl.kv_values(w, "v", s) for s in range(w.num_seqs)]), slots,
                       w.num_blocks, vof, "v")
    o_ref, l_ref = oatt.decode_multi_reference(q.astype(np.float64), okp, ovp, w.block_tables, w.context_lens,
                                               kof, vof, w.scale, 16)
    cells = [(s, i, h) for s in range(w.num_seqs) for i in range(NQ) for h in range(hq)]
    check_multi(o, l, o_ref, l_ref, odt, cells)


def test_multi_query_full_size_8b_shape():
    """The 8B-shaped cache at full size, two queries per sequence (4 q heads
    per kv head: all 8 columns), the benchmark's split count; sampled
    sequences against the oracle."""
    w = wl.decode_workload(2)
    P = BENCH_SPLITS[2]
    NQ = 2
    print(f"case workload 2, {NQ} queries, splits {P}", flush=True)
    kp, vp, kf, vf = build_gpu_cache(w)
    q = multi_q(w, NQ)
    o, l = run_multi(w, kp, vp, kf, vf, q, P, w.out_dtype)
    kof, vof = oracle_format(w.kfmt), oracle_format(w.vfmt)
    G = w.num_q_heads // w.num_kv_heads
    seqs = (0, 13, 31)
    o_ref = np.zeros(o.shape)
    l_ref = np.full(l.shape, -math.inf)
    for s in seqs:
        n = int(w.context_lens[s])
        xk, xv = wl.kv_values(w, "k", s), wl.kv_values(w, "v", s)
        bt = np.arange((n + 15) // 16)
        sl = bt[np.arange(n) // 16] * 16 + np.arange(n) % 16
        for kvh in range(w.num_kv_heads):
            Kp = np.zeros((len(bt), 1, opg.tile_layout(kof, 16)[2]), np.uint8)
            Vp = np.zeros((len(bt), 1, opg.tile_layout(vof, 16)[2]), np.uint8)
            opg.write_pages(xk[:, kvh:kvh + 1], sl, Kp, kof, 16)
            opg.write_pages(xv[:, kvh:kvh + 1], sl, Vp, vof, 16, "v")
            K = opg.reconstruct_sequence(Kp, bt, n, 0, kof, 16)
            V = opg.reconstruct_sequence(Vp, bt, n, 0, vof, 16, role="v")
            for i in range(NQ):
                c = n - (NQ - 1 - i)
                for h in range(kvh * G, (kvh + 1) * G):
                    o_ref[s, i, h], l_ref[s, i, h] = oatt.attention(q[s, i, h].astype(np.float64), K[:c], V[:c],
                                                                    w.scale)
    cells = [(s, i, h) for s in seqs for i in range(NQ) for h in range(w.num_q_heads)]
    check_multi(o, l, o_ref, l_ref, w.out_dtype, cells)


SINGLE_WIDE = [
    # d, kbits, vbits, Hq, Hkv, ctx, splits, out dtype: one query, more than 8 q heads per kv head
    (128, [4], [4], 32, 2, [1, 200, 1000], 1, "f32"),
    (128, [4, 3], [2], 256, 2, [70, 500], 3, "bf16"),
    (64, [2], [4], 48, 1, [33, 900], 2, "f32"),
]


@pytest.mark.parametrize("case", SINGLE_WIDE, ids=[f"d{c[0]}K{c[1]}V{c[2]}G{c[3]//c[4]}P{c[6]}" for c in SINGLE_WIDE])
def test_single_query_wide_groups(case):
    """One query per sequence with 16 to 128 q heads per kv head (q [B, H_q,
    d]) against the fp64 oracle."""
    import torch
    import quantized_paged_kv_amd as tq
    d, kb, vb, hq, hkv, ctx, P, odt = case
    print(f"case {case}", flush=True)
    w = wl.small_decode_workload(900 + hq + P, len(ctx), hq, hkv, d, ctx, kb, vb, out_dtype=odt, num_splits=P,
                                 max_blocks_per_seq=(max(ctx) + 15) // 16 + 1)
    kp, vp, kf, vf = build_gpu_cache(w)
    q = multi_q(w, 1)[:, 0]
    bt = torch.from_numpy(w.block_tables.astype(np.int32)).cuda()
    cl = torch.from_numpy(w.context_lens.astype(np.int32)).cuda()
    od = torch.float32 if odt == "f32" else torch.bfloat16
    o, l = tq.decode_paged(to_device(q, w.q_dtype), kp, vp, bt, cl, kf, vf, w.scale, num_splits=P, out_dtype=od,
                           check=True)
    torch.cuda.synchronize()
    o, l = o.float().cpu().numpy()[:, None], l.cpu().numpy()[:, None]
    kof, vof = oracle_format(w.kfmt), oracle_format(w.vfmt)
    slots = np.concatenate(slots_of(w.block_tables, w.context_lens))
    okp = oracle_pages(np.concatenate([wl.kv_values(w, "k", s) for s in range(w.num_seqs)]), slots,
                       w.num_blocks, kof, "k")
    ovp = oracle_pages(np.concatenate([wl.kv_values(w, "v", s) for s in range(w.num_seqs)]), slots,
                       w.num_blocks, vof, "v")
    o_ref, l_ref = oatt.decode_multi_reference(q[:, None].astype(np.float64), okp, ovp, w.block_tables,
                                               w.context_lens, kof, vof, w.scale, 16)
    cells = [(s, 0, h) for s in range(w.num_seqs) for h in range(hq)]
    check_multi(o, l, o_ref, l_ref, odt, cells)


def test_multi_query_full_size_70b_shape():
    """The 70B-shaped cache at full size (8 sequences x 32768 tokens, 8 q
    heads per kv head) with 16 queries per sequence: 128 columns per kv
    head, the benchmark's split count; every (query, q head) output of
    sampled (sequence, kv head) pairs, every kv head once, against the
    oracle."""
    w = wl.decode_workload(4)
    P = BENCH_SPLITS[4]
    NQ = 16
    print(f"case workload 4, {NQ} queries, splits {P}", flush=True)
    kp, vp, kf, vf = build_gpu_cache(w)
    q = multi_q(w, NQ)
    o, l = run_multi(w, kp, vp, kf, vf, q, P, w.out_dtype)
    kof, vof = oracle_format(w.kfmt), oracle_format(w.vfmt)
    G = w.num_q_heads // w.num_kv_heads
    pairs = {0: range(0, 4), 5: range(4, 8)}   # sequence -> kv heads
    o_ref = np.zeros(o.shape)
    l_ref = np.full(l.shape, -math.inf)
    cells = []
    for s, heads in pairs.items():
        n = int(w.context_lens[s])
        xk, xv = wl.kv_values(w, "k", s), wl.kv_values(w, "v", s)
        bt = np.arange((n + 15) // 16)
        sl = bt[np.arange(n) // 16] * 16 + np.arange(n) % 16
        for kvh in heads:
            cells += [(s, i, h) for i in range(NQ) for h in range(kvh * G, (kvh + 1) * G)]
            Kp = np.zeros((len(bt), 1, opg.tile_layout(kof, 16)[2]), np.uint8)
            Vp = np.zeros((len(bt), 1, opg.tile_layout(vof, 16)[2]), np.uint8)
            opg.write_pages(xk[:, kvh:kvh + 1], sl, Kp, kof, 16)
            opg.write_pages(xv[:, kvh:kvh + 1], sl, Vp, vof, 16, "v")
            K = opg.reconstruct_sequence(Kp, bt, n, 0, kof, 16)
            V = opg.reconstruct_sequence(Vp, bt, n, 0, vof, 16, role="v")
            for i in range(NQ):
                c = n - (NQ - 1 - i)
                for h in range(kvh * G, (kvh + 1) * G):
                    o_ref[s, i, h], l_ref[s, i, h] = oatt.attention(q[s, i, h].astype(np.float64), K[:c], V[:c],
                                                                    w.scale)
        print(f"  sequence {s} referenced", flush=True)
    check_multi(o, l, o_ref, l_ref, w.out_dtype, cells)
