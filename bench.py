"""Benchmark of one decode layer-step over a packed, paged KV cache.

A step = quantise-on-write of the current token of every sequence
(tq_write_kv) + paged decode attention over the whole context
(tq_decode_paged, split-K with its merge), for one layer.  The timed loop
cycles over several layers' caches whose pools together exceed the 256 MB
Infinity Cache, so every step streams its pages from HBM, as a real
multi-layer decode does.

Default workload: the Llama-3-8B-shaped layer (batch 32, 32 q / 8 kv heads,
d = 128, context lengths uniform in [1024, 8192], K4/V4).  The
Llama-3.1-70B-shaped layer share (batch 8, 64 q / 8 kv heads, context
32768, K4/V2) is measured in the same run and reported under "secondary".

Prints one JSON line.  Inputs are seeded synthetic tensors of the
workloads' shapes and distributions (data: "synthetic").
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
PEAK_F16_TFLOPS = 2500.0   # dense fp16 matrix-core peak
SPLITS = {2: 16, 4: 16, 5: 64, 6: 64, 7: 64, 1: 1}
LAYERS = {2: 3, 4: 2, 5: 1, 6: 1, 7: 1, 1: 1}
FLUSH_BYTES = 1 << 30
NAMES = {"8b": 2, "70b": 4, "long": 5, "long25": 6, "long_qjl": 7, "tiny": 1}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def algorithmic_bytes(w, kf, vf):
    """Bytes the method must move in one layer-step (decode + write)."""
    import numpy as np
    krow = kf.tile_bytes()[0] + 2 * kf.num_groups * (2 if kf.qjl else 1)   # index bytes + norms (+ residual norms)
    vrow = vf.tile_bytes()[0] + 2 * vf.num_groups
    ctx = w.context_lens.astype(np.int64)
    cache = int(ctx.sum()) * w.num_kv_heads * (krow + vrow)
    esz = 2 if w.q_dtype == "bf16" else 4
    q = w.num_seqs * w.num_q_heads * w.head_dim * esz
    out = w.num_seqs * w.num_q_heads * w.head_dim * (2 if w.out_dtype == "bf16" else 4)
    lse = w.num_seqs * w.num_q_heads * 4
    bt = int(((ctx + 15) // 16).sum()) * 4 + w.num_seqs * 4
    decode = cache + q + out + lse + bt
    write = w.num_seqs * w.num_kv_heads * (2 * w.head_dim * esz + krow + vrow) + w.num_seqs * 8
    return decode, write


def kernel_source_hash():
    h = hashlib.sha256()
    for f in ("decode.hip", "tq_internal.h", "window_item.h"):
        h.update(open(os.path.join(ROOT, "quantized_paged_kv_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def stored_traffic(tag):
    """HBM bytes per decode launch from committed rocprofv3 counter runs, if
    they were taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", f"decode_{tag}_counters.json")
    if not os.path.exists(path):
        return None
    d = json.load(open(path))
    if d.get("kernel_sha") != kernel_source_hash():
        return None
    return d.get("hbm_bytes_per_launch")


class Bench:
    def __init__(self, index, layers=None, splits=None, device="cuda"):
        import numpy as np
        import torch
        import quantized_paged_kv_amd as tq
        import workloads as wl
        self.tq, self.torch, self.np = tq, torch, np
        self.w = w = wl.decode_workload(index)
        self.index = index
        self.P = splits or SPLITS[index]
        self.L = layers or LAYERS[index]
        proj = None if w.kfmt.qjl_proj is None else torch.from_numpy(w.kfmt.qjl_proj.copy()).cuda()
        kf = tq.Format(w.head_dim, w.kfmt.group_bits, w.kfmt.signs, w.kfmt.group_channels, qjl_proj=proj)
        vf = tq.Format(w.head_dim, w.vfmt.group_bits, w.vfmt.signs, w.vfmt.group_channels)
        self.kf, self.vf = kf, vf
        dt = torch.bfloat16 if w.in_dtype == "bf16" else torch.float32
        self.pools = [(tq.alloc_pages(w.num_blocks, w.num_kv_heads, kf), tq.alloc_pages(w.num_blocks, w.num_kv_heads, vf))
                      for _ in range(self.L)]
        err = tq.new_error_word()
        last_k, last_v, last_slot = [], [], []
        for s in range(w.num_seqs):
            n = int(w.context_lens[s])
            t = np.arange(n)
            sl = torch.from_numpy(w.block_tables[s, t // 16].astype(np.int64) * 16 + t % 16).cuda()
            xk = self._dev(wl.kv_values(w, "k", s), w.in_dtype)
            xv = self._dev(wl.kv_values(w, "v", s), w.in_dtype)
            for kp, vp in self.pools:
                tq.write_kv(xk, xv, sl, kp, vp, kf, vf, dev_err=err)
            last_k.append(xk[-1:])
            last_v.append(xv[-1:])
            last_slot.append(sl[-1:])
            del xk, xv
        tq.raise_device_error(err, "cache build")
        log(f"cache built: {w.name}, {self.L} layer pools")
        # the current token of every sequence (the last cached position)
        self.new_k = torch.cat(last_k).contiguous()
        self.new_v = torch.cat(last_v).contiguous()
        self.new_slots = torch.cat(last_slot).contiguous()
        self.q = self._dev(wl.q_values(w), w.q_dtype)
        self.bt = torch.from_numpy(w.block_tables).cuda()
        self.cl = torch.from_numpy(w.context_lens).cuda()
        od = torch.bfloat16 if w.out_dtype == "bf16" else torch.float32
        self.out = torch.empty((w.num_seqs, w.num_q_heads, w.head_dim), dtype=od, device="cuda")
        self.lse = torch.empty((w.num_seqs, w.num_q_heads), dtype=torch.float32, device="cuda")
        nbytes = tq.workspace_bytes(w.num_seqs, w.num_q_heads, w.head_dim, self.P)
        self.ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")
        self.decode_bytes, self.write_bytes = algorithmic_bytes(w, kf, vf)
        torch.cuda.synchronize()

    def _dev(self, x, dtype):
        import workloads as wl
        np, torch = self.np, self.torch
        if dtype == "bf16":
            return torch.from_numpy(wl.to_bf16_bits(x).view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()

    def write(self, layer):
        kp, vp = self.pools[layer]
        self.tq.write_kv(self.new_k, self.new_v, self.new_slots, kp, vp, self.kf, self.vf)

    def decode(self, layer):
        kp, vp = self.pools[layer]
        w = self.w
        self.tq.decode_paged(self.q, kp, vp, self.bt, self.cl, self.kf, self.vf, w.scale, num_splits=self.P,
                             out=self.out, lse=self.lse, workspace=self.ws)

    def step(self, i):
        layer = i % self.L
        self.write(layer)
        self.decode(layer)

    def timed_cold(self, launches, warmup, flush):
        """Decode call durations (ms, sorted) with cold caches: before each
        timed call a flush reads `flush` (1 GiB, evicting L2 and the 256 MB
        Infinity Cache with clean lines, so that the timed call does not pay
        for writing back someone else's dirty data), then a GPU-side spin
        keeps the host's enqueue time out of the interval the HIP events
        bracket."""
        torch = self.torch
        for i in range(warmup):
            self.decode(i % self.L)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(launches)]
        for i in range(launches):
            layer = i % self.L
            flush_caches(flush)
            torch.cuda._sleep(200000)
            ev[i][0].record()
            self.decode(layer)
            ev[i][1].record()
        torch.cuda.synchronize()
        return sorted(a.elapsed_time(b) for a, b in ev)

    def capture(self):
        """One graph per layer pool holding that layer's step (the write of
        the current tokens, the decode and its merge): replaying it issues
        the same kernels with the same arguments, without the host's
        per-call enqueue work."""
        torch = self.torch
        for i in range(2 * self.L):   # eager warm-up (library state, allocator)
            self.step(i)
        torch.cuda.synchronize()
        self.graphs = []
        for layer in range(self.L):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                self.step(layer)
            self.graphs.append(g)
        torch.cuda.synchronize()

    def timed_graph(self, steps, warmup):
        """Wall time per layer step (ms) replaying the captured steps."""
        torch = self.torch
        if not getattr(self, "graphs", None):
            self.capture()
        for i in range(warmup):
            self.graphs[i % self.L].replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            self.graphs[(warmup + i) % self.L].replay()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / steps * 1e3

    def timed(self, steps, warmup):
        torch = self.torch
        for i in range(warmup):
            self.step(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            self.step(warmup + i)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        # per-launch decode duration with HIP events on the launch stream; a
        # short GPU-side spin before each start event keeps the host's
        # enqueue time of the call out of the measured interval
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for i in range(steps):
            layer = (warmup + i) % self.L
            self.write(layer)
            torch.cuda._sleep(200000)
            ev[i][0].record()
            self.decode(layer)
            ev[i][1].record()
        torch.cuda.synchronize()
        dec_ms = sorted(a.elapsed_time(b) for a, b in ev)
        return wall / steps * 1e3, dec_ms


def flush_caches(flush):
    """Read every byte of `flush` (int64 view; one small result)."""
    flush.view(__import__("torch").int64).max()


def write_cold(launches, warmup, flush):
    """Quantise-on-write of the write workload (16 sequences x 2048 new
    tokens, 8 kv heads, d = 128, K4/V4, Student-t(5) bf16 input) into a shared
    pool, each timed launch after a cache flush."""
    import numpy as np
    import torch
    import quantized_paged_kv_amd as tq
    import workloads as wl
    w = wl.write_workload(0)
    kf = tq.Format(w.head_dim, w.kfmt.group_bits, w.kfmt.signs, w.kfmt.group_channels)
    vf = tq.Format(w.head_dim, w.vfmt.group_bits, w.vfmt.signs, w.vfmt.group_channels)
    kp, vp = tq.alloc_pages(w.num_blocks, w.num_kv_heads, kf), tq.alloc_pages(w.num_blocks, w.num_kv_heads, vf)
    dev = lambda x: torch.from_numpy(wl.to_bf16_bits(x).view(np.int16)).view(torch.bfloat16).cuda()
    xk, xv = dev(wl.write_values(w, "k")), dev(wl.write_values(w, "v"))
    slots = torch.from_numpy(w.slot_mapping).cuda()
    for _ in range(warmup):
        tq.write_kv(xk, xv, slots, kp, vp, kf, vf)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(launches)]
    for i in range(launches):
        flush_caches(flush)
        torch.cuda._sleep(200000)
        ev[i][0].record()
        tq.write_kv(xk, xv, slots, kp, vp, kf, vf)
        ev[i][1].record()
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in ev)
    rows = w.num_tokens * w.num_kv_heads
    krow = kf.tile_bytes()[0] + 2 * kf.num_groups * (2 if kf.qjl else 1)   # index bytes + norms (+ residual norms)
    vrow = vf.tile_bytes()[0] + 2 * vf.num_groups
    nbytes = rows * (2 * w.head_dim * 2 + krow + vrow) + w.num_tokens * 8
    return w, ms, nbytes


def window_cold(b, launches, warmup, flush, cap=132):
    """Dense window next to the packed history (the 8B-shaped cache of `b`):
    every sequence keeps cap = 4 boundary + 128 recent tokens in bf16, attended
    by tq_decode_dense and merged with the history's float32 (o, lse).  Times,
    with cold caches, the window call alone and the whole window-augmented
    decode (tq_decode_paged with float32 output, then tq_decode_dense), and
    the same result from one tq_decode_paged_window call."""
    import numpy as np
    import torch
    import workloads as wl
    tq, w = b.tq, b.w
    B, Hq, Hkv, d = w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim
    kw = b._dev(wl.window_values(w.seed, B, cap, Hkv, d, "k"), "bf16")
    vw = b._dev(wl.window_values(w.seed, B, cap, Hkv, d, "v"), "bf16")
    lens = torch.full((B,), cap, dtype=torch.int32, device="cuda")
    ho = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")
    hl = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    out = torch.empty((B, Hq, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    kp, vp = b.pools[0]

    def history():
        tq.decode_paged(b.q, kp, vp, b.bt, b.cl, b.kf, b.vf, w.scale, num_splits=b.P, out=ho, lse=hl,
                        workspace=b.ws)

    def window():
        tq.decode_dense(b.q, kw, vw, lens, w.scale, hist_out=ho, hist_lse=hl, out=out, lse=lse)

    ws_f = torch.empty(max(tq.workspace_bytes(B, Hq, d, b.P + 1), 1), dtype=torch.uint8, device="cuda")

    def fused():
        tq.decode_paged_window(b.q, kp, vp, b.bt, b.cl, b.kf, b.vf, kw, vw, lens, w.scale, num_splits=b.P,
                               out=out, lse=lse, workspace=ws_f)

    res = {}
    for key, fns in (("window_us", (window,)), ("decode_plus_window_us", (history, window)),
                     ("decode_with_window_one_call_us", (fused,))):
        history()
        for _ in range(warmup):
            for f in fns:
                f()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(launches)]
        for i in range(launches):
            flush_caches(flush)
            torch.cuda._sleep(200000)
            ev[i][0].record()
            for f in fns:
                f()
            ev[i][1].record()
        torch.cuda.synchronize()
        res[key] = sorted(a.elapsed_time(c) for a, c in ev)
    win_bytes = 2 * B * cap * Hkv * d * 2                       # window K and V rows (bf16)
    io_bytes = B * Hq * d * 2 + B * Hq * (d + 1) * 4 + B * Hq * d * 2 + B * Hq * 4 + B * 4   # q, history, out, lse, lens
    return res, win_bytes + io_bytes, cap


def multi_cold(b, launches, warmup, flush, nq=2):
    """Multi-query decode on the cache of `b`: nq queries per sequence (the
    last nq cached tokens are theirs) in one call; times it with cold caches.
    Returns (sorted ms, algorithmic bytes, algorithmic flops): the flops are
    4 d per (query, q head, visible token), q.K and P.V at 2 d each."""
    import numpy as np
    import torch
    import workloads as wl
    tq, w = b.tq, b.w
    B, Hq, d = w.num_seqs, w.num_q_heads, w.head_dim
    q = b._dev(wl.bf16_round(wl.rng(w.seed, 41).standard_normal((B, nq, Hq, d), dtype=np.float32)), "bf16")
    out = torch.empty((B, nq, Hq, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, nq, Hq), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(tq.workspace_bytes(B * nq, Hq, d, b.P), 1), dtype=torch.uint8, device="cuda")

    def call(layer):
        kp, vp = b.pools[layer]
        tq.decode_paged(q, kp, vp, b.bt, b.cl, b.kf, b.vf, w.scale, num_splits=b.P, out=out, lse=lse, workspace=ws)

    for i in range(warmup):
        call(i % b.L)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(launches)]
    for i in range(launches):
        flush_caches(flush)
        torch.cuda._sleep(200000)
        ev[i][0].record()
        call(i % b.L)
        ev[i][1].record()
    torch.cuda.synchronize()
    extra = (nq - 1) * B * Hq * (2 * d * 2 + 4)   # the other queries' q, out and lse
    ctx = w.context_lens.astype(np.int64)
    visible = sum(int(np.maximum(ctx - (nq - 1 - i), 0).sum()) for i in range(nq))
    flops = 4 * d * Hq * visible
    return sorted(a.elapsed_time(c) for a, c in ev), b.decode_bytes + extra, flops


def phase_trace(index, launches, flush):
    """Per-phase times of the decode kernel from the phase-timestamp build
    (libtq_trace.so, TQ_PHASE_TRACE): each persistent workgroup records the
    100 MHz real-time counter at its phase boundaries; cold calls (flush
    before each).  Returns medians / maxima over workgroups in us."""
    import numpy as np
    import torch
    b = Bench(index)
    tq = b.tq
    n_wg = torch.cuda.get_device_properties(0).multi_processor_count
    buf = torch.zeros(16 * n_wg, dtype=torch.int64, device="cuda")
    if not tq.set_phase_trace(buf):
        raise SystemExit("the loaded library has no phase trace: run with the libtq_trace.so build")
    runs = []
    for i in range(launches):
        buf.zero_()
        flush_caches(flush)
        torch.cuda._sleep(200000)
        b.decode(i % b.L)
        torch.cuda.synchronize()
        runs.append(buf.view(n_wg, 16).cpu().numpy().astype(np.int64))
    tq.set_phase_trace(None)
    us = 0.01   # 100 MHz counter ticks
    out = {}
    keys = {"plan": (0, 1), "first_piece_prologue": (2, 3), "first_piece_loop": (3, 4),
            "first_piece_epilogue": (4, 5), "second_piece_prologue": (6, 7), "second_piece_loop": (7, 8),
            "second_piece_epilogue": (8, 9)}
    for name, (a, c) in keys.items():
        vals = []
        for r in runs:
            ok = (r[:, a] > 0) & (r[:, c] > 0)
            vals.extend(((r[ok, c] - r[ok, a]) * us).tolist())
        if vals:
            v = np.array(vals)
            out[name] = {"median": round(float(np.median(v)), 2), "max": round(float(v.max()), 2),
                         "workgroups": int(len(v) / len(runs))}
    ent, span, tail, pieces = [], [], [], []
    for r in runs:
        live = r[:, 0] > 0
        t0 = r[live, 0].min()
        ent.append(float(np.median(r[live, 0] - t0)) * us)
        span.append(float(r[live, 14].max() - t0) * us)
        tail.append(float(r[live, 14].max() - np.median(r[live, 14])) * us)
        pieces.append(float(r[live, 15].mean()))
    out["entry_after_first_workgroup"] = round(float(np.median(ent)), 2)
    out["kernel_span"] = round(float(np.median(span)), 2)
    out["exit_tail_after_median"] = round(float(np.median(tail)), 2)
    out["pieces_per_workgroup"] = round(float(np.mean(pieces)), 3)
    out["workload"] = b.w.name
    out["launches"] = launches
    return out


def stats_us(ms):
    n = len(ms)
    return {"avg": round(sum(ms) / n * 1e3, 2), "p10": round(ms[n // 10] * 1e3, 2),
            "p50": round(ms[n // 2] * 1e3, 2), "p90": round(ms[9 * n // 10] * 1e3, 2)}


def cpu_baseline(index, budget_s=12.0, gpu_out=None, gpu_lse=None):
    """The oracle (as it stands) decoding whole sequences of the workload on
    the host: dense reconstruction from oracle-written pages + fp64
    attention for every q head.  Pages are prepared untimed.

    With gpu_out / gpu_lse (the outputs of the timed tq_decode_paged calls
    of this run), every (sequence, q head) the oracle decodes is also
    compared with them: lse within 1e-4, out within 2e-3 normwise, bf16 out
    taken modulo its rounding (the distance from the fp64 reference to the
    interval of reals that round to each output value)."""
    import numpy as np
    import oracle
    from oracle import attn as oatt
    from oracle import pages as opg
    import workloads as wl
    w = wl.decode_workload(index)
    kof = oracle.Format.make(w.head_dim, w.kfmt.group_bits, w.kfmt.signs, w.kfmt.group_channels)
    vof = oracle.Format.make(w.head_dim, w.vfmt.group_bits, w.vfmt.signs, w.vfmt.group_channels)
    q = wl.q_values(w)
    G = w.num_q_heads // w.num_kv_heads
    krow = opg.tile_layout(kof, 16)[0] + 2 * kof.num_groups
    vrow = opg.tile_layout(vof, 16)[0] + 2 * vof.num_groups
    from tests.helpers import out_error
    total_bytes, total_t, done = 0, 0.0, []
    worst_out = worst_raw = worst_lse = 0.0
    checked = 0
    for s in range(w.num_seqs):
        n = int(w.context_lens[s])
        bt = np.arange((n + 15) // 16)
        sl = bt[np.arange(n) // 16] * 16 + np.arange(n) % 16
        xk, xv = wl.kv_values(w, "k", s), wl.kv_values(w, "v", s)
        pools = []
        for h in range(w.num_kv_heads):
            Kp = np.zeros((len(bt), 1, opg.tile_layout(kof, 16)[2]), np.uint8)
            Vp = np.zeros((len(bt), 1, opg.tile_layout(vof, 16)[2]), np.uint8)
            for a in range(0, n, 16384):
                opg.write_pages(xk[a:a + 16384, h:h + 1], sl[a:a + 16384], Kp, kof, 16)
                opg.write_pages(xv[a:a + 16384, h:h + 1], sl[a:a + 16384], Vp, vof, 16, "v")
            pools.append((Kp, Vp))
        t0 = time.perf_counter()
        refs = []
        for h in range(w.num_kv_heads):
            Kp, Vp = pools[h]
            K = opg.reconstruct_sequence(Kp, bt, n, 0, kof, 16)
            V = opg.reconstruct_sequence(Vp, bt, n, 0, vof, 16, role="v")
            for g in range(G):
                refs.append((h * G + g, oatt.attention(q[s, h * G + g].astype(np.float64), K, V, w.scale)))
        total_t += time.perf_counter() - t0
        if gpu_out is not None:
            for hq, (o_ref, l_ref) in refs:
                e = float(out_error(gpu_out[s, hq][None], o_ref[None], w.out_dtype == "bf16")[0])
                worst_out = max(worst_out, e)
                worst_raw = max(worst_raw, float(out_error(gpu_out[s, hq][None], o_ref[None])[0]))
                worst_lse = max(worst_lse, abs(float(gpu_lse[s, hq]) - l_ref))
                checked += 1
        total_bytes += n * w.num_kv_heads * (krow + vrow)
        done.append(s)
        if total_t >= budget_s:
            break
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        threads = 1
    cores = len(os.sched_getaffinity(0))
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as fh:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in fh if ln.startswith("model name")), "")
    except OSError:
        pass
    res = {"value": round(total_bytes / total_t / 1e9, 4), "unit": "GB/s", "cores": min(cores, threads),
            "kind": "oracle", "route": "oracle-dense-fp64 (diagnostic)",
            "allowed_cores": cores, "blas_threads": threads, "cpu_model": cpu_model,
            "numpy": np.__version__,
            "sample": f"{len(done)} whole sequence(s) of the workload ({sum(int(w.context_lens[s]) for s in done)} "
                      f"tokens x {w.num_kv_heads} kv heads x {w.num_q_heads // w.num_kv_heads} q heads each): "
                      f"dense reconstruction + fp64 attention, {total_t:.1f} s on {cores} allowed cores"}
    if gpu_out is not None:
        res["parity_same_run"] = {
            "route_checked": "tq_decode_paged (serving)", "reference": "oracle-dense-fp64 (diagnostic)",
            "rows_checked": checked, "worst_out_err": round(worst_out, 7), "worst_out_err_raw": round(worst_raw, 7),
            "worst_lse_err": round(float(worst_lse), 8),
            "reading": "per (sequence, q head): lse abs <= 1e-4; out normwise <= 2e-3 against the fp64 reference, "
                       "bf16 out modulo its rounding (distance to the interval of reals rounding to each output "
                       "element); raw = bf16 out against fp64 without that allowance",
            "pass": bool(worst_lse <= 1e-4 and worst_out <= 2e-3)}
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="8b", choices=sorted(NAMES) + ["write"],
                    help="decode workload of the step; 'write' times only the quantise-on-write workload")
    ap.add_argument("--splits", type=int, default=None)
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--phase-trace", action="store_true",
                    help="only report per-phase decode times from the phase-timestamp build (libtq_trace.so)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only copy BYTES device to device 5 times (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.calibrate_copy:
        import torch
        src = torch.ones(args.calibrate_copy, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": args.calibrate_copy, "launches": 5}), flush=True)
        return
    if args.phase_trace:
        os.environ["TQ_LIB_PATH"] = os.path.join(ROOT, "quantized_paged_kv_amd", "libtq_trace.so")
        import torch
        flush = torch.ones(FLUSH_BYTES, dtype=torch.uint8, device="cuda")
        print(json.dumps({"phase_trace_us": phase_trace(NAMES[args.workload], args.steps, flush)}), flush=True)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the decode shards by kv head or "
              f"sequence with no exchange", file=sys.stderr)
        sys.exit(2)
    import torch
    flush = torch.ones(FLUSH_BYTES, dtype=torch.uint8, device="cuda")
    if args.workload == "write":
        ww, wms, wbytes = write_cold(args.steps, args.warmup, flush)
        wavg = sum(wms) / len(wms)
        print(json.dumps({"write": {"workload": ww.name, "us": stats_us(wms), "algorithmic_bytes": wbytes,
                                    "GBs": round(wbytes / (wavg * 1e-3) / 1e9, 1),
                                    "frac_of_peak": round(wbytes / (wavg * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}}),
              flush=True)
        return
    index = NAMES[args.workload]
    b = Bench(index, splits=args.splits)
    ms_step, dec_warm = b.timed(args.steps, args.warmup)
    ms_graph = b.timed_graph(args.steps, args.warmup)
    log(f"timed {args.steps} steps: {ms_step * 1e3:.1f} us/step, {ms_graph * 1e3:.1f} us/step replayed as a graph")
    dec_ms = b.timed_cold(args.steps, args.warmup, flush)
    torch.cuda.synchronize()
    timed_out = b.out.float().cpu().numpy()   # outputs of the last timed call (the same for every layer)
    timed_lse = b.lse.cpu().numpy()
    w = b.w
    step_bytes = b.decode_bytes + b.write_bytes
    value = step_bytes / (ms_step * 1e-3) / 1e9
    dec_avg = sum(dec_ms) / len(dec_ms)
    achieved = b.decode_bytes / (dec_avg * 1e-3) / 1e9
    tag = args.workload
    traffic = stored_traffic(tag)
    result = {
        "metric": "tq_decode_paged HBM GB/s (% of peak) and us/layer-step at 8B/70B shapes",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp16-mfma/fp32-acc over u8 pages", "data": "synthetic",
        "config": {"workload": w.name, "batch": w.num_seqs, "q_heads": w.num_q_heads, "kv_heads": w.num_kv_heads,
                   "head_dim": w.head_dim, "context_tokens": int(w.context_lens.sum()),
                   "k_bits": w.kfmt.group_bits, "v_bits": w.vfmt.group_bits, "num_splits": b.P,
                   "layers_cycled": b.L, "step": "tq_write_kv(current token) + tq_decode_paged",
                   "parallelism": "single GPU"},
        "us_per_layer_step": round(ms_step * 1e3, 2),
        "us_per_layer_step_graph": round(ms_graph * 1e3, 2),
        "step_launch": "calls issued one by one (value, us_per_layer_step); us_per_layer_step_graph replays the "
                       "same step captured as a HIP graph (within a few us of the eager launches, either way)",
        "decode_us": stats_us(dec_ms),
        "decode_us_layers_cycled": stats_us(dec_warm),
        "decode_GBs_median": round(b.decode_bytes / (dec_ms[len(dec_ms) // 2] * 1e-3) / 1e9, 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": traffic, "kernel": "tq_decode_paged (decode kernel + split merge)",
                     "route": "tq_decode_paged (serving)",
                     "algorithmic_bytes_per_launch": b.decode_bytes,
                     "timing": "cold caches (1 GiB read before each launch)"},
    }
    if not args.no_secondary and index == 2:
        wres, wbytes_win, cap = window_cold(b, max(10, args.steps // 2), args.warmup, flush)
        wavg = sum(wres["window_us"]) / len(wres["window_us"])
        result["window"] = {
            "workload": f"{w.name} + dense window of {cap} bf16 tokens per sequence (4 boundary + 128 recent)",
            "window_us": stats_us(wres["window_us"]),
            "decode_plus_window_us": stats_us(wres["decode_plus_window_us"]),
            "decode_with_window_one_call_us": stats_us(wres["decode_with_window_one_call_us"]),
            "window_algorithmic_bytes": wbytes_win,
            "roofline": {"bound": "hbm", "achieved": round(wbytes_win / (wavg * 1e-3) / 1e9, 1),
                         "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(wbytes_win / (wavg * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                         "kernel": "tq_decode_dense (window attention + merge with the history)"}}
        fz = wres["decode_with_window_one_call_us"]
        log(f"window: {wavg * 1e3:.1f} us; decode + window in one call: {fz[len(fz) // 2] * 1e3:.1f} us")
        mq_ms, mq_bytes, _ = multi_cold(b, max(10, args.steps // 2), args.warmup, flush)
        mq_avg = sum(mq_ms) / len(mq_ms)
        result["multi_query"] = {
            "workload": f"{w.name}, 2 queries per sequence (causal over the cache, one call)",
            "decode_us": stats_us(mq_ms), "algorithmic_bytes": mq_bytes,
            "GBs": round(mq_bytes / (mq_avg * 1e-3) / 1e9, 1),
            "frac_of_peak": round(mq_bytes / (mq_avg * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
        log(f"multi-query: {mq_avg * 1e3:.1f} us")
    del b
    torch.cuda.empty_cache()
    if not args.no_secondary and index == 2:
        b4 = Bench(4)
        n4 = max(10, args.steps // 2)
        ms4, d4w = b4.timed(n4, args.warmup)
        ms4g = b4.timed_graph(n4, args.warmup)
        log(f"secondary timed: {ms4 * 1e3:.1f} us/step, {ms4g * 1e3:.1f} as a graph")
        d4 = b4.timed_cold(n4, args.warmup, flush)
        a4 = sum(d4) / len(d4)
        result["secondary"] = {"workload": b4.w.name, "us_per_layer_step": round(ms4 * 1e3, 2),
                               "us_per_layer_step_graph": round(ms4g * 1e3, 2),
                               "decode_us": stats_us(d4), "decode_us_layers_cycled": stats_us(d4w),
                               "decode_us_avg": round(a4 * 1e3, 2),
                               "decode_GBs": round(b4.decode_bytes / (a4 * 1e-3) / 1e9, 1),
                               "frac_of_peak": round(b4.decode_bytes / (a4 * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                               "num_splits": b4.P, "traffic": stored_traffic("70b")}
        # chunked prefill over the same cache: 16 queries per sequence, 128
        # (query, q head) columns per kv head, one call
        nq = 16
        mq_ms, mq_bytes, mq_flops = multi_cold(b4, n4, args.warmup, flush, nq=nq)
        mq_avg = sum(mq_ms) / len(mq_ms)
        mq_tf = mq_flops / (mq_avg * 1e-3) / 1e12
        result["multi_query_70b"] = {
            "workload": f"{b4.w.name}, {nq} queries per sequence (causal over the cache, one call)",
            "decode_us": stats_us(mq_ms), "num_splits": b4.P, "algorithmic_bytes": mq_bytes,
            "algorithmic_flops": mq_flops,
            "GBs": round(mq_bytes / (mq_avg * 1e-3) / 1e9, 1),
            "frac_of_hbm_peak": round(mq_bytes / (mq_avg * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "TFLOPs": round(mq_tf, 1),
            "frac_of_fp16_mfma_peak": round(mq_tf / PEAK_F16_TFLOPS, 4)}
        log(f"multi-query 70b x{nq}: {mq_avg * 1e3:.1f} us, {mq_tf:.0f} TFLOP/s")
        del b4
        torch.cuda.empty_cache()
        # the other workloads: the write path and the tiny / long-context decodes
        # (the long context also with the 2.5-bit K recipe, and with the 3+2-bit
        # recipe plus the QJL residual stage)
        ww, wms, wbytes = write_cold(args.steps, args.warmup, flush)
        wavg = sum(wms) / len(wms)
        result["write"] = {"workload": ww.name, "us": stats_us(wms), "algorithmic_bytes": wbytes,
                           "GBs": round(wbytes / (wavg * 1e-3) / 1e9, 1),
                           "frac_of_peak": round(wbytes / (wavg * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
        log(f"write: {wavg * 1e3:.1f} us")
        torch.cuda.empty_cache()
        for idx, key in ((5, "long"), (6, "long25"), (7, "long_qjl"), (1, "tiny")):
            bx = Bench(idx)
            dx = bx.timed_cold(max(10, args.steps // 2), args.warmup, flush)
            ax = sum(dx) / len(dx)
            result[key] = {"workload": bx.w.name, "decode_us": stats_us(dx), "num_splits": bx.P,
                           "algorithmic_bytes": bx.decode_bytes,
                           "GBs": round(bx.decode_bytes / (ax * 1e-3) / 1e9, 1)}
            log(f"{key}: {ax * 1e3:.1f} us")
            del bx
            torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        result["cpu_baseline"] = cpu_baseline(index, gpu_out=timed_out, gpu_lse=timed_lse)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
