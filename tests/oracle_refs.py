"""Oracle references for decode parity tests, one (sequence, kv head) at a
time: the oracle encodes that head's rows into a pool of its own and runs
its fp64 attention over the dense reconstruction for the head's q heads.

Large workloads are spread over worker processes started with "spawn"
(fresh interpreters that import only numpy, the oracle and the workload
generators; never the GPU runtime).  Test infrastructure only."""
from __future__ import annotations

import math
import multiprocessing as mp
import os

import numpy as np

from oracle import attn as oatt
from oracle import encode as oenc
from oracle import pages as opg
import workloads as wl


def _fmt(spec) -> oenc.Format:
    return oenc.Format.make(spec.head_dim, spec.group_bits, spec.signs, spec.group_channels, qjl_proj=spec.qjl_proj)


def head_refs(w, q: np.ndarray, s: int, kvh: int, heads):
    """{(s, h): (o_ref float64 [d], lse_ref)} for q heads `heads` of kv head
    kvh of sequence s (q: [S, H_q, d] float32)."""
    n = int(w.context_lens[s])
    if n == 0:
        return {(s, h): (np.zeros(w.head_dim), -math.inf) for h in heads}
    kof, vof = _fmt(w.kfmt), _fmt(w.vfmt)
    bt = np.arange((n + 15) // 16)
    sl = bt[np.arange(n) // 16] * 16 + np.arange(n) % 16
    xk = wl.kv_values(w, "k", s)[:, kvh:kvh + 1]
    xv = wl.kv_values(w, "v", s)[:, kvh:kvh + 1]
    Kp = np.zeros((len(bt), 1, opg.tile_layout(kof, 16)[2]), np.uint8)
    Vp = np.zeros((len(bt), 1, opg.tile_layout(vof, 16)[2]), np.uint8)
    for a in range(0, n, 16384):
        opg.write_pages(xk[a:a + 16384], sl[a:a + 16384], Kp, kof, 16)
        opg.write_pages(xv[a:a + 16384], sl[a:a + 16384], Vp, vof, 16, "v")
    K = opg.reconstruct_sequence(Kp, bt, n, 0, kof, 16)
    V = opg.reconstruct_sequence(Vp, bt, n, 0, vof, 16, role="v")
    return {(s, h): oatt.attention(q[s, h].astype(np.float64), K, V, w.scale) for h in heads}


def _task(args):
    w, q, s, kvh, heads = args
    return head_refs(w, q, s, kvh, heads)


def decode_refs(w, q: np.ndarray, pairs, procs: int = 0):
    """References for every (sequence, q head) pair; procs > 1 spreads the
    (sequence, kv head) units over that many spawned processes."""
    G = w.num_q_heads // w.num_kv_heads
    units = {}
    for s, h in pairs:
        units.setdefault((s, h // G), []).append(h)
    tasks = [(w, q, s, kvh, heads) for (s, kvh), heads in sorted(units.items())]
    out = {}
    if procs > 1 and len(tasks) > 1:
        # longest units first, so the pool drains evenly
        tasks.sort(key=lambda t: -int(w.context_lens[t[2]]))
        with mp.get_context("spawn").Pool(min(procs, len(tasks))) as pool:
            for r in pool.imap_unordered(_task, tasks):
                out.update(r)
    else:
        for t in tasks:
            out.update(_task(t))
    return out


def cpu_procs() -> int:
    """Worker processes for the oracle: the allowed cores, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))
