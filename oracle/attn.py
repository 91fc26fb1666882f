"""Attention over the decoded cache, split partials and their merge.

The method's attention is exact softmax attention over the dequantised
cache, so the oracle writes it out by its plain definition in float64 in
the original (un-rotated) domain:

    s_t = scale * q . K_t,   lse = ln sum_t exp(s_t),   o = sum_t exp(s_t - lse) V_t

Readings of open points: kv head = q head // (H_q / H_kv); the LSE is a
natural log.
A sequence with no cached tokens gives o = 0 and lse = -inf.

Split-K (flash-decoding): the logical blocks of a sequence are cut into
contiguous chunks of `chunk_blocks` blocks; each chunk yields its own
normalised o_p and lse_p (empty chunks: o_p = 0, lse_p = -inf) and the merge
is the log-sum-exp identity

    lse = M + ln sum_p exp(lse_p - M),   o = sum_p exp(lse_p - lse) o_p.

[D "Serving Route Design"]: the workspace of the split is bounded by the
runtime shape (sequences x heads x splits x d), never by context length.

Dense window ([D "Format Strategy"]: a recent dense window and boundary-token
preservation; [D "Data Ownership"]: the compressed cache owns its recent
windows).  Reading: a sequence's cache is its packed history plus a small set
of tokens kept unquantised (its first tokens and its most recent ones), and
attention runs over the union, by the same plain definition.
"""
from __future__ import annotations

import math

import numpy as np

from .pages import reconstruct_sequence


def attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float):
    """q[d], K[n, d], V[n, d] -> (o[d], lse) in float64."""
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    n = K.shape[0]
    if n == 0:
        return np.zeros(q.shape[-1]), -math.inf
    s = scale * (K @ q)
    mx = np.max(s)
    e = np.exp(s - mx)
    tot = np.sum(e)
    lse = mx + math.log(tot)
    o = (e / tot) @ V
    return o, lse


def split_partials(q, K, V, scale, block_size: int, chunk_blocks: int, num_splits: int):
    """Partials (o_p[P, d], lse_p[P]) of one (sequence, q head) for chunks of
    chunk_blocks logical blocks."""
    n = K.shape[0]
    d = K.shape[1]
    o = np.zeros((num_splits, d))
    lse = np.full(num_splits, -math.inf)
    span = chunk_blocks * block_size
    for p in range(num_splits):
        lo, hi = p * span, min((p + 1) * span, n)
        if lo < hi:
            o[p], lse[p] = attention(q, K[lo:hi], V[lo:hi], scale)
    return o, lse


def merge_partials(o_p: np.ndarray, lse_p: np.ndarray):
    """LSE-weighted merge of partials o_p[P, d], lse_p[P]."""
    o_p = np.asarray(o_p, dtype=np.float64)
    lse_p = np.asarray(lse_p, dtype=np.float64)
    if not np.any(np.isfinite(lse_p)):
        return np.zeros(o_p.shape[-1]), -math.inf
    M = np.max(lse_p)
    w = np.exp(lse_p - M)
    lse = M + math.log(np.sum(w))
    o = np.sum(np.exp(lse_p - lse)[:, None] * o_p, axis=0)
    return o, lse


def decode_reference(q: np.ndarray, k_pages, v_pages, block_tables, context_lens, kfmt, vfmt,
                     scale: float, block_size: int, pairs=None):
    """fp64 decode of q[B, H_q, d] against packed pages.  Returns
    (out[B, H_q, d], lse[B, H_q]); with `pairs` (list of (seq, q_head)) only
    those entries are computed (others stay NaN)."""
    B, Hq, d = q.shape
    Hkv = k_pages.shape[1]
    G = Hq // Hkv
    out = np.full((B, Hq, d), np.nan)
    lse = np.full((B, Hq), np.nan)
    todo = pairs if pairs is not None else [(s, h) for s in range(B) for h in range(Hq)]
    cache = {}
    for s, h in todo:
        kvh = h // G
        key = (s, kvh)
        if key not in cache:
            n = int(context_lens[s])
            K = reconstruct_sequence(k_pages, block_tables[s], n, kvh, kfmt, block_size)
            V = reconstruct_sequence(v_pages, block_tables[s], n, kvh, vfmt, block_size, role="v")
            cache = {key: (K, V)}
        K, V = cache[key]
        out[s, h], lse[s, h] = attention(q[s, h], K, V, scale)
    return out, lse


def decode_window_reference(q: np.ndarray, k_win: np.ndarray, v_win: np.ndarray, win_lens, scale: float,
                            k_pages=None, v_pages=None, block_tables=None, context_lens=None, kfmt=None,
                            vfmt=None, block_size: int = 16, pairs=None):
    """fp64 attention of q[B, H_q, d] over each sequence's dense window rows
    k_win[s, :win_lens[s], kv_head] / v_win (exact values, any float dtype)
    together with its decoded packed history (when pages are given), as one
    set of tokens.  Returns (out[B, H_q, d], lse[B, H_q]); with `pairs` only
    those (seq, q_head) entries are computed (others stay NaN)."""
    B, Hq, d = q.shape
    Hkv = k_win.shape[2]
    G = Hq // Hkv
    out = np.full((B, Hq, d), np.nan)
    lse = np.full((B, Hq), np.nan)
    todo = pairs if pairs is not None else [(s, h) for s in range(B) for h in range(Hq)]
    cache = {}
    for s, h in todo:
        kvh = h // G
        key = (s, kvh)
        if key not in cache:
            n = int(win_lens[s])
            K = np.asarray(k_win[s, :n, kvh], dtype=np.float64)
            V = np.asarray(v_win[s, :n, kvh], dtype=np.float64)
            if k_pages is not None:
                c = int(context_lens[s])
                Kh = reconstruct_sequence(k_pages, block_tables[s], c, kvh, kfmt, block_size)
                Vh = reconstruct_sequence(v_pages, block_tables[s], c, kvh, vfmt, block_size, role="v")
                K = np.concatenate([Kh, K]) if c else K
                V = np.concatenate([Vh, V]) if c else V
            cache = {key: (K, V)}
        K, V = cache[key]
        out[s, h], lse[s, h] = attention(q[s, h], K, V, scale)
    return out, lse


def decode_multi_reference(q: np.ndarray, k_pages, v_pages, block_tables, context_lens, kfmt, vfmt,
                           scale: float, block_size: int):
    """fp64 multi-query decode of q[B, NQ, H_q, d]: the sequence's last NQ
    cached tokens are the queries' own, so query i (0-based) attends the
    first context_lens[s] - (NQ - 1 - i) tokens (none: o = 0, lse = -inf).
    Returns (out[B, NQ, H_q, d], lse[B, NQ, H_q])."""
    B, NQ, Hq, d = q.shape
    Hkv = k_pages.shape[1]
    G = Hq // Hkv
    out = np.zeros((B, NQ, Hq, d))
    lse = np.full((B, NQ, Hq), -math.inf)
    for s in range(B):
        n = int(context_lens[s])
        for kvh in range(Hkv):
            K = reconstruct_sequence(k_pages, block_tables[s], n, kvh, kfmt, block_size) if n else np.zeros((0, d))
            V = reconstruct_sequence(v_pages, block_tables[s], n, kvh, vfmt, block_size, role="v") if n else np.zeros((0, d))
            for i in range(NQ):
                c = max(n - (NQ - 1 - i), 0)
                for h in range(kvh * G, (kvh + 1) * G):
                    out[s, i, h], lse[s, i, h] = attention(q[s, i, h], K[:c], V[:c], scale)
    return out, lse
