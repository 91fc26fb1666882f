"""Seeded synthetic inputs shared by the oracle side and the GPU side.

This module draws random numbers and lays out shapes; it holds none of the
method's arithmetic (no rotation, codebook, quantisation, packing or
attention).  Everything the method itself would otherwise draw at random
(the +-1 rotation signs, the high-precision channel subset, block-table
permutations) is produced here and handed to both sides as an input.

Two generators are used:

* SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
  generators", OOPSLA 2014): a published counter-style 64-bit generator that
  is written out below, so signs, permutations and channel subsets do not
  depend on the numpy version.
* numpy ``default_rng([seed, stream])`` (PCG64) for the bulk K/V/q values.

The five workloads mirror the shapes of the decode layer steps described on
the TurboQuant server page (Llama-3-8B / Llama-3.1-70B shapes, 32k benchmark
prompt, 131072 maximum context) and the TurboQuant design page's serving
route (block = slot // block_size, offset = slot % block_size).
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional

import numpy as np

MASK64 = (1 << 64) - 1
GOLDEN_GAMMA = 0x9E3779B97F4A7C15

# stream ids per purpose, fixed so that each purpose draws independent numbers
STREAM_K_SIGNS = 1
STREAM_V_SIGNS = 2
STREAM_CHANNELS = 3
STREAM_BLOCKS = 4
STREAM_OUTLIERS = 5
STREAM_QJL = 6
STREAM_V_CHANNELS = 7
STREAM_K = 11
STREAM_V = 12
STREAM_Q = 13
STREAM_CTX = 14
STREAM_NEW_K = 21
STREAM_NEW_V = 22
STREAM_WIN_K = 31
STREAM_WIN_V = 32


class SplitMix64:
    """SplitMix64 as published: state += gamma; then two xor-shift-multiply
    rounds and a final xor-shift."""

    def __init__(self, seed: int, stream: int = 0):
        self.state = ((seed & 0xFFFFFFFF) << 32 ^ (stream * GOLDEN_GAMMA)) & MASK64

    def next(self) -> int:
        self.state = (self.state + GOLDEN_GAMMA) & MASK64
        z = self.state
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
        return z ^ (z >> 31)

    def below(self, n: int) -> int:
        """Uniform integer in [0, n) (modulo reduction; bias < n / 2^64)."""
        return self.next() % n


def signs(seed: int, stream: int, n: int) -> np.ndarray:
    """n values in {+1, -1}: -1 where the top bit of a SplitMix64 output is set."""
    g = SplitMix64(seed, stream)
    return np.array([-1 if (g.next() >> 63) else 1 for _ in range(n)], dtype=np.int8)


def permutation(seed: int, stream: int, n: int) -> np.ndarray:
    """Fisher-Yates shuffle of 0..n-1 driven by SplitMix64."""
    g = SplitMix64(seed, stream)
    p = list(range(n))
    for i in range(n - 1, 0, -1):
        j = g.below(i + 1)
        p[i], p[j] = p[j], p[i]
    return np.array(p, dtype=np.int64)


def channel_subset(seed: int, stream: int, n: int, k: int) -> np.ndarray:
    """k distinct channel ids from 0..n-1, ascending (first k of a shuffle)."""
    return np.sort(permutation(seed, stream, n)[:k])


def rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.default_rng([seed, stream])


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even) and
    return the 16-bit patterns.  Inputs must be finite."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32).astype(np.uint64)
    rounded = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 array holding the bfloat16-rounded values of x."""
    return bf16_bits_to_f32(to_bf16_bits(x))


# --------------------------------------------------------------------------
# workload descriptions
# --------------------------------------------------------------------------

@dataclasses.dataclass
class FormatSpec:
    """Shape of one tensor's format: bit width per channel group and, for two
    groups, the seeded channel subset of the first (high-precision) group."""
    head_dim: int
    group_bits: List[int]
    group_channels: Optional[np.ndarray] = None  # full ordered list, group 0 then group 1
    signs: Optional[np.ndarray] = None
    qjl_proj: Optional[np.ndarray] = None        # float32 [groups, m, m]: QJL projections (K only)

    @property
    def num_groups(self) -> int:
        return len(self.group_bits)

    @property
    def group_sizes(self) -> List[int]:
        return [self.head_dim // self.num_groups] * self.num_groups


@dataclasses.dataclass
class DecodeWorkload:
    name: str
    seed: int
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    context_lens: np.ndarray          # int32 [B]
    num_blocks: int                   # physical pool size
    block_tables: np.ndarray          # int32 [B, max_blocks_per_seq], unused = -1
    kfmt: FormatSpec
    vfmt: FormatSpec
    kv_dist: str                      # "normal", "t3", "t5u", "normal_outliers"
    in_dtype: str                     # "bf16" or "f32"
    q_dtype: str
    out_dtype: str
    scale: float
    num_splits: int
    outlier_channels: Optional[np.ndarray] = None

    @property
    def max_blocks_per_seq(self) -> int:
        return self.block_tables.shape[1]

    @property
    def group_size(self) -> int:
        return self.num_q_heads // self.num_kv_heads


def qjl_projection(seed: int, num_groups: int, m: int) -> np.ndarray:
    """QJL projections: float32 [num_groups, m, m] of N(0, 1) draws."""
    return rng(seed, STREAM_QJL).standard_normal((num_groups, m, m), dtype=np.float32)


def _formats(seed: int, head_dim: int, kbits: List[int], vbits: List[int], qjl: bool = False):
    # The same seeded sign vector serves K and V ("a seeded rotation").
    s = signs(seed, STREAM_K_SIGNS, head_dim)
    kch = None
    if len(kbits) == 2:
        hi = channel_subset(seed, STREAM_CHANNELS, head_dim, head_dim // 2)
        lo = np.array(sorted(set(range(head_dim)) - set(hi.tolist())), dtype=np.int64)
        kch = np.concatenate([hi, lo])
    vch = None
    if len(vbits) == 2:   # V's own channel groups, drawn independently of K's
        hi = channel_subset(seed, STREAM_V_CHANNELS, head_dim, head_dim // 2)
        lo = np.array(sorted(set(range(head_dim)) - set(hi.tolist())), dtype=np.int64)
        vch = np.concatenate([hi, lo])
    proj = qjl_projection(seed, len(kbits), head_dim // len(kbits)) if qjl else None
    kf = FormatSpec(head_dim, list(kbits), kch, s.copy(), proj)
    vf = FormatSpec(head_dim, list(vbits), vch, s.copy())
    return kf, vf


def _paged_tables(seed: int, context_lens: np.ndarray, block_size: int,
                  max_blocks_per_seq: int, pool_factor: float = 1.25):
    need = [int(math.ceil(int(c) / block_size)) for c in context_lens]
    num_blocks = int(math.ceil(pool_factor * sum(need)))
    perm = permutation(seed, STREAM_BLOCKS, num_blocks)
    bt = np.full((len(context_lens), max_blocks_per_seq), -1, dtype=np.int32)
    pos = 0
    for s, n in enumerate(need):
        bt[s, :n] = perm[pos:pos + n]
        pos += n
    return num_blocks, bt


def decode_workload(index: int, seed: int = 0) -> DecodeWorkload:
    """The decode workloads (index 1, 2, 4, 5; index 3 is the write workload;
    index 6 is workload 5 with the 2.5-bit K recipe: 64 channels at 3 bits
    and 64 at 2 bits; index 7 is workload 6 with the QJL residual stage on
    both K groups: 3.5 bits per K channel)."""
    bs = 16
    if index == 1:
        ctx = np.array([256], dtype=np.int32)
        kf, vf = _formats(seed, 64, [4], [4])
        # 16 physical blocks in a seeded permutation: the pool is exactly full.
        perm = permutation(seed, STREAM_BLOCKS, 16)
        bt = perm.astype(np.int32)[None, :]
        return DecodeWorkload("tiny d64 ctx256 K4/V4", seed, 1, 1, 1, 64, bs, ctx, 16, bt,
                              kf, vf, "normal", "f32", "f32", "f32", 1.0 / 8.0, 1)
    if index == 2:
        ctx = rng(seed, STREAM_CTX).integers(1024, 8192, size=32, endpoint=True).astype(np.int32)
        nb, bt = _paged_tables(seed, ctx, bs, 8192 // bs)
        kf, vf = _formats(seed, 128, [4], [4])
        return DecodeWorkload("llama3-8b-shape B32 Hq32 Hkv8 ctx U[1024,8192] K4/V4", seed, 32, 32, 8,
                              128, bs, ctx, nb, bt, kf, vf, "normal", "bf16", "bf16", "bf16",
                              1.0 / math.sqrt(128.0), 16)
    if index == 4:
        ctx = np.full(8, 32768, dtype=np.int32)
        nb, bt = _paged_tables(seed, ctx, bs, 32768 // bs)
        kf, vf = _formats(seed, 128, [4], [2])
        oc = np.sort(permutation(seed, STREAM_OUTLIERS, 128)[:4])
        return DecodeWorkload("llama3.1-70b-shape B8 Hq64 Hkv8 ctx32768 K4/V2", seed, 8, 64, 8, 128, bs,
                              ctx, nb, bt, kf, vf, "normal_outliers", "bf16", "bf16", "bf16",
                              1.0 / math.sqrt(128.0), 16, outlier_channels=oc)
    if index == 5:
        ctx = np.array([131072], dtype=np.int32)
        nb, bt = _paged_tables(seed, ctx, bs, 131072 // bs)
        kf, vf = _formats(seed, 128, [4, 3], [2])
        return DecodeWorkload("long-context B1 Hq64 Hkv8 ctx131072 K(4+3)/V2 64 splits", seed, 1, 64, 8,
                              128, bs, ctx, nb, bt, kf, vf, "t3", "bf16", "bf16", "bf16",
                              1.0 / math.sqrt(128.0), 64)
    if index == 6:
        ctx = np.array([131072], dtype=np.int32)
        nb, bt = _paged_tables(seed, ctx, bs, 131072 // bs)
        kf, vf = _formats(seed, 128, [3, 2], [2])
        return DecodeWorkload("long-context B1 Hq64 Hkv8 ctx131072 K(3+2)/V2 64 splits", seed, 1, 64, 8,
                              128, bs, ctx, nb, bt, kf, vf, "t3", "bf16", "bf16", "bf16",
                              1.0 / math.sqrt(128.0), 64)
    if index == 7:
        ctx = np.array([131072], dtype=np.int32)
        nb, bt = _paged_tables(seed, ctx, bs, 131072 // bs)
        kf, vf = _formats(seed, 128, [3, 2], [2], qjl=True)
        return DecodeWorkload("long-context B1 Hq64 Hkv8 ctx131072 K(3+2)+QJL/V2 64 splits", seed, 1, 64, 8,
                              128, bs, ctx, nb, bt, kf, vf, "t3", "bf16", "bf16", "bf16",
                              1.0 / math.sqrt(128.0), 64)
    raise ValueError(f"no decode workload {index}")


def small_decode_workload(seed: int, num_seqs: int, num_q_heads: int, num_kv_heads: int,
                          head_dim: int, context_lens, kbits, vbits, *, kv_dist="normal",
                          in_dtype="bf16", out_dtype="bf16", num_splits=1,
                          max_blocks_per_seq: Optional[int] = None, pool_factor=1.25,
                          qjl: bool = False) -> DecodeWorkload:
    """Small seeded case for parity tests (ragged lengths, partial last block)."""
    bs = 16
    ctx = np.asarray(context_lens, dtype=np.int32)
    mb = max_blocks_per_seq or max(1, int(math.ceil(int(ctx.max()) / bs)))
    nb, bt = _paged_tables(seed, ctx, bs, mb, pool_factor)
    nb = max(nb, 1)
    kf, vf = _formats(seed, head_dim, list(kbits), list(vbits), qjl)
    return DecodeWorkload(f"small seed{seed}", seed, num_seqs, num_q_heads, num_kv_heads, head_dim, bs,
                          ctx, nb, bt, kf, vf, kv_dist, in_dtype, in_dtype, out_dtype,
                          1.0 / math.sqrt(head_dim), num_splits)


def _draw(dist: str, g: np.random.Generator, shape, outliers=None) -> np.ndarray:
    if dist == "normal" or dist == "normal_outliers":
        x = g.standard_normal(shape, dtype=np.float32)
    elif dist == "t3":
        x = g.standard_t(3, size=shape).astype(np.float32)
    elif dist == "t5u":
        x = (g.standard_t(5, size=shape) * math.sqrt(3.0 / 5.0)).astype(np.float32)
    elif dist == "tiny":
        # rows of tiny norm: N(0, 1) directions, each row scaled so its L2
        # norm is log-uniform in [1e-7, 5e-5] (fp16 norms subnormal or near)
        x = g.standard_normal(shape, dtype=np.float32)
        lo, hi = math.log(1e-7), math.log(5e-5)
        target = np.exp(g.uniform(lo, hi, size=shape[:-1] + (1,)))
        x = (x / np.linalg.norm(x, axis=-1, keepdims=True) * target).astype(np.float32)
    else:
        raise ValueError(dist)
    return x


def kv_values(w: DecodeWorkload, which: str, seq: int, dtype_out="f32") -> np.ndarray:
    """K or V rows of one sequence: float32 array [ctx, H_kv, d] holding values
    exactly representable in the workload's input dtype.  Each sequence draws
    from its own stream, so one sequence can be regenerated alone."""
    stream = STREAM_K if which == "k" else STREAM_V
    g = rng(w.seed, stream * 1000003 + seq)
    n = int(w.context_lens[seq])
    x = _draw(w.kv_dist, g, (n, w.num_kv_heads, w.head_dim))
    if w.in_dtype == "bf16":
        x = bf16_round(x)
        if w.outlier_channels is not None:
            x[:, :, w.outlier_channels] *= np.float32(8.0)  # power of two: stays exact
    return x


def q_values(w: DecodeWorkload) -> np.ndarray:
    g = rng(w.seed, STREAM_Q)
    q = g.standard_normal((w.num_seqs, w.num_q_heads, w.head_dim), dtype=np.float32)
    if w.q_dtype == "bf16":
        q = bf16_round(q)
    return q


@dataclasses.dataclass
class WriteWorkload:
    name: str
    seed: int
    num_tokens: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    slot_mapping: np.ndarray  # int64 [T]
    kfmt: FormatSpec
    vfmt: FormatSpec
    kv_dist: str
    in_dtype: str


def write_workload(seed: int = 0, num_seqs: int = 16, new_tokens: int = 2048,
                   num_kv_heads: int = 8, head_dim: int = 128, kbits=(4,), vbits=(4,),
                   kv_dist="t5u", in_dtype="bf16", qjl: bool = False) -> WriteWorkload:
    """Quantise-on-write: num_seqs sequences each appending new_tokens tokens
    through a seeded slot mapping into one shared pool (1.25x the need)."""
    bs = 16
    per_seq = int(math.ceil(new_tokens / bs))
    num_blocks = int(math.ceil(1.25 * per_seq * num_seqs))
    perm = permutation(seed, STREAM_BLOCKS, num_blocks)
    slots = np.empty(num_seqs * new_tokens, dtype=np.int64)
    for s in range(num_seqs):
        blk = perm[s * per_seq:(s + 1) * per_seq]
        i = np.arange(new_tokens)
        slots[s * new_tokens:(s + 1) * new_tokens] = blk[i // bs] * bs + i % bs
    kf, vf = _formats(seed, head_dim, list(kbits), list(vbits), qjl)
    return WriteWorkload(f"write {num_seqs}x{new_tokens} Hkv{num_kv_heads} d{head_dim}", seed,
                         num_seqs * new_tokens, num_kv_heads, head_dim, bs, num_blocks, slots,
                         kf, vf, kv_dist, in_dtype)


def write_values(w: WriteWorkload, which: str) -> np.ndarray:
    stream = STREAM_NEW_K if which == "k" else STREAM_NEW_V
    g = rng(w.seed, stream)
    x = _draw(w.kv_dist, g, (w.num_tokens, w.num_kv_heads, w.head_dim))
    if w.in_dtype == "bf16":
        x = bf16_round(x)
    return x


def window_values(seed: int, num_seqs: int, capacity: int, num_kv_heads: int, head_dim: int, which: str,
                  dtype: str = "bf16", dist: str = "normal") -> np.ndarray:
    """Dense-window K or V rows: float32 array [num_seqs, capacity, H_kv, d]
    holding values exactly representable in `dtype` (N(0, 1) by default)."""
    g = rng(seed, STREAM_WIN_K if which == "k" else STREAM_WIN_V)
    x = _draw(dist, g, (num_seqs, capacity, num_kv_heads, head_dim))
    return bf16_round(x) if dtype == "bf16" else x
