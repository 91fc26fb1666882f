"""Test glue: turns seeded workloads into oracle formats, product formats and
GPU tensors.  Lives in tests/ because it touches both sides."""
from __future__ import annotations

import numpy as np

import oracle
from oracle import encode as oenc
from oracle import pages as opg
from workloads import FormatSpec, bf16_bits_to_f32, to_bf16_bits


def oracle_format(spec: FormatSpec) -> oenc.Format:
    return oenc.Format.make(spec.head_dim, spec.group_bits, spec.signs, spec.group_channels,
                            qjl_proj=spec.qjl_proj)


def product_format(spec: FormatSpec):
    import quantized_paged_kv_amd as tq
    proj = None
    if spec.qjl_proj is not None:
        import torch
        proj = torch.from_numpy(spec.qjl_proj.copy()).cuda()
    return tq.Format(spec.head_dim, spec.group_bits, spec.signs, spec.group_channels, qjl_proj=proj)


def to_device(x: np.ndarray, dtype: str, device="cuda"):
    """float32 numpy holding exactly representable values -> torch tensor."""
    import torch
    if dtype == "bf16":
        bits = to_bf16_bits(x)
        assert np.array_equal(bf16_bits_to_f32(bits), x.astype(np.float32)), "values not bf16-exact"
        t = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(device)


def oracle_pages(x: np.ndarray, slots: np.ndarray, num_blocks: int, fmt: oenc.Format, role: str, fill=0xA5):
    """Pool written by the oracle (sentinel-filled first)."""
    T, H, d = x.shape
    _, _, tile = opg.tile_layout(fmt, 16)
    pages = np.full((num_blocks, H, tile), fill, dtype=np.uint8)
    opg.write_pages(x, slots, pages, fmt, 16, role)
    return pages


def written_mask(slots: np.ndarray, num_blocks: int, H: int, fmt: oenc.Format, role: str) -> np.ndarray:
    """Boolean mask of the bytes a write of `slots` owns (rows + norm slots)."""
    rb, noff, tile = opg.tile_layout(fmt, 16)
    mask = np.zeros((num_blocks, H, tile), dtype=bool)
    for s in slots:
        b, o = divmod(int(s), 16)
        mask[b, :, opg.index_positions(fmt, role, [o])[0]] = True
        sl = 4 * (o % 4) + o // 4
        for g in range(fmt.num_groups * (2 if fmt.qjl else 1)):   # vector (and residual) norms
            pos = noff + 2 * (16 * g + sl)
            mask[b, :, pos:pos + 2] = True
    return mask


def slots_of(block_tables: np.ndarray, context_lens: np.ndarray):
    """Slot of every cached token of every sequence, sequence-major."""
    out = []
    for s, n in enumerate(context_lens):
        t = np.arange(int(n))
        out.append(block_tables[s, t // 16].astype(np.int64) * 16 + t % 16)
    return out


def bf16_neighbours(o: np.ndarray):
    """For bf16 values o (held in float32), the next bf16 values below and
    above, as float64 (infinite past the largest finite value)."""
    bits = to_bf16_bits(np.asarray(o, dtype=np.float32)).astype(np.int64)
    mag, neg = bits & 0x7FFF, (bits & 0x8000) != 0
    up = np.where(neg, mag - 1, mag + 1)          # towards +inf in magnitude terms
    dn = np.where(neg, mag + 1, mag - 1)
    def val(m, sign_neg):
        m = np.clip(m, 0, 0x7F80)
        b = (m | np.where(sign_neg, 0x8000, 0)).astype(np.uint16)
        return bf16_bits_to_f32(b).astype(np.float64)
    zero = mag == 0
    hi = np.where(zero, val(np.ones_like(mag), False), np.where(neg, val(up, True), val(up, False)))
    lo = np.where(zero, -val(np.ones_like(mag), False), np.where(neg, val(dn, True), val(dn, False)))
    return lo, hi


def out_error(o_gpu: np.ndarray, o_ref: np.ndarray, bf16: bool = False):
    """Per (seq, head) vector: normwise relative error against the fp64
    reference, ||o - ref|| / ||ref||.

    With bf16=True the output is a bf16 vector and the error is taken modulo
    its rounding: per element, the distance from ref to the interval of reals
    that round to o (half-way to each bf16 neighbour), i.e. the smallest
    perturbation of the exact result whose bf16 rounding is the output;
    ||that|| / ||ref||.  (bf16 rounding of the exact result alone moves it by
    up to 2^-8 relative per element, ~1e-3 to 2.5e-3 normwise, which is not
    the kernel's error.)"""
    ref = o_ref.astype(np.float64)
    den = np.linalg.norm(ref, axis=-1)
    den = np.where(den == 0, 1.0, den)
    o = o_gpu.astype(np.float64)
    if not bf16:
        return np.linalg.norm(o - ref, axis=-1) / den
    lo_n, hi_n = bf16_neighbours(o_gpu)
    lo, hi = (o + lo_n) / 2, (o + hi_n) / 2
    e = np.maximum(0.0, np.maximum(lo - ref, ref - hi))
    return np.linalg.norm(e, axis=-1) / den


def elem_error(o_gpu: np.ndarray, o_ref: np.ndarray):
    """Elementwise |o - o_ref| relative to the vector's max |o_ref|."""
    ref = o_ref.astype(np.float64)
    scale = np.max(np.abs(ref), axis=-1, keepdims=True)
    scale = np.where(scale == 0, 1.0, scale)
    return np.abs(o_gpu.astype(np.float64) - ref) / scale
