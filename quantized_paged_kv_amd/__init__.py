"""Python binding of libtq (ctypes).  Argument marshalling only: every step
of the quantise-on-write / paged-decode / split-merge path runs in the HIP
kernels of libtq.so; torch supplies device memory and the current stream.

The library must have been built (``python quantized_paged_kv_amd/_build.py``
or ``__graft_entry__.build()``); importing this package without it raises,
there is no fallback of any kind.

Errors follow the TurboQuant design page's "Error Model": ValueError,
IndexError, UnsupportedFormatError (a format no kernel serves; nothing is
silently densified), FileNotFoundError (missing format metadata).
"""
from __future__ import annotations

import ctypes
import json
import math
import os
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# TQ_LIB_PATH selects another build of the library (for example the
# phase-timestamp variant libtq_trace.so); the default is the in-tree libtq.so
LIB_PATH = os.environ.get("TQ_LIB_PATH") or os.path.join(_HERE, "libtq.so")

TQ_OK, TQ_ERR_VALUE, TQ_ERR_INDEX, TQ_ERR_UNSUPPORTED_FORMAT, TQ_ERR_NOT_FOUND, TQ_ERR_DEVICE = range(6)
TQ_F32, TQ_BF16 = 0, 1
BLOCK_SIZE = 16


class UnsupportedFormatError(Exception):
    """A valid format that no decode/write kernel serves."""


class DeviceError(RuntimeError):
    """HIP launch or runtime failure inside libtq."""


class tq_format(ctypes.Structure):
    _fields_ = [
        ("head_dim", ctypes.c_int32),
        ("num_groups", ctypes.c_int32),
        ("group_bits", ctypes.c_int32 * 2),
        ("group_channels", ctypes.c_uint8 * 128),
        ("codebook", (ctypes.c_uint16 * 16) * 2),
        ("signs", ctypes.c_int8 * 128),
        ("qjl", ctypes.c_int32),
        ("qjl_proj", ctypes.c_void_p),
    ]


def _load(path: str = LIB_PATH):
    # torch first: its bundled HIP runtime is registered under the soname that
    # libtq.so asks for, so libtq binds to that same runtime instance (the one
    # that owns torch's device memory and stream handles) instead of loading a
    # second copy of the runtime.
    import torch  # noqa: F401
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run `python quantized_paged_kv_amd/_build.py`")
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    i32, i64, u64, f32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_float
    fmtp = ctypes.POINTER(tq_format)
    sig = {
        "tq_last_error": ([], ctypes.c_char_p),
        "tq_lloyd_max_codebook": ([i32, P], i32),
        "tq_format_check": ([fmtp], i32),
        "tq_tile_bytes": ([fmtp, i32, P, P], i32),
        "tq_write_kv": ([P, P, i32, i64, i32, P, P, P, i64, i32, fmtp, fmtp, P, P], i32),
        "tq_decode_workspace_bytes": ([i32, i32, i32, i32, P], i32),
        "tq_selftest_fp64": ([P, P, i64, P, P, P, P, P], i32),
        "tq_decode_paged": ([P, i32, i32, i32, i32, P, P, i64, i32, P, i32, P, fmtp, fmtp, f32, i32, P, u64,
                             P, i32, P, P, P], i32),
        "tq_decode_paged_multi": ([P, i32, i32, i32, i32, i32, P, P, i64, i32, P, i32, P, fmtp, fmtp, f32, i32,
                                   P, u64, P, i32, P, P, P], i32),
        "tq_split_merge": ([P, P, i32, i32, i32, i32, P, i32, P, P], i32),
        "tq_decode_dense": ([P, i32, i32, i32, i32, i32, P, P, i32, i32, P, f32, P, P, P, i32, P, P, P], i32),
        "tq_decode_paged_window": ([P, i32, i32, i32, i32, P, P, i64, i32, P, i32, P, fmtp, fmtp, P, P, i32, i32,
                                    P, f32, i32, P, u64, P, i32, P, P, P], i32),
        "tq_debug_phase_trace": ([P], i32),
        "tq_decode_paged_noalloc": ([P, i32, i32, i32, i32, P, P, i64, i32, P, i32, P, fmtp, fmtp, f32, i32, P, i32,
                                     P, P, P], i32),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


_lib = _load()


def _check(status: int):
    if status == TQ_OK:
        return
    msg = _lib.tq_last_error().decode()
    if status == TQ_ERR_VALUE:
        raise ValueError(msg)
    if status == TQ_ERR_INDEX:
        raise IndexError(msg)
    if status == TQ_ERR_UNSUPPORTED_FORMAT:
        raise UnsupportedFormatError(msg)
    if status == TQ_ERR_NOT_FOUND:
        raise FileNotFoundError(msg)
    raise DeviceError(msg)


def lloyd_max_codebook(bits: int) -> np.ndarray:
    """fp16 Lloyd-Max levels of a unit Gaussian (computed by libtq on the host)."""
    out = (ctypes.c_uint16 * 16)()
    _check(_lib.tq_lloyd_max_codebook(bits, ctypes.cast(out, ctypes.c_void_p)))
    return np.frombuffer(bytes(out), dtype=np.uint16)[:1 << bits].copy()


class Format:
    """One tensor's storage format.  K and V carry separate formats."""

    def __init__(self, head_dim: int, group_bits: Sequence[int], signs, group_channels=None,
                 codebooks: Optional[Sequence[np.ndarray]] = None, qjl_proj=None):
        """qjl_proj: for a K format with the QJL residual stage, a contiguous
        float32 GPU tensor [num_groups, m, m] of N(0, 1) projections (kept
        alive by this object; the library reads it during each call)."""
        self.head_dim = int(head_dim)
        self.group_bits = [int(b) for b in group_bits]
        self.signs = np.asarray(signs, dtype=np.int8).reshape(-1)
        ng = len(self.group_bits)
        if group_channels is None:
            group_channels = np.arange(self.head_dim)
        self.group_channels = np.asarray(group_channels, dtype=np.int64).reshape(-1)
        if codebooks is None:
            codebooks = [lloyd_max_codebook(b) if 2 <= b <= 4 else np.zeros(0, np.uint16) for b in self.group_bits]
        self.codebooks = [np.asarray(c, dtype=np.uint16) for c in codebooks]
        c = tq_format()
        c.head_dim = self.head_dim
        c.num_groups = ng
        if ng not in (1, 2) or self.signs.size != self.head_dim or self.group_channels.size != self.head_dim:
            raise ValueError("format arrays do not match head_dim / group count")
        if self.head_dim > 128 or np.any(self.group_channels < 0) or np.any(self.group_channels > 255):
            raise ValueError("head_dim above 128 or channel id out of range")
        for g in range(ng):
            c.group_bits[g] = self.group_bits[g]
            for i, v in enumerate(self.codebooks[g][:16]):
                c.codebook[g][i] = int(v)
        for j in range(self.head_dim):
            c.group_channels[j] = int(self.group_channels[j])
            c.signs[j] = int(self.signs[j])
        self.qjl_proj = qjl_proj
        if qjl_proj is not None:
            import torch
            m = self.head_dim // ng
            if not (qjl_proj.is_cuda and qjl_proj.dtype == torch.float32 and qjl_proj.is_contiguous()
                    and tuple(qjl_proj.shape) == (ng, m, m)):
                raise ValueError("qjl_proj must be a contiguous float32 GPU tensor [num_groups, m, m]")
            c.qjl = 1
            c.qjl_proj = qjl_proj.data_ptr()
        self.c = c
        _check(_lib.tq_format_check(ctypes.byref(c)))

    @property
    def num_groups(self) -> int:
        return len(self.group_bits)

    def tile_bytes(self, block_size: int = BLOCK_SIZE):
        rib, tb = ctypes.c_int32(), ctypes.c_int32()
        _check(_lib.tq_tile_bytes(ctypes.byref(self.c), block_size, ctypes.byref(rib), ctypes.byref(tb)))
        return rib.value, tb.value

    # metadata persistence ([D "Recipe Strategy"]: runtime loads metadata and
    # validates head dimension and group sizes)
    @property
    def qjl(self) -> bool:
        return self.qjl_proj is not None

    def to_json(self) -> dict:
        d = {"head_dim": self.head_dim, "group_bits": self.group_bits,
             "group_channels": self.group_channels.tolist(), "signs": self.signs.tolist(),
             "codebooks_f16": [c.tolist() for c in self.codebooks]}
        if self.qjl_proj is not None:
            d["qjl_proj"] = self.qjl_proj.cpu().numpy().tolist()
        return d

    def save(self, path: str):
        with open(path, "w") as fh:
            json.dump(self.to_json(), fh)

    @staticmethod
    def load(path: str) -> "Format":
        if not os.path.exists(path):
            raise FileNotFoundError(f"format metadata {path} not found")
        with open(path) as fh:
            d = json.load(fh)
        try:
            proj = None
            if "qjl_proj" in d:
                import torch
                proj = torch.tensor(np.array(d["qjl_proj"], dtype=np.float32), device="cuda")
            return Format(d["head_dim"], d["group_bits"], d["signs"], d["group_channels"],
                          [np.array(c, dtype=np.uint16) for c in d["codebooks_f16"]], proj)
        except KeyError as e:
            raise ValueError(f"malformed format metadata: missing {e}") from None


def _ptr(t) -> int:
    return 0 if t is None else t.data_ptr()


def _stream(stream=None) -> int:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return TQ_BF16
    if t.dtype == torch.float32:
        return TQ_F32
    raise ValueError(f"unsupported dtype {t.dtype}")


def _need(cond, msg):
    if not cond:
        raise ValueError(msg)


def alloc_pages(num_blocks: int, num_kv_heads: int, fmt: Format, device="cuda"):
    """A page pool [num_blocks][num_kv_heads][tile_bytes] of uint8 (uninitialised)."""
    import torch
    _, tb = fmt.tile_bytes()
    return torch.empty((num_blocks, num_kv_heads, tb), dtype=torch.uint8, device=device)


def new_error_word(device="cuda"):
    import torch
    return torch.zeros(2, dtype=torch.int32, device=device)


def raise_device_error(dev_err, what: str = ""):
    """Synchronise on the error word and raise IndexError if a kernel set it."""
    code, pos = [int(x) for x in dev_err.cpu().tolist()]
    if code == TQ_ERR_INDEX:
        raise IndexError(f"{what}: entry out of range at position {pos}")
    if code != 0:
        raise DeviceError(f"{what}: device error code {code} at {pos}")


def write_kv(k, v, slot_mapping, k_pages, v_pages, kfmt: Format, vfmt: Format, dev_err=None,
             check: bool = False, stream=None):
    """Quantise k/v rows [T, H_kv, d] (bf16 or fp32, contiguous, on the GPU)
    into the page pools at slot_mapping (int64 [T])."""
    ref = k if k is not None else v
    _need(ref is not None, "k and v are both None")
    for t in (k, v):
        if t is not None:
            _need(t.is_cuda and t.is_contiguous() and t.dim() == 3, "k/v must be contiguous [T, H, d] GPU tensors")
            _need(t.shape == ref.shape and t.dtype == ref.dtype, "k and v differ in shape or dtype")
    import torch
    _need(slot_mapping.dtype == torch.int64 and slot_mapping.is_cuda and slot_mapping.numel() == ref.shape[0],
          "slot_mapping must be an int64 GPU tensor with one slot per token")
    pages = k_pages if k_pages is not None else v_pages
    _need(pages is not None and pages.dtype == torch.uint8 and pages.dim() == 3, "page pools must be uint8 [NB, H, tile]")
    for t, pg, f in ((k, k_pages, kfmt), (v, v_pages, vfmt)):
        if t is not None:
            _need(pg is not None and pg.is_contiguous() and pg.shape[1] == t.shape[1]
                  and pg.shape[2] == f.tile_bytes()[1], "page pool shape does not match the format")
            _need(f.head_dim == t.shape[2], "row length differs from the format's head_dim")
    if k is not None and v is not None:
        _need(k_pages.shape[0] == v_pages.shape[0], "K and V pools differ in block count")
    own_err = dev_err is None and check
    if own_err:
        dev_err = new_error_word(ref.device)
    _check(_lib.tq_write_kv(_ptr(k), _ptr(v), _dtype_code(ref), ref.shape[0], ref.shape[1], _ptr(slot_mapping),
                            _ptr(k_pages if k is not None else None), _ptr(v_pages if v is not None else None),
                            pages.shape[0], BLOCK_SIZE, ctypes.byref(kfmt.c) if k is not None else None,
                            ctypes.byref(vfmt.c) if v is not None else None, _ptr(dev_err), _stream(stream)))
    if check:
        raise_device_error(dev_err, "tq_write_kv")


def selftest_fp64(a, b, stream=None):
    """The write path's fp64 operations on the device: for float64 GPU
    tensors a, b of one shape returns (sqrt(a), a / b, a * b, binary16 bits
    of a as int16), computed by a kernel built like the write kernel."""
    import torch
    _need(a.is_cuda and b.is_cuda and a.dtype == torch.float64 and b.dtype == torch.float64 and a.shape == b.shape
          and a.is_contiguous() and b.is_contiguous(), "a and b must be contiguous float64 GPU tensors of one shape")
    outs = [torch.empty_like(a) for _ in range(3)] + [torch.empty(a.shape, dtype=torch.int16, device=a.device)]
    _check(_lib.tq_selftest_fp64(_ptr(a), _ptr(b), a.numel(), *[_ptr(t) for t in outs], _stream(stream)))
    return tuple(outs)


def workspace_bytes(num_seqs: int, num_q_heads: int, head_dim: int, num_splits: int) -> int:
    b = ctypes.c_uint64()
    _check(_lib.tq_decode_workspace_bytes(num_seqs, num_q_heads, head_dim, num_splits, ctypes.byref(b)))
    return b.value


def decode_paged(q, k_pages, v_pages, block_tables, context_lens, kfmt: Format, vfmt: Format, scale: float,
                 num_splits: int = 1, out=None, lse=None, workspace=None, out_dtype=None, dev_err=None,
                 check: bool = False, stream=None):
    """Decode attention of q [B, H_q, d] against the packed pages.  Returns
    (out [B, H_q, d], lse [B, H_q] float32).  With q [B, NQ, H_q, d] the NQ
    queries of each sequence attend causally (query i sees its first
    context_lens - (NQ - 1 - i) tokens): out [B, NQ, H_q, d], lse [B, NQ, H_q]."""
    import torch
    _need(q.is_cuda and q.is_contiguous() and q.dim() in (3, 4),
          "q must be a contiguous [B, H_q, d] or [B, NQ, H_q, d] GPU tensor")
    NQ = q.shape[1] if q.dim() == 4 else 1
    B, Hq, d = q.shape[0], q.shape[-2], q.shape[-1]
    _need(k_pages.dim() == 3 and v_pages.dim() == 3 and k_pages.dtype == torch.uint8 and v_pages.dtype == torch.uint8,
          "page pools must be uint8 [NB, H_kv, tile]")
    Hkv = k_pages.shape[1]
    _need(v_pages.shape[:2] == k_pages.shape[:2], "K and V pools differ in blocks or heads")
    _need(k_pages.shape[2] == kfmt.tile_bytes()[1] and v_pages.shape[2] == vfmt.tile_bytes()[1],
          "page pool tile size does not match the format")
    _need(kfmt.head_dim == d and vfmt.head_dim == d, "q head_dim differs from the formats")
    _need(block_tables.dtype == torch.int32 and block_tables.dim() == 2 and block_tables.shape[0] == B
          and block_tables.is_contiguous(), "block_tables must be contiguous int32 [B, max_blocks]")
    _need(context_lens.dtype == torch.int32 and context_lens.numel() == B, "context_lens must be int32 [B]")
    rows = tuple(q.shape[:-1])
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or q.dtype, device=q.device)
    _need(out.shape == q.shape and out.is_contiguous(), "out must be contiguous and shaped like q")
    if lse is None:
        lse = torch.empty(rows, dtype=torch.float32, device=q.device)
    _need(lse.shape == rows and lse.dtype == torch.float32, "lse must be float32 shaped like q without d")
    need = workspace_bytes(B * NQ, Hq, d, num_splits)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    own_err = dev_err is None and check
    if own_err:
        dev_err = new_error_word(q.device)
    _check(_lib.tq_decode_paged_multi(_ptr(q), _dtype_code(q), B, NQ, Hq, Hkv, _ptr(k_pages), _ptr(v_pages),
                                      k_pages.shape[0], BLOCK_SIZE, _ptr(block_tables), block_tables.shape[1],
                                      _ptr(context_lens), ctypes.byref(kfmt.c), ctypes.byref(vfmt.c), float(scale),
                                      int(num_splits), _ptr(workspace), ws_bytes, _ptr(out), _dtype_code(out),
                                      _ptr(lse), _ptr(dev_err), _stream(stream)))
    if check:
        raise_device_error(dev_err, "tq_decode_paged")
    return out, lse


NOALLOC_SCRATCH_BYTES = 16 << 20


def decode_paged_noalloc(q, k_pages, v_pages, block_tables, context_lens, kfmt: Format, vfmt: Format,
                         scale: float, out, lse=None, num_splits: int = 1, dev_err=None, stream=None):
    """tq_decode_paged_noalloc: decode of q [B, H_q, d] into the caller's out
    [B, H_q, d] (and lse [B, H_q] float32 if given) with the split partials
    in the library's per-GPU array; this wrapper allocates nothing either.
    Calls that overlap on one GPU race (they share that array)."""
    import torch
    _need(q.is_cuda and q.is_contiguous() and q.dim() == 3, "q must be a contiguous [B, H_q, d] GPU tensor")
    B, Hq, d = q.shape
    _need(k_pages.dim() == 3 and v_pages.dim() == 3 and k_pages.dtype == torch.uint8 and v_pages.dtype == torch.uint8,
          "page pools must be uint8 [NB, H_kv, tile]")
    _need(v_pages.shape[:2] == k_pages.shape[:2], "K and V pools differ in blocks or heads")
    _need(block_tables.dtype == torch.int32 and block_tables.dim() == 2 and block_tables.shape[0] == B
          and block_tables.is_contiguous(), "block_tables must be contiguous int32 [B, max_blocks]")
    _need(context_lens.dtype == torch.int32 and context_lens.numel() == B, "context_lens must be int32 [B]")
    _need(out is not None and out.shape == q.shape and out.is_contiguous(), "out must be contiguous and shaped like q")
    _need(lse is None or (lse.shape == (B, Hq) and lse.dtype == torch.float32), "lse must be float32 [B, H_q]")
    _check(_lib.tq_decode_paged_noalloc(_ptr(q), _dtype_code(q), B, Hq, k_pages.shape[1], _ptr(k_pages),
                                        _ptr(v_pages), k_pages.shape[0], BLOCK_SIZE, _ptr(block_tables),
                                        block_tables.shape[1], _ptr(context_lens), ctypes.byref(kfmt.c),
                                        ctypes.byref(vfmt.c), float(scale), int(num_splits), _ptr(out),
                                        _dtype_code(out), _ptr(lse), _ptr(dev_err), _stream(stream)))
    return out, lse


def split_merge(part_out, part_lse, out=None, lse=None, out_dtype=None, stream=None):
    """Log-sum-exp merge of partials part_out [S, H, P, d], part_lse [S, H, P]."""
    import torch
    _need(part_out.dtype == torch.float32 and part_lse.dtype == torch.float32, "partials must be float32")
    _need(part_out.dim() == 4 and part_out.is_contiguous() and part_lse.is_contiguous(), "bad partial layout")
    S, H, P, d = part_out.shape
    _need(part_lse.shape == (S, H, P), "part_lse shape differs from part_out")
    if out is None:
        out = torch.empty((S, H, d), dtype=out_dtype or torch.float32, device=part_out.device)
    if lse is None:
        lse = torch.empty((S, H), dtype=torch.float32, device=part_out.device)
    _check(_lib.tq_split_merge(_ptr(part_out), _ptr(part_lse), S, H, P, d, _ptr(out), _dtype_code(out), _ptr(lse),
                               _stream(stream)))
    return out, lse


def decode_dense(q, k_win, v_win, lens, scale: float, hist_out=None, hist_lse=None, out=None, lse=None,
                 out_dtype=None, dev_err=None, check: bool = False, stream=None):
    """Exact attention of q [B, H_q, d] over a dense window k_win / v_win
    [B, capacity, H_kv, d] (bf16 or float32) holding lens[s] tokens of
    sequence s, merged by log-sum-exp with (hist_out [B, H_q, d] float32,
    hist_lse [B, H_q]) when given.  out may be hist_out and lse hist_lse.
    Returns (out, lse)."""
    import torch
    _need(q.is_cuda and q.is_contiguous() and q.dim() == 3, "q must be a contiguous [B, H_q, d] GPU tensor")
    B, Hq, d = q.shape
    _need(k_win.dim() == 4 and k_win.shape == v_win.shape and k_win.dtype == v_win.dtype
          and k_win.is_contiguous() and v_win.is_contiguous() and k_win.shape[0] == B and k_win.shape[3] == d,
          "window K/V must be contiguous [B, capacity, H_kv, d] of one dtype")
    _need(lens.dtype == torch.int32 and lens.numel() == B, "lens must be int32 [B]")
    _need((hist_out is None) == (hist_lse is None), "hist_out and hist_lse go together")
    if hist_out is not None:
        _need(hist_out.dtype == torch.float32 and hist_out.shape == (B, Hq, d) and hist_out.is_contiguous()
              and hist_lse.dtype == torch.float32 and hist_lse.shape == (B, Hq) and hist_lse.is_contiguous(),
              "history must be float32 out [B, H_q, d] and lse [B, H_q]")
    if out is None:
        out = torch.empty((B, Hq, d), dtype=out_dtype or q.dtype, device=q.device)
    _need(out.shape == (B, Hq, d) and out.is_contiguous(), "out must be contiguous [B, H_q, d]")
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    own_err = dev_err is None and check
    if own_err:
        dev_err = new_error_word(q.device)
    _check(_lib.tq_decode_dense(_ptr(q), _dtype_code(q), B, Hq, k_win.shape[2], d, _ptr(k_win), _ptr(v_win),
                                _dtype_code(k_win), k_win.shape[1], _ptr(lens), float(scale), _ptr(hist_out),
                                _ptr(hist_lse), _ptr(out), _dtype_code(out), _ptr(lse), _ptr(dev_err),
                                _stream(stream)))
    if check:
        raise_device_error(dev_err, "tq_decode_dense")
    return out, lse


def decode_paged_window(q, k_pages, v_pages, block_tables, context_lens, kfmt: Format, vfmt: Format, k_win, v_win,
                        win_lens, scale: float, num_splits: int = 1, out=None, lse=None, workspace=None,
                        out_dtype=None, dev_err=None, check: bool = False, stream=None):
    """Decode attention of q [B, H_q, d] over the packed pages AND a dense
    bf16 window k_win / v_win [B, capacity, H_kv, d] holding win_lens[s]
    tokens of sequence s, in one call (the window's tokens are not also in
    the pages).  Returns (out [B, H_q, d], lse [B, H_q] float32)."""
    import torch
    _need(q.is_cuda and q.is_contiguous() and q.dim() == 3, "q must be a contiguous [B, H_q, d] GPU tensor")
    B, Hq, d = q.shape
    _need(k_pages.dim() == 3 and v_pages.dim() == 3 and k_pages.dtype == torch.uint8 and v_pages.dtype == torch.uint8,
          "page pools must be uint8 [NB, H_kv, tile]")
    Hkv = k_pages.shape[1]
    _need(v_pages.shape[:2] == k_pages.shape[:2], "K and V pools differ in blocks or heads")
    _need(k_pages.shape[2] == kfmt.tile_bytes()[1] and v_pages.shape[2] == vfmt.tile_bytes()[1],
          "page pool tile size does not match the format")
    _need(kfmt.head_dim == d and vfmt.head_dim == d, "q head_dim differs from the formats")
    _need(block_tables.dtype == torch.int32 and block_tables.dim() == 2 and block_tables.shape[0] == B
          and block_tables.is_contiguous(), "block_tables must be contiguous int32 [B, max_blocks]")
    _need(context_lens.dtype == torch.int32 and context_lens.numel() == B, "context_lens must be int32 [B]")
    _need(k_win.dim() == 4 and k_win.shape == v_win.shape and k_win.dtype == v_win.dtype
          and k_win.is_contiguous() and v_win.is_contiguous() and k_win.shape[0] == B
          and k_win.shape[2] == Hkv and k_win.shape[3] == d,
          "window K/V must be contiguous [B, capacity, H_kv, d] of one dtype")
    _need(win_lens.dtype == torch.int32 and win_lens.numel() == B, "win_lens must be int32 [B]")
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or q.dtype, device=q.device)
    _need(out.shape == q.shape and out.is_contiguous(), "out must be contiguous and shaped like q")
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    _need(lse.shape == (B, Hq) and lse.dtype == torch.float32, "lse must be float32 [B, H_q]")
    need = workspace_bytes(B, Hq, d, num_splits + 1)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    own_err = dev_err is None and check
    if own_err:
        dev_err = new_error_word(q.device)
    _check(_lib.tq_decode_paged_window(_ptr(q), _dtype_code(q), B, Hq, Hkv, _ptr(k_pages), _ptr(v_pages),
                                       k_pages.shape[0], BLOCK_SIZE, _ptr(block_tables), block_tables.shape[1],
                                       _ptr(context_lens), ctypes.byref(kfmt.c), ctypes.byref(vfmt.c),
                                       _ptr(k_win), _ptr(v_win), _dtype_code(k_win), k_win.shape[1],
                                       _ptr(win_lens), float(scale), int(num_splits), _ptr(workspace), ws_bytes,
                                       _ptr(out), _dtype_code(out), _ptr(lse), _ptr(dev_err), _stream(stream)))
    if check:
        raise_device_error(dev_err, "tq_decode_paged_window")
    return out, lse


def set_phase_trace(buf) -> bool:
    """Phase-timestamp buffer (device uint64 tensor, 16 values per CU) for the
    decode kernel; None stops recording.  Returns False when the loaded
    library was built without TQ_PHASE_TRACE."""
    st = _lib.tq_debug_phase_trace(_ptr(buf))
    if st == TQ_ERR_UNSUPPORTED_FORMAT:
        return False
    _check(st)
    return True


__all__ = ["Format", "UnsupportedFormatError", "DeviceError", "lloyd_max_codebook", "alloc_pages",
           "new_error_word", "raise_device_error", "write_kv", "workspace_bytes", "decode_paged", "decode_paged_noalloc",
           "split_merge", "decode_dense", "decode_paged_window", "set_phase_trace", "selftest_fp64",
           "LIB_PATH", "BLOCK_SIZE"]
