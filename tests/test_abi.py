"""The C-ABI library: loads, exports what include/tq.h declares, and its host
logic (codebook, byte math, validation) — no GPU compute is launched here."""
import ctypes
import json
import os
import re

import numpy as np
import pytest

import oracle
from oracle import pages as opg
from workloads import signs, channel_subset

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

tq = pytest.importorskip("quantized_paged_kv_amd")


def header_functions():
    text = open(os.path.join(ROOT, "include", "tq.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tq_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = header_functions()
    assert len(names) >= 8
    lib = ctypes.CDLL(tq.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_library_codebook_equals_oracle(bits):
    """Two independent Lloyd-Max solvers (Max's shooting method in the
    library, Lloyd iteration + root polish in the oracle) give the same fp16
    codebook."""
    lib = tq.lloyd_max_codebook(bits)
    if bits == 1:
        ref = np.float16(oracle.lloyd_max_gaussian(2)).view(np.uint16)
    else:
        ref = oracle.codebook_f16(bits).view(np.uint16)
    np.testing.assert_array_equal(lib, ref)


def _fmts():
    s = signs(0, 1, 128)
    hi = channel_subset(0, 3, 128, 64)
    lo = np.array(sorted(set(range(128)) - set(hi.tolist())))
    return [((128, [4], s, None)), ((128, [2], s, None)), ((128, [4, 3], s, np.concatenate([hi, lo]))),
            ((64, [4], signs(0, 1, 64), None)), ((128, [3], s, None)), ((64, [4, 2], signs(0, 1, 64),
                                                                          np.arange(64)))]


@pytest.mark.parametrize("i", range(6))
def test_tile_bytes_match_oracle(i):
    d, bits, s, ch = _fmts()[i]
    f = tq.Format(d, bits, s, ch)
    of = oracle.Format.make(d, bits, s, ch)
    rb, _, tile = opg.tile_layout(of, 16)
    assert f.tile_bytes() == (rb, tile)


def test_workspace_bytes():
    assert tq.workspace_bytes(1, 64, 128, 64) == 64 * 64 * 129 * 4
    assert tq.workspace_bytes(32, 32, 128, 1) == 0


def test_format_validation_errors():
    s = signs(0, 1, 128)
    with pytest.raises(ValueError):
        tq.Format(128, [5], s)
    with pytest.raises(ValueError):
        tq.Format(96, [4], s[:96])
    bad = s.copy()
    bad[0] = 0
    with pytest.raises(ValueError):
        tq.Format(128, [4], bad)
    cb = tq.lloyd_max_codebook(4)[::-1].copy()          # descending
    with pytest.raises(ValueError):
        tq.Format(128, [4], s, None, [cb])
    ch = np.arange(128)
    ch[[3, 70]] = ch[[70, 3]]                            # not ascending within the groups
    with pytest.raises(ValueError):
        tq.Format(128, [4, 3], s, ch)
    with pytest.raises(ValueError):
        tq.Format(128, [4], s, np.roll(np.arange(128), 1))


def test_metadata_roundtrip_and_not_found(tmp_path):
    d, bits, s, ch = _fmts()[2]
    f = tq.Format(d, bits, s, ch)
    p = tmp_path / "fmt.json"
    f.save(str(p))
    g = tq.Format.load(str(p))
    assert bytes(g.c) == bytes(f.c)
    with pytest.raises(FileNotFoundError):
        tq.Format.load(str(tmp_path / "missing.json"))
    bad = json.loads(p.read_text())
    bad["group_bits"] = [4, 5]
    p.write_text(json.dumps(bad))
    with pytest.raises(ValueError):
        tq.Format.load(str(p))


def _call_write(**kw):
    f = tq.Format(128, [4], signs(0, 1, 128))
    args = dict(k=1, v=1, in_dtype=tq.TQ_BF16, T=4, H=8, slots=1, kp=1, vp=1, nb=10, bs=16, kf=f, vf=f)
    args.update(kw)
    return tq._lib.tq_write_kv(args["k"], args["v"], args["in_dtype"], args["T"], args["H"], args["slots"],
                               args["kp"], args["vp"], args["nb"], args["bs"],
                               ctypes.byref(args["kf"].c) if args["kf"] else None,
                               ctypes.byref(args["vf"].c) if args["vf"] else None, None, None)


def test_write_status_codes_without_launch():
    assert _call_write(k=None, v=None) == tq.TQ_ERR_VALUE
    assert _call_write(in_dtype=7) == tq.TQ_ERR_VALUE
    assert _call_write(bs=32) == tq.TQ_ERR_UNSUPPORTED_FORMAT
    assert _call_write(H=0) == tq.TQ_ERR_VALUE
    assert _call_write(slots=None) == tq.TQ_ERR_VALUE
    assert _call_write(kp=None) == tq.TQ_ERR_VALUE
    f64 = tq.Format(64, [4], signs(0, 1, 64))
    assert _call_write(vf=f64) == tq.TQ_ERR_VALUE     # K and V head_dim differ
    assert _call_write(T=0) == tq.TQ_OK               # nothing to do, nothing launched
    assert "head_dim" in tq._lib.tq_last_error().decode() or True


def _call_decode(**kw):
    s = signs(0, 1, 128)
    f4 = tq.Format(128, [4], s)
    a = dict(q=1, qd=tq.TQ_BF16, B=2, Hq=8, Hkv=2, kp=1, vp=1, nb=10, bs=16, bt=1, mb=4, cl=1, kf=f4, vf=f4,
             scale=0.1, P=1, ws=None, wsb=0, out=1, od=tq.TQ_BF16, lse=None)
    a.update(kw)
    return tq._lib.tq_decode_paged(a["q"], a["qd"], a["B"], a["Hq"], a["Hkv"], a["kp"], a["vp"], a["nb"], a["bs"],
                                   a["bt"], a["mb"], a["cl"], ctypes.byref(a["kf"].c), ctypes.byref(a["vf"].c),
                                   a["scale"], a["P"], a["ws"], a["wsb"], a["out"], a["od"], a["lse"], None, None)


def test_decode_status_codes_without_launch():
    s = signs(0, 1, 128)
    assert _call_decode(Hq=7) == tq.TQ_ERR_VALUE
    assert _call_decode(bs=8) == tq.TQ_ERR_UNSUPPORTED_FORMAT
    assert _call_decode(Hq=130, Hkv=1) == tq.TQ_ERR_UNSUPPORTED_FORMAT    # GQA group above 128
    assert _call_decode(kf=tq.Format(128, [3], s)) == tq.TQ_ERR_UNSUPPORTED_FORMAT
    assert _call_decode(vf=tq.Format(128, [3], s)) == tq.TQ_ERR_UNSUPPORTED_FORMAT
    assert "no decode kernel" in tq._lib.tq_last_error().decode()
    assert _call_decode(P=0) == tq.TQ_ERR_VALUE
    assert _call_decode(P=4) == tq.TQ_ERR_VALUE                  # workspace missing
    assert _call_decode(qd=3) == tq.TQ_ERR_VALUE
    assert _call_decode(q=None) == tq.TQ_ERR_VALUE
    assert _call_decode(vf=tq.Format(64, [4], signs(0, 1, 64))) == tq.TQ_ERR_VALUE
    assert _call_decode(B=0) == tq.TQ_OK


def test_noalloc_decode_status_codes_without_launch():
    """The allocation-free decode rejects a split workspace past its array
    (VALUE, with the sizes in the message) and a NULL format before any
    device call; with no sequences it returns OK."""
    L = tq._lib
    s = signs(0, 1, 128)
    kf = tq.Format(128, [4], s)
    args = lambda B, P, f: (1, tq.TQ_BF16, B, 64, 8, 1, 1, 10, 16, 1, 4, 1, f, ctypes.byref(kf.c), 0.1, P, 1,
                            tq.TQ_BF16, None, None, None)
    assert L.tq_decode_paged_noalloc(*args(600, 128, ctypes.byref(kf.c))) == tq.TQ_ERR_VALUE
    msg = L.tq_last_error().decode()
    assert "exceeds" in msg and str(16 << 20) in msg
    assert L.tq_decode_paged_noalloc(*args(4, 4, None)) == tq.TQ_ERR_VALUE
    assert L.tq_decode_paged_noalloc(*args(0, 1, ctypes.byref(kf.c))) == tq.TQ_OK
    assert tq.NOALLOC_SCRATCH_BYTES == 16 << 20


def test_merge_status_codes_without_launch():
    L = tq._lib
    assert L.tq_split_merge(1, 1, 2, 2, 0, 128, 1, tq.TQ_F32, None, None) == tq.TQ_ERR_VALUE
    assert L.tq_split_merge(1, 1, 2, 2, 2, 96, 1, tq.TQ_F32, None, None) == tq.TQ_ERR_VALUE
    assert L.tq_split_merge(None, 1, 2, 2, 2, 128, 1, tq.TQ_F32, None, None) == tq.TQ_ERR_VALUE
    assert L.tq_split_merge(1, 1, 0, 2, 2, 128, 1, tq.TQ_F32, None, None) == tq.TQ_OK


def _call_dense(q=16, qd=None, B=2, Hq=8, Hkv=2, d=128, k=16, v=16, kvd=None, cap=4, lens=16, scale=0.1,
                ho=None, hl=None, out=16, od=None):
    """tq_decode_dense with fake (never dereferenced) pointers: every call here
    must be refused by host validation or return before any launch."""
    qd = tq.TQ_BF16 if qd is None else qd
    kvd = tq.TQ_BF16 if kvd is None else kvd
    od = tq.TQ_F32 if od is None else od
    return tq._lib.tq_decode_dense(q, qd, B, Hq, Hkv, d, k, v, kvd, cap, lens, scale, ho, hl, out, od,
                                   None, None, None)


def test_dense_window_status_codes_without_launch():
    assert _call_dense(Hq=7) == tq.TQ_ERR_VALUE                      # not a multiple of H_kv
    assert _call_dense(Hq=34, Hkv=2) == tq.TQ_ERR_UNSUPPORTED_FORMAT  # 17 q heads per kv head
    assert _call_dense(d=96) == tq.TQ_ERR_UNSUPPORTED_FORMAT
    assert _call_dense(qd=3) == tq.TQ_ERR_VALUE
    assert _call_dense(kvd=3) == tq.TQ_ERR_VALUE
    assert _call_dense(scale=0.0) == tq.TQ_ERR_VALUE
    assert _call_dense(scale=float("nan")) == tq.TQ_ERR_VALUE
    assert _call_dense(cap=-1) == tq.TQ_ERR_VALUE
    assert _call_dense(ho=16) == tq.TQ_ERR_VALUE                      # hist_out without hist_lse
    assert _call_dense(q=None) == tq.TQ_ERR_VALUE
    assert _call_dense(lens=None) == tq.TQ_ERR_VALUE
    assert _call_dense(k=None) == tq.TQ_ERR_VALUE
    assert _call_dense(k=24) == tq.TQ_ERR_VALUE                       # not 16-byte aligned
    assert _call_dense(out=12) == tq.TQ_ERR_VALUE                     # not 8-byte aligned
    assert "aligned" in tq._lib.tq_last_error().decode()
    assert _call_dense(B=0) == tq.TQ_OK


def test_multi_query_status_codes_without_launch():
    s = signs(0, 1, 128)
    f = tq.Format(128, [4], s)
    L = tq._lib

    def call(NQ=2, Hq=8, Hkv=2, B=2):
        return L.tq_decode_paged_multi(16, tq.TQ_BF16, B, NQ, Hq, Hkv, 16, 16, 10, 16, 16, 4, 16,
                                       ctypes.byref(f.c), ctypes.byref(f.c), 0.1, 1, None, 0, 16, tq.TQ_BF16,
                                       None, None, None)
    assert call(NQ=0) == tq.TQ_ERR_VALUE
    assert call(NQ=33, B=0) == tq.TQ_ERR_UNSUPPORTED_FORMAT    # 33 queries x 4 q heads > 128 columns
    assert "pairs per kv head" in L.tq_last_error().decode()
    assert call(NQ=129, Hq=2, Hkv=2, B=0) == tq.TQ_ERR_UNSUPPORTED_FORMAT
    assert call(NQ=32, B=0) == tq.TQ_OK                         # exactly 128 columns
    assert call(NQ=1, Hq=256, Hkv=2, B=0) == tq.TQ_OK           # 128 q heads per kv head
    assert call(B=0) == tq.TQ_OK
    qc = _qjl_c(f)
    def call_qjl(NQ, Hq):
        return L.tq_decode_paged_multi(16, tq.TQ_BF16, 0, NQ, Hq, 2, 16, 16, 10, 16, 16, 4, 16,
                                       ctypes.byref(qc), ctypes.byref(f.c), 0.1, 1, None, 0, 16, tq.TQ_BF16,
                                       None, None, None)
    assert call_qjl(2, 8) == tq.TQ_OK                           # 4-bit K + QJL: the main kernel, several queries
    assert call_qjl(1, 128) == tq.TQ_OK                         # 64 q heads per kv head
    assert call_qjl(33, 4) == tq.TQ_ERR_UNSUPPORTED_FORMAT      # 66 columns: past the 64 of the QJL path
    assert "64" in L.tq_last_error().decode()
    f3 = tq.Format(128, [3], s)                                 # a layout only the separate QJL kernel reads
    q3 = _qjl_c(f3)
    def call_q3(NQ, Hq):
        return L.tq_decode_paged_multi(16, tq.TQ_BF16, 0, NQ, Hq, 2, 16, 16, 10, 16, 16, 4, 16,
                                       ctypes.byref(q3), ctypes.byref(f.c), 0.1, 1, None, 0, 16, tq.TQ_BF16,
                                       None, None, None)
    assert call_q3(2, 8) == tq.TQ_ERR_UNSUPPORTED_FORMAT        # one query there
    assert call_q3(1, 32) == tq.TQ_ERR_UNSUPPORTED_FORMAT       # and at most 8 q heads per kv head
    assert call_q3(1, 16) == tq.TQ_OK


def _qjl_c(f, proj=0x1000):
    """The format's C struct with the QJL stage switched on (a stand-in
    device pointer: no call here dereferences it)."""
    c = tq.tq_format()
    ctypes.memmove(ctypes.byref(c), ctypes.byref(f.c), ctypes.sizeof(c))
    c.qjl = 1
    c.qjl_proj = proj
    return c


@pytest.mark.parametrize("i", range(6))
def test_qjl_tile_bytes_match_oracle(i):
    d, bits, s, ch = _fmts()[i]
    c = _qjl_c(tq.Format(d, bits, s, ch))
    m = d // len(bits)
    of = oracle.Format.make(d, bits, s, ch, qjl_proj=np.zeros((len(bits), m, m), np.float32))
    rb, _, tile = opg.tile_layout(of, 16)
    rib, tb = ctypes.c_int32(), ctypes.c_int32()
    assert tq._lib.tq_tile_bytes(ctypes.byref(c), 16, ctypes.byref(rib), ctypes.byref(tb)) == tq.TQ_OK
    assert (rib.value, tb.value) == (rb, tile)


def test_qjl_status_codes_without_launch():
    s = signs(0, 1, 128)
    f4 = tq.Format(128, [4], s)
    assert ctypes.sizeof(tq.tq_format) == 352            # the C struct: 336 bytes, then qjl, padding, the pointer
    c = _qjl_c(f4, proj=None)
    assert tq._lib.tq_format_check(ctypes.byref(c)) == tq.TQ_ERR_VALUE     # projection missing
    c = _qjl_c(f4)
    c.qjl = 2
    assert tq._lib.tq_format_check(ctypes.byref(c)) == tq.TQ_ERR_VALUE
    kq = _qjl_c(f4)
    assert tq._lib.tq_format_check(ctypes.byref(kq)) == tq.TQ_OK

    class _F:   # a Format-like holder for the call helpers
        def __init__(self, cs):
            self.c = cs
    fq = _F(kq)
    assert _call_decode(vf=fq) == tq.TQ_ERR_VALUE                     # QJL on V
    assert _call_decode(kf=fq, B=0) == tq.TQ_OK
    assert _call_decode(kf=fq, P=4) == tq.TQ_ERR_VALUE                # workspace missing
    L = tq._lib
    st = L.tq_decode_paged_multi(1, tq.TQ_BF16, 2, 17, 8, 2, 1, 1, 10, 16, 1, 4, 1, ctypes.byref(kq),
                                 ctypes.byref(f4.c), 0.1, 1, None, 0, 1, tq.TQ_BF16, None, None, None)
    assert st == tq.TQ_ERR_UNSUPPORTED_FORMAT                         # 68 columns: past the QJL path's 64
    assert _call_write(vf=fq) == tq.TQ_ERR_VALUE                      # QJL on V


def test_qjl_alignment_checked_before_launch():
    s = signs(0, 1, 128)
    f4 = tq.Format(128, [4], s)
    kq = _qjl_c(f4, proj=0x1004)   # not 16-byte aligned

    class _F:
        def __init__(self, cs):
            self.c = cs
    assert _call_decode(kf=_F(kq), kp=0x1000, vp=0x2000) == tq.TQ_ERR_VALUE
    assert "aligned" in tq._lib.tq_last_error().decode()


def test_qjl_write_alignment_checked_before_launch():
    s = signs(0, 1, 128)
    f4 = tq.Format(128, [4], s)

    class _F:
        def __init__(self, cs):
            self.c = cs
    assert _call_write(kf=_F(_qjl_c(f4, proj=0x1008))) == tq.TQ_ERR_VALUE
    assert "aligned" in tq._lib.tq_last_error().decode()


def test_fused_window_status_codes_without_launch():
    """tq_decode_paged_window with stand-in pointers: every call here is
    refused by host validation or returns before any launch."""
    s = signs(0, 1, 128)
    f = tq.Format(128, [4], s)
    L = tq._lib

    def call(B=2, Hq=8, Hkv=2, kf=None, k=16, v=16, wd=None, cap=4, lens=16, ws=None, wsb=0):
        kc = f.c if kf is None else kf
        wd = tq.TQ_BF16 if wd is None else wd
        return L.tq_decode_paged_window(16, tq.TQ_BF16, B, Hq, Hkv, 16, 16, 10, 16, 16, 4, 16, ctypes.byref(kc),
                                        ctypes.byref(f.c), k, v, wd, cap, lens, 0.1, 1, ws, wsb, 16, tq.TQ_BF16,
                                        None, None, None)
    assert call(wd=tq.TQ_F32) == tq.TQ_ERR_UNSUPPORTED_FORMAT       # f32 windows: tq_decode_dense
    assert call(Hq=34, Hkv=2) == tq.TQ_ERR_UNSUPPORTED_FORMAT       # 17 q heads per kv head
    assert "16 q heads" in L.tq_last_error().decode()
    assert call(cap=-1) == tq.TQ_ERR_VALUE
    assert call(lens=None) == tq.TQ_ERR_VALUE
    assert call(k=None) == tq.TQ_ERR_VALUE
    assert call(k=24) == tq.TQ_ERR_VALUE                             # not 16-byte aligned
    assert "aligned" in L.tq_last_error().decode()
    assert call() == tq.TQ_ERR_VALUE                                 # one split still needs the window's slot
    assert "workspace" in L.tq_last_error().decode()
    need = tq.workspace_bytes(2, 8, 128, 2)
    assert need > 0
    assert call(ws=16, wsb=need - 1) == tq.TQ_ERR_VALUE
    q3 = _qjl_c(tq.Format(128, [3], s))                              # the separate QJL kernel's layout
    assert call(kf=q3) == tq.TQ_ERR_UNSUPPORTED_FORMAT
    assert call(B=0) == tq.TQ_OK
