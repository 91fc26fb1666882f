"""GPU parity of tq_write_kv: packed bytes and norms bit-exact against the
oracle (whole pools compared, including bytes a write must not touch)."""
import numpy as np
import pytest

from oracle import encode as oenc
from oracle import pages as opg
from tests.conftest import gpu_available
from tests.helpers import oracle_format, product_format, to_device, oracle_pages
import workloads as wl

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def _gpu_write(x_k, x_v, slots, num_blocks, kspec, vspec, dtype, fill=0xA5, chunk=None):
    import torch
    import quantized_paged_kv_amd as tq
    kf, vf = product_format(kspec), product_format(vspec)
    H = (x_k if x_k is not None else x_v).shape[1]
    kp = torch.full((num_blocks, H, kf.tile_bytes()[1]), fill, dtype=torch.uint8, device="cuda")
    vp = torch.full((num_blocks, H, vf.tile_bytes()[1]), fill, dtype=torch.uint8, device="cuda")
    T = len(slots)
    chunk = chunk or T
    for a in range(0, T, chunk):
        b = min(T, a + chunk)
        k = to_device(x_k[a:b], dtype) if x_k is not None else None
        v = to_device(x_v[a:b], dtype) if x_v is not None else None
        sl = torch.from_numpy(np.asarray(slots[a:b], dtype=np.int64)).cuda()
        tq.write_kv(k, v, sl, kp if k is not None else None, vp if v is not None else None, kf, vf, check=True)
    torch.cuda.synchronize()
    return kp.cpu().numpy(), vp.cpu().numpy()


def _oracle_pool(x, slots, num_blocks, spec, role, chunk=8192):
    f = oracle_format(spec)
    _, _, tile = opg.tile_layout(f, 16)
    pages = np.full((num_blocks, x.shape[1], tile), 0xA5, dtype=np.uint8)
    for a in range(0, len(slots), chunk):
        opg.write_pages(x[a:a + chunk], slots[a:a + chunk], pages, f, 16, role)
    return pages


def _assert_pool_equal(got, ref, what):
    if not np.array_equal(got, ref):
        bad = np.argwhere(got != ref)
        raise AssertionError(f"{what}: {len(bad)} bytes differ, first at {bad[:5].tolist()}")


def test_tiny_fp32_d64():
    """The tiny workload: 256 tokens, d=64, K4/V4, fp32 rows, permuted pool."""
    w = wl.decode_workload(1)
    xk, xv = wl.kv_values(w, "k", 0), wl.kv_values(w, "v", 0)
    slots = w.block_tables[0, np.arange(256) // 16].astype(np.int64) * 16 + np.arange(256) % 16
    print("case tiny d64 fp32", flush=True)
    kp, vp = _gpu_write(xk, xv, slots, w.num_blocks, w.kfmt, w.vfmt, "f32")
    _assert_pool_equal(kp, _oracle_pool(xk, slots, w.num_blocks, w.kfmt, "k"), "K")
    _assert_pool_equal(vp, _oracle_pool(xv, slots, w.num_blocks, w.vfmt, "v"), "V")


@pytest.mark.parametrize("kbits,vbits,d,dist,dtype", [
    ([4], [4], 128, "t5u", "bf16"),
    ([4], [2], 128, "normal_outliers", "bf16"),
    ([4, 3], [2], 128, "t3", "bf16"),
    ([2], [3], 128, "normal", "f32"),
    ([3, 2], [4, 2], 128, "normal", "bf16"),
    ([4, 2], [2, 4], 64, "t3", "f32"),
    ([2], [4], 64, "normal", "bf16"),
    ([4], [4, 3], 128, "normal", "bf16"),
    ([3, 2], [3, 2], 64, "t3", "f32"),
])
def test_formats_random_slots(kbits, vbits, d, dist, dtype):
    seed = 7 + d + sum(kbits) * 3 + sum(vbits)
    w = wl.write_workload(seed=seed, num_seqs=3, new_tokens=200, num_kv_heads=3, head_dim=d, kbits=kbits,
                          vbits=vbits, kv_dist=dist if dist != "normal_outliers" else "normal", in_dtype=dtype)
    xk, xv = wl.write_values(w, "k"), wl.write_values(w, "v")
    if dist == "normal_outliers":
        xk[:, :, [3, 50, 77, 120]] *= 8
    kspec, vspec = w.kfmt, w.vfmt
    if len(vbits) == 2:
        hi = wl.channel_subset(seed, 9, d, d // 2)
        lo = np.array(sorted(set(range(d)) - set(hi.tolist())))
        vspec = wl.FormatSpec(d, list(vbits), np.concatenate([hi, lo]), w.vfmt.signs)
    print(f"case formats K{kbits} V{vbits} d{d} {dist} {dtype}", flush=True)
    kp, vp = _gpu_write(xk, xv, w.slot_mapping, w.num_blocks, kspec, vspec, dtype)
    _assert_pool_equal(kp, _oracle_pool(xk, w.slot_mapping, w.num_blocks, kspec, "k"), "K")
    _assert_pool_equal(vp, _oracle_pool(xv, w.slot_mapping, w.num_blocks, vspec, "v"), "V")


def test_exact_threshold_ties_and_zero_rows():
    """One-hot rows give |w_j| = c for every channel and r = c exactly; with a
    codebook whose thresholds are -1, 0, +1 every channel sits on a threshold,
    so the tie rule (strictly below) decides every index.  Zero rows take the
    written-out special case."""
    import quantized_paged_kv_amd as tq
    d, H = 128, 2
    s = wl.signs(5, 1, d)
    cb = np.array([-1.5, -0.5, 0.5, 1.5], dtype=np.float16)
    rows = []
    for k in range(0, d, 9):
        for c in (1.0, 0.75, 2.0 ** -20, 1024.0, -3.0):
            r = np.zeros(d, dtype=np.float32)
            r[k] = c
            rows.append(r)
    rows.append(np.zeros(d, dtype=np.float32))
    x = np.stack(rows)[:, None, :].repeat(H, axis=1)
    x[:, 1] *= -1
    T = x.shape[0]
    nb = (T + 15) // 16 + 1
    slots = np.arange(T, dtype=np.int64) + 16
    spec = wl.FormatSpec(d, [2], None, s)
    of = oenc.Format(d, [2], np.arange(d), [cb], s)
    of.validate()
    _, _, tile = opg.tile_layout(of, 16)
    ref = np.full((nb, H, tile), 0xA5, dtype=np.uint8)
    opg.write_pages(x, slots, ref, of, 16)
    # every index is 0 or 2 (exactly on a threshold), zero row is L/2-1 = 1
    idx, norms = oenc.encode_rows(x, of)
    assert set(np.unique(idx[0][:-1]).tolist()) <= {0, 2}
    assert np.all(idx[0][-1] == 1) and np.all(norms[-1] == 0)
    import torch
    pf = tq.Format(d, [2], s, None, [cb.view(np.uint16)])
    kp = torch.full((nb, H, tile), 0xA5, dtype=torch.uint8, device="cuda")
    tq.write_kv(to_device(x, "f32"), None, torch.from_numpy(slots).cuda(), kp, None, pf, pf, check=True)
    _assert_pool_equal(kp.cpu().numpy(), ref, "ties")


@pytest.mark.parametrize("cb_vals", [[-1.5, -0.5, 0.5, 1.5], [-0.01, 0.0, 0.01, 1.0]],
                         ids=["bucketed-search", "thresholds-too-close-for-buckets"])
def test_level_search_extreme_scales(cb_vals):
    """The level index is found by a bucketed search when the codebook allows
    it and the row scale is inside the float range, else by comparing every
    threshold; both give the oracle's bytes, also for rows scaled by 1e36 and
    1e-36 (outside the bucketed search's range) and near thresholds."""
    import torch
    import quantized_paged_kv_amd as tq
    d, H = 128, 2
    s = wl.signs(7, 1, d)
    cb = np.array(cb_vals, dtype=np.float16)
    rng = np.random.default_rng(11)
    base = rng.standard_normal((96, H, d)).astype(np.float32)
    scales = np.array([1.0, 1e36, 1e-36, 3.0, 2.0 ** -60, 2.0 ** 60] * 16, dtype=np.float32)[:, None, None]
    x = wl.bf16_round(base * scales)
    T = x.shape[0]
    nb = (T + 15) // 16 + 1
    slots = np.arange(T, dtype=np.int64) + 16
    of = oenc.Format(d, [2], np.arange(d), [cb], s)
    of.validate()
    _, _, tile = opg.tile_layout(of, 16)
    ref = np.full((nb, H, tile), 0xA5, dtype=np.uint8)
    opg.write_pages(x, slots, ref, of, 16)
    pf = tq.Format(d, [2], s, None, [cb.view(np.uint16)])
    kp = torch.full((nb, H, tile), 0xA5, dtype=torch.uint8, device="cuda")
    tq.write_kv(to_device(x, "bf16"), None, torch.from_numpy(slots).cuda(), kp, None, pf, pf, check=True)
    _assert_pool_equal(kp.cpu().numpy(), ref, "extreme scales")


def test_out_of_range_slot_reports_index_error_and_skips_row():
    import torch
    import quantized_paged_kv_amd as tq
    w = wl.write_workload(seed=3, num_seqs=1, new_tokens=40, num_kv_heads=2, head_dim=128)
    xk = wl.write_values(w, "k")
    slots = w.slot_mapping.copy()
    slots[7] = w.num_blocks * 16          # one past the pool
    kf = product_format(w.kfmt)
    kp = torch.full((w.num_blocks, 2, kf.tile_bytes()[1]), 0xA5, dtype=torch.uint8, device="cuda")
    with pytest.raises(IndexError, match="position 7"):
        tq.write_kv(to_device(xk, "bf16"), None, torch.from_numpy(slots).cuda(), kp, None, kf, kf, check=True)
    good = np.delete(np.arange(40), 7)
    ref = _oracle_pool(xk[good], slots[good], w.num_blocks, w.kfmt, "k")
    _assert_pool_equal(kp.cpu().numpy(), ref, "K with one bad slot")
    slots[7] = -1
    kp2 = torch.full_like(kp, 0xA5)
    with pytest.raises(IndexError):
        tq.write_kv(to_device(xk, "bf16"), None, torch.from_numpy(slots).cuda(), kp2, None, kf, kf, check=True)


def test_write_workload_full_size():
    """Quantise-on-write at full size: 16 sequences x 2048 new tokens, 8 kv
    heads, d=128, Student-t(5) rows, K4/V4: whole pools bit-exact."""
    w = wl.write_workload(seed=0)
    xk, xv = wl.write_values(w, "k"), wl.write_values(w, "v")
    print("case write full size", flush=True)
    kp, vp = _gpu_write(xk, xv, w.slot_mapping, w.num_blocks, w.kfmt, w.vfmt, "bf16")
    _assert_pool_equal(kp, _oracle_pool(xk, w.slot_mapping, w.num_blocks, w.kfmt, "k"), "K")
    _assert_pool_equal(vp, _oracle_pool(xv, w.slot_mapping, w.num_blocks, w.vfmt, "v"), "V")


def test_two_streams_write_disjoint_slots_concurrently():
    """Two write batches with disjoint slots on two streams, with no order
    between them: every other token of the same blocks, so both batches write
    rows of the same tiles at the same time.  Rows are whole bytes and each
    norm its own 2-byte slot, so concurrent writers touch no common byte: the
    pools equal the oracle's whole pools."""
    import torch
    import quantized_paged_kv_amd as tq
    w = wl.write_workload(seed=91, num_seqs=4, new_tokens=512, num_kv_heads=8, head_dim=128, kbits=[4, 3],
                          vbits=[2])
    xk, xv = wl.write_values(w, "k"), wl.write_values(w, "v")
    kf, vf = product_format(w.kfmt), product_format(w.vfmt)
    kp = torch.full((w.num_blocks, 8, kf.tile_bytes()[1]), 0xA5, dtype=torch.uint8, device="cuda")
    vp = torch.full((w.num_blocks, 8, vf.tile_bytes()[1]), 0xA5, dtype=torch.uint8, device="cuda")
    halves = []
    for part in (0, 1):
        idx = np.arange(part, len(w.slot_mapping), 2)
        halves.append((to_device(xk[idx], "bf16"), to_device(xv[idx], "bf16"),
                       torch.from_numpy(w.slot_mapping[idx].astype(np.int64)).cuda(), tq.new_error_word()))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    print("case two streams, interleaved slots", flush=True)
    for (k, v, sl, err), st in zip(halves, streams):
        tq.write_kv(k, v, sl, kp, vp, kf, vf, dev_err=err, stream=st)
    torch.cuda.synchronize()
    for _, _, _, err in halves:
        tq.raise_device_error(err, "concurrent write")
    _assert_pool_equal(kp.cpu().numpy(), _oracle_pool(xk, w.slot_mapping, w.num_blocks, w.kfmt, "k"), "K")
    _assert_pool_equal(vp.cpu().numpy(), _oracle_pool(xv, w.slot_mapping, w.num_blocks, w.vfmt, "v"), "V")
