"""tq_decode_paged_noalloc (the allocation-free decode, split partials in the
library's per-GPU array) against tq_decode_paged with a caller workspace on
the same inputs, to the decode's parity bar (lse within 1e-4, out 2e-3
normwise and elementwise at fp32 output), and against the oracle: two calls
in a row, the second with a smaller input (fewer sequences, shorter
contexts, fewer splits), so the second reads an array the first left
behind.  Sizes past the array are rejected before any launch."""
import math

import numpy as np
import pytest

from tests.conftest import gpu_available
from tests.helpers import product_format, to_device, out_error, elem_error, slots_of
from tests.oracle_refs import decode_refs
import workloads as wl

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def _cache(w):
    import torch
    import quantized_paged_kv_amd as tq
    kf, vf = product_format(w.kfmt), product_format(w.vfmt)
    kp = torch.full((w.num_blocks, w.num_kv_heads, kf.tile_bytes()[1]), 0xA5, dtype=torch.uint8, device="cuda")
    vp = torch.full((w.num_blocks, w.num_kv_heads, vf.tile_bytes()[1]), 0xA5, dtype=torch.uint8, device="cuda")
    for s, sl in enumerate(slots_of(w.block_tables, w.context_lens)):
        if len(sl):
            tq.write_kv(to_device(wl.kv_values(w, "k", s), w.in_dtype), to_device(wl.kv_values(w, "v", s), w.in_dtype),
                        torch.from_numpy(sl).cuda(), kp, vp, kf, vf, check=True)
    return kp, vp, kf, vf


def _compare(w, P):
    import torch
    import quantized_paged_kv_amd as tq
    kp, vp, kf, vf = _cache(w)
    q = wl.q_values(w)
    qd = to_device(q, w.q_dtype)
    bt = torch.from_numpy(w.block_tables).cuda()
    cl = torch.from_numpy(w.context_lens).cuda()
    o_ws, l_ws = tq.decode_paged(qd, kp, vp, bt, cl, kf, vf, w.scale, num_splits=P, out_dtype=torch.float32,
                                 check=True)
    out = torch.full_like(o_ws, math.nan)
    lse = torch.full_like(l_ws, math.nan)
    err = tq.new_error_word()
    tq.decode_paged_noalloc(qd, kp, vp, bt, cl, kf, vf, w.scale, out, lse, num_splits=P, dev_err=err)
    tq.raise_device_error(err, "tq_decode_paged_noalloc")
    torch.cuda.synchronize()
    o_ws, l_ws, o, l = o_ws.cpu().numpy(), l_ws.cpu().numpy(), out.cpu().numpy(), lse.cpu().numpy()
    ref = decode_refs(w, q, [(s, h) for s in range(w.num_seqs) for h in range(w.num_q_heads)])
    worst = 0.0
    for s in range(w.num_seqs):
        for h in range(w.num_q_heads):
            o_ref, l_ref = ref[(s, h)]
            if l_ref == -math.inf:
                assert l[s, h] == -math.inf and np.all(o[s, h] == 0)
                assert l_ws[s, h] == -math.inf
                continue
            for a, b in ((o[s, h], o_ws[s, h]), (o[s, h], o_ref)):
                worst = max(worst, out_error(a[None], b[None])[0], float(np.max(elem_error(a[None], b[None]))))
                assert out_error(a[None], b[None])[0] <= 2e-3
                assert np.max(elem_error(a[None], b[None])) <= 2e-3
            assert abs(float(l[s, h]) - float(l_ws[s, h])) <= 1e-4
            assert abs(float(l[s, h]) - l_ref) <= 1e-4
    print(f"worst out {worst:.2e}", flush=True)


def test_noalloc_equals_workspace_call_two_calls_in_a_row():
    print("case noalloc: 5 sequences, P 6; then 2 sequences, P 3", flush=True)
    w1 = wl.small_decode_workload(810, 5, 8, 2, 128, [1500, 0, 333, 17, 900], [4], [2], num_splits=6,
                                  max_blocks_per_seq=100)
    _compare(w1, 6)
    w2 = wl.small_decode_workload(811, 2, 4, 1, 64, [200, 45], [4, 3], [4], num_splits=3, max_blocks_per_seq=16,
                                  kv_dist="t3")
    _compare(w2, 3)


def test_noalloc_rejects_a_workspace_past_its_array():
    import torch
    import quantized_paged_kv_amd as tq
    w = wl.small_decode_workload(812, 1, 8, 2, 128, [40], [4], [4])
    kp, vp, kf, vf = _cache(w)
    q = torch.zeros((600, 64, 128), dtype=torch.bfloat16, device="cuda")   # 600 * 64 * 128 splits * 129 * 4 B > 16 MiB
    bt = torch.zeros((600, 4), dtype=torch.int32, device="cuda")
    cl = torch.zeros(600, dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    with pytest.raises(ValueError, match="exceeds"):
        tq.decode_paged_noalloc(q, kp, vp, bt, cl, kf, vf, 0.1, out, num_splits=128)
