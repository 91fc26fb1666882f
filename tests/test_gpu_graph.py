"""A layer step (tq_write_kv of the current tokens, then tq_decode_paged with
its split merge) captured as a HIP graph and replayed: every replay, with
eager work and synchronisations between replays, gives the eager step's
result (the decode's block sharing between waves may reorder fp32 sums, so
bf16 outputs may differ by one bf16 step and lse by 1e-5; pages bit for
bit)."""
import numpy as np
import pytest

from tests.conftest import gpu_available
from tests.helpers import product_format, to_device, slots_of
import workloads as wl

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


@pytest.mark.parametrize("kbits,vbits,P,qjl", [([4], [4], 4, False), ([3, 2], [2], 3, True)])
def test_layer_step_graph_replays_match_eager(kbits, vbits, P, qjl):
    import torch
    import quantized_paged_kv_amd as tq
    print(f"case graph K{kbits} V{vbits} P{P} qjl={qjl}", flush=True)
    w = wl.small_decode_workload(77, 3, 8, 2, 128, [300, 1000, 17], kbits, vbits, num_splits=P, qjl=qjl)
    kf, vf = product_format(w.kfmt), product_format(w.vfmt)
    kp = torch.zeros((w.num_blocks, 2, kf.tile_bytes()[1]), dtype=torch.uint8, device="cuda")
    vp = torch.zeros((w.num_blocks, 2, vf.tile_bytes()[1]), dtype=torch.uint8, device="cuda")
    new_k, new_v, new_s = [], [], []
    for s, sl in enumerate(slots_of(w.block_tables, w.context_lens)):
        xk, xv = to_device(wl.kv_values(w, "k", s), "bf16"), to_device(wl.kv_values(w, "v", s), "bf16")
        slt = torch.from_numpy(sl).cuda()
        tq.write_kv(xk[:-1], xv[:-1], slt[:-1], kp, vp, kf, vf)   # history; the last token is the step's
        new_k.append(xk[-1:]); new_v.append(xv[-1:]); new_s.append(slt[-1:])
    nk, nv, ns = torch.cat(new_k).contiguous(), torch.cat(new_v).contiguous(), torch.cat(new_s).contiguous()
    q = to_device(wl.q_values(w), "bf16")
    bt = torch.from_numpy(w.block_tables).cuda()
    cl = torch.from_numpy(w.context_lens).cuda()
    out = torch.empty((3, 8, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((3, 8), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(tq.workspace_bytes(3, 8, 128, P), 1), dtype=torch.uint8, device="cuda")

    def step():
        tq.write_kv(nk, nv, ns, kp, vp, kf, vf)
        tq.decode_paged(q, kp, vp, bt, cl, kf, vf, w.scale, num_splits=P, out=out, lse=lse, workspace=ws)

    step()
    torch.cuda.synchronize()
    ref_o, ref_l = out.float().cpu().numpy(), lse.cpu().numpy()
    ref_k, ref_v = kp.cpu().numpy(), vp.cpu().numpy()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    other = torch.empty_like(out)
    for r in range(4):
        out.zero_()
        lse.fill_(0.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        o, l = out.float().cpu().numpy(), lse.cpu().numpy()
        assert np.array_equal(kp.cpu().numpy(), ref_k) and np.array_equal(vp.cpu().numpy(), ref_v), r
        assert np.max(np.abs(l - ref_l)) <= 1e-5, (r, np.max(np.abs(l - ref_l)))
        # bf16 outputs: a reordered fp32 sum may move a value by one bf16 step
        assert np.all(np.abs(o - ref_o) <= 2.0 ** -8 * np.abs(ref_o) + 1e-6), r
        # eager work between replays: a decode into another buffer
        tq.decode_paged(q, kp, vp, bt, cl, kf, vf, w.scale, num_splits=P, out=other, workspace=ws)
        torch.cuda.synchronize()
