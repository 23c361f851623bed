"""coli_moe_route_forward_timeline (the self-routing fp32 step whose kernels
also write per-wave real-time marks): its outputs equal those of
coli_moe_route_forward bit for bit, and every recorded wave's marks are
ordered (entry <= the phase marks it reached <= exit)."""
import numpy as np
import pytest

from conftest import gpu_available

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]

import int4_routed_expert_bias_amd as coli  # noqa: E402
import synth  # noqa: E402

CAP = 8192


def _outs(b, T):
    n_kept = int(b.offsets[int(b.n_union[0].item())].item())
    return {"ids": b.ids[:T].cpu().numpy(), "w": b.w[:T].cpu().numpy().view(np.uint32),
            "union_ids": b.union_ids.cpu().numpy(), "offsets": b.offsets.cpu().numpy(),
            "slots": b.slots[:n_kept].cpu().numpy(), "n_union": b.n_union[:1].cpu().numpy(),
            "y": b.y[:T].cpu().numpy().view(np.uint32)}


@pytest.mark.parametrize("T", [1, 2, 4])
def test_timeline_step_equals_route_forward(T):
    import torch
    w = synth.WORKLOADS["decode"]
    lay = coli.DeviceLayer(synth.workload_layer(w), k=w.k, n_shared=w.n_shared)
    x = torch.from_numpy(synth.activations(w.H, T, wid=300 + T)).cuda()
    names = coli.route_forward_kernel_names(coli.ACT_F32, T)
    print(f"timeline T={T} kernels={names}", flush=True)
    res = []
    rec = torch.zeros((len(names), CAP, 8), dtype=torch.int64, device="cuda")
    for timed in (True, False):
        b = coli.Buffers(lay, T, coli.ACT_F32)
        b.y.fill_(-7.0)
        if timed:
            coli.route_forward_timeline(lay, x, T, b.ids, b.w, b.union_ids, b.offsets, b.slots,
                                        b.n_union, coli.ACT_F32, b.y, b.workspace, rec, CAP)
        else:
            coli.route_forward(lay, x, T, b.ids, b.w, b.union_ids, b.offsets, b.slots,
                               b.n_union, coli.ACT_F32, b.y, b.workspace)
        torch.cuda.synchronize()
        res.append(_outs(b, T))
    for name in res[0]:
        assert np.array_equal(res[0][name], res[1][name]), name
    r = rec.cpu().numpy()
    for i, nm in enumerate(names):
        live = r[i, :, 0] > 0
        if nm == "combine_kernel":
            assert not live.any()  # writes no marks
            continue
        assert live.any(), nm
        m = r[i, live]
        assert (m[:, 7] >= m[:, 0]).all(), nm
        for j in (1, 2, 3):
            hit = m[:, j] > 0
            assert (m[hit, j] >= m[hit, 0]).all() and (m[hit, j] <= m[hit, 7]).all(), (nm, j)
    # the kernels ran in order: each one's first entry after the previous one's first entry
    firsts = [r[i, r[i, :, 0] > 0, 0].min() for i, nm in enumerate(names) if nm != "combine_kernel"]
    assert firsts == sorted(firsts)
