"""coli_moe_route_forward_noalloc (the layer step with its scratch in the
library's static device array) against coli_moe_route_forward with a
caller workspace: the same routing, union and output, bit for bit, on two
calls in a row (the second with fewer tokens, so the array holds the first
call's larger contents), in both arithmetic families."""
import numpy as np
import pytest

from conftest import gpu_available

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]

import int4_routed_expert_bias_amd as coli  # noqa: E402
import synth  # noqa: E402


def _outs(b, T):
    n_kept = int(b.offsets[int(b.n_union[0].item())].item())
    return {"ids": b.ids[:T].cpu().numpy(), "w": b.w[:T].cpu().numpy().view(np.uint32),
            "union_ids": b.union_ids.cpu().numpy(), "offsets": b.offsets.cpu().numpy(),
            "slots": b.slots[:n_kept].cpu().numpy(), "n_union": b.n_union[:1].cpu().numpy(),
            "y": b.y[:T].cpu().numpy().view(np.uint32)}


def _run(lay, x, T, mode, top_p, noalloc):
    import torch
    b = coli.Buffers(lay, T, mode)
    for t in (b.ids, b.union_ids, b.offsets, b.slots, b.n_union):
        t.fill_(-7)
    b.w.fill_(-7.0)
    b.y.fill_(-7.0)
    if noalloc:
        coli.route_forward_noalloc(lay, x, T, b.ids, b.w, b.union_ids, b.offsets, b.slots,
                                   b.n_union, mode, b.y, top_p=top_p)
    else:
        coli.route_forward(lay, x, T, b.ids, b.w, b.union_ids, b.offsets, b.slots, b.n_union,
                           mode, b.y, b.workspace, top_p=top_p)
    torch.cuda.synchronize()
    return _outs(b, T)


@pytest.mark.parametrize("mode,Ts", [(coli.ACT_F32, (4, 1)), (coli.ACT_I8, (4, 1)),
                                     (coli.ACT_I8, (40, 3)), (coli.ACT_F32, (19, 2))])
@pytest.mark.parametrize("top_p", [None, 0.7])
def test_noalloc_equals_route_forward(mode, Ts, top_p):
    import torch
    w = synth.WORKLOADS["decode"]
    lay = coli.DeviceLayer(synth.workload_layer(w), k=w.k, n_shared=w.n_shared)
    for i, T in enumerate(Ts):
        print(f"noalloc mode={mode} T={T} top_p={top_p}", flush=True)
        x = torch.from_numpy(synth.activations(w.H, T, wid=90 + i + T)).cuda()
        a = _run(lay, x, T, mode, top_p, noalloc=True)
        c = _run(lay, x, T, mode, top_p, noalloc=False)
        for name in a:
            assert np.array_equal(a[name], c[name]), (mode, T, name)


def test_noalloc_rejects_beyond_scratch():
    import torch
    w = synth.WORKLOADS["decode"]
    lay = coli.DeviceLayer(synth.workload_layer(w, experts=[0]), k=w.k, n_shared=w.n_shared)
    T = 114
    b = coli.Buffers(lay, 1, coli.ACT_F32)
    x = torch.zeros((T, w.H), device="cuda")
    ids = torch.empty((T, w.k), dtype=torch.int32, device="cuda")
    wt = torch.empty((T, w.k), device="cuda")
    y = torch.empty((T, w.H), device="cuda")
    sl = torch.empty((T * w.k,), dtype=torch.int32, device="cuda")
    with pytest.raises(coli.ColiError) as e:
        coli.route_forward_noalloc(lay, x, T, ids, wt, b.union_ids, b.offsets, sl, b.n_union,
                                   coli.ACT_F32, y)
    assert e.value.status == coli.COLI_E_SCRATCH
