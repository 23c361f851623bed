"""GPU tests of Place + Overlap (coli_moe_forward_placed, include/coli_place.h).

Placement changes speed only: for every call the placed forward must give
bitwise the y of the resident forward (coli_moe_forward on a layer with all
experts in device memory), whatever the cache state, the pass split or the
streams, and so stay within the oracle's tolerance.  Sequences of calls move
the cache through empty, partly filled, full and thrashing states."""
import numpy as np
import pytest

from conftest import gpu_available

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]

import int4_routed_expert_bias_amd as coli  # noqa: E402
import oracle as oracle_mod  # noqa: E402
import synth  # noqa: E402
from gpu_util import GpuLayer, assert_close, make_layer  # noqa: E402

ORC = None


def orc():
    global ORC
    if ORC is None:
        ORC = oracle_mod.default()
    return ORC


class Placed:
    """A PlacedLayer on the same arrays as a resident GpuLayer."""

    def __init__(self, lay: GpuLayer, n_slots, T_max, chunk=1, host=None):
        import torch
        self.lay = lay
        self.pl = coli.PlacedLayer(lay.arrays, lay.k, n_slots, T_max, chunk,
                                   n_shared=lay.n_shared, host=host)
        self.copy = torch.cuda.Stream()
        self.pws = {}

    def run(self, x_np, mode, top_p=None, same_stream=False):
        import torch
        T = x_np.shape[0]
        x = torch.from_numpy(np.ascontiguousarray(x_np)).cuda()
        b = coli.Buffers(self.pl, T, mode)
        nb = coli.place_ws_bytes(self.pl.E, self.pl.k, T)
        pws = torch.empty((nb,), dtype=torch.uint8, device="cuda")
        stats = coli.run_layer_placed(self.pl, x, b, pws, top_p=top_p,
                                      copy_stream=None if same_stream else self.copy)
        torch.cuda.synchronize()
        return b.y[:T].cpu().numpy(), b.ids[:T].cpu().numpy(), stats

    def resident(self):
        return {e: self.pl.placer.slot_of(e) for e in range(self.pl.E)
                if self.pl.placer.slot_of(e) >= 0}


def resident_y(lay: GpuLayer, x_np, mode, top_p=None):
    import torch
    T = x_np.shape[0]
    x = torch.from_numpy(np.ascontiguousarray(x_np)).cuda()
    b = coli.Buffers(lay.dev, T, mode)
    coli.run_layer(lay.dev, x, b, top_p=top_p)
    torch.cuda.synchronize()
    return b.y[:T].cpu().numpy(), b.ids[:T].cpu().numpy()


def check_call(P: Placed, x, mode, top_p=None, same_stream=False):
    before = P.resident()
    y, ids, st = P.run(x, mode, top_p=top_p, same_stream=same_stream)
    y_res, ids_res = resident_y(P.lay, x, mode, top_p=top_p)
    assert np.array_equal(ids, ids_res)
    assert np.array_equal(y.view(np.int32), y_res.view(np.int32)), \
        f"placed y differs from resident y (max {np.abs(y - y_res).max():.3e})"
    union = sorted(set(ids[ids >= 0].tolist()))
    assert st["n_union"] == len(union)
    assert st["hits"] == sum(e in before for e in union)
    assert st["loads"] == st["n_union"] - st["hits"]
    assert st["passes"] == 1 + -(-st["loads"] // P.pl.placer.chunk)
    after = P.resident()
    if len(union) <= P.pl.n_slots:
        assert all(e in after for e in union)
    return y, ids, st


@pytest.mark.parametrize("mode", [coli.ACT_F32, coli.ACT_I8])
@pytest.mark.parametrize("n_slots,chunk", [(3, 1), (5, 2), (16, 4)])
def test_tiny_sequence_bitwise(mode, n_slots, chunk):
    w = synth.WORKLOADS["tiny"]
    lay = GpuLayer(synth.workload_layer(w), w.k, w.n_shared)
    P = Placed(lay, n_slots, T_max=64, chunk=chunk)
    kinds = set()
    for i, T in enumerate([4, 4, 1, 3, 17, 4, 2, 33, 4, 1]):
        x = synth.activations(lay.H, T, wid=70 + i, layer=i % 3)
        y, ids, st = check_call(P, x, mode)
        kinds.add((st["hits"] > 0, st["loads"] > 0, st["passes"] > 2))
        if i == 0:  # and the oracle agrees (teacher-forced on the GPU's routing)
            ref = orc().forward_rows(lay.orc, x, ids, resident_w(lay, x), np.arange(T), mode)
            assert_close(y, ref, "placed y vs oracle")
    assert any(k[0] for k in kinds) and any(k[1] for k in kinds)  # hits and loads happened


def resident_w(lay, x):
    import torch
    T = x.shape[0]
    b = coli.Buffers(lay.dev, T, coli.ACT_F32)
    coli.route(lay.dev, torch.from_numpy(x).cuda(), T, b.ids, b.w, b.workspace)
    torch.cuda.synchronize()
    return b.w[:T].cpu().numpy()


@pytest.mark.parametrize("mode", [coli.ACT_F32, coli.ACT_I8])
def test_ragged_shape_thrashing_cache(mode):
    # union larger than the slot pool: later passes reuse slots of earlier ones
    lay = make_layer(320, 192, 10, 3, wid=71)
    P = Placed(lay, n_slots=2, T_max=40, chunk=1)
    saw_reuse = False
    for i, T in enumerate([9, 1, 2, 4, 5, 37, 3]):
        x = synth.activations(lay.H, T, wid=72 + i)
        _, _, st = check_call(P, x, mode)
        saw_reuse |= st["n_union"] > 2
    assert saw_reuse


def test_no_shared_expert_and_same_stream():
    lay = make_layer(256, 128, 12, 3, wid=73, n_shared=0)
    P = Placed(lay, n_slots=4, T_max=24, chunk=2)
    for i, T in enumerate([1, 4, 21, 2]):
        x = synth.activations(lay.H, T, wid=74 + i)
        for mode in (coli.ACT_F32, coli.ACT_I8):
            check_call(P, x, mode, same_stream=(i % 2 == 1))


@pytest.mark.parametrize("mode", [coli.ACT_F32, coli.ACT_I8])
def test_topp_placed(mode):
    lay = make_layer(512, 256, 32, 8, wid=75)
    P = Placed(lay, n_slots=12, T_max=8, chunk=3)
    for i, T in enumerate([4, 1, 4, 3]):
        x = synth.activations(lay.H, T, wid=76 + i)
        check_call(P, x, mode, top_p=0.7)


def test_prefetch_makes_next_call_all_hits():
    import torch
    lay = make_layer(256, 128, 16, 2, wid=77)
    P = Placed(lay, n_slots=8, T_max=4)
    x = synth.activations(lay.H, 4, wid=77)
    _, ids_res = resident_y(lay, x, coli.ACT_F32)
    union = sorted(set(ids_res.ravel().tolist()))
    coli.place_prefetch(P.pl, union, copy_stream=P.copy)
    assert all(P.pl.placer.slot_of(e) >= 0 for e in union)
    _, _, st = check_call(P, x, coli.ACT_F32)
    assert st["hits"] == st["n_union"] and st["loads"] == 0 and st["passes"] == 1
    torch.cuda.synchronize()


def test_decode_full_size_sequence():
    """The H6144/I2048/E256 top-8 layer at T = 1 and 4 with a 24-slot pool."""
    w = synth.WORKLOADS["decode"]
    lay = GpuLayer(synth.workload_layer(w, layer=0), w.k, w.n_shared)
    P = Placed(lay, n_slots=24, T_max=4, chunk=2)
    for i, T in enumerate([1, 1, 4, 1, 4]):
        x = synth.activations(lay.H, T, wid=78 + i)
        for mode in (coli.ACT_F32, coli.ACT_I8):
            check_call(P, x, mode)


def test_new_slot_memory_starts_empty():
    # a descriptor naming other slot memory makes the placer forget its residency
    import torch
    lay = make_layer(256, 128, 16, 2, wid=79)
    P = Placed(lay, n_slots=6, T_max=4)
    x = synth.activations(lay.H, 4, wid=79)
    _, _, st1 = check_call(P, x, coli.ACT_F32)
    _, _, st2 = check_call(P, x, coli.ACT_F32)
    assert st2["loads"] == 0
    pl = P.pl
    pl.slots = {n: torch.zeros_like(t) for n, t in pl.slots.items()}
    pl.slot_table = torch.zeros_like(pl.slot_table)
    for n in ("w13", "s13", "w2", "s2"):
        setattr(pl.tiers, "slot_" + n, pl.slots[n].data_ptr())
    pl.tiers.slot_table = pl.slot_table.data_ptr()
    # (the host-side view still lists the old residency until the call sees
    # the new memory, so the call is checked directly)
    y, _, st3 = P.run(x, coli.ACT_F32)
    y_res, _ = resident_y(lay, x, coli.ACT_F32)
    assert np.array_equal(y.view(np.int32), y_res.view(np.int32))
    assert st3["hits"] == 0 and st3["loads"] == st3["n_union"] == st1["n_union"]
