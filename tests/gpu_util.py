"""Shared helpers of the GPU parity tests: run the HIP library through its C
ABI on seeded synthetic layers and compare with the CPU oracle."""
from __future__ import annotations

import numpy as np

import int4_routed_expert_bias_amd as coli
import oracle as oracle_mod
import synth

TOL = 1e-3  # max|gpu - ref| <= TOL * max|ref| per output tensor


def rel_err(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    m = np.abs(ref).max()
    return float(np.abs(got - ref).max() / (m if m > 0 else 1.0))


def assert_close(got, ref, what, tol=TOL):
    e = rel_err(got, ref)
    assert e <= tol, f"{what}: max|gpu-ref|/max|ref| = {e:.3e} > {tol}"
    return e


def f32_ulp_diff(a, b):
    ai = np.asarray(a, np.float32).view(np.int32).astype(np.int64)
    bi = np.asarray(b, np.float32).view(np.int32).astype(np.int64)
    ai = np.where(ai < 0, -(ai & 0x7FFFFFFF), ai)
    bi = np.where(bi < 0, -(bi & 0x7FFFFFFF), bi)
    return np.abs(ai - bi)


def check_route(gpu_ids, gpu_w, orc_ids, orc_w, orc_scores, bias):
    """Ids must equal the oracle's.  A token may differ only at a near-tie of
    the selection keys (within 4 ulps at the k-th position), where both
    orders are correct; such tokens are counted and returned."""
    gpu_ids = np.asarray(gpu_ids)
    near = 0
    for t in range(orc_ids.shape[0]):
        if np.array_equal(gpu_ids[t], orc_ids[t]):
            continue
        key = (orc_scores[t] + bias).astype(np.float32)
        kth = key[orc_ids[t, -1]]
        diff = set(gpu_ids[t].tolist()) ^ set(orc_ids[t].tolist())
        order_only = not diff
        cands = diff if diff else set(orc_ids[t].tolist())
        ok = all(f32_ulp_diff(key[e], kth) <= 4 for e in cands) or order_only and all(
            f32_ulp_diff(key[gpu_ids[t, j]], key[orc_ids[t, j]]) <= 4 for j in range(len(gpu_ids[t])))
        assert ok, f"token {t}: gpu ids {gpu_ids[t]} != oracle {orc_ids[t]} (not a near tie)"
        near += 1
    assert_close(gpu_w, orc_w, "topk_w")
    return near


class GpuLayer:
    """A synthetic layer on the GPU plus its host arrays for the oracle."""

    def __init__(self, arrays: dict, k: int, n_shared: int = 1):
        self.arrays = arrays
        self.k = k
        self.n_shared = n_shared
        self.dev = coli.DeviceLayer(arrays, k=k, n_shared=n_shared)
        self.orc = oracle_mod.Layer(arrays, k=k, n_shared=n_shared)
        self.H, self.I, self.E = arrays["H"], arrays["I"], arrays["E"]

    def run(self, x_np: np.ndarray, act_mode: int, dump: bool = False):
        import torch
        T = x_np.shape[0]
        x = torch.from_numpy(np.ascontiguousarray(x_np)).cuda()
        b = coli.Buffers(self.dev, T, act_mode, dump=dump)
        coli.run_layer(self.dev, x, b)
        torch.cuda.synchronize()
        nu = int(b.n_union[0].item())
        out = dict(ids=b.ids[:T].cpu().numpy(), w=b.w[:T].cpu().numpy(), y=b.y[:T].cpu().numpy(),
                   union_ids=b.union_ids.cpu().numpy(), offsets=b.offsets.cpu().numpy(),
                   slots=b.slots[:T * self.k].cpu().numpy(), n_union=nu)
        if dump:
            out["dump"] = coli.dump_views(b.dump.cpu().numpy(), self.H, self.I, self.k, T,
                                          self.n_shared)
        return out


def make_layer(H, I, E, k, wid, layer=0, n_shared=1, bias_kind="normal"):
    A = synth.layer_arrays(H, I, E, k, wid=wid, layer=layer, n_shared=n_shared,
                           bias_kind=bias_kind)
    return GpuLayer(A, k, n_shared)
