"""Shared helpers of the GPU parity tests: run the HIP library through its C
ABI on seeded synthetic layers and compare with the CPU oracle."""
from __future__ import annotations

import os

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


def pool_map(fn, items, workers=None):
    """fn over items on a thread pool (the oracle's C calls release the GIL);
    results in item order.  At most 16 workers (one GPU's CPU share)."""
    from concurrent.futures import ThreadPoolExecutor
    items = list(items)
    n = workers or max(1, min(16, os.cpu_count() or 1, len(items)))
    with ThreadPoolExecutor(n) as ex:
        return list(ex.map(fn, items))


def orc_route_all(orc, lay_orc, x, chunk=64):
    """The oracle's routing of every row of x (ids, w, logits, scores), rows
    split over threads."""
    x = np.ascontiguousarray(x, np.float32)
    parts = pool_map(lambda a: orc.route(lay_orc, x[a:a + chunk]), range(0, x.shape[0], chunk))
    return tuple(np.concatenate([p[i] for p in parts]) for i in range(4))


def check_route(gpu_ids, gpu_w, orc_ids, orc_w):
    """Router selections must equal the oracle's bit for bit, every token and
    every position (the selection order included); the routing weights agree
    within the tolerance."""
    gpu_ids = np.asarray(gpu_ids)
    bad = np.nonzero(~np.all(gpu_ids == orc_ids, axis=1))[0]
    assert bad.size == 0, (f"{bad.size} token(s) routed differently from the oracle, first "
                           f"{bad[0]}: gpu {gpu_ids[bad[0]]} vs oracle {orc_ids[bad[0]]}")
    assert_close(gpu_w, orc_w, "topk_w")


def tile_rows(ids, union_ids, offsets, slots, n_union, T, k, n_shared, tile=128):
    """Rows of the expert outputs o to check so that the first and the last
    tile of every union entry's row list hold a checked row (its first row,
    the last rows of the first tile's two halves, its last row): a list of
    (o row, token, expert) with o row = slot t*k+j for a routed expert and
    T*k+t for the shared expert (expert -1)."""
    rows = []
    for u in range(n_union):
        a, b = int(offsets[u]), int(offsets[u + 1])
        for p in sorted({a, min(a + tile // 2 - 1, b - 1), min(a + tile - 1, b - 1), b - 1}):
            sl = int(slots[p])
            t, j = sl // k, sl % k
            assert ids[t, j] == union_ids[u]
            rows.append((sl, t, int(union_ids[u])))
    if n_shared:
        for t in sorted({0, min(tile // 2 - 1, T - 1), min(tile - 1, T - 1), T - 1}):
            rows.append((T * k + t, t, -1))
    return rows


PERM8_INV = np.array([0, 4, 1, 5, 2, 6, 3, 7])  # natural element b sits at position PERM8_INV[b]


def check_expert_rows_i8(orc, arrays, x, bufs, rows, T, k, n_shared, what):
    """Int8 family, grouped GEMM (T > 4): for each listed (o row, token,
    expert), the GPU's int8 codes of h and their scales (read from the
    forward's workspace) against the oracle's -- every code within one of
    the oracle's (a flip at a rounding boundary), flips rare overall -- and
    the GPU's expert output against the oracle's down projection on the
    GPU's own codes (the accumulators are exact given the operands).
    Returns the fraction of flipped codes."""
    H, I = arrays["H"], arrays["I"]
    E = arrays["E"]
    off = coli.i8_workspace_offsets(H, I, E, k, T, n_shared)
    ws = bufs.workspace
    R = T * k + n_shared * T
    kept = int(bufs.offsets[int(bufs.n_union[0].item())].item())
    slots = bufs.slots[:kept].cpu().numpy()
    pos_of = np.full(T * k, -1, np.int64)
    pos_of[slots] = np.arange(kept)
    pos = np.array([pos_of[r[0]] if r[2] >= 0 else r[0] for r in rows])
    assert (pos >= 0).all()
    import torch
    G2 = I // 64
    qh_all = ws[off["qh"]:off["qh"] + R * I].view(R, I)
    sh_all = ws[off["sh"]:off["sh"] + R * G2 * 4].view(torch.float32).view(R, G2)
    o_all = ws[off["o"]:off["o"] + R * H * 4].view(torch.float32).view(R, H)
    pt = torch.tensor(pos, device=ws.device)
    qh = qh_all[pt].cpu().numpy().view(np.int8).reshape(len(rows), -1, 8)[:, :, PERM8_INV]
    qh = np.ascontiguousarray(qh.reshape(len(rows), I))
    sh = sh_all[pt].cpu().numpy()
    o = o_all[torch.tensor([r[0] for r in rows], device=ws.device)].cpu().numpy()

    def weights(e):
        if e >= 0:
            return arrays["w13"][e], arrays["s13"][e], arrays["w2"][e], arrays["s2"][e]
        return arrays["sh_w13"], arrays["sh_s13"], arrays["sh_w2"], arrays["sh_s2"]

    def ref(i):
        _, t, e = rows[i]
        w13, s13, w2, s2 = weights(e)
        full = orc.expert_i8(w13, s13, w2, s2, x[t])
        return full["qh"], full["sh"], orc.down_i8(w2, s2, qh[i], sh[i])

    refs = pool_map(ref, range(len(rows)))
    flips = 0
    for i, (r, (qr, sr, og)) in enumerate(zip(rows, refs)):
        tag = f"{what}: o row {r[0]} (token {r[1]}, expert {r[2]})"
        d = np.abs(qh[i].astype(np.int32) - qr.astype(np.int32))
        assert d.max() <= 1, f"{tag}: a code of h differs by {d.max()}"
        flips += int((d > 0).sum())
        assert_close(sh[i], sr, f"{tag}: scales of h")
        assert_close(o[i], og, f"{tag}: down projection on the GPU's codes")
    frac = flips / (len(rows) * I)
    assert frac < 0.01, f"{what}: {frac:.2%} of the codes of h flipped"
    return frac


def orc_y_rows(orc, lay_orc, x_rows, ids_rows, w_rows, mode):
    """The oracle's layer output for each given token (its input row, ids
    and weights), one token per thread."""
    x_rows = np.ascontiguousarray(x_rows, np.float32)
    ys = pool_map(lambda i: orc.forward_rows(lay_orc, x_rows[i:i + 1], ids_rows[i:i + 1],
                                             w_rows[i:i + 1], np.zeros(1, np.int32), mode)[0],
                  range(x_rows.shape[0]))
    return np.stack(ys)


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
