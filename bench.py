#!/usr/bin/env python3
"""Throughput of the int4 routed-expert MoE layer on one MI355X.

A step is one pass of the whole path -- route, union and forward -- over one
batch of seeded synthetic tokens: one coli_moe_route_forward call for up to
4 tokens (the gate/up kernel routes the tokens itself; one token in the fp32
family: three launches -- router GEMV, gate/up, down with the combine), else
coli_moe_route_union and coli_moe_forward.

Workloads (--workload):
  decode         H6144 I2048 E256 top-8 + 1 shared, T=1, fp32 family
                 (the default); steps cycle over --layers resident copies of
                 the layer (distinct weights, like consecutive layers of a
                 model) so each step reads its experts from HBM and not from
                 the 256 MB Infinity Cache.
  verify         same layer, T=4 tokens sharing a common component, fp32.
  prefill512     same layer, T=512, Zipf(1.1) popularity, int8 family.
  prefill4096x8  T=4096 through 8 stacked layers (RMS pre-norm, residual),
                 int8 family; a step is the whole stack.
  tiny           H256 I128 E16 top-2, T=4 (parity-size workload).

The timed steps are captured once in a HIP graph and replayed between two
synchronisations (wall clock).  The dominant kernel's duration comes from
HIP events that each kernel's own dispatch records at its start and end
(coli_moe_route_forward_profiled / coli_moe_forward_profiled launch through
hipExtLaunchKernel on the library's stream), over the same inputs.  Prints
one JSON line.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0     # MI355X HBM3E
I8_PEAK_TOPS = 5000.0     # dense int8 MFMA
METRIC = "MoE layer tokens/s + achieved HBM GB/s (decode) / int8 TOPS (prefill)"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Hip:
    """HIP events through the runtime torch already loaded."""

    def __init__(self):
        import torch  # noqa: F401  (loads libamdhip64.so.7 first)
        self.L = ctypes.CDLL("libamdhip64.so.7")
        self.L.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.L.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                               ctypes.c_void_p]
        self.L.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.L.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        e = ctypes.c_void_p()
        assert self.L.hipEventCreate(ctypes.byref(e)) == 0
        return e.value

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        assert self.L.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
        return ms.value

    def destroy(self, e):
        self.L.hipEventDestroy(e)


def expert_bytes(H, I):
    return 3 * I * H // 2 + 3 * I * (H // 64) * 2


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default="decode",
                    choices=["decode", "verify", "prefill512", "prefill4096x8", "tiny",
                             "mla", "mla_verify", "mla_dsa"])
    ap.add_argument("--layers", type=int, default=None, help="resident layer copies cycled (decode/verify)")
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of a HIP graph")
    ap.add_argument("--act-mode", choices=["f32", "i8"], default=None,
                    help="arithmetic family (default: the workload's own)")
    ap.add_argument("--topp", type=float, default=None,
                    help="adaptive expert top-p router (coli_moe_route_topp) instead of top-k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target oracle sample time")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (the reference for HBM counters)")
    ap.add_argument("--place-slots", type=int, default=None,
                    help="Place + Overlap: routed experts in pinned host memory, this many "
                         "device slots per layer (coli_moe_forward_placed)")
    ap.add_argument("--place-chunk", type=int, default=1, help="loaded experts per compute pass")
    ap.add_argument("--no-overlap", action="store_true",
                    help="placed mode: copies on the compute stream (no copy/compute overlap)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; the multi-GPU sharding "
                                   "of the layer is a design (see the design notes), not built",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import numpy as np
    import torch

    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")  # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": src.numel() * 4, "copies": 3}))
        return

    import int4_routed_expert_bias_amd as coli
    from int4_routed_expert_bias_amd import profiling
    import synth

    assert torch.cuda.is_available(), "needs a GPU"
    torch.cuda.set_device(0)
    if coli.device_check() != coli.COLI_OK:
        raise SystemExit("device is not gfx950: " + coli.strerror(coli.device_check()))

    if args.workload.startswith("mla"):
        return bench_mla(args)
    w = synth.WORKLOADS[args.workload]
    H, I, E, k, T = w.H, w.I, w.E, w.k, w.T
    fam = args.act_mode or w.act_mode
    mode = coli.ACT_I8 if fam == "i8" else coli.ACT_F32
    if args.place_slots is not None:
        return bench_placed(args, w, mode)
    stacked = w.layers > 1
    defaults = {"decode": (256, 32), "verify": (128, 16), "prefill512": (20, 4),
                "prefill4096x8": (4, 1), "tiny": (256, 32)}
    K = args.steps if args.steps is not None else defaults[w.name][0]
    W = args.warmup if args.warmup is not None else defaults[w.name][1]
    if stacked:
        NL = w.layers
    else:
        NL = args.layers if args.layers is not None else (8 if w.name in ("decode", "verify") else 1)

    # ---- resident layers -------------------------------------------------
    t0 = time.time()
    layers = []
    host0 = None
    for l in range(NL):
        A = synth.workload_layer(w, layer=l)
        if l == 0:
            host0 = A
        layers.append(coli.DeviceLayer(A, k=k, n_shared=w.n_shared))
        if l > 0:
            del A
    log(f"[bench] {NL} layer(s) resident ({NL * (w.E + 1) * expert_bytes(H, I) / 1e9:.1f} GB experts) "
        f"in {time.time() - t0:.1f}s")

    # ---- inputs and buffers ----------------------------------------------
    nsteps_in = W + K
    if stacked:
        xs = [torch.from_numpy(synth.workload_x(w, layer=0)).cuda()]
    elif w.x_kind == "overlap":
        xs = [torch.from_numpy(synth.activations(H, T, wid=w.wid, layer=100 + s, kind="overlap")).cuda()
              for s in range(nsteps_in)]
    else:
        xall = torch.from_numpy(synth.activations(H, T * nsteps_in, wid=w.wid)).cuda()
        xs = [xall[s * T:(s + 1) * T] for s in range(nsteps_in)]
    bufs = coli.Buffers(layers[0], T, mode)
    if stacked:
        resid = torch.empty((T, H), dtype=torch.float32, device="cuda")
        xhat = torch.empty_like(resid)

    one_call = coli.route_forward_fused(layers[0], T, mode)  # coli_moe_route_forward

    def step(s):
        if stacked:
            resid.copy_(xs[0])
            for l, lay in enumerate(layers):
                coli.rmsnorm(resid, xhat, T, H, 1e-6)
                coli.run_layer(lay, xhat, bufs, top_p=args.topp)
                coli.add_inplace(resid, bufs.y, T * H)
        else:
            coli.run_layer(layers[s % NL], xs[s], bufs, top_p=args.topp,
                           fused="step" if one_call else True)

    # ---- warmup ----------------------------------------------------------
    for s in range(W):
        step(s)
    torch.cuda.synchronize()

    # ---- timed region ----------------------------------------------------
    use_graph = not args.no_graph
    if use_graph:
        g = torch.cuda.CUDAGraph()
        cap_stream = torch.cuda.Stream()
        cap_stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cap_stream):
            with torch.cuda.graph(g, stream=cap_stream):
                for s in range(K):
                    step(W + s if not stacked else s)
        torch.cuda.synchronize()
        g.replay()  # one untimed replay (graph upload)
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        g.replay()
        torch.cuda.synchronize()
        t_end = time.perf_counter()
    else:
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        for s in range(K):
            step(W + s if not stacked else s)
        torch.cuda.synchronize()
        t_end = time.perf_counter()
    elapsed = t_end - t_start
    layer_passes = K * (w.layers if stacked else 1)
    value = layer_passes * T / elapsed
    ms_per_step = elapsed * 1e3 / K

    # ---- dominant kernel: per-kernel events on the library's stream ------
    hip = Hip()
    names = coli.route_forward_kernel_names(mode, T) if one_call else coli.forward_kernel_names(mode, T)
    nk = len(names)
    dom = next(j for j, nm in enumerate(names) if "gateup" in nm)
    prof_steps = min(K, 64)
    ev = [[hip.event() for _ in range(2 * nk)] for _ in range(prof_steps * (w.layers if stacked else 1))]
    union_sizes = []
    torch.cuda._sleep(200_000_000)  # keep the GPU busy while the host enqueues
    i = 0
    for s in range(prof_steps):
        if stacked:
            resid.copy_(xs[0])
            lays = list(enumerate(layers))
        else:
            lays = [(0, layers[(W + s) % NL])]
        for _, lay in lays:
            x_in = xs[W + s] if not stacked else xhat
            if stacked:
                coli.rmsnorm(resid, xhat, T, H, 1e-6)
            if one_call:
                coli.route_forward_profiled(lay, x_in, T, bufs.ids, bufs.w, bufs.union_ids,
                                            bufs.offsets, bufs.slots, bufs.n_union, mode, bufs.y,
                                            bufs.workspace, ev[i], top_p=args.topp)
            else:
                coli.route_union(lay, x_in, T, bufs.ids, bufs.w, bufs.union_ids, bufs.offsets,
                                 bufs.slots, bufs.n_union, bufs.workspace, top_p=args.topp)
                coli.forward_profiled(lay, x_in, T, bufs.ids, bufs.w, bufs.union_ids,
                                      bufs.offsets, bufs.slots, bufs.n_union, mode, bufs.y,
                                      bufs.workspace, ev[i])
            union_sizes.append(bufs.n_union[:1].clone())
            if stacked:
                coli.add_inplace(resid, bufs.y, T * H)
            i += 1
    torch.cuda.synchronize()
    per_kernel = np.zeros(nk)
    for e in ev:
        for j in range(nk):
            per_kernel[j] += hip.elapsed_ms(e[2 * j], e[2 * j + 1])
    per_kernel /= len(ev)
    for e in ev:
        for x_ in e:
            hip.destroy(x_)
    U = np.array([int(u.item()) for u in union_sizes])
    dur_s = per_kernel[dom] * 1e-3
    n_exp = U.mean() + w.n_shared
    R = T * k + w.n_shared * T
    gateup_bytes = n_exp * (2 * I * (H // 2) + 2 * I * (H // 64) * 2)
    if mode == coli.ACT_F32:
        algo_bytes = gateup_bytes + T * H * 4 + R * I * 4
    elif "i8v" in names[dom]:  # small-batch integer kernels hand h on in fp32
        algo_bytes = gateup_bytes + T * H + T * (H // 64) * 4 + R * I * 4
    else:
        algo_bytes = gateup_bytes + T * H + T * (H // 64) * 4 + R * I + R * (I // 64) * 4
    algo_ops = 2.0 * R * 2 * I * H  # int8 ops (or fp32 flops) of the gate/up matmul
    t_hbm = algo_bytes / (HBM_PEAK_GBS * 1e9)
    t_mfma = algo_ops / (I8_PEAK_TOPS * 1e12) if mode == coli.ACT_I8 else 0.0
    if t_mfma > t_hbm:
        ach = algo_ops / dur_s / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 2), "peak": I8_PEAK_TOPS, "unit": "TOP/s",
                "frac": round(ach / I8_PEAK_TOPS, 4), "traffic": None}
    else:
        ach = algo_bytes / dur_s / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": None}
    traffic = None
    tpath = os.path.join(ROOT, "profiles", "traffic.json")
    if os.path.exists(tpath):
        with open(tpath) as fp:
            rec = json.load(fp).get(f"{w.name}:{names[dom]}")
        # the counters were taken with plain top-k routing
        if rec and rec.get("source_hash") == profiling.source_hash() and args.topp is None:
            traffic = rec["hbm_bytes_per_launch"]
    roof["traffic"] = traffic
    roof["kernel"] = names[dom]
    roof["kernel_us"] = round(per_kernel[dom] * 1e3, 2)
    roof["algorithmic_bytes_per_launch"] = int(algo_bytes)
    roof["algorithmic_ops_per_launch"] = int(algo_ops)
    kernels_us = {names[j]: round(per_kernel[j] * 1e3, 2) for j in range(nk)}

    # ---- CPU baseline: the oracle on a bounded sample ---------------------
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        orc = oracle.default()
        olay = oracle.Layer(host0, k=k, n_shared=w.n_shared)
        xh = synth.workload_x(w, layer=0) if (stacked or w.x_kind == "overlap") else \
            synth.activations(H, T, wid=w.wid)
        done, t_cpu0 = 0, time.perf_counter()
        omode = oracle.ACT_I8 if mode == coli.ACT_I8 else oracle.ACT_F32
        while True:
            xt = xh[done % T:done % T + 1]
            ids, wt, _, _ = (orc.route(olay, xt) if args.topp is None
                             else orc.route_topp(olay, xt, args.topp))
            orc.union(ids, E)
            orc.forward(olay, xt, ids, wt, omode)
            done += 1
            if time.perf_counter() - t_cpu0 >= args.cpu_seconds or done >= 1000:
                break
        t_cpu = time.perf_counter() - t_cpu0
        cpu = {"value": round(done / t_cpu, 4), "unit": "tokens/s", "cores": 1, "kind": "oracle",
               "sample": f"{done} token(s) of the {w.name} workload through route, union and "
                         f"forward on layer 0 ({t_cpu:.1f} s, single-threaded C oracle)"}

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "tokens/s", "n_gpus": 1,
        "steps": K, "warmup": W, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "i8" if mode == coli.ACT_I8 else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "description": w.note, "H": H, "I": I, "E": E, "k": k,
                   "T": T, "n_shared": w.n_shared, "layers": NL,
                   "act_mode": "i8" if mode == coli.ACT_I8 else "f32", "top_p": args.topp,
                   "graph": use_graph, "union_size_mean": round(float(U.mean()), 2),
                   "union_size_minmax": [int(U.min()), int(U.max())],
                   "kernels_us": kernels_us},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


PCIE_PEAK_GBS = 64.0  # PCIe 5.0 x16, one direction (the MI355X host link)


def bench_placed(args, w, mode):
    """Place + Overlap: every layer's routed experts live in pinned host
    memory, --place-slots of them at a time in device slots (LRU).  Steps run
    eagerly (the placed forward synchronises once per layer to read the
    union).  The layers' routers and shared experts differ; their host tiers
    alias one pinned copy of the routed experts (the copy traffic is the
    same as with distinct copies)."""
    import numpy as np
    import torch

    import int4_routed_expert_bias_amd as coli
    import synth

    H, I, E, k, T = w.H, w.I, w.E, w.k, w.T
    if w.layers > 1:
        raise SystemExit("placed mode runs the single-layer workloads (decode, verify, prefill512, tiny)")
    NL = args.layers if args.layers is not None else (8 if w.name in ("decode", "verify") else 1)
    defaults = {"decode": (64, 16), "verify": (32, 8), "prefill512": (8, 4), "tiny": (64, 16)}
    K = args.steps if args.steps is not None else defaults[w.name][0]
    W = args.warmup if args.warmup is not None else defaults[w.name][1]
    n_slots = args.place_slots
    t0 = time.time()
    host = None
    layers = []
    for l in range(NL):
        # layers after the first take their routed experts from layer 0's host tier
        A = synth.workload_layer(w, layer=l, experts=None if l == 0 else [0])
        pl = coli.PlacedLayer(A, k, n_slots, T_max=T, chunk=args.place_chunk,
                              n_shared=w.n_shared, host=host)
        host = pl.host
        layers.append(pl)
        del A
    eb = expert_bytes(H, I)
    log(f"[bench] placed: {NL} layer(s), host tier {E * eb / 1e9:.1f} GB pinned, "
        f"{n_slots} slots/layer ({NL * n_slots * eb / 1e9:.1f} GB device) in {time.time() - t0:.1f}s")

    # plain pinned host -> device copy rate (the ceiling of the staging)
    src = torch.empty(1 << 30, dtype=torch.uint8).pin_memory()
    dst = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    dst.copy_(src, non_blocking=True)
    torch.cuda.synchronize()
    t_c = time.perf_counter()
    for _ in range(3):
        dst.copy_(src, non_blocking=True)
    torch.cuda.synchronize()
    h2d_gbs = 3 * (1 << 30) / (time.perf_counter() - t_c) / 1e9
    del src, dst

    nsteps_in = W + K
    if w.x_kind == "overlap":
        xs = [torch.from_numpy(synth.activations(H, T, wid=w.wid, layer=100 + s, kind="overlap")).cuda()
              for s in range(nsteps_in)]
    else:
        xall = torch.from_numpy(synth.activations(H, T * nsteps_in, wid=w.wid)).cuda()
        xs = [xall[s * T:(s + 1) * T] for s in range(nsteps_in)]
    bufs = coli.Buffers(layers[0], T, mode)
    pws = torch.empty((coli.place_ws_bytes(E, k, T),), dtype=torch.uint8, device="cuda")
    copy_stream = None if args.no_overlap else torch.cuda.Stream()
    # fill every layer's slots (experts 0..n_slots-1), then warm the LRU state
    for pl in layers:
        coli.place_prefetch(pl, list(range(n_slots)), copy_stream=copy_stream)
    torch.cuda.synchronize()

    def step(s, stats):
        for pl in layers:
            st = coli.run_layer_placed(pl, xs[s], bufs, pws, copy_stream=copy_stream,
                                       top_p=args.topp)
            stats.append(st)

    warm = []
    for s in range(W):
        step(s, warm)
    torch.cuda.synchronize()
    stats = []
    t_start = time.perf_counter()
    for s in range(K):
        step(W + s, stats)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    U = np.array([st["n_union"] for st in stats])
    hits = np.array([st["hits"] for st in stats])
    loads = np.array([st["loads"] for st in stats])
    loaded_bytes = loads.sum() * eb
    pcie = loaded_bytes / elapsed / 1e9
    out = {
        "metric": METRIC, "value": round(K * NL * T / elapsed, 2), "unit": "tokens/s",
        "n_gpus": 1, "steps": K, "warmup": W, "ms_per_step": round(elapsed * 1e3 / K, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "i8" if mode == coli.ACT_I8 else "f32", "data": "synthetic",
        "config": {"workload": w.name + "-placed", "description": w.note + "; routed experts in "
                   "pinned host memory, LRU slots in device memory; a step is the token batch "
                   f"through {NL} layer(s), value counts tokens per layer pass", "H": H, "I": I, "E": E, "k": k, "T": T,
                   "n_shared": w.n_shared, "layers": NL,
                   "act_mode": "i8" if mode == coli.ACT_I8 else "f32", "top_p": args.topp,
                   "graph": False, "union_size_mean": round(float(U.mean()), 2),
                   "union_size_minmax": [int(U.min()), int(U.max())]},
        "placement": {"n_slots": n_slots, "chunk": args.place_chunk,
                      "overlap": not args.no_overlap,
                      "hit_rate": round(float(hits.sum() / U.sum()), 4),
                      "loads_per_layer_call": round(float(loads.mean()), 3),
                      "passes_per_layer_call": round(float(np.mean([st["passes"] for st in stats])), 3),
                      "h2d_bytes_per_step": int(loaded_bytes / K),
                      "h2d_copy_gbs_measured": round(h2d_gbs, 2),
                      # share of the wall time the link needs for these bytes at the
                      # measured plain-copy rate
                      "copy_busy_frac": round(loaded_bytes / (h2d_gbs * 1e9) / elapsed, 4)},
        "roofline": {"bound": "pcie", "achieved": round(pcie, 2), "peak": PCIE_PEAK_GBS,
                     "unit": "GB/s", "frac": round(pcie / PCIE_PEAK_GBS, 4), "traffic": None,
                     "kernel": "expert staging (host-to-device copies)"},
        "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)


FP32_PEAK_TFLOPS = 157.3  # MI355X dense fp32 matrix / vector peak

# Decode attention over the compressed (576-float) MLA cache: query tokens,
# heads, cache length, sparse key-list width (0: the whole prefix).
MLA_WORKLOADS = {
    "mla": dict(B=1, H=64, T=32768, n_sel=0,
                note="one decode token, 64 heads, 32,768 cached tokens"),
    "mla_verify": dict(B=4, H=64, T=32768, n_sel=0,
                       note="a 4-token verify batch (causal prefixes) over 32,768 cached tokens"),
    "mla_dsa": dict(B=1, H=64, T=131072, n_sel=2048,
                    note="one decode token, 64 heads, 2,048 keys selected from 131,072 cached"),
}


def bench_mla(args):
    """Steps are coli_mla_decode calls that cycle over --layers distinct caches
    (so each step reads its cache from HBM, not from the 256 MB Infinity
    Cache), captured in one HIP graph.  Kernel durations come from events the
    kernels' own dispatches record (coli_mla_decode_profiled)."""
    import numpy as np
    import torch

    import int4_routed_expert_bias_amd as coli
    import synth

    cfg = MLA_WORKLOADS[args.workload]
    B, Hh, T, n_sel = cfg["B"], cfg["H"], cfg["T"], cfg["n_sel"]
    NL = args.layers if args.layers is not None else 8
    K = args.steps if args.steps is not None else 256
    W = args.warmup if args.warmup is not None else 32
    scale = float(np.float32(1.0 / np.sqrt(192.0)))
    wid = 400 + list(MLA_WORKLOADS).index(args.workload) * 10
    t0 = time.time()
    q = torch.from_numpy(synth.activations(576, B * Hh, wid=wid).reshape(B, Hh, 576)).cuda()
    kvs = [torch.from_numpy(synth.activations(576, T, wid=wid + 1, layer=l)).cuda()
           for l in range(NL)]
    lens = torch.tensor([T - B + 1 + b for b in range(B)], dtype=torch.int32, device="cuda")
    idx = None
    if n_sel:
        rng = np.random.default_rng(wid)
        idx = torch.from_numpy(np.stack([np.sort(rng.choice(T, n_sel, replace=False))
                                         for _ in range(B)]).astype(np.int32)).cuda()
    out = torch.empty((B, Hh, 512), device="cuda")
    ws = torch.empty((coli.mla_workspace_bytes(B, Hh, T, n_sel),), dtype=torch.uint8, device="cuda")
    log(f"[bench] mla: {NL} caches of {T} x 576 fp32 ({NL * T * 2304 / 1e9:.2f} GB) "
        f"in {time.time() - t0:.1f}s")

    def step(s):
        coli.mla_decode(q, kvs[s % NL], out, ws, scale, lens=None if idx is not None else lens,
                        idx=idx)

    for s in range(W):
        step(s)
    torch.cuda.synchronize()
    use_graph = not args.no_graph
    if use_graph:
        g = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cap):
            with torch.cuda.graph(g, stream=cap):
                for s in range(K):
                    step(W + s)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        g.replay()
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t_start
    else:
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        for s in range(K):
            step(W + s)
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t_start

    hip = Hip()
    prof = min(K, 64)
    evs = [[hip.event() for _ in range(4)] for _ in range(prof)]
    torch.cuda._sleep(100_000_000)
    for s in range(prof):
        coli.mla_decode_profiled(q, kvs[(W + s) % NL], out, ws, scale, evs[s],
                                 lens=None if idx is not None else lens, idx=idx)
    torch.cuda.synchronize()
    attn_ms = np.mean([hip.elapsed_ms(e[0], e[1]) for e in evs])
    merge_ms = np.mean([hip.elapsed_ms(e[2], e[3]) for e in evs])
    for e in evs:
        for x in e:
            hip.destroy(x)
    nk = [n_sel] * B if n_sel else [T - B + 1 + b for b in range(B)]
    flops = sum(2.0 * Hh * kk * (576 + 512) for kk in nk)
    keys_read = n_sel * B if n_sel else T   # the prefixes overlap: one read of the cache
    hbm = keys_read * 576 * 4 + B * Hh * 576 * 4
    t_attn = attn_ms * 1e-3
    ach = flops / t_attn / 1e12
    bound = "mfma" if flops / (FP32_PEAK_TFLOPS * 1e12) > hbm / (HBM_PEAK_GBS * 1e9) else "hbm"
    if bound == "mfma":
        roof = {"bound": "mfma", "achieved": round(ach, 2), "peak": FP32_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / FP32_PEAK_TFLOPS, 4), "traffic": None}
    else:
        gbs = hbm / t_attn / 1e9
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None}
    roof.update({"kernel": "mla_attn_kernel", "kernel_us": round(attn_ms * 1e3, 2),
                 "algorithmic_flops_per_launch": int(flops), "algorithmic_bytes_per_launch": int(hbm)})

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        orc = oracle.default()
        qh = q.cpu().numpy()
        kvh = kvs[0].cpu().numpy()
        idxh = None if idx is None else idx.cpu().numpy()
        done, t_c = 0, time.perf_counter()
        while True:  # one query token (all heads) at a time
            b = done % B
            if idxh is None:
                orc.mla_decode(qh[b:b + 1], kvh, scale, lens=np.array([nk[b]], np.int32))
            else:
                orc.mla_decode(qh[b:b + 1], kvh, scale, idx=idxh[b:b + 1])
            done += 1
            if time.perf_counter() - t_c >= args.cpu_seconds or done >= 1000:
                break
        t_cpu = time.perf_counter() - t_c
        cpu = {"value": round(done / t_cpu, 4), "unit": "tokens/s", "cores": 1, "kind": "oracle",
               "sample": f"{done} query token(s) of the {args.workload} workload, all {Hh} heads "
                         f"({t_cpu:.1f} s, single-threaded C oracle)"}

    res = {
        "metric": "MLA decode attention query tokens/s + achieved fp32 matrix TFLOP/s",
        "value": round(K * B / elapsed, 2), "unit": "tokens/s", "n_gpus": 1, "steps": K,
        "warmup": W, "ms_per_step": round(elapsed * 1e3 / K, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": args.workload, "description": cfg["note"], "B": B, "heads": Hh,
                   "T": T, "n_sel": n_sel, "dim": 576, "latent": 512, "scale": scale,
                   "caches": NL, "graph": use_graph,
                   "kernels_us": {"mla_attn_kernel": round(attn_ms * 1e3, 2),
                                  "mla_merge_kernel": round(merge_ms * 1e3, 2)}},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
