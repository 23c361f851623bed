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

Without --workload the run reports decode as the headline line (value,
roofline, cpu_baseline) and verify, prefill512 and prefill4096x8 beside it
under "workloads", each with its own tokens/s, roofline (int8 TOP/s for the
prefill GEMM when it is matrix-core bound) and oracle baseline; plus the
plain HBM read rate with the streaming kernels' load pattern
("hbm_read_ceiling"), the GPU clocks and the host CPU.

Per workload, the timed steps are captured once in a HIP graph and replayed
between two synchronisations (wall clock): value = tokens / that time.  The
dominant kernel's duration comes from HIP events that each kernel's own
dispatch records at its start and end (coli_moe_route_forward_profiled /
coli_moe_forward_profiled launch through hipExtLaunchKernel on the library's
stream), over the same inputs.  The step time's median and p10/p90 come
from 50 further replays of the timed graph (warm) and from 64 replays of a
one-step graph, each after a 1 GiB read of other memory that evicts L2 and
the Infinity Cache (cold).  The oracle baseline runs single-threaded on one
pinned host CPU.  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

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
        self.L.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]

    def event(self):
        e = ctypes.c_void_p()
        assert self.L.hipEventCreate(ctypes.byref(e)) == 0
        return e.value

    def record(self, e, stream=None):
        import torch
        st = torch.cuda.current_stream().cuda_stream if stream is None else stream
        assert self.L.hipEventRecord(ctypes.c_void_p(e), ctypes.c_void_p(st)) == 0

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        assert self.L.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
        return ms.value

    def destroy(self, e):
        self.L.hipEventDestroy(e)


def expert_bytes(H, I):
    return 3 * I * H // 2 + 3 * I * (H // 64) * 2


DEFAULT_STEPS = {"decode": (256, 32), "verify": (128, 16), "prefill512": (20, 4),
                 "prefill4096x8": (4, 1), "tiny": (256, 32)}
# the workloads reported beside the headline (decode) in a default run
EXTRA_WORKLOADS = ("verify", "prefill512", "prefill4096x8")


def host_info():
    """CPU model and counts of the host the oracle baseline runs on."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    aff = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None
    return {"cpu_model": model, "nproc": os.cpu_count(), "cpus_allowed": aff}


def gpu_clocks():
    """Current shader and memory clocks (MHz) of GPU 0: the level marked '*'
    in the driver's DPM tables, else rocm-smi's report; None if neither."""
    import glob
    import re
    import subprocess
    out = {}
    for card in sorted(glob.glob("/sys/class/drm/card*/device")):
        try:
            for key, fn in (("sclk", "pp_dpm_sclk"), ("mclk", "pp_dpm_mclk")):
                with open(os.path.join(card, fn)) as f:
                    for line in f:
                        if "*" in line:
                            m = re.search(r"(\d+)\s*[Mm][Hh]z", line)
                            if m:
                                out[key] = int(m.group(1))
            if out:
                out["source"] = card + "/pp_dpm_*"
                return out
        except OSError:
            continue
    try:
        r = subprocess.run(["rocm-smi", "--showclocks"], capture_output=True, text=True,
                           timeout=20)
        for line in r.stdout.splitlines():
            m = re.search(r"\b(sclk|mclk)\b.*?\((\d+)\s*Mhz\)", line, re.I)
            if m and m.group(1).lower() not in out:
                out[m.group(1).lower()] = int(m.group(2))
        if out:
            out["source"] = "rocm-smi --showclocks"
            return out
    except (OSError, subprocess.SubprocessError):
        pass
    return None


class ClockSampler:
    """Samples gpu_clocks() every `period` seconds on a thread while the GPU
    works, so that the reported clocks are the ones under load."""

    def __init__(self, period=0.02):
        import threading
        self.period, self.samples = period, []
        self._stop = threading.Event()
        self._t = threading.Thread(target=self._run, daemon=True)

    def _run(self):
        while not self._stop.is_set():
            c = gpu_clocks()
            if c:
                self.samples.append(c)
            self._stop.wait(self.period)

    def __enter__(self):
        self._t.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        self._t.join()

    def summary(self):
        if not self.samples:
            return None
        out = {"samples": len(self.samples), "source": self.samples[0].get("source")}
        for key in ("sclk", "mclk"):
            v = [c[key] for c in self.samples if key in c]
            if v:
                out[key] = {"median": float(np.median(v)), "min": min(v), "max": max(v)}
        return out


def stream_read_rate(hip, n_bufs=8, nbytes=188 << 20, reps=3):
    """Plain HBM read rate with the streaming kernels' load pattern
    (coli_stream_read) over n_bufs distinct buffers of the decode step's
    size (so that no read is served by the 256 MB Infinity Cache), for a
    range of workgroup counts; GB/s of the best count and all counts."""
    import torch
    import int4_routed_expert_bias_amd as coli
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    bufs = [torch.randint(0, 255, (nbytes,), dtype=torch.uint8, device="cuda") for _ in range(n_bufs)]
    out = torch.empty((64 * cus,), dtype=torch.int32, device="cuda")
    res = {}
    for mult in (1, 2, 4, 8):
        g = mult * cus
        for b in bufs:  # warm
            coli.stream_read(b, out, g)
        torch.cuda.synchronize()
        e0, e1 = hip.event(), hip.event()
        hip.record(e0)
        for _ in range(reps):
            for b in bufs:
                coli.stream_read(b, out, g)
        hip.record(e1)
        torch.cuda.synchronize()
        ms = hip.elapsed_ms(e0, e1)
        hip.destroy(e0)
        hip.destroy(e1)
        res[f"{mult}x_cus"] = round(reps * n_bufs * nbytes / (ms * 1e-3) / 1e9, 1)
    del bufs
    torch.cuda.empty_cache()
    best = max(res, key=res.get)
    return {"gbs": res[best], "workgroups": best, "by_workgroups": res,
            "bytes_per_read": nbytes, "buffers": n_bufs,
            "kernel": "stream_read_kernel (coli_stream_read)"}


def issue_sharing():
    """Do the matrix core and the vector ALU of one SIMD issue in parallel?
    coli_issue_probe's modes on one workgroup per CU: MFMA only, FMA only,
    one wave of each kind per SIMD, both in every wave; and the vector
    issue rate itself: the FMAs of one wave per SIMD instead of two, and
    three-VGPR-source FMAs (us per workgroup, median over the workgroups;
    ns per wave64 instruction per SIMD)."""
    import torch
    import int4_routed_expert_bias_amd as coli
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    ticks = torch.zeros((cus,), dtype=torch.int64, device="cuda")
    sink = torch.zeros((1,), dtype=torch.int32, device="cuda")
    us = {}
    for mode, name in enumerate(("mfma_only", "fma_only", "mfma_and_fma_waves", "mfma_and_fma_interleaved",
                                 "fma_one_wave_per_simd", "fma_three_vgpr_sources")):
        for _ in range(2):
            coli.issue_probe(mode, ticks, sink)
        torch.cuda.synchronize()
        us[name] = round(float(np.median(ticks.cpu().numpy())) / 100.0, 2)
    # per SIMD: mode 2 runs half of mode 0's MFMAs and half of mode 1's FMAs
    serial2 = (us["mfma_only"] + us["fma_only"]) / 2
    return {"us_per_workgroup": us,
            "mixed_waves_vs_serial_sum": round(us["mfma_and_fma_waves"] / serial2, 3),
            "interleaved_vs_serial_sum": round(us["mfma_and_fma_interleaved"] /
                                               (us["mfma_only"] + us["fma_only"]), 3),
            # 2048 iterations x 16 FMAs per wave; 2 waves per SIMD (1 in mode 4)
            "ns_per_valu_instr_per_simd": {
                "two_waves": round(us["fma_only"] * 1e3 / (2 * 2048 * 16), 3),
                "one_wave": round(us["fma_one_wave_per_simd"] * 1e3 / (2048 * 16), 3),
                "two_waves_three_vgpr_sources": round(us["fma_three_vgpr_sources"] * 1e3 / (2 * 2048 * 16), 3)},
            "kernel": "issue_probe_kernel (coli_issue_probe)"}


def percentiles(v):
    v = np.asarray(v, np.float64)
    return {"median": round(float(np.median(v)), 2), "p10": round(float(np.percentile(v, 10)), 2),
            "p90": round(float(np.percentile(v, 90)), 2), "n": int(v.size)}


def oracle_baseline(w, host0, mode, topp, cpu_seconds):
    """The oracle, single-threaded and pinned to one host CPU, on tokens of
    the workload one at a time (route, union and forward) for about
    cpu_seconds."""
    import oracle
    import synth
    import int4_routed_expert_bias_amd as coli
    orc = oracle.default()
    olay = oracle.Layer(host0, k=w.k, n_shared=w.n_shared)
    stacked = w.layers > 1
    xh = synth.workload_x(w, layer=0) if (stacked or w.x_kind == "overlap") else \
        synth.activations(w.H, w.T, wid=w.wid)
    omode = oracle.ACT_I8 if mode == coli.ACT_I8 else oracle.ACT_F32
    pinned = None
    old_aff = None
    if hasattr(os, "sched_setaffinity"):
        old_aff = os.sched_getaffinity(0)
        pinned = min(old_aff)
        os.sched_setaffinity(0, {pinned})
    try:
        done, t0 = 0, time.perf_counter()
        while True:
            xt = xh[done % w.T:done % w.T + 1]
            ids, wt, _, _ = orc.route(olay, xt) if topp is None else orc.route_topp(olay, xt, topp)
            orc.union(ids, w.E)
            orc.forward(olay, xt, ids, wt, omode)
            done += 1
            if time.perf_counter() - t0 >= cpu_seconds or done >= 1000:
                break
        t_cpu = time.perf_counter() - t0
    finally:
        if old_aff is not None:
            os.sched_setaffinity(0, old_aff)
    return {"value": round(done / t_cpu, 4), "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "pinned_cpu": pinned,
            "sample": f"{done} token(s) of the {w.name} workload, one at a time through route, "
                      f"union and forward on layer 0 ({t_cpu:.1f} s, single-threaded C oracle "
                      f"pinned to one CPU)"}


def expert_popularity(offsets, U, E):
    """Realised popularity of the routed experts: per layer call, the slot
    counts of the union entries sorted descending; their mean by rank over
    the calls, and the least-squares slope of log(count) on log(rank) over
    ranks 3..64 (the Zipf(1.1) bias aims at about -1.05 there)."""
    by_rank = np.zeros(E)
    for off, u in zip(offsets, U):
        o = off[:u + 1].cpu().numpy().astype(np.int64)
        c = np.sort(np.diff(o))[::-1]
        by_rank[:len(c)] += c
    by_rank /= len(offsets)
    r = np.arange(3, min(64, int(U.min())) + 1)
    c = by_rank[r - 1]
    ok = c > 0
    slope = float(np.polyfit(np.log(r[ok]), np.log(c[ok]), 1)[0]) if ok.sum() >= 2 else None
    return {"mean_slots_by_rank_top16": [round(float(v), 1) for v in by_rank[:16]],
            "mean_slots_rank_64_128_256": [round(float(by_rank[i - 1]), 2) for i in (64, 128, 256)],
            "loglog_slope_ranks_3_64": round(slope, 3) if slope is not None else None,
            "calls": len(offsets)}


TL_CAP = 8192      # waves recorded per kernel by the timeline entry point
TL_TICK_US = 0.01  # the real-time counter runs at 100 MHz


def timeline_summary(rec, names, per_kernel_us):
    """Markdown summary of per-wave timeline marks rec[step, kernel, wave,
    mark] (counter ticks, 0 = not reached): per kernel, the spread of wave
    entries and exits relative to the step's first wave entry, each wave's
    time to its marks, and the gap to the previous kernel; medians over the
    steps."""
    steps, nk = rec.shape[0], rec.shape[1]
    rows = {}
    for s in range(steps):
        base = None
        for i in range(nk):
            m0 = rec[s, i, :, 0]
            if (m0 > 0).any():
                b = m0[m0 > 0].min()
                base = b if base is None else min(base, b)
        prev_exit = None
        for i in range(nk):
            r = rec[s, i].astype(np.int64)
            live = r[:, 0] > 0
            if not live.any():
                continue
            e0 = (r[live, 0] - base) * TL_TICK_US
            ex = r[live, 7]
            ex = (ex[ex > 0] - base) * TL_TICK_US
            d = rows.setdefault(i, {})
            d.setdefault("waves", []).append(int(live.sum()))
            # most waves of the kernel resident at once (entry +1, exit -1)
            done = r[live, 7] > 0
            ev = np.concatenate([np.stack([r[live, 0][done], np.ones(done.sum(), np.int64)], 1),
                                 np.stack([r[live, 7][done], -np.ones(done.sum(), np.int64)], 1)])
            ev = ev[np.lexsort((ev[:, 1], ev[:, 0]))]
            d.setdefault("peak", []).append(int(np.cumsum(ev[:, 1]).max()) if len(ev) else 0)
            d.setdefault("entry_first", []).append(e0.min())
            d.setdefault("entry_med", []).append(np.median(e0))
            d.setdefault("entry_last", []).append(e0.max())
            if len(ex):
                d.setdefault("exit_first", []).append(ex.min())
                d.setdefault("exit_med", []).append(np.median(ex))
                d.setdefault("exit_last", []).append(ex.max())
            if prev_exit is not None:
                d.setdefault("gap", []).append(e0.min() - prev_exit)
            if len(ex):
                prev_exit = ex.max()
            for j in (1, 2, 3, 4, 5, 6):
                mj = r[live, j]
                ok = mj > 0
                if ok.any():
                    dt = (mj[ok] - r[live, 0][ok]) * TL_TICK_US
                    d.setdefault(f"m{j}_med", []).append(np.median(dt))
                    d.setdefault(f"m{j}_max", []).append(dt.max())
    med = lambda v: f"{np.median(v):.2f}" if v else "-"
    marks = [j for j in (1, 2, 3, 4, 5, 6) if any(f"m{j}_med" in d for d in rows.values())]
    out = ["| kernel | event us | waves | most resident at once | gap after previous | "
           "entries first / median / last | "
           "exits first / median / last | " + " | ".join(f"wave to mark {j} (median / max)" for j in marks) + " |",
           "|---|---|---|---|---|---|---|" + "---|" * len(marks)]
    for i in range(nk):
        d = rows.get(i)
        if not d:
            continue
        out.append(f"| `{names[i]}` | {per_kernel_us[i]:.2f} | {int(np.median(d['waves']))} | "
                   f"{int(np.median(d['peak']))} | "
                   f"{med(d.get('gap'))} | {med(d['entry_first'])} / {med(d['entry_med'])} / "
                   f"{med(d['entry_last'])} | {med(d.get('exit_first'))} / {med(d.get('exit_med'))} / "
                   f"{med(d.get('exit_last'))} | " +
                   " | ".join(f"{med(d.get(f'm{j}_med'))} / {med(d.get(f'm{j}_max'))}" for j in marks) + " |")
    return "\n".join(out)


def bench_resident(name, K, W, *, act_mode=None, topp=None, layers=None, use_graph=True,
                   cpu_seconds=12.0, with_cpu=True, prof_steps=None, timeline=None):
    """One resident-layer workload: K graph-replayed steps after W warmup
    steps, then the per-kernel and per-step times from dispatch-recorded
    events (warm, and cold after a 1 GiB write that flushes the caches), the
    roofline of the dominant kernel and the oracle baseline."""
    import torch
    import int4_routed_expert_bias_amd as coli
    from int4_routed_expert_bias_amd import profiling
    import synth

    w = synth.WORKLOADS[name]
    H, I, E, k, T = w.H, w.I, w.E, w.k, w.T
    fam = act_mode or w.act_mode
    mode = coli.ACT_I8 if fam == "i8" else coli.ACT_F32
    stacked = w.layers > 1
    NL = w.layers if stacked else (layers if layers is not None else
                                   (8 if name in ("decode", "verify") else 1))

    # ---- resident layers -------------------------------------------------
    t0 = time.time()
    devl = []
    host0 = None
    for l in range(NL):
        A = synth.workload_layer(w, layer=l)
        if l == 0:
            host0 = A
        devl.append(coli.DeviceLayer(A, k=k, n_shared=w.n_shared))
        if l > 0:
            del A
    log(f"[bench] {name}: {NL} layer(s) resident ({NL * (E + 1) * expert_bytes(H, I) / 1e9:.1f} GB "
        f"experts) in {time.time() - t0:.1f}s")

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
    bufs = coli.Buffers(devl[0], T, mode)
    if stacked:
        resid = torch.empty((T, H), dtype=torch.float32, device="cuda")
        xhat = torch.empty_like(resid)

    one_call = coli.route_forward_fused(devl[0], T, mode)  # coli_moe_route_forward

    def step(s):
        if stacked:
            # pre-norm of layer 0; between layers the residual add and the
            # next pre-norm in one pass (coli_add_rmsnorm)
            resid.copy_(xs[0])
            coli.rmsnorm(resid, xhat, T, H, 1e-6)
            for li, lay in enumerate(devl):
                coli.run_layer(lay, xhat, bufs, top_p=topp)
                if li + 1 < len(devl):
                    coli.add_rmsnorm(resid, bufs.y, xhat, T, H, 1e-6)
                else:
                    coli.add_inplace(resid, bufs.y, T * H)
        else:
            coli.run_layer(devl[s % NL], xs[s], bufs, top_p=topp,
                           fused="step" if one_call else True)

    for s in range(W):
        step(s)
    torch.cuda.synchronize()

    # ---- timed region: K steps in one HIP graph, replayed ------------------
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
        # distribution of the step time: more replays of the same graph, each
        # bracketed by events (per-step time = replay time / K)
        hip = Hip()
        reps = 12 if stacked else 50
        evs = [(hip.event(), hip.event()) for _ in range(reps)]
        for e0, e1 in evs:
            hip.record(e0)
            g.replay()
            hip.record(e1)
        torch.cuda.synchronize()
        step_warm = [hip.elapsed_ms(e0, e1) * 1e3 / K for e0, e1 in evs]
        for e in evs:
            hip.destroy(e[0])
            hip.destroy(e[1])
        del g
        # cold steps: one step per replay, after a read of 1 GiB of other
        # memory that evicts L2 and the Infinity Cache without dirtying them
        g1 = torch.cuda.CUDAGraph()
        cap_stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cap_stream):
            with torch.cuda.graph(g1, stream=cap_stream):
                step(W if not stacked else 0)
        torch.cuda.synchronize()
        sweep = torch.empty((1 << 30,), dtype=torch.uint8, device="cuda")
        sweep_out = torch.empty((4096,), dtype=torch.int32, device="cuda")
        cus = torch.cuda.get_device_properties(0).multi_processor_count
        g1.replay()
        reps = 16 if stacked else 64
        evs = [(hip.event(), hip.event()) for _ in range(reps)]
        for e0, e1 in evs:
            coli.stream_read(sweep, sweep_out, cus)
            hip.record(e0)
            g1.replay()
            hip.record(e1)
        torch.cuda.synchronize()
        step_cold = [hip.elapsed_ms(e0, e1) * 1e3 for e0, e1 in evs]
        for e in evs:
            hip.destroy(e[0])
            hip.destroy(e[1])
        del g1, sweep, sweep_out
    else:
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        for s in range(K):
            step(W + s if not stacked else s)
        torch.cuda.synchronize()
        t_end = time.perf_counter()
        step_warm = step_cold = None
    elapsed = t_end - t_start
    layer_passes = K * (w.layers if stacked else 1)
    value = layer_passes * T / elapsed
    ms_per_step = elapsed * 1e3 / K

    # ---- per-kernel times: dispatch-recorded events ------------------------
    hip = Hip()
    names = coli.route_forward_kernel_names(mode, T) if one_call else coli.forward_kernel_names(mode, T)
    nk = len(names)
    # the gate/up matmul: one launch, or the grouped GEMM's full-tile and
    # partial-tile launches together
    doms = [j for j, nm in enumerate(names) if "gateup" in nm]
    dom = doms[0]
    dom_label = names[dom] if len(doms) == 1 else names[dom].split(",")[0] + ">"
    if prof_steps is None:
        prof_steps = 8 if stacked else 64
    union_sizes = []
    union_offsets = []
    ev = [[hip.event() for _ in range(2 * nk)] for _ in range(prof_steps * (w.layers if stacked else 1))]
    torch.cuda._sleep(200_000_000)  # keep the GPU busy while the host enqueues
    i = 0
    for s in range(prof_steps):
        if stacked:
            resid.copy_(xs[0])
            lays = devl
        else:
            lays = [devl[(W + s) % NL]]
        if stacked:
            coli.rmsnorm(resid, xhat, T, H, 1e-6)
        for li, lay in enumerate(lays):
            x_in = xs[(W + s) % len(xs)] if not stacked else xhat
            if one_call:
                coli.route_forward_profiled(lay, x_in, T, bufs.ids, bufs.w, bufs.union_ids,
                                            bufs.offsets, bufs.slots, bufs.n_union, mode, bufs.y,
                                            bufs.workspace, ev[i], top_p=topp)
            else:
                coli.route_union(lay, x_in, T, bufs.ids, bufs.w, bufs.union_ids, bufs.offsets,
                                 bufs.slots, bufs.n_union, bufs.workspace, top_p=topp)
                coli.forward_profiled(lay, x_in, T, bufs.ids, bufs.w, bufs.union_ids,
                                      bufs.offsets, bufs.slots, bufs.n_union, mode, bufs.y,
                                      bufs.workspace, ev[i])
            union_sizes.append(bufs.n_union[:1].clone())
            if w.bias_kind == "zipf":
                union_offsets.append(bufs.offsets.clone())
            if stacked and li + 1 < len(lays):
                coli.add_rmsnorm(resid, bufs.y, xhat, T, H, 1e-6)
            elif stacked:
                coli.add_inplace(resid, bufs.y, T * H)
            i += 1
    torch.cuda.synchronize()
    per_kernel = np.zeros(nk)
    span_ms = 0.0  # several dominant launches: their wall span (they may overlap)
    for e in ev:
        for j in range(nk):
            per_kernel[j] += hip.elapsed_ms(e[2 * j], e[2 * j + 1])
        if len(doms) > 1:
            # times from the start of the call's first launch, earliest
            # start to latest end
            ref = e[0]
            span_ms += (max(hip.elapsed_ms(ref, e[2 * j + 1]) for j in doms)
                        - min(hip.elapsed_ms(ref, e[2 * j]) for j in doms))
        for x_ in e:
            hip.destroy(x_)
    per_kernel /= len(ev)
    span_ms /= len(ev)
    U = np.array([int(u.item()) for u in union_sizes])
    popularity = expert_popularity(union_offsets, U, E) if union_offsets else None
    dur_s = (span_ms if len(doms) > 1 else per_kernel[dom]) * 1e-3
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
    # HBM bytes per launch from the committed counter record (profiles/):
    # reported only while the kernel sources are those the counters were
    # taken on, and labelled as that stored record
    tpath = os.path.join(ROOT, "profiles", "traffic.json")
    if os.path.exists(tpath) and topp is None:
        with open(tpath) as fp:
            rec = json.load(fp).get(f"{w.name}:{dom_label}")
        if rec and rec.get("source_hash") == profiling.source_hash(
                tuple(rec.get("sources", profiling.ALL_SOURCES))):
            roof["traffic"] = rec["hbm_bytes_per_launch"]
            roof["traffic_source"] = ("profiles/traffic.json (rocprofv3 FETCH_SIZE/WRITE_SIZE, "
                                      "copy-calibrated; same kernel sources)")
    roof["kernel"] = dom_label + (f" ({len(doms)} launches: the tile lists; kernel_us is their wall "
                                  f"span, earliest start to latest end)" if len(doms) > 1 else "")
    roof["kernel_us"] = round(dur_s * 1e6, 2)
    roof["algorithmic_bytes_per_launch"] = int(algo_bytes)
    roof["algorithmic_ops_per_launch"] = int(algo_ops)
    if mode == coli.ACT_I8:
        roof["hbm_gbs_of_kernel"] = round(algo_bytes / dur_s / 1e9, 1)
        roof["int8_tops_of_kernel"] = round(algo_ops / dur_s / 1e12, 2)
    kernels_us = {names[j]: round(per_kernel[j] * 1e3, 2) for j in range(nk)}

    if timeline:
        # per-wave phase marks of the same kernels (coli_moe_route_forward_timeline)
        if not (one_call and mode == coli.ACT_F32 and not stacked):
            raise SystemExit("--timeline: the self-routing fp32 workloads (decode, verify) only")
        n_tl = 32
        rec = torch.zeros((n_tl, nk, TL_CAP, 8), dtype=torch.int64, device="cuda")
        torch.cuda._sleep(200_000_000)
        for s in range(n_tl):
            lay = devl[(W + s) % NL]
            coli.route_forward_timeline(lay, xs[(W + s) % len(xs)], T, bufs.ids, bufs.w,
                                        bufs.union_ids, bufs.offsets, bufs.slots, bufs.n_union,
                                        mode, bufs.y, bufs.workspace, rec[s], TL_CAP, top_p=topp)
        torch.cuda.synchronize()
        table = timeline_summary(rec.cpu().numpy(), names, [per_kernel[j] * 1e3 for j in range(nk)])
        with open(timeline, "w") as fp:
            fp.write(f"# Timeline of the {w.name} step ({n_tl} eager steps, one layer call each)\n\n"
                     "Times in us from the step's first wave entry; medians over the steps.  "
                     "'event us' is the kernel's dispatch-event duration from the same run.  "
                     "Marks (coli_moe_route_forward_timeline): self-routing gate/up 1 routing done, "
                     "2 activations staged, 3 first reduction batch written, 4 router keys loaded, "
                     "5 selection found, 6 selection and union written; fused down + combine "
                     "1 first entry's rows done, 2 / 3 before / after the workgroup barrier.\n\n")
            fp.write(table + "\n")
        log(table)
        del rec

    cpu = oracle_baseline(w, host0, mode, topp, cpu_seconds) if with_cpu else None
    res = {
        "value": round(value, 2), "unit": "tokens/s", "steps": K, "warmup": W,
        "ms_per_step": round(ms_per_step, 5), "dtype": "i8" if mode == coli.ACT_I8 else "f32",
        "config": {"workload": w.name, "description": w.note, "H": H, "I": I, "E": E, "k": k,
                   "T": T, "n_shared": w.n_shared, "layers": NL,
                   "act_mode": "i8" if mode == coli.ACT_I8 else "f32", "top_p": topp,
                   "graph": use_graph, "union_size_mean": round(float(U.mean()), 2),
                   "union_size_minmax": [int(U.min()), int(U.max())],
                   "kernels_us": kernels_us},
        **({"expert_popularity": popularity} if popularity else {}),
        # step time (us): warm = graph replays of the K timed steps (replay
        # time / K); cold = single-step graph replays, each after a 1 GiB read
        # of other memory (evicts L2 and Infinity Cache), graph launch included
        "step_us": ({"warm": percentiles(step_warm), "cold": percentiles(step_cold)}
                    if step_warm is not None else None),
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    del devl, bufs, xs
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default=None,
                    choices=["decode", "verify", "prefill512", "prefill4096x8", "tiny",
                             "mla", "mla_verify", "mla_dsa"],
                    help="run only this workload (default: decode as the headline, with verify, "
                         "prefill512 and prefill4096x8 reported beside it)")
    ap.add_argument("--layers", type=int, default=None, help="resident layer copies cycled (decode/verify)")
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of a HIP graph")
    ap.add_argument("--act-mode", choices=["f32", "i8"], default=None,
                    help="arithmetic family (default: the workload's own)")
    ap.add_argument("--topp", type=float, default=None,
                    help="adaptive expert top-p router (coli_moe_route_topp) instead of top-k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target oracle sample time")
    ap.add_argument("--prof-steps", type=int, default=None,
                    help="event-timed steps per phase (default 64; 8 for the 8-layer stack)")
    ap.add_argument("--timeline", default=None, metavar="PATH",
                    help="decode/verify: also write per-wave kernel phase marks "
                         "(coli_moe_route_forward_timeline), summarised as markdown, to PATH")
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
    import synth

    assert torch.cuda.is_available(), "needs a GPU"
    torch.cuda.set_device(0)
    if coli.device_check() != coli.COLI_OK:
        raise SystemExit("device is not gfx950: " + coli.strerror(coli.device_check()))

    if args.workload is not None and args.workload.startswith("mla"):
        return bench_mla(args)
    name = args.workload or "decode"
    w = synth.WORKLOADS[name]
    if args.place_slots is not None:
        fam = args.act_mode or w.act_mode
        return bench_placed(args, w, coli.ACT_I8 if fam == "i8" else coli.ACT_F32)
    K = args.steps if args.steps is not None else DEFAULT_STEPS[name][0]
    W = args.warmup if args.warmup is not None else DEFAULT_STEPS[name][1]
    with ClockSampler() as clk:
        head = bench_resident(name, K, W, act_mode=args.act_mode, topp=args.topp,
                              layers=args.layers, use_graph=not args.no_graph,
                              cpu_seconds=0.0, with_cpu=False, prof_steps=args.prof_steps,
                              timeline=args.timeline)
    if not args.no_cpu_baseline:  # after the GPU work, outside the clock sampling
        import synth as _s
        hw = _s.WORKLOADS[name]
        head["cpu_baseline"] = oracle_baseline(hw, _s.workload_layer(hw, layer=0),
                                               coli.ACT_I8 if head["dtype"] == "i8" else coli.ACT_F32,
                                               args.topp, args.cpu_seconds)
    out = {"metric": METRIC, "value": head["value"], "unit": "tokens/s", "n_gpus": 1,
           "steps": K, "warmup": W, "ms_per_step": head["ms_per_step"], "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": head["dtype"], "data": "synthetic"}
    for key in ("config", "step_us", "roofline", "cpu_baseline"):
        out[key] = head[key]
    if "expert_popularity" in head:
        out["expert_popularity"] = head["expert_popularity"]
    if args.workload is None:
        # the other workloads of the metric, each with its own default steps
        extra = {}
        for nm in EXTRA_WORKLOADS:
            kk, ww = DEFAULT_STEPS[nm]
            r = bench_resident(nm, kk, ww, cpu_seconds=args.cpu_seconds,
                               with_cpu=not args.no_cpu_baseline)
            extra[nm] = r
            log(f"[bench] {nm}: {r['value']:.0f} tokens/s, {r['roofline']['kernel']} "
                f"{r['roofline']['kernel_us']} us = {r['roofline']['frac']:.3f} of its roofline")
        out["workloads"] = extra
        out["hbm_read_ceiling"] = stream_read_rate(Hip())
        out["simd_issue_sharing"] = issue_sharing()
    # clocks sampled every 20 ms while the headline workload ran on the GPU
    out["clocks_mhz"] = clk.summary()
    out["host"] = host_info()
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
