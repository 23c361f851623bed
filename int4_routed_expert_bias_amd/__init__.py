"""Python binding of libcoli_moe.so -- the int4 routed-expert MoE layer on
MI355X (gfx950).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  PyTorch provides device memory and streams.  The functions carry
the C ABI names (include/coli_moe.h) without the ``coli_moe_`` prefix and
raise ``ColiError`` on a nonzero status.  If the library is not built, the
import of ``lib()`` fails loudly: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcoli_moe.so")

ACT_F32, ACT_I8 = 0, 1
COLI_OK, COLI_E_ARG, COLI_E_SHAPE, COLI_E_ALIGN, COLI_E_WORKSPACE, COLI_E_DEVICE, \
    COLI_E_UNSUPPORTED, COLI_E_SCRATCH = range(8)
NOALLOC_SCRATCH_BYTES = 32 << 20  # COLI_NOALLOC_SCRATCH_BYTES

# every symbol declared in include/coli_moe.h
EXPORTS = ("coli_moe_abi_version", "coli_moe_workspace_bytes", "coli_moe_route",
           "coli_moe_route_topp", "coli_moe_route_union", "coli_moe_union", "coli_moe_forward", "coli_moe_forward_profiled",
           "coli_moe_route_forward", "coli_moe_route_forward_profiled",
           "coli_moe_route_forward_noalloc", "coli_moe_route_forward_timeline",
           "coli_moe_route_forward_kernel_count", "coli_moe_route_forward_kernel_name",
           "coli_moe_forward_kernel_count", "coli_moe_forward_kernel_name",
           "coli_moe_acc_dump_bytes", "coli_moe_i8_workspace_offsets", "coli_moe_strerror",
           "coli_moe_device_check",
           "coli_rmsnorm", "coli_add_inplace", "coli_add_rmsnorm", "coli_stream_read", "coli_issue_probe")
# every symbol declared in include/coli_mla.h
MLA_EXPORTS = ("coli_mla_workspace_bytes", "coli_mla_decode", "coli_mla_decode_profiled")
# every symbol declared in include/coli_place.h
PLACE_EXPORTS = ("coli_moe_placer_create", "coli_moe_placer_destroy", "coli_moe_placer_reset",
                 "coli_moe_placer_slot_of", "coli_moe_place_plan", "coli_moe_place_ws_bytes",
                 "coli_moe_forward_placed", "coli_moe_place_prefetch")


class ColiError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


class ColiLayer(ctypes.Structure):
    _fields_ = [("H", ctypes.c_int32), ("I", ctypes.c_int32), ("E", ctypes.c_int32),
                ("k", ctypes.c_int32), ("n_shared", ctypes.c_int32)] + [
        (n, ctypes.c_void_p) for n in ("router_w", "router_bias", "w13", "s13", "w2", "s2",
                                       "sh_w13", "sh_s13", "sh_w2", "sh_s2")]


_lib = None


def lib():
    """Load libcoli_moe.so (built in-tree by __graft_entry__.build())."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
        # Load torch's HIP runtime first so that the library binds to the same
        # runtime instance (one libamdhip64.so.7 per process).
        import torch  # noqa: F401
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        sig = {
            "coli_moe_abi_version": ([], ctypes.c_int),
            "coli_moe_workspace_bytes": ([i32, i32, i32, i32, i32, i32], sz),
            "coli_moe_route": ([vp, vp, i32, vp, vp, vp, sz, vp], ctypes.c_int),
            "coli_moe_route_topp": ([vp, vp, i32, ctypes.c_float, vp, vp, vp, sz, vp], ctypes.c_int),
            "coli_moe_union": ([vp, i32, i32, i32, vp, vp, vp, vp, vp], ctypes.c_int),
            "coli_moe_route_union": ([vp, vp, i32, ctypes.c_float, vp, vp, vp, vp, vp, vp, vp, sz,
                                      vp], ctypes.c_int),
            "coli_moe_forward": ([vp, vp, i32, vp, vp, vp, vp, vp, vp, i32, vp, vp, sz, vp, vp],
                                 ctypes.c_int),
            "coli_moe_forward_profiled": ([vp, vp, i32, vp, vp, vp, vp, vp, vp, i32, vp, vp, sz, vp,
                                           vp, i32, vp], ctypes.c_int),
            "coli_moe_route_forward": ([vp, vp, i32, ctypes.c_float, vp, vp, vp, vp, vp, vp, i32,
                                        vp, vp, sz, vp], ctypes.c_int),
            "coli_moe_route_forward_profiled": ([vp, vp, i32, ctypes.c_float, vp, vp, vp, vp, vp,
                                                 vp, i32, vp, vp, sz, vp, i32, vp], ctypes.c_int),
            "coli_moe_route_forward_timeline": ([vp, vp, i32, ctypes.c_float, vp, vp, vp, vp, vp,
                                                 vp, i32, vp, vp, sz, vp, i32, vp], ctypes.c_int),
            "coli_moe_route_forward_noalloc": ([vp, vp, i32, ctypes.c_float, vp, vp, vp, vp, vp,
                                                vp, i32, vp, vp], ctypes.c_int),
            "coli_moe_route_forward_kernel_count": ([i32, i32], ctypes.c_int),
            "coli_moe_route_forward_kernel_name": ([i32, i32, i32], ctypes.c_char_p),
            "coli_moe_forward_kernel_count": ([i32, i32], ctypes.c_int),
            "coli_moe_forward_kernel_name": ([i32, i32, i32], ctypes.c_char_p),
            "coli_moe_acc_dump_bytes": ([i32, i32, i32, i32, i32], sz),
            "coli_moe_i8_workspace_offsets": ([i32, i32, i32, i32, i32, i32, vp], ctypes.c_int),
            "coli_moe_strerror": ([ctypes.c_int], ctypes.c_char_p),
            "coli_moe_device_check": ([], ctypes.c_int),
            "coli_rmsnorm": ([vp, vp, i32, i32, ctypes.c_float, vp], ctypes.c_int),
            "coli_add_inplace": ([vp, vp, i64, vp], ctypes.c_int),
            "coli_add_rmsnorm": ([vp, vp, vp, i32, i32, ctypes.c_float, vp], ctypes.c_int),
            "coli_stream_read": ([vp, sz, vp, i32, vp], ctypes.c_int),
            "coli_issue_probe": ([i32, i32, vp, vp, vp], ctypes.c_int),
            "coli_moe_placer_create": ([i32, i32, i32, i32, i32, i32, i32, vp], ctypes.c_int),
            "coli_moe_placer_destroy": ([vp], None),
            "coli_moe_placer_reset": ([vp], ctypes.c_int),
            "coli_moe_placer_slot_of": ([vp, i32], i32),
            "coli_moe_place_plan": ([vp, vp, i32, vp, vp, vp, vp, vp], ctypes.c_int),
            "coli_moe_place_ws_bytes": ([i32, i32, i32], sz),
            "coli_moe_forward_placed": ([vp, vp, vp, vp, i32, vp, vp, vp, vp, vp, vp, i32, vp, vp,
                                         sz, vp, sz, vp, vp, vp], ctypes.c_int),
            "coli_moe_place_prefetch": ([vp, vp, vp, i32, vp, vp], ctypes.c_int),
            "coli_mla_workspace_bytes": ([i32, i32, i32, i32], sz),
            "coli_mla_decode": ([vp, i32, i32, vp, i32, vp, vp, i32, ctypes.c_float, vp, vp, sz,
                                 vp], ctypes.c_int),
            "coli_mla_decode_profiled": ([vp, i32, i32, vp, i32, vp, vp, i32, ctypes.c_float, vp,
                                          vp, sz, vp, i32, vp], ctypes.c_int),
        }
        for name, (args, res) in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


def strerror(status: int) -> str:
    return lib().coli_moe_strerror(status).decode()


def _check(status: int, what: str):
    if status != COLI_OK:
        raise ColiError(status, f"{what}: {strerror(status)}")


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def workspace_bytes(H, I, E, k, T, act_mode) -> int:
    return lib().coli_moe_workspace_bytes(H, I, E, k, T, act_mode)


def acc_dump_bytes(H, I, k, T, n_shared) -> int:
    return lib().coli_moe_acc_dump_bytes(H, I, k, T, n_shared)


def i8_workspace_offsets(H, I, E, k, T, n_shared=1):
    """Byte offsets of o, qh and sh inside an int8-family forward workspace
    (T > 4; see coli_moe_i8_workspace_offsets)."""
    out = (ctypes.c_size_t * 3)()
    _check(lib().coli_moe_i8_workspace_offsets(H, I, E, k, T, n_shared, out),
           "coli_moe_i8_workspace_offsets")
    return {"o": out[0], "qh": out[1], "sh": out[2]}


def device_check() -> int:
    return lib().coli_moe_device_check()


def route(layer, x, T, ids, w, workspace, workspace_nbytes=None, stream=None):
    nb = workspace.numel() * workspace.element_size() if workspace_nbytes is None else workspace_nbytes
    _check(lib().coli_moe_route(layer.ref, _ptr(x), T, _ptr(ids), _ptr(w), _ptr(workspace), nb,
                                _stream(stream)), "coli_moe_route")


def route_topp(layer, x, T, top_p, ids, w, workspace, workspace_nbytes=None, stream=None):
    nb = workspace.numel() * workspace.element_size() if workspace_nbytes is None else workspace_nbytes
    _check(lib().coli_moe_route_topp(layer.ref, _ptr(x), T, float(top_p), _ptr(ids), _ptr(w),
                                     _ptr(workspace), nb, _stream(stream)), "coli_moe_route_topp")


def route_union(layer, x, T, ids, w, union_ids, offsets, slots, n_union, workspace, top_p=None,
                workspace_nbytes=None, stream=None):
    """coli_moe_route_union: route (top-k, or top-p when top_p is given) and
    union in one call (one launch for T <= 4)."""
    nb = workspace.numel() * workspace.element_size() if workspace_nbytes is None else workspace_nbytes
    p = 1.0 if top_p is None else float(top_p)
    _check(lib().coli_moe_route_union(layer.ref, _ptr(x), T, p, _ptr(ids), _ptr(w),
                                      _ptr(union_ids), _ptr(offsets), _ptr(slots), _ptr(n_union),
                                      _ptr(workspace), nb, _stream(stream)), "coli_moe_route_union")


def union(ids, T, k, E, union_ids, offsets, slots, n_union, stream=None):
    _check(lib().coli_moe_union(_ptr(ids), T, k, E, _ptr(union_ids), _ptr(offsets), _ptr(slots),
                                _ptr(n_union), _stream(stream)), "coli_moe_union")


def forward(layer, x, T, ids, w, union_ids, offsets, slots, n_union, act_mode, y, workspace,
            workspace_nbytes=None, acc_dump=None, stream=None):
    nb = workspace.numel() * workspace.element_size() if workspace_nbytes is None else workspace_nbytes
    _check(lib().coli_moe_forward(layer.ref, _ptr(x), T, _ptr(ids), _ptr(w), _ptr(union_ids),
                                  _ptr(offsets), _ptr(slots), _ptr(n_union), act_mode, _ptr(y),
                                  _ptr(workspace), nb, _ptr(acc_dump), _stream(stream)),
           "coli_moe_forward")


def forward_profiled(layer, x, T, ids, w, union_ids, offsets, slots, n_union, act_mode, y,
                     workspace, events, stream=None):
    """coli_moe_forward that records ``events`` (raw hipEvent_t handles)."""
    nb = workspace.numel() * workspace.element_size()
    arr = (ctypes.c_void_p * len(events))(*events)
    _check(lib().coli_moe_forward_profiled(layer.ref, _ptr(x), T, _ptr(ids), _ptr(w),
                                           _ptr(union_ids), _ptr(offsets), _ptr(slots),
                                           _ptr(n_union), act_mode, _ptr(y), _ptr(workspace), nb,
                                           None, arr, len(events), _stream(stream)),
           "coli_moe_forward_profiled")


def route_forward(layer, x, T, ids, w, union_ids, offsets, slots, n_union, act_mode, y, workspace,
                  top_p=None, workspace_nbytes=None, stream=None):
    """coli_moe_route_forward: route, union and forward in one call (for up to
    4 tokens with E <= 256 the gate/up kernel routes the tokens itself)."""
    nb = workspace.numel() * workspace.element_size() if workspace_nbytes is None else workspace_nbytes
    p = 1.0 if top_p is None else float(top_p)
    _check(lib().coli_moe_route_forward(layer.ref, _ptr(x), T, p, _ptr(ids), _ptr(w),
                                        _ptr(union_ids), _ptr(offsets), _ptr(slots), _ptr(n_union),
                                        act_mode, _ptr(y), _ptr(workspace), nb, _stream(stream)),
           "coli_moe_route_forward")


def route_forward_noalloc(layer, x, T, ids, w, union_ids, offsets, slots, n_union, act_mode, y,
                          top_p=None, stream=None):
    """coli_moe_route_forward_noalloc: coli_moe_route_forward with the
    library's static scratch array instead of a workspace (no allocation)."""
    p = 1.0 if top_p is None else float(top_p)
    _check(lib().coli_moe_route_forward_noalloc(layer.ref, _ptr(x), T, p, _ptr(ids), _ptr(w),
                                                _ptr(union_ids), _ptr(offsets), _ptr(slots),
                                                _ptr(n_union), act_mode, _ptr(y),
                                                _stream(stream)),
           "coli_moe_route_forward_noalloc")


def route_forward_profiled(layer, x, T, ids, w, union_ids, offsets, slots, n_union, act_mode, y,
                           workspace, events, top_p=None, stream=None):
    """coli_moe_route_forward (self-routing case) recording ``events``."""
    nb = workspace.numel() * workspace.element_size()
    p = 1.0 if top_p is None else float(top_p)
    arr = (ctypes.c_void_p * len(events))(*events)
    _check(lib().coli_moe_route_forward_profiled(layer.ref, _ptr(x), T, p, _ptr(ids), _ptr(w),
                                                 _ptr(union_ids), _ptr(offsets), _ptr(slots),
                                                 _ptr(n_union), act_mode, _ptr(y), _ptr(workspace),
                                                 nb, arr, len(events), _stream(stream)),
           "coli_moe_route_forward_profiled")


def route_forward_timeline(layer, x, T, ids, w, union_ids, offsets, slots, n_union, act_mode, y,
                           workspace, timeline, waves_cap, top_p=None, stream=None):
    """coli_moe_route_forward (self-routing fp32 case) writing per-wave
    timeline marks into ``timeline`` (uint64/int64 device tensor of
    kernels x waves_cap x 8, zeroed by the caller)."""
    nb = workspace.numel() * workspace.element_size()
    p = 1.0 if top_p is None else float(top_p)
    if timeline.numel() < len(route_forward_kernel_names(act_mode, T)) * waves_cap * 8:
        raise ValueError("timeline holds fewer than kernels x waves_cap x 8 marks")
    _check(lib().coli_moe_route_forward_timeline(layer.ref, _ptr(x), T, p, _ptr(ids), _ptr(w),
                                                 _ptr(union_ids), _ptr(offsets), _ptr(slots),
                                                 _ptr(n_union), act_mode, _ptr(y), _ptr(workspace),
                                                 nb, _ptr(timeline), waves_cap, _stream(stream)),
           "coli_moe_route_forward_timeline")


def route_forward_kernel_names(act_mode, T=1):
    n = lib().coli_moe_route_forward_kernel_count(act_mode, T)
    return [lib().coli_moe_route_forward_kernel_name(act_mode, T, i).decode() for i in range(n)]


def route_forward_fused(layer, T, act_mode):
    """Whether coli_moe_route_forward routes inside the gate/up kernel."""
    return 1 <= T <= 4 and layer.E <= 256 and (act_mode == ACT_F32 or T == 1)


def forward_kernel_names(act_mode, T=2):
    n = lib().coli_moe_forward_kernel_count(act_mode, T)
    return [lib().coli_moe_forward_kernel_name(act_mode, T, i).decode() for i in range(n)]


def rmsnorm(x, xhat, T, H, eps=1e-6, stream=None):
    _check(lib().coli_rmsnorm(_ptr(x), _ptr(xhat), T, H, eps, _stream(stream)), "coli_rmsnorm")


def add_inplace(x, y, n, stream=None):
    _check(lib().coli_add_inplace(_ptr(x), _ptr(y), n, _stream(stream)), "coli_add_inplace")


def add_rmsnorm(x, y, xhat, T, H, eps=1e-6, stream=None):
    """x += y, then xhat = rmsnorm(x), in one pass (coli_add_rmsnorm)."""
    _check(lib().coli_add_rmsnorm(_ptr(x), _ptr(y), _ptr(xhat), T, H, eps, _stream(stream)),
           "coli_add_rmsnorm")


def stream_read(buf, out, n_groups, nbytes=None, stream=None):
    """coli_stream_read (measurement only): read ``buf`` with the streaming
    kernels' load pattern; one checksum per workgroup into ``out``."""
    nb = buf.numel() * buf.element_size() if nbytes is None else nbytes
    _check(lib().coli_stream_read(_ptr(buf), nb, _ptr(out), n_groups, _stream(stream)),
           "coli_stream_read")


def issue_probe(mode, ticks, sink, n_groups=None, stream=None):
    """coli_issue_probe (measurement only): MFMA-only, FMA-only and mixed
    workloads on the SIMDs; each workgroup's ticks into ``ticks``."""
    n = ticks.numel() if n_groups is None else n_groups
    _check(lib().coli_issue_probe(mode, n, _ptr(ticks), _ptr(sink), _stream(stream)),
           "coli_issue_probe")


class DeviceLayer:
    """One layer's tensors in device memory plus the C descriptor.

    ``arrays`` uses the synthetic-layer layout (router_w, router_b, w13, s13,
    w2, s2 and optionally sh_*), as numpy arrays or torch tensors."""

    def __init__(self, arrays: dict, k: int, n_shared: int = 1, device="cuda"):
        import numpy as np
        import torch

        def dev(a):
            if isinstance(a, np.ndarray):
                if a.dtype == np.uint16:
                    a = a.view(np.int16)
                a = torch.from_numpy(np.ascontiguousarray(a))
            return a.to(device, non_blocking=False).contiguous()

        self.H, self.I, self.E, self.k, self.n_shared = (int(arrays["H"]), int(arrays["I"]),
                                                        int(arrays["E"]), k, n_shared)
        self.t = {}
        for n in ("router_w", "router_b", "w13", "s13", "w2", "s2"):
            self.t[n] = dev(arrays[n])
        if n_shared:
            for n in ("sh_w13", "sh_s13", "sh_w2", "sh_s2"):
                self.t[n] = dev(arrays[n])
        s = ColiLayer(self.H, self.I, self.E, k, n_shared)
        s.router_w = _ptr(self.t["router_w"])
        s.router_bias = _ptr(self.t["router_b"])
        for n in ("w13", "s13", "w2", "s2"):
            setattr(s, n, _ptr(self.t[n]))
        if n_shared:
            for n in ("sh_w13", "sh_s13", "sh_w2", "sh_s2"):
                setattr(s, n, _ptr(self.t[n]))
        self.struct = s

    @property
    def ref(self):
        return ctypes.byref(self.struct)


class Buffers:
    """Device buffers of one (layer shape, T, act_mode) call sequence."""

    def __init__(self, layer: DeviceLayer, T: int, act_mode: int, device="cuda", dump=False):
        import torch
        H, I, E, k = layer.H, layer.I, layer.E, layer.k
        self.T, self.act_mode = T, act_mode
        cap = max(1, min(E, T * k))
        i32, f32 = torch.int32, torch.float32
        self.ids = torch.empty((max(T, 1), k), dtype=i32, device=device)
        self.w = torch.empty((max(T, 1), k), dtype=f32, device=device)
        self.union_ids = torch.empty((cap,), dtype=i32, device=device)
        self.offsets = torch.empty((cap + 1,), dtype=i32, device=device)
        self.slots = torch.empty((max(1, T * k),), dtype=i32, device=device)
        self.n_union = torch.zeros((4,), dtype=i32, device=device)
        self.y = torch.empty((max(T, 1), H), dtype=f32, device=device)
        nb = workspace_bytes(H, I, E, k, T, act_mode)
        self.workspace = torch.empty((max(nb, 256),), dtype=torch.uint8, device=device)
        self.dump = None
        if dump:
            db = acc_dump_bytes(H, I, k, T, layer.n_shared)
            self.dump = torch.empty((max(db, 256),), dtype=torch.uint8, device=device)


def run_layer(layer: DeviceLayer, x, bufs: Buffers, stream=None, top_p=None, fused=True):
    """route -> union -> forward for x [T][H] (device fp32); top_p selects
    the adaptive top-p router; fused routes and unions in one call
    (coli_moe_route_union), else in two; fused="step" runs the whole step in
    one call (coli_moe_route_forward; not with an acc_dump buffer)."""
    T = bufs.T
    if fused == "step":
        if bufs.dump is not None:
            raise ValueError("coli_moe_route_forward takes no acc_dump buffer")
        route_forward(layer, x, T, bufs.ids, bufs.w, bufs.union_ids, bufs.offsets, bufs.slots,
                      bufs.n_union, bufs.act_mode, bufs.y, bufs.workspace, top_p=top_p,
                      stream=stream)
        return bufs.y
    if fused:
        route_union(layer, x, T, bufs.ids, bufs.w, bufs.union_ids, bufs.offsets, bufs.slots,
                    bufs.n_union, bufs.workspace, top_p=top_p, stream=stream)
    else:
        if top_p is None:
            route(layer, x, T, bufs.ids, bufs.w, bufs.workspace, stream=stream)
        else:
            route_topp(layer, x, T, top_p, bufs.ids, bufs.w, bufs.workspace, stream=stream)
        union(bufs.ids, T, layer.k, layer.E, bufs.union_ids, bufs.offsets, bufs.slots,
              bufs.n_union, stream=stream)
    forward(layer, x, T, bufs.ids, bufs.w, bufs.union_ids, bufs.offsets, bufs.slots,
            bufs.n_union, bufs.act_mode, bufs.y, bufs.workspace, acc_dump=bufs.dump,
            stream=stream)
    return bufs.y


def dump_regions(H, I, k, T, n_shared):
    """Byte offset, dtype and shape of each region of the acc_dump buffer
    (include/coli_moe.h): acc13 [R][2I][H/64], acc2 [R][H][I/64], qh [R][I],
    sh [R][I/64], qx [T][H], sx [T][H/64], each 256-byte aligned."""
    import numpy as np
    R = T * k + n_shared * T
    regs = [("acc13", np.int32, (R, 2 * I, H // 64)), ("acc2", np.int32, (R, H, I // 64)),
            ("qh", np.int8, (R, I)), ("sh", np.float32, (R, I // 64)),
            ("qx", np.int8, (T, H)), ("sx", np.float32, (T, H // 64))]
    out, off = {}, 0
    for name, dt, shape in regs:
        out[name] = (off, dt, shape)
        n = int(np.prod(shape)) * np.dtype(dt).itemsize
        off = (off + n + 255) & ~255
    return out


def dump_views(dump_host, H, I, k, T, n_shared):
    """Split a host copy (numpy uint8) of the acc_dump buffer into its
    documented regions (see dump_regions)."""
    import numpy as np
    out = {}
    for name, (off, dt, shape) in dump_regions(H, I, k, T, n_shared).items():
        n = int(np.prod(shape)) * np.dtype(dt).itemsize
        out[name] = dump_host[off:off + n].view(dt).reshape(shape)
    return out


# ---- placement across pinned host memory and device slots (coli_place.h) ----

class ColiTiers(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("host_w13", "host_s13", "host_w2", "host_s2",
                                               "slot_w13", "slot_s13", "slot_w2", "slot_s2",
                                               "slot_table")]


class PlaceStats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("n_union", "hits", "loads", "passes")]


def place_ws_bytes(E, k, T) -> int:
    return lib().coli_moe_place_ws_bytes(E, k, T)


class Placer:
    """Residency state of one layer's experts (coli_moe_placer)."""

    def __init__(self, H, I, E, k, n_slots, T_max, chunk=1):
        h = ctypes.c_void_p()
        _check(lib().coli_moe_placer_create(H, I, E, k, n_slots, T_max, chunk, ctypes.byref(h)),
               "coli_moe_placer_create")
        self.handle = h.value
        self.E, self.n_slots, self.chunk = E, n_slots, chunk

    def close(self):
        if getattr(self, "handle", None):
            lib().coli_moe_placer_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def reset(self):
        _check(lib().coli_moe_placer_reset(self.handle), "coli_moe_placer_reset")

    def slot_of(self, e) -> int:
        return lib().coli_moe_placer_slot_of(self.handle, e)

    def plan(self, union_ids):
        """coli_moe_place_plan on a host list; returns the plan as lists."""
        U = len(union_ids)
        A = ctypes.c_int32 * max(U, 1)
        uid, es, ep, le, lw = A(*union_ids), A(), A(), A(), A()
        counts = (ctypes.c_int32 * 3)()
        _check(lib().coli_moe_place_plan(self.handle, uid, U, es, ep, le, lw, counts),
               "coli_moe_place_plan")
        hits, nl, npass = counts
        return dict(slot=list(es[:U]), pass_=list(ep[:U]),
                    loads=[(le[i], lw[i]) for i in range(nl)], hits=hits, passes=npass)


class PlacedLayer:
    """A layer whose routed experts live in pinned host memory, with a pool
    of n_slots device slots in front of them.  Router and shared expert are
    in device memory.  ``host`` may pass the pinned host tier of another
    PlacedLayer (dict of tensors) to share it."""

    def __init__(self, arrays: dict, k: int, n_slots: int, T_max: int, chunk: int = 1,
                 n_shared: int = 1, device="cuda", host=None):
        import numpy as np
        import torch

        def t(a):
            if isinstance(a, np.ndarray):
                if a.dtype == np.uint16:
                    a = a.view(np.int16)
                a = torch.from_numpy(np.ascontiguousarray(a))
            return a

        self.H, self.I, self.E, self.k, self.n_shared = (int(arrays["H"]), int(arrays["I"]),
                                                        int(arrays["E"]), k, n_shared)
        self.n_slots = n_slots
        self.t = {}
        for n in ("router_w", "router_b"):
            self.t[n] = t(arrays[n]).to(device).contiguous()
        if n_shared:
            for n in ("sh_w13", "sh_s13", "sh_w2", "sh_s2"):
                self.t[n] = t(arrays[n]).to(device).contiguous()
        if host is None:
            host = {n: t(arrays[n]).contiguous().pin_memory() for n in ("w13", "s13", "w2", "s2")}
        self.host = host
        self.slots = {n: torch.empty((n_slots,) + tuple(host[n].shape[1:]), dtype=host[n].dtype,
                                     device=device) for n in ("w13", "s13", "w2", "s2")}
        self.slot_table = torch.empty((max(self.E, 4),), dtype=torch.int32, device=device)
        s = ColiLayer(self.H, self.I, self.E, k, n_shared)
        s.router_w = _ptr(self.t["router_w"])
        s.router_bias = _ptr(self.t["router_b"])
        if n_shared:
            for n in ("sh_w13", "sh_s13", "sh_w2", "sh_s2"):
                setattr(s, n, _ptr(self.t[n]))
        self.struct = s
        tr = ColiTiers()
        for n in ("w13", "s13", "w2", "s2"):
            setattr(tr, "host_" + n, _ptr(host[n]))
            setattr(tr, "slot_" + n, _ptr(self.slots[n]))
        tr.slot_table = _ptr(self.slot_table)
        self.tiers = tr
        self.placer = Placer(self.H, self.I, self.E, k, n_slots, T_max, chunk)

    @property
    def ref(self):
        return ctypes.byref(self.struct)


def forward_placed(layer: PlacedLayer, x, T, ids, w, union_ids, offsets, slots, n_union,
                   act_mode, y, workspace, place_ws, stream=None, copy_stream=None):
    """coli_moe_forward_placed; returns the call's PlaceStats as a dict."""
    nb = workspace.numel() * workspace.element_size()
    pb = place_ws.numel() * place_ws.element_size()
    st = PlaceStats()
    cs = _stream(stream) if copy_stream is None else _stream(copy_stream)
    _check(lib().coli_moe_forward_placed(layer.ref, ctypes.byref(layer.tiers),
                                         layer.placer.handle, _ptr(x), T, _ptr(ids), _ptr(w),
                                         _ptr(union_ids), _ptr(offsets), _ptr(slots),
                                         _ptr(n_union), act_mode, _ptr(y), _ptr(workspace), nb,
                                         _ptr(place_ws), pb, ctypes.byref(st), _stream(stream),
                                         cs), "coli_moe_forward_placed")
    return dict(n_union=st.n_union, hits=st.hits, loads=st.loads, passes=st.passes)


def place_prefetch(layer: PlacedLayer, experts, stream=None, copy_stream=None):
    n = len(experts)
    arr = (ctypes.c_int32 * max(n, 1))(*experts)
    cs = _stream(stream) if copy_stream is None else _stream(copy_stream)
    _check(lib().coli_moe_place_prefetch(layer.placer.handle, ctypes.byref(layer.tiers), arr, n,
                                         _stream(stream), cs), "coli_moe_place_prefetch")


def run_layer_placed(layer: PlacedLayer, x, bufs: "Buffers", place_ws, stream=None,
                     copy_stream=None, top_p=None):
    """route -> union -> forward_placed; returns the call's placement stats."""
    T = bufs.T
    route_union(layer, x, T, bufs.ids, bufs.w, bufs.union_ids, bufs.offsets, bufs.slots,
                bufs.n_union, bufs.workspace, top_p=top_p, stream=stream)
    return forward_placed(layer, x, T, bufs.ids, bufs.w, bufs.union_ids, bufs.offsets,
                          bufs.slots, bufs.n_union, bufs.act_mode, bufs.y, bufs.workspace,
                          place_ws, stream=stream, copy_stream=copy_stream)


# ---- decode attention over the compressed MLA KV cache (coli_mla.h) ---------

MLA_DIM, MLA_LATENT = 576, 512


def mla_workspace_bytes(B, n_heads, T, n_sel=0) -> int:
    return lib().coli_mla_workspace_bytes(B, n_heads, T, n_sel)


def mla_decode(q, kv, out, workspace, scale, lens=None, idx=None, stream=None):
    """coli_mla_decode: q [B][n_heads][576], kv [T][576], out [B][n_heads][512]
    (device fp32); lens [B] or idx [B][n_sel] (device int32)."""
    B, nh = q.shape[0], q.shape[1]
    n_sel = 0 if idx is None else idx.shape[1]
    nb = workspace.numel() * workspace.element_size()
    _check(lib().coli_mla_decode(_ptr(q), B, nh, _ptr(kv), kv.shape[0], _ptr(lens), _ptr(idx),
                                 n_sel, float(scale), _ptr(out), _ptr(workspace), nb,
                                 _stream(stream)), "coli_mla_decode")


def mla_decode_profiled(q, kv, out, workspace, scale, events, lens=None, idx=None, stream=None):
    B, nh = q.shape[0], q.shape[1]
    n_sel = 0 if idx is None else idx.shape[1]
    nb = workspace.numel() * workspace.element_size()
    arr = (ctypes.c_void_p * len(events))(*events)
    _check(lib().coli_mla_decode_profiled(_ptr(q), B, nh, _ptr(kv), kv.shape[0], _ptr(lens),
                                          _ptr(idx), n_sel, float(scale), _ptr(out),
                                          _ptr(workspace), nb, arr, len(events),
                                          _stream(stream)), "coli_mla_decode_profiled")
