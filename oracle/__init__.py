"""ctypes access to the plain-C CPU oracle (liborc.so).

TEST INFRASTRUCTURE ONLY: used by tests/, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py``.  The product path never imports this
package; it shares no code with the GPU library.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liborc.so")
_lib = None

ACT_F32, ACT_I8 = 0, 1

CFLAGS = ["-std=c99", "-O2", "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra"]


def build(extra_flags=(), out=None) -> str:
    """Compile the oracle with gcc (never with fast-math)."""
    out = out or _LIB_PATH
    cmd = (["gcc"] + CFLAGS + list(extra_flags) +
           ["-fPIC", "-shared", "-o", out, os.path.join(_HERE, "coli_oracle.c"), "-lm"])
    subprocess.run(cmd, check=True)
    return out


class OrcLayer(ctypes.Structure):
    _fields_ = [("H", ctypes.c_int32), ("I", ctypes.c_int32), ("E", ctypes.c_int32),
                ("k", ctypes.c_int32), ("n_shared", ctypes.c_int32)] + [
        (n, ctypes.c_void_p) for n in ("router_w", "router_b", "w13", "s13", "w2", "s2",
                                       "sh_w13", "sh_s13", "sh_w2", "sh_s2")]


def _setup(L):
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    sig = {
        "orc_f16_to_f32": ([ctypes.c_uint16], ctypes.c_float),
        "orc_int4": ([vp, i64], ctypes.c_int),
        "orc_logits": ([vp, vp, i32, vp], None),
        "orc_select": ([i32, i32, i32, vp, vp, vp, vp, vp], None),
        "orc_route": ([vp, vp, i32, vp, vp, vp, vp], None),
        "orc_union": ([i32, i32, i32, vp, vp, vp, vp, vp], None),
        "orc_prune_topp": ([i32, i32, i32, ctypes.c_float, vp, vp, vp], None),
        "orc_quant_i8": ([i64, vp, vp, vp], None),
        "orc_expert_f32": ([i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp], None),
        "orc_expert_i8": ([i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp], None),
        "orc_down_acc_i8": ([i32, i32, vp, vp, vp], None),
        "orc_down_i8": ([i32, i32, vp, vp, vp, vp, vp], None),
        "orc_token_forward": ([vp, vp, vp, vp, i32, vp], None),
        "orc_forward": ([vp, vp, i32, vp, vp, i32, vp], None),
        "orc_forward_rows": ([vp, vp, vp, vp, i32, i32, vp, vp], None),
        "orc_rmsnorm": ([i32, i32, vp, vp], None),
        "orc_mla_decode": ([i32, i32, vp, i32, vp, vp, vp, i32, ctypes.c_float, vp], None),
        "orc_swiglu": ([ctypes.c_float, ctypes.c_float], ctypes.c_float),
    }
    for name, (args, res) in sig.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = res
    return L


def load(path=None):
    return _setup(ctypes.CDLL(path or _LIB_PATH))


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        _lib = load()
    return _lib


def _p(a):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data


class Layer:
    """Holds numpy arrays of one layer (synth layout) and the orc_layer view."""

    def __init__(self, arrays: dict, k: int, n_shared: int = 1):
        self.a = arrays
        self.H, self.I, self.E, self.k = arrays["H"], arrays["I"], arrays["E"], k
        self.n_shared = n_shared
        s = OrcLayer(self.H, self.I, self.E, k, n_shared)
        for n in ("router_w", "router_b", "w13", "s13", "w2", "s2"):
            setattr(s, n, _p(arrays[n]))
        if n_shared:
            for n in ("sh_w13", "sh_s13", "sh_w2", "sh_s2"):
                setattr(s, n, _p(arrays[n]))
        self.struct = s

    @property
    def ref(self):
        return ctypes.byref(self.struct)


class Oracle:
    """The oracle's functions bound to one loaded library (the real build or
    a planted-mistake build made by the tests)."""

    def __init__(self, L):
        self.L = L

    def f16_to_f32(self, h: int) -> float:
        return self.L.orc_f16_to_f32(h)

    def swiglu(self, g: float, u: float) -> float:
        return self.L.orc_swiglu(g, u)

    def int4_at(self, row: np.ndarray, kk: int) -> int:
        return self.L.orc_int4(_p(row), kk)

    def logits(self, layer: Layer, x: np.ndarray) -> np.ndarray:
        x = np.ascontiguousarray(x, np.float32)
        out = np.empty((x.shape[0], layer.E), np.float32)
        self.L.orc_logits(layer.ref, _p(x), x.shape[0], _p(out))
        return out

    def select(self, logits_: np.ndarray, bias: np.ndarray, k: int):
        lg = np.ascontiguousarray(logits_, np.float32)
        b = np.ascontiguousarray(bias, np.float32)
        T, E = lg.shape
        ids = np.empty((T, k), np.int32)
        w = np.empty((T, k), np.float32)
        s = np.empty((T, E), np.float32)
        self.L.orc_select(E, k, T, _p(lg), _p(b), _p(ids), _p(w), _p(s))
        return ids, w, s

    def route(self, layer: Layer, x: np.ndarray):
        x = np.ascontiguousarray(x, np.float32)
        T = x.shape[0]
        ids = np.empty((T, layer.k), np.int32)
        w = np.empty((T, layer.k), np.float32)
        lg = np.empty((T, layer.E), np.float32)
        s = np.empty((T, layer.E), np.float32)
        self.L.orc_route(layer.ref, _p(x), T, _p(ids), _p(w), _p(lg), _p(s))
        return ids, w, lg, s

    def prune_topp(self, ids: np.ndarray, w: np.ndarray, scores: np.ndarray, p: float):
        """Top-p pruning of a top-k selection (copies; see orc_prune_topp)."""
        ids = np.array(ids, np.int32, copy=True)
        w = np.array(w, np.float32, copy=True)
        s = np.ascontiguousarray(scores, np.float32)
        T, k = ids.shape
        self.L.orc_prune_topp(s.shape[1], k, T, float(p), _p(s), _p(ids), _p(w))
        return ids, w

    def route_topp(self, layer: Layer, x: np.ndarray, p: float):
        ids, w, lg, s = self.route(layer, x)
        ids, w = self.prune_topp(ids, w, s, p)
        return ids, w, lg, s

    def union(self, ids: np.ndarray, E: int):
        ids = np.ascontiguousarray(ids, np.int32)
        T, k = ids.shape
        cap = min(E, T * k)
        u = np.empty((cap,), np.int32)
        off = np.empty((cap + 1,), np.int32)
        slots = np.empty((T * k,), np.int32)
        nu = np.zeros((1,), np.int32)
        self.L.orc_union(T, k, E, _p(ids), _p(u), _p(off), _p(slots), _p(nu))
        return u, off, slots, int(nu[0])

    def quant_i8(self, x: np.ndarray):
        x = np.ascontiguousarray(x, np.float32).reshape(-1)
        q = np.empty(x.shape, np.int8)
        s = np.empty((x.size // 64,), np.float32)
        self.L.orc_quant_i8(x.size, _p(x), _p(q), _p(s))
        return q, s

    def expert_f32(self, w13, s13, w2, s2, x):
        H = x.shape[-1]
        I = w2.shape[1] * 2
        g = np.empty((I,), np.float32); u = np.empty((I,), np.float32)
        h = np.empty((I,), np.float32); o = np.empty((H,), np.float64)
        self.L.orc_expert_f32(H, I, _p(w13), _p(s13), _p(w2), _p(s2),
                             _p(np.ascontiguousarray(x, np.float32)), _p(g), _p(u), _p(h), _p(o))
        return dict(g=g, u=u, h=h, o=o)

    def expert_i8(self, w13, s13, w2, s2, x):
        H = x.shape[-1]
        I = w2.shape[1] * 2
        acc13 = np.empty((2 * I, H // 64), np.int32)
        g = np.empty((I,), np.float32); u = np.empty((I,), np.float32)
        h = np.empty((I,), np.float32); qh = np.empty((I,), np.int8)
        sh = np.empty((I // 64,), np.float32); acc2 = np.empty((H, I // 64), np.int32)
        o = np.empty((H,), np.float64)
        self.L.orc_expert_i8(H, I, _p(w13), _p(s13), _p(w2), _p(s2),
                            _p(np.ascontiguousarray(x, np.float32)), _p(acc13), _p(g), _p(u),
                            _p(h), _p(qh), _p(sh), _p(acc2), _p(o))
        return dict(acc13=acc13, g=g, u=u, h=h, qh=qh, sh=sh, acc2=acc2, o=o)

    def down_i8(self, w2, s2, qh, sh):
        """Down projection (double) from given int8 codes of h (natural order)
        and their scales."""
        H, I = w2.shape[0], w2.shape[1] * 2
        o = np.empty(H, np.float64)
        self.L.orc_down_i8(H, I, _p(w2), _p(s2), _p(np.ascontiguousarray(qh, np.int8)),
                           _p(np.ascontiguousarray(sh, np.float32)), _p(o))
        return o

    def down_acc_i8(self, w2, qh):
        H, I = w2.shape[0], w2.shape[1] * 2
        acc2 = np.empty((H, I // 64), np.int32)
        self.L.orc_down_acc_i8(H, I, _p(w2), _p(np.ascontiguousarray(qh, np.int8)), _p(acc2))
        return acc2

    def forward(self, layer: Layer, x, ids, w, act_mode=ACT_F32):
        x = np.ascontiguousarray(x, np.float32)
        y = np.empty_like(x)
        self.L.orc_forward(layer.ref, _p(x), x.shape[0], _p(np.ascontiguousarray(ids, np.int32)),
                          _p(np.ascontiguousarray(w, np.float32)), act_mode, _p(y))
        return y

    def forward_rows(self, layer: Layer, x, ids, w, sel, act_mode=ACT_F32):
        x = np.ascontiguousarray(x, np.float32)
        sel = np.ascontiguousarray(sel, np.int32)
        y = np.empty((sel.size, layer.H), np.float32)
        self.L.orc_forward_rows(layer.ref, _p(x), _p(np.ascontiguousarray(ids, np.int32)),
                               _p(np.ascontiguousarray(w, np.float32)), act_mode, sel.size,
                               _p(sel), _p(y))
        return y

    def rmsnorm(self, x):
        x = np.ascontiguousarray(x, np.float32)
        out = np.empty_like(x)
        self.L.orc_rmsnorm(x.shape[0], x.shape[1], _p(x), _p(out))
        return out

    def mla_decode(self, q: np.ndarray, kv: np.ndarray, scale: float, lens=None, idx=None):
        """q [B][n_heads][576], kv [T][576]; lens [B] or idx [B][n_sel]
        -> out [B][n_heads][512] (orc_mla_decode)."""
        q = np.ascontiguousarray(q, np.float32)
        kv = np.ascontiguousarray(kv, np.float32)
        B, nh, _ = q.shape
        out = np.empty((B, nh, 512), np.float32)
        ln = None if lens is None else np.ascontiguousarray(lens, np.int32)
        ix = None if idx is None else np.ascontiguousarray(idx, np.int32)
        n_sel = 0 if ix is None else ix.shape[1]
        self.L.orc_mla_decode(B, nh, _p(q), kv.shape[0], _p(kv), _p(ln), _p(ix), n_sel,
                              float(scale), _p(out))
        return out


_default = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle(lib())
    return _default
