"""Seeded synthetic inputs of the int4 routed-expert MoE layer.

One module feeds both the CPU oracle and the GPU library, so the two always
see identical bytes.  It contains no arithmetic of the layer: only the
counter-based generator in ``synth.c`` (SplitMix64 + Box-Muller), the
distributions of each tensor, and the workload definitions.

Tensor layouts (row-major, host numpy arrays):

===========  =======================  ======================================
name         shape / dtype            meaning
===========  =======================  ======================================
router_w     [E, H] float32           router weights, N(0, 0.02)
router_b     [E] float32              per-expert selection bias
w13          [E, 2I, H/2] uint8       packed int4, rows [0,I) gate, [I,2I) up;
                                      byte b of a row holds k=2b (low nibble)
                                      and k=2b+1 (high nibble), two's complement
s13          [E, 2I, H/64] uint16     fp16 bit patterns, exp(N(-4, 0.3)), one
                                      per row per 64-group along K
w2           [E, H, I/2] uint8        down projection, same encoding
s2           [E, H, I/64] uint16
sh_*         as above without E       the shared expert
===========  =======================  ======================================
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None


def build() -> str:
    """Compile libsynth.so with gcc (plain C99, no fast-math)."""
    import subprocess

    cmd = ["gcc", "-std=c99", "-O2", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-o", _LIB_PATH, os.path.join(_HERE, "synth.c"), "-lm", "-lpthread"]
    subprocess.run(cmd, check=True)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        u64, i32, f64 = ctypes.c_uint64, ctypes.c_int32, ctypes.c_double
        vp = ctypes.c_void_p
        L.synth_key.argtypes = [u64, u64]; L.synth_key.restype = u64
        L.synth_u64.argtypes = [u64, u64, u64]; L.synth_u64.restype = u64
        L.synth_normal.argtypes = [u64, u64, u64]; L.synth_normal.restype = f64
        L.synth_f16_from_double.argtypes = [f64]; L.synth_f16_from_double.restype = ctypes.c_uint16
        L.synth_fill_bytes.argtypes = [u64, u64, vp, u64, u64, ctypes.c_int]
        L.synth_fill_normal_f32.argtypes = [u64, u64, vp, u64, u64, f64, f64, ctypes.c_int]
        L.synth_fill_lognormal_f16.argtypes = [u64, u64, vp, u64, u64, f64, f64, ctypes.c_int]
        L.synth_fill_overlap_x.argtypes = [u64, u64, u64, vp, i32, i32]
        L.synth_permutation.argtypes = [u64, u64, i32, vp]
        L.synth_zipf_bias.argtypes = [u64, u64, i32, f64, f64, vp]
        for f in ("synth_fill_bytes", "synth_fill_normal_f32", "synth_fill_lognormal_f16",
                  "synth_fill_overlap_x", "synth_permutation", "synth_zipf_bias"):
            getattr(L, f).restype = None
        _lib = L
    return _lib


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


# tensor ids inside a (workload, layer) stream block
T_ROUTER_W, T_ROUTER_B, T_W13, T_S13, T_W2, T_S2 = 1, 2, 3, 4, 5, 6
T_SH_W13, T_SH_S13, T_SH_W2, T_SH_S2 = 7, 8, 9, 10
T_X, T_X_SHARED, T_PERM = 11, 12, 13


def stream_id(workload_id: int, layer: int, tensor: int) -> int:
    return (workload_id * 1000 + layer) * 100 + tensor


@dataclass(frozen=True)
class Workload:
    """A seeded synthetic workload of the MoE layer."""
    name: str
    wid: int            # stream namespace
    H: int
    I: int
    E: int
    k: int
    T: int
    layers: int = 1
    n_shared: int = 1
    x_kind: str = "normal"     # "normal" | "overlap"
    bias_kind: str = "normal"  # "normal" | "zipf"
    act_mode: str = "f32"      # arithmetic family the workload is defined on
    seed: int = 0
    note: str = field(default="", compare=False)


WORKLOADS = {
    w.name: w for w in [
        Workload("tiny", 0, 256, 128, 16, 2, 4, act_mode="both",
                 note="H256 I128 E16 top-2, 1 shared, T=4"),
        Workload("decode", 1, 6144, 2048, 256, 8, 1, act_mode="f32",
                 note="single-token decode on the H6144/I2048/E256 top-8 layer"),
        Workload("verify", 2, 6144, 2048, 256, 8, 4, x_kind="overlap", act_mode="f32",
                 note="4-token verify batch whose tokens share a common component"),
        Workload("prefill512", 3, 6144, 2048, 256, 8, 512, bias_kind="zipf", act_mode="i8",
                 note="512-token prefill, Zipf(1.1) expert popularity"),
        Workload("prefill4096x8", 4, 6144, 2048, 256, 8, 4096, layers=8, bias_kind="zipf",
                 act_mode="i8",
                 note="4096-token prefill through 8 stacked layers, popularity reshuffled per layer"),
    ]
}

ZIPF_S = 1.1
ZIPF_TAU = 0.1
SCALE_MU, SCALE_SIGMA = -4.0, 0.3
ROUTER_STD, BIAS_STD = 0.02, 0.1


def expert_bytes(H: int, I: int) -> int:
    """Bytes of one int4 gs64 SwiGLU expert with fp16 scales."""
    return 3 * I * H // 2 + 3 * I * (H // 64) * 2


def layer_arrays(H, I, E, k=None, *, wid: int, layer: int = 0, seed: int = 0,
                 n_shared: int = 1, bias_kind: str = "normal", experts=None) -> dict:
    """Generate one layer's parameters.

    ``experts`` optionally restricts the routed-expert tensors to a list of
    expert indices (the arrays then have len(experts) in their first axis);
    the bytes are the same as in the full tensors at those indices.
    """
    assert H % 64 == 0 and I % 64 == 0
    L = lib()
    th = _threads()
    sid = lambda t: stream_id(wid, layer, t)
    out = {"H": H, "I": I, "E": E}
    rw = np.empty((E, H), np.float32)
    L.synth_fill_normal_f32(seed, sid(T_ROUTER_W), _ptr(rw), rw.size, 0, 0.0, ROUTER_STD, th)
    rb = np.empty((E,), np.float32)
    if bias_kind == "zipf":
        L.synth_zipf_bias(seed, sid(T_PERM), E, ZIPF_S, ZIPF_TAU, _ptr(rb))
    else:
        L.synth_fill_normal_f32(seed, sid(T_ROUTER_B), _ptr(rb), E, 0, 0.0, BIAS_STD, th)
    out["router_w"], out["router_b"] = rw, rb

    ids = list(range(E)) if experts is None else list(experts)
    n = len(ids)
    w13_row, s13_row = 2 * I * (H // 2), 2 * I * (H // 64)
    w2_row, s2_row = H * (I // 2), H * (I // 64)
    w13 = np.empty((n, 2 * I, H // 2), np.uint8)
    s13 = np.empty((n, 2 * I, H // 64), np.uint16)
    w2 = np.empty((n, H, I // 2), np.uint8)
    s2 = np.empty((n, H, I // 64), np.uint16)
    if experts is None:
        ids = []  # whole tensors in one threaded call each (same bytes)
        L.synth_fill_bytes(seed, sid(T_W13), _ptr(w13), w13.size, 0, th)
        L.synth_fill_lognormal_f16(seed, sid(T_S13), _ptr(s13), s13.size, 0,
                                   SCALE_MU, SCALE_SIGMA, th)
        L.synth_fill_bytes(seed, sid(T_W2), _ptr(w2), w2.size, 0, th)
        L.synth_fill_lognormal_f16(seed, sid(T_S2), _ptr(s2), s2.size, 0,
                                   SCALE_MU, SCALE_SIGMA, th)
    for i, e in enumerate(ids):
        L.synth_fill_bytes(seed, sid(T_W13), w13[i].ctypes.data, w13_row, e * w13_row, th)
        L.synth_fill_lognormal_f16(seed, sid(T_S13), s13[i].ctypes.data, s13_row, e * s13_row,
                                   SCALE_MU, SCALE_SIGMA, th)
        L.synth_fill_bytes(seed, sid(T_W2), w2[i].ctypes.data, w2_row, e * w2_row, th)
        L.synth_fill_lognormal_f16(seed, sid(T_S2), s2[i].ctypes.data, s2_row, e * s2_row,
                                   SCALE_MU, SCALE_SIGMA, th)
    out.update(w13=w13, s13=s13, w2=w2, s2=s2)
    if n_shared:
        sh_w13 = np.empty((2 * I, H // 2), np.uint8)
        sh_s13 = np.empty((2 * I, H // 64), np.uint16)
        sh_w2 = np.empty((H, I // 2), np.uint8)
        sh_s2 = np.empty((H, I // 64), np.uint16)
        L.synth_fill_bytes(seed, sid(T_SH_W13), _ptr(sh_w13), sh_w13.size, 0, th)
        L.synth_fill_lognormal_f16(seed, sid(T_SH_S13), _ptr(sh_s13), sh_s13.size, 0,
                                   SCALE_MU, SCALE_SIGMA, th)
        L.synth_fill_bytes(seed, sid(T_SH_W2), _ptr(sh_w2), sh_w2.size, 0, th)
        L.synth_fill_lognormal_f16(seed, sid(T_SH_S2), _ptr(sh_s2), sh_s2.size, 0,
                                   SCALE_MU, SCALE_SIGMA, th)
        out.update(sh_w13=sh_w13, sh_s13=sh_s13, sh_w2=sh_w2, sh_s2=sh_s2)
    return out


def activations(H, T, *, wid: int, layer: int = 0, seed: int = 0, kind: str = "normal",
                token_offset: int = 0) -> np.ndarray:
    """x [T, H] float32.  ``normal``: iid N(0,1).  ``overlap``: tokens share a
    common N(0,1) component, x_t = (s + 0.5 z_t) / sqrt(1.25)."""
    L = lib()
    x = np.empty((T, H), np.float32)
    if T == 0:
        return x
    if kind == "overlap":
        assert token_offset == 0
        L.synth_fill_overlap_x(seed, stream_id(wid, layer, T_X_SHARED), stream_id(wid, layer, T_X),
                               _ptr(x), T, H)
    else:
        L.synth_fill_normal_f32(seed, stream_id(wid, layer, T_X), _ptr(x), x.size,
                                token_offset * H, 0.0, 1.0, _threads())
    return x


def workload_layer(w: Workload | str, layer: int = 0, experts=None) -> dict:
    if isinstance(w, str):
        w = WORKLOADS[w]
    return layer_arrays(w.H, w.I, w.E, w.k, wid=w.wid, layer=layer, seed=w.seed,
                        n_shared=w.n_shared, bias_kind=w.bias_kind, experts=experts)


def workload_x(w: Workload | str, layer: int = 0, T=None, token_offset: int = 0) -> np.ndarray:
    if isinstance(w, str):
        w = WORKLOADS[w]
    return activations(w.H, w.T if T is None else T, wid=w.wid, layer=layer, seed=w.seed,
                       kind=w.x_kind, token_offset=token_offset)


def permutation(seed: int, stream: int, n: int) -> np.ndarray:
    p = np.empty((n,), np.int32)
    lib().synth_permutation(seed, stream, n, _ptr(p))
    return p
