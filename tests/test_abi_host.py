"""Host-side tests of the C ABI (no GPU needed): the library loads, exports
every symbol the public header declares, and rejects bad arguments with the
documented status codes before any HIP call.

Every call here carries at least one invalid argument, so no call reaches
the device (fake pointers are never dereferenced)."""
import ctypes
import glob
import os
import re

import pytest

import int4_routed_expert_bias_amd as coli
from conftest import ROOT, gpu_available

HEADERS = {os.path.join(ROOT, "include", "coli_moe.h"): "EXPORTS",
           os.path.join(ROOT, "include", "coli_place.h"): "PLACE_EXPORTS",
           os.path.join(ROOT, "include", "coli_mla.h"): "MLA_EXPORTS"}


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(coli.LIB_PATH):
        from int4_routed_expert_bias_amd import build as b
        b.build()
    return coli.lib()


def header_functions(path):
    src = open(path).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(coli_\w+)\s*\(", src)))


def test_exports_every_declared_symbol(L):
    for path, attr in HEADERS.items():
        names = header_functions(path)
        assert set(names) == set(getattr(coli, attr)), (path, names)
        for n in names:
            assert hasattr(L, n), n
    assert set(glob.glob(os.path.join(ROOT, "include", "*.h"))) == set(HEADERS)
    assert L.coli_moe_abi_version() == 1


def test_strerror(L):
    for s in range(8):
        assert coli.strerror(s).startswith("COLI_")
    assert "unknown" in coli.strerror(99)


def test_workspace_bytes(L):
    assert coli.workspace_bytes(6144, 2048, 256, 8, 1, 0) > 0
    assert coli.workspace_bytes(6144, 2048, 256, 8, 4096, 1) > 0
    assert coli.workspace_bytes(6000, 2048, 256, 8, 1, 0) == 0      # H % 64
    assert coli.workspace_bytes(6144, 2048, 256, 9, 1, 2) == 0      # mode
    assert coli.workspace_bytes(6144, 2048, 4, 8, 1, 0) == 0        # k > E
    assert coli.workspace_bytes(6144, 2048, 256, 17, 1, 0) == 0     # k > 16
    assert coli.acc_dump_bytes(256, 128, 2, 4, 1) > 0
    assert coli.acc_dump_bytes(256, 128, 2, 4, 2) == 0


def test_issue_probe_argument_errors(L):
    """The measurement probe rejects modes outside 0..5, group counts
    outside 1..65536 and null or misaligned pointers before any device
    work."""
    fake = ctypes.c_void_p(FAKE)
    for mode, n in ((-1, 1), (6, 1), (0, 0), (5, 65537)):
        assert L.coli_issue_probe(mode, n, fake, fake, None) == coli.COLI_E_ARG, (mode, n)
    assert L.coli_issue_probe(0, 1, None, fake, None) == coli.COLI_E_ARG
    assert L.coli_issue_probe(0, 1, ctypes.c_void_p(FAKE + 4), fake, None) == coli.COLI_E_ALIGN


def test_i8_workspace_offsets(L):
    """The int8 family's intermediate regions lie inside the workspace, in
    order, without overlap; batches of up to 4 tokens have none."""
    H, I, E, k, T = 6144, 2048, 256, 8, 4096
    off = coli.i8_workspace_offsets(H, I, E, k, T)
    R = T * k + T
    assert off["o"] + R * H * 4 <= off["qh"]
    assert off["qh"] + R * I <= off["sh"]
    assert off["sh"] + R * (I // 64) * 4 <= coli.workspace_bytes(H, I, E, k, T, coli.ACT_I8)
    for bad in ((H, I, E, k, 4, 1), (H, I, E, k, T, 2), (6000, I, E, k, T, 1)):
        with pytest.raises(coli.ColiError):
            coli.i8_workspace_offsets(*bad)


FAKE = 0x100000  # aligned, never dereferenced
MIS = 0x100004   # 4-byte aligned only


def layer(**kw):
    d = dict(H=256, I=128, E=16, k=2, n_shared=1, router_w=FAKE, router_bias=FAKE, w13=FAKE,
             s13=FAKE, w2=FAKE, s2=FAKE, sh_w13=FAKE, sh_s13=FAKE, sh_w2=FAKE, sh_s2=FAKE)
    d.update(kw)
    s = coli.ColiLayer(d["H"], d["I"], d["E"], d["k"], d["n_shared"])
    for n in ("router_w", "router_bias", "w13", "s13", "w2", "s2", "sh_w13", "sh_s13",
              "sh_w2", "sh_s2"):
        setattr(s, n, d[n])
    return s


def route(L, lay, T=4, x=FAKE, ids=FAKE, w=FAKE, ws=FAKE, nb=1 << 20):
    return L.coli_moe_route(ctypes.byref(lay) if lay is not None else None, x, T, ids, w, ws, nb,
                            None)


def forward(L, lay, T=4, mode=0, y=FAKE, ws=FAKE, nb=1 << 30, dump=None, **p):
    a = dict(x=FAKE, ids=FAKE, w=FAKE, u=FAKE, off=FAKE, sl=FAKE, nu=FAKE)
    a.update(p)
    return L.coli_moe_forward(ctypes.byref(lay) if lay is not None else None, a["x"], T, a["ids"],
                              a["w"], a["u"], a["off"], a["sl"], a["nu"], mode, y, ws, nb, dump,
                              None)


def test_route_argument_errors(L):
    assert route(L, None) == coli.COLI_E_ARG
    assert route(L, layer(H=100)) == coli.COLI_E_SHAPE
    assert route(L, layer(I=0)) == coli.COLI_E_SHAPE
    assert route(L, layer(E=0)) == coli.COLI_E_SHAPE
    assert route(L, layer(E=2000)) == coli.COLI_E_SHAPE
    assert route(L, layer(k=17, E=32)) == coli.COLI_E_SHAPE
    assert route(L, layer(k=3, E=2)) == coli.COLI_E_SHAPE
    assert route(L, layer(n_shared=2)) == coli.COLI_E_SHAPE
    assert route(L, layer(), T=-1) == coli.COLI_E_SHAPE
    assert route(L, layer(), T=70000) == coli.COLI_E_SHAPE
    assert route(L, layer(router_w=0)) == coli.COLI_E_ARG
    assert route(L, layer(), x=0) == coli.COLI_E_ARG
    assert route(L, layer(), ws=0) == coli.COLI_E_ARG
    assert route(L, layer(), x=MIS) == coli.COLI_E_ALIGN
    assert route(L, layer(router_bias=MIS)) == coli.COLI_E_ALIGN
    assert route(L, layer(), nb=16) == coli.COLI_E_WORKSPACE
    assert route(L, layer(), T=0) == coli.COLI_OK  # no-op, nothing enqueued


def test_route_topp_argument_errors(L):
    def rt(lay, p, T=4, x=FAKE, nb=1 << 20):
        return L.coli_moe_route_topp(ctypes.byref(lay) if lay is not None else None, x, T,
                                     ctypes.c_float(p), FAKE, FAKE, FAKE, nb, None)
    assert rt(None, 0.7) == coli.COLI_E_ARG
    assert rt(layer(H=100), 0.7) == coli.COLI_E_SHAPE
    assert rt(layer(), 0.0) == coli.COLI_E_ARG
    assert rt(layer(), -0.5) == coli.COLI_E_ARG
    assert rt(layer(), float("nan")) == coli.COLI_E_ARG
    assert rt(layer(), 0.7, x=MIS) == coli.COLI_E_ALIGN
    assert rt(layer(), 0.7, nb=16) == coli.COLI_E_WORKSPACE
    assert rt(layer(), 0.7, T=0) == coli.COLI_OK


def test_union_argument_errors(L):
    U = L.coli_moe_union
    assert U(FAKE, 4, 2, 0, FAKE, FAKE, FAKE, FAKE, None) == coli.COLI_E_SHAPE
    assert U(FAKE, 4, 0, 16, FAKE, FAKE, FAKE, FAKE, None) == coli.COLI_E_SHAPE
    assert U(FAKE, 4, 17, 1024, FAKE, FAKE, FAKE, FAKE, None) == coli.COLI_E_SHAPE
    assert U(FAKE, -2, 2, 16, FAKE, FAKE, FAKE, FAKE, None) == coli.COLI_E_SHAPE
    assert U(None, 4, 2, 16, FAKE, FAKE, FAKE, FAKE, None) == coli.COLI_E_ARG
    assert U(FAKE, 4, 2, 16, FAKE, FAKE, None, FAKE, None) == coli.COLI_E_ARG
    assert U(FAKE, 4, 2, 16, FAKE, FAKE, FAKE, None, None) == coli.COLI_E_ARG
    assert U(FAKE, 4, 2, 16, MIS, FAKE, FAKE, FAKE, None) == coli.COLI_E_ALIGN


def test_forward_argument_errors(L):
    assert forward(L, None) == coli.COLI_E_ARG
    assert forward(L, layer(w13=0)) == coli.COLI_E_ARG
    assert forward(L, layer(n_shared=0)) == coli.COLI_E_ARG         # shared pointers given
    assert forward(L, layer(sh_w2=0)) == coli.COLI_E_ARG            # shared incomplete
    assert forward(L, layer(s2=MIS)) == coli.COLI_E_ALIGN
    assert forward(L, layer(), mode=3) == coli.COLI_E_UNSUPPORTED
    assert forward(L, layer(), mode=0, dump=FAKE) == coli.COLI_E_ARG
    assert forward(L, layer(), y=0) == coli.COLI_E_ARG
    assert forward(L, layer(), nu=0) == coli.COLI_E_ARG
    assert forward(L, layer(), sl=MIS) == coli.COLI_E_ALIGN
    assert forward(L, layer(), nb=1024) == coli.COLI_E_WORKSPACE
    assert forward(L, layer(), mode=1, nb=1024) == coli.COLI_E_WORKSPACE
    assert forward(L, layer(), T=0) == coli.COLI_OK


def test_glue_argument_errors(L):
    assert L.coli_rmsnorm(FAKE, FAKE, 4, 100, ctypes.c_float(1e-6), None) == coli.COLI_E_SHAPE
    assert L.coli_rmsnorm(FAKE, FAKE, 4, 128, ctypes.c_float(-1.0), None) == coli.COLI_E_ARG
    assert L.coli_rmsnorm(MIS, FAKE, 4, 128, ctypes.c_float(1e-6), None) == coli.COLI_E_ALIGN
    assert L.coli_add_inplace(FAKE, None, 8, None) == coli.COLI_E_ARG
    assert L.coli_add_inplace(FAKE, FAKE, -1, None) == coli.COLI_E_ARG
    assert L.coli_add_rmsnorm(FAKE, FAKE, FAKE, 4, 100, ctypes.c_float(1e-6), None) == coli.COLI_E_SHAPE
    assert L.coli_add_rmsnorm(FAKE, FAKE, FAKE, 4, 128, ctypes.c_float(-1.0), None) == coli.COLI_E_ARG
    assert L.coli_add_rmsnorm(FAKE, None, FAKE, 4, 128, ctypes.c_float(1e-6), None) == coli.COLI_E_ARG
    assert L.coli_add_rmsnorm(FAKE, MIS, FAKE, 4, 128, ctypes.c_float(1e-6), None) == coli.COLI_E_ALIGN
    assert L.coli_add_rmsnorm(FAKE, FAKE, FAKE, 0, 128, ctypes.c_float(1e-6), None) == coli.COLI_OK


@pytest.mark.skipif(gpu_available(), reason="checks the no-device path of a GPU-less host")
def test_no_device_reports_device_error(L):
    assert L.coli_moe_device_check() in (coli.COLI_E_DEVICE, coli.COLI_E_UNSUPPORTED)


def test_forward_profiled_needs_two_events_per_kernel(L):
    lay = layer()
    for mode, T in ((0, 1), (0, 4), (0, 9), (1, 2), (1, 9)):
        n = coli.lib().coli_moe_forward_kernel_count(mode, T)
        short = (ctypes.c_void_p * (2 * n - 1))(*([FAKE] * (2 * n - 1)))
        st = L.coli_moe_forward_profiled(ctypes.byref(lay), FAKE, T, FAKE, FAKE, FAKE, FAKE, FAKE,
                                         FAKE, mode, FAKE, FAKE, 1 << 30, None, short, 2 * n - 1,
                                         None)
        assert st == coli.COLI_E_ARG, (mode, T)
        holes = (ctypes.c_void_p * (2 * n))(*([FAKE] * (2 * n - 1) + [None]))
        st = L.coli_moe_forward_profiled(ctypes.byref(lay), FAKE, T, FAKE, FAKE, FAKE, FAKE, FAKE,
                                         FAKE, mode, FAKE, FAKE, 1 << 30, None, holes, 2 * n,
                                         None)
        assert st == coli.COLI_E_ARG, (mode, T)



def test_mla_argument_errors(L):
    def call(q=FAKE, B=1, nh=64, kv=FAKE, T=100, lens=FAKE, idx=None, n_sel=0, scale=0.07,
             out=FAKE, ws=FAKE, nb=1 << 30):
        return L.coli_mla_decode(q, B, nh, kv, T, lens, idx, n_sel, ctypes.c_float(scale), out,
                                 ws, nb, None)
    assert call(B=0) == coli.COLI_E_SHAPE
    assert call(B=257) == coli.COLI_E_SHAPE
    assert call(nh=0) == coli.COLI_E_SHAPE
    assert call(nh=129) == coli.COLI_E_SHAPE
    assert call(T=0) == coli.COLI_E_SHAPE
    assert call(idx=FAKE, n_sel=0) == coli.COLI_E_SHAPE
    assert call(scale=float("inf")) == coli.COLI_E_ARG
    assert call(scale=float("nan")) == coli.COLI_E_ARG
    assert call(q=None) == coli.COLI_E_ARG
    assert call(lens=None) == coli.COLI_E_ARG          # neither lens nor a key list
    assert call(ws=None) == coli.COLI_E_ARG
    assert call(kv=MIS) == coli.COLI_E_ALIGN
    assert call(lens=MIS) == coli.COLI_E_ALIGN
    assert call(nb=16) == coli.COLI_E_WORKSPACE
    ev = (ctypes.c_void_p * 3)(FAKE, FAKE, FAKE)
    assert L.coli_mla_decode_profiled(FAKE, 1, 64, FAKE, 100, FAKE, None, 0, ctypes.c_float(0.1),
                                      FAKE, FAKE, 1 << 30, ev, 3, None) == coli.COLI_E_ARG
    assert coli.mla_workspace_bytes(1, 64, 32768) >= 64 * 516 * 4
    assert coli.mla_workspace_bytes(4, 128, 100, 2048) > 0
    assert coli.mla_workspace_bytes(0, 64, 100) == 0
    assert coli.mla_workspace_bytes(1, 64, 0) == 0


def test_route_forward_argument_errors(L):
    def rf(lay, T=1, p=1.0, mode=0, x=FAKE, u=FAKE, sl=FAKE, y=FAKE, nb=1 << 30):
        return L.coli_moe_route_forward(ctypes.byref(lay) if lay is not None else None, x, T,
                                        ctypes.c_float(p), FAKE, FAKE, u, FAKE, sl, FAKE, mode, y,
                                        FAKE, nb, None)
    assert rf(None) == coli.COLI_E_ARG
    assert rf(layer(H=100)) == coli.COLI_E_SHAPE
    assert rf(layer(), T=-1) == coli.COLI_E_SHAPE
    assert rf(layer(), mode=5) == coli.COLI_E_UNSUPPORTED
    assert rf(layer(), p=0.0) == coli.COLI_E_ARG
    assert rf(layer(), u=None) == coli.COLI_E_ARG
    assert rf(layer(), sl=None) == coli.COLI_E_ARG
    assert rf(layer(), y=None) == coli.COLI_E_ARG
    assert rf(layer(), x=MIS) == coli.COLI_E_ALIGN
    assert rf(layer(), nb=16) == coli.COLI_E_WORKSPACE
    assert rf(layer(), T=3, nb=16) == coli.COLI_E_WORKSPACE
    noexp = layer()
    noexp.w13 = None
    assert rf(noexp) == coli.COLI_E_ARG

    def rfp(T=1, mode=0, n=6, holes=False):
        ev = (ctypes.c_void_p * max(n, 1))(*([FAKE] * max(n, 1)))
        if holes:
            ev[n - 1] = None
        return L.coli_moe_route_forward_profiled(ctypes.byref(layer()), FAKE, T, ctypes.c_float(1.0),
                                                 FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, mode, FAKE,
                                                 FAKE, 1 << 30, ev, n, None)
    assert rfp(T=5) == coli.COLI_E_UNSUPPORTED      # only the self-routing cases
    assert rfp(T=2, mode=1, n=12) == coli.COLI_E_UNSUPPORTED
    assert rfp(n=5) == coli.COLI_E_ARG
    assert rfp(holes=True) == coli.COLI_E_ARG
    assert rfp(T=4, n=7) == coli.COLI_E_ARG          # four kernels: 8 events
    assert rfp(mode=1, n=9) == coli.COLI_E_ARG       # five int8 kernels: 10 events
    assert rfp(mode=1, n=10, holes=True) == coli.COLI_E_ARG
    lib_ = coli.lib()
    cnt = lib_.coli_moe_route_forward_kernel_count
    assert [cnt(0, 1), cnt(0, 2), cnt(0, 4), cnt(0, 5), cnt(1, 1), cnt(1, 2), cnt(2, 1)] == \
        [3, 4, 4, 0, 5, 0, 0]
    name = lib_.coli_moe_route_forward_kernel_name
    assert [name(0, 1, i) for i in (-1, 3)] == [None, None]
    assert name(0, 1, 1) == b"gateup_t1_kernel" and name(0, 4, 1) == b"gateup_mt_kernel"
    assert name(0, 4, 3) == b"combine_kernel" and name(1, 1, 2) == b"gateup_i8v_kernel"


def test_route_union_argument_errors(L):
    def ru(lay, T=4, p=1.0, x=FAKE, u=FAKE, off=FAKE, sl=FAKE, nu=FAKE, nb=1 << 20):
        return L.coli_moe_route_union(ctypes.byref(lay) if lay is not None else None, x, T,
                                      ctypes.c_float(p), FAKE, FAKE, u, off, sl, nu, FAKE, nb, None)
    assert ru(None) == coli.COLI_E_ARG
    assert ru(layer(H=100)) == coli.COLI_E_SHAPE
    assert ru(layer(), T=-1) == coli.COLI_E_SHAPE
    assert ru(layer(), p=0.0) == coli.COLI_E_ARG
    assert ru(layer(), p=float("nan")) == coli.COLI_E_ARG
    assert ru(layer(), nu=None) == coli.COLI_E_ARG
    assert ru(layer(), u=None) == coli.COLI_E_ARG
    assert ru(layer(), sl=None) == coli.COLI_E_ARG
    assert ru(layer(), x=None) == coli.COLI_E_ARG
    assert ru(layer(), off=MIS) == coli.COLI_E_ALIGN
    assert ru(layer(), x=MIS) == coli.COLI_E_ALIGN
    assert ru(layer(), nb=16) == coli.COLI_E_WORKSPACE


def test_route_forward_noalloc_argument_errors(L):
    """The no-allocation step runs every host check of coli_moe_route_forward
    and rejects a shape beyond its static scratch before any HIP call."""
    def rf(lay, T=4, mode=0, p=1.0, x=FAKE, y=FAKE):
        return L.coli_moe_route_forward_noalloc(
            ctypes.byref(lay) if lay is not None else None, x, T, ctypes.c_float(p), FAKE, FAKE,
            FAKE, FAKE, FAKE, FAKE, mode, y, None)
    assert rf(None) == coli.COLI_E_ARG
    assert rf(layer(H=100)) == coli.COLI_E_SHAPE
    assert rf(layer(), mode=2) == coli.COLI_E_UNSUPPORTED
    assert rf(layer(), p=0.0) == coli.COLI_E_ARG
    assert rf(layer(), y=0) == coli.COLI_E_ARG
    assert rf(layer(), x=MIS) == coli.COLI_E_ALIGN
    big = layer(H=6144, I=2048, E=256, k=8)
    for mode, t_max in ((0, 113), (1, 135)):
        assert coli.workspace_bytes(6144, 2048, 256, 8, t_max, mode) <= coli.NOALLOC_SCRATCH_BYTES
        assert rf(big, T=t_max + 1, mode=mode) == coli.COLI_E_SCRATCH
        assert rf(big, T=4096, mode=mode) == coli.COLI_E_SCRATCH


def test_route_forward_timeline_argument_errors(L):
    """The timeline entry point takes the self-routing fp32 cases only and a
    buffer with at least one wave's record per kernel."""
    def rft(T=1, mode=0, tl=FAKE, cap=1024, x=FAKE):
        return L.coli_moe_route_forward_timeline(ctypes.byref(layer()), x, T, ctypes.c_float(1.0),
                                                 FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, mode, FAKE,
                                                 FAKE, 1 << 30, tl, cap, None)
    assert rft(tl=None) == coli.COLI_E_ARG
    assert rft(cap=0) == coli.COLI_E_ARG
    assert rft(tl=MIS) == coli.COLI_E_ARG           # 8-byte records
    assert rft(T=5) == coli.COLI_E_UNSUPPORTED      # not self-routing
    assert rft(mode=1) == coli.COLI_E_UNSUPPORTED   # the int8 family writes no timeline
    assert rft(x=MIS) == coli.COLI_E_ALIGN
