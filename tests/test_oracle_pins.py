"""Pins of the CPU oracle to things other than itself.

Each ``pin_*`` takes an ``oracle.Oracle`` and raises AssertionError on a
mismatch.  They check the oracle against library routines (numpy's fp16
conversion and float32 IEEE arithmetic, Python's exact rationals and
high-precision decimals), brute force on tiny inputs, closed forms and
special cases.  ``test_planted_mistakes`` rebuilds the oracle with one
plausible mistake at a time and requires that some pin catches it.
"""
import itertools
import os
import subprocess
import tempfile
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest

import oracle as oracle_mod
import synth

RNG = np.random.default_rng(20261203)

# ----------------------------------------------------------------------------
# helpers


def f32_round(fr: Fraction) -> np.float32:
    """Correctly rounded (nearest, ties to even) float32 of an exact rational."""
    a = np.float32(float(fr))
    cands = {a, np.nextafter(a, np.float32(np.inf)), np.nextafter(a, np.float32(-np.inf))}
    cands = [c for c in cands if np.isfinite(c)]
    best = min(cands, key=lambda c: (abs(Fraction(float(c)) - fr),
                                     int(np.array(c).view(np.uint32)) & 1))
    return np.float32(best)


def near_f32_midpoint(fr: Fraction, rel=2.0 ** -40) -> bool:
    """True if fr lies within rel*|fr| of a rounding boundary of float32."""
    r = f32_round(fr)
    for nb in (np.nextafter(r, np.float32(np.inf)), np.nextafter(r, np.float32(-np.inf))):
        if not np.isfinite(nb):
            continue
        mid = (Fraction(float(r)) + Fraction(float(nb))) / 2
        if abs(fr - mid) <= abs(fr) * Fraction(rel):
            return True
    return False


def f32_bits(a):
    return np.asarray(a, np.float32).view(np.uint32)


def unpack_int4(packed: np.ndarray) -> np.ndarray:
    """Packed rows [..., K/2] -> int codes [..., K]: low nibble first, two's
    complement (written with numpy bit operations, independent of the C)."""
    p = packed.astype(np.int16)
    lo = p & 0xF
    hi = (p >> 4) & 0xF
    out = np.stack([lo, hi], axis=-1).reshape(*packed.shape[:-1], packed.shape[-1] * 2)
    return np.where(out >= 8, out - 16, out).astype(np.int64)


def f16_scales(bits: np.ndarray) -> np.ndarray:
    return bits.view(np.float16).astype(np.float64)


def tiny_layer(H=128, I=64, E=6, k=2, layer=0, wid=90):
    A = synth.layer_arrays(H, I, E, k, wid=wid, layer=layer)
    return A, oracle_mod.Layer(A, k=k)


def np_quant(x: np.ndarray):
    """float32 IEEE reference quantiser (numpy): per 64-group symmetric int8."""
    x = np.asarray(x, np.float32).reshape(-1, 64)
    amax = np.max(np.abs(x), axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        sc = (amax / np.float32(127.0)).astype(np.float32)
        q = np.rint(x / sc[:, None]).astype(np.float32)
    q = np.clip(q, -127, 127)
    q[amax == 0] = 0
    sc[amax == 0] = 0
    return q.astype(np.int8).reshape(-1), sc


# ----------------------------------------------------------------------------
# pins


def pin_f16(o):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float32)
    got = np.array([o.f16_to_f32(int(b)) for b in bits], np.float32)
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    m = ~np.isnan(ref)
    assert np.array_equal(f32_bits(ref[m]), f32_bits(got[m])), "fp16 decode differs from numpy"


def pin_int4(o):
    for lo in range(-8, 8):
        for hi in range(-8, 8):
            byte = (lo & 0xF) | ((hi & 0xF) << 4)
            row = np.array([0x5A, byte, 0xA5], np.uint8)
            assert o.int4_at(row, 2) == lo and o.int4_at(row, 3) == hi, (lo, hi)


def pin_logits(o):
    for H, E, T in ((64, 5, 3), (192, 4, 2)):
        A, lay = tiny_layer(H=H, I=64, E=E, k=2, wid=91)
        x = RNG.standard_normal((T, H)).astype(np.float32) * np.float32(3.0)
        got = o.logits(lay, x)
        Wr = A["router_w"]
        for t in range(T):
            for e in range(E):
                ex = sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(x[t], Wr[e]))
                if near_f32_midpoint(ex):
                    continue
                assert f32_bits(got[t, e]) == f32_bits(f32_round(ex)), (t, e)


def exact_sigmoid_f32(l: np.float32) -> np.float32:
    getcontext().prec = 80
    d = Decimal(float(l))
    s = Decimal(1) / (Decimal(1) + (-d).exp())
    fr = Fraction(s)
    return f32_round(fr), near_f32_midpoint(fr)


def pin_sigmoid(o):
    ls = np.array([0.0, 1e-8, -1e-8, 0.25, -0.25, 1.0, -1.0, 3.7, -3.7, 10.0, -10.0,
                   17.0, -30.0, 88.0, -88.0, 120.0, -120.0], np.float32)
    ls = np.concatenate([ls, RNG.standard_normal(60).astype(np.float32) * 4]).astype(np.float32)
    E = ls.size
    _, _, s = o.select(ls[None, :], np.zeros(E, np.float32), 1)
    for e in range(E):
        ref, near = exact_sigmoid_f32(ls[e])
        if not near:
            assert f32_bits(s[0, e]) == f32_bits(ref), (ls[e], s[0, e], ref)


def _check_selection(o, lg, b, k):
    ids, w, s = o.select(lg, b, k)
    T, E = lg.shape
    for t in range(T):
        key = (s[t] + b).astype(np.float32)  # IEEE fp32 add (numpy)
        expect = sorted(range(E), key=lambda e: (-float(key[e]), e))[:k]
        assert list(ids[t]) == expect, (t, list(ids[t]), expect)
        acc = np.float32(0.0)
        for j in range(k):
            acc = np.float32(acc + s[t, ids[t, j]])
        ref_w = np.array([np.float32(s[t, ids[t, j]]) / acc for j in range(k)], np.float32)
        assert np.array_equal(f32_bits(w[t]), f32_bits(ref_w)), t


def pin_select_brute(o):
    for E in (5, 8, 11):
        for k in range(1, E + 1):
            lg = RNG.standard_normal((4, E)).astype(np.float32)
            lg[1] = lg[1][0]                       # all logits equal: ties broken by index
            lg[2, ::2] = lg[2, 1]                  # partial ties
            b = (RNG.standard_normal(E) * 0.1).astype(np.float32)
            b[::3] = b[0]
            _check_selection(o, lg, b, k)
            # exhaustive: the chosen set beats every other k-subset lexicographically
            ids, _, s = o.select(lg, b, k)
            key = (s + b).astype(np.float32)
            for t in range(lg.shape[0]):
                chosen = set(ids[t].tolist())
                for c in chosen:
                    for u in set(range(E)) - chosen:
                        assert key[t, c] > key[t, u] or (key[t, c] == key[t, u] and c < u)


def pin_select_special(o):
    for E, k in ((16, 2), (12, 3), (8, 8)):
        A, lay = tiny_layer(H=64, I=64, E=E, k=k, wid=92)
        A["router_w"][:] = 0.0
        x = RNG.standard_normal((3, 64)).astype(np.float32)
        ids, w, lg, s = o.route(lay, x)
        assert np.all(lg == 0) and np.all(s == np.float32(0.5))
        assert np.all(w == np.float32(1.0) / np.float32(k)), w
        b = A["router_b"]
        expect = sorted(range(E), key=lambda e: (-float(np.float32(0.5) + b[e]), e))[:k]
        assert all(list(r) == expect for r in ids)
        A["router_b"][:] = 0.25                 # all keys equal -> lowest indices
        ids, w, _, _ = o.route(lay, x)
        assert all(list(r) == list(range(k)) for r in ids)
        forced = RNG.choice(E, size=k, replace=False)
        A["router_b"][:] = 0.0
        A["router_b"][forced] = 10.0
        A["router_w"][:] = (RNG.standard_normal(A["router_w"].shape) * 0.02).astype(np.float32)
        ids, w, _, _ = o.route(lay, x)
        assert all(set(r.tolist()) == set(forced.tolist()) for r in ids)
        assert np.allclose(w.sum(1), 1.0, atol=k * 2e-7)


def _random_ids(T, k, E):
    return np.stack([RNG.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)


def pin_union(o):
    cases = [(1, 8, 256), (4, 2, 16), (7, 3, 10), (64, 8, 256), (33, 5, 6), (5, 1, 3)]
    for T, k, E in cases:
        ids = _random_ids(T, k, E)
        u, off, slots, nu = o.union(ids, E)
        flat = ids.reshape(-1)
        expect_u = sorted(set(flat.tolist()))
        cap = min(E, T * k)
        assert nu == len(expect_u)
        assert list(u[:nu]) == expect_u and all(v == -1 for v in u[nu:])
        counts = [int((flat == e).sum()) for e in expect_u]
        assert list(off[:nu + 1]) == [0] + list(np.cumsum(counts))
        assert all(v == T * k for v in off[nu:cap + 1])
        for i, e in enumerate(expect_u):
            expect_slots = [s for s in range(T * k) if flat[s] == e]
            assert list(slots[off[i]:off[i + 1]]) == expect_slots
        assert sorted(slots.tolist()) == list(range(T * k))
        if T == 1:
            assert list(u[:nu]) == sorted(ids[0].tolist())
    ids = np.tile(np.array([[3, 1, 7]], np.int32), (5, 1))  # identical tokens
    u, off, slots, nu = o.union(ids, 9)
    assert nu == 3 and list(np.diff(off[:4])) == [5, 5, 5]


def pin_quant(o):
    x = (RNG.standard_normal((20000, 64)) * np.exp(RNG.uniform(-6, 6, (20000, 1)))).astype(np.float32)
    x[5] = 0.0
    x[6] = np.float32(127.0)
    x[6, :8] = np.array([2.5, 3.5, -2.5, -3.5, 126.5, -0.5, 0.5, -127.0], np.float32)
    x[7, :] = np.float32(-1e-3)
    q, s = o.quant_i8(x)
    rq, rs = np_quant(x)
    assert np.array_equal(f32_bits(s), f32_bits(rs))
    assert np.array_equal(q, rq)
    assert list(q.reshape(-1, 64)[6, :8]) == [2, 4, -2, -4, 126, 0, 0, -127]
    assert np.all(q.reshape(-1, 64)[5] == 0) and s[5] == 0
    assert np.all(q.reshape(-1, 64)[7] == -127)


def pin_swiglu(o):
    assert o.swiglu(0.0, 5.0) == 0.0
    assert o.swiglu(100.0, 3.0) == np.float32(300.0)
    v = o.swiglu(-100.0, 3.0)
    assert v == 0.0 and np.signbit(v)
    gs = np.concatenate([RNG.standard_normal(400) * 4, [1e-20, -1e-20, 20.0, -20.0, 60.0]])
    us = RNG.standard_normal(gs.size) * 3
    for g, u in zip(gs.astype(np.float32), us.astype(np.float32)):
        ref = float(g) / (1.0 + np.exp(-float(g))) * float(u)
        got = o.swiglu(float(g), float(u))
        ulp = np.spacing(np.float32(abs(ref))) if ref != 0 else np.float32(1e-45)
        assert abs(got - ref) <= 4 * ulp, (g, u, got, ref)


def _exact_dot(wcodes, wscale, v):
    return sum(Fraction(int(c)) * Fraction(float(sc)) * Fraction(float(vv))
               for c, sc, vv in zip(wcodes, wscale, v))


def pin_f32_expert_exact(o):
    H, I = 256, 128
    A, _ = tiny_layer(H=H, I=I, E=1, k=1, wid=93)
    pow2 = np.array([0x2C00, 0x2800, 0x2400, 0x2000], np.uint16)  # 2^-4 .. 2^-7
    s13 = pow2[RNG.integers(0, 4, A["s13"][0].shape)]
    s2 = pow2[RNG.integers(0, 4, A["s2"][0].shape)]
    w13, w2 = A["w13"][0], A["w2"][0]
    x = RNG.integers(-8, 8, H).astype(np.float32)
    r = o.expert_f32(w13, s13, w2, s2, x)
    codes13 = unpack_int4(w13)
    sc13 = f16_scales(s13)
    # integer arithmetic in units of 2^-7: exact
    scaled = (np.repeat(sc13, 64, axis=1) * 128).astype(np.int64)
    gu = (codes13 * scaled * x.astype(np.int64)).sum(1)
    gu_f = (gu / 128.0).astype(np.float32)
    assert np.array_equal(f32_bits(r["g"]), f32_bits(gu_f[:I]))
    assert np.array_equal(f32_bits(r["u"]), f32_bits(gu_f[I:]))
    hv = np.array([o.swiglu(float(a), float(b)) for a, b in zip(r["g"], r["u"])], np.float32)
    assert np.array_equal(f32_bits(hv), f32_bits(r["h"]))
    codes2 = unpack_int4(w2)
    sc2 = np.repeat(f16_scales(s2), 64, axis=1)
    for n in range(0, H, 37):
        ex = _exact_dot(codes2[n], sc2[n], r["h"])
        assert abs(Fraction(float(r["o"][n])) - ex) <= abs(ex) * Fraction(1, 10 ** 13) + Fraction(1, 10 ** 30)
    # one-hot input selects one dequantised column exactly
    A2, _ = tiny_layer(H=H, I=I, E=1, k=1, wid=94)
    for kk in (0, 1, 63, 64, 200, 255):
        x1 = np.zeros(H, np.float32)
        x1[kk] = 1.0
        r1 = o.expert_f32(A2["w13"][0], A2["s13"][0], A2["w2"][0], A2["s2"][0], x1)
        col = unpack_int4(A2["w13"][0])[:, kk] * f16_scales(A2["s13"][0])[:, kk // 64]
        assert np.array_equal(r1["g"], col[:I].astype(np.float32))
        assert np.array_equal(r1["u"], col[I:].astype(np.float32))


def pin_i8_expert(o):
    H, I = 192, 128
    A, _ = tiny_layer(H=H, I=I, E=1, k=1, wid=95)
    w13, s13, w2, s2 = A["w13"][0], A["s13"][0], A["w2"][0], A["s2"][0]
    x = (RNG.standard_normal(H) * 1.7).astype(np.float32)
    r = o.expert_i8(w13, s13, w2, s2, x)
    qx, sx = np_quant(x)
    codes13 = unpack_int4(w13).reshape(2 * I, H // 64, 64)
    acc13 = (codes13 * qx.astype(np.int64).reshape(1, H // 64, 64)).sum(-1)
    assert np.array_equal(r["acc13"], acc13)
    sc13 = f16_scales(s13)
    for rr in range(2 * I):
        ex = sum(Fraction(int(acc13[rr, g])) * Fraction(float(sx[g])) * Fraction(float(sc13[rr, g]))
                 for g in range(H // 64))
        if near_f32_midpoint(ex):
            continue
        got = r["g"][rr] if rr < I else r["u"][rr - I]
        assert f32_bits(got) == f32_bits(f32_round(ex)), rr
    hv = np.array([o.swiglu(float(a), float(b)) for a, b in zip(r["g"], r["u"])], np.float32)
    assert np.array_equal(f32_bits(hv), f32_bits(r["h"]))
    qh, sh = np_quant(r["h"])
    assert np.array_equal(qh, r["qh"]) and np.array_equal(f32_bits(sh), f32_bits(r["sh"]))
    codes2 = unpack_int4(w2).reshape(H, I // 64, 64)
    acc2 = (codes2 * qh.astype(np.int64).reshape(1, I // 64, 64)).sum(-1)
    assert np.array_equal(r["acc2"], acc2)
    assert np.array_equal(o.down_acc_i8(w2, qh), acc2)
    sc2 = f16_scales(s2)
    for n in range(H):
        ex = sum(Fraction(int(acc2[n, g])) * Fraction(float(sh[g])) * Fraction(float(sc2[n, g]))
                 for g in range(I // 64))
        assert abs(Fraction(float(r["o"][n])) - ex) <= abs(ex) * Fraction(1, 10 ** 14)
    # the down stage on given codes: the oracle's own codes reproduce its o,
    # arbitrary codes and scales follow the exact rational sum
    assert np.array_equal(o.down_i8(w2, s2, r["qh"], r["sh"]), r["o"])
    qr = RNG.integers(-127, 128, I).astype(np.int8)
    sr = (RNG.random(I // 64) * 0.05).astype(np.float32)
    od = o.down_i8(w2, s2, qr, sr)
    accr = (codes2 * qr.astype(np.int64).reshape(1, I // 64, 64)).sum(-1)
    for n in range(H):
        ex = sum(Fraction(int(accr[n, g])) * Fraction(float(sr[g])) * Fraction(float(sc2[n, g]))
                 for g in range(I // 64))
        assert abs(Fraction(float(od[n])) - ex) <= abs(ex) * Fraction(1, 10 ** 14)
    # extreme accumulator: all weight codes -8, all activation codes -127
    w13e = np.full_like(w13, 0x88)
    xe = np.full(H, -3.0, np.float32)
    re = o.expert_i8(w13e, s13, w2, s2, xe)
    assert np.all(re["acc13"] == 64 * 127 * 8)


def pin_combine(o):
    for mode in (oracle_mod.ACT_F32, oracle_mod.ACT_I8):
        A, lay = tiny_layer(H=128, I=128, E=6, k=3, wid=96)
        x = RNG.standard_normal((3, 128)).astype(np.float32)
        ids, w, _, _ = o.route(lay, x)
        y = o.forward(lay, x, ids, w, mode)
        ex = o.expert_i8 if mode == oracle_mod.ACT_I8 else o.expert_f32
        for t in range(3):
            acc = np.zeros(128, np.float64)
            for j in range(3):
                e = ids[t, j]
                oj = ex(A["w13"][e], A["s13"][e], A["w2"][e], A["s2"][e], x[t])["o"]
                acc += np.float64(w[t, j]) * oj
            acc += ex(A["sh_w13"], A["sh_s13"], A["sh_w2"], A["sh_s2"], x[t])["o"]
            assert np.array_equal(f32_bits(y[t]), f32_bits(acc.astype(np.float32))), (mode, t)
        # every routed expert identical: routed part equals that expert's output
        for n in ("w13", "s13", "w2", "s2"):
            A[n][:] = A[n][0]
        y = o.forward(lay, x, ids, w, mode)
        for t in range(3):
            o0 = ex(A["w13"][0], A["s13"][0], A["w2"][0], A["s2"][0], x[t])["o"]
            osh = ex(A["sh_w13"], A["sh_s13"], A["sh_w2"], A["sh_s2"], x[t])["o"]
            assert np.allclose(y[t], o0 + osh, rtol=1e-5, atol=1e-5 * np.abs(o0).max())
    # k = E with a zero router: uniform weights 1/E
    A, lay = tiny_layer(H=64, I=64, E=8, k=8, wid=97)
    A["router_w"][:] = 0.0
    ids, w, _, _ = o.route(lay, RNG.standard_normal((2, 64)).astype(np.float32))
    assert np.all(w == np.float32(0.125))


def pin_rmsnorm(o):
    x = (RNG.standard_normal((6, 384)) * np.array([[1e-3], [1], [50], [1e3], [0.5], [7]])).astype(np.float32)
    x[4] = 0.0
    got = o.rmsnorm(x)
    x64 = x.astype(np.float64)
    ref = (x64 / np.sqrt((x64 ** 2).mean(1, keepdims=True) + 1e-6)).astype(np.float32)
    d = np.abs(f32_bits(got).astype(np.int64) - f32_bits(ref).astype(np.int64))
    assert d.max() <= 1, d.max()
    assert np.all(got[4] == 0)


def pin_relabel_and_independence(o):
    for mode in (oracle_mod.ACT_F32, oracle_mod.ACT_I8):
        A, lay = tiny_layer(H=128, I=64, E=7, k=2, wid=98)
        x = RNG.standard_normal((5, 128)).astype(np.float32)
        ids, w, _, _ = o.route(lay, x)
        y = o.forward(lay, x, ids, w, mode)
        perm = RNG.permutation(7)  # new label of old expert e is perm[e]
        inv = np.argsort(perm)
        B = dict(A)
        for n in ("router_w", "router_b", "w13", "s13", "w2", "s2"):
            B[n] = np.ascontiguousarray(A[n][inv])
        lay2 = oracle_mod.Layer(B, k=2)
        ids2, w2_, _, _ = o.route(lay2, x)
        assert np.array_equal(ids2, perm[ids]) and np.array_equal(w2_, w)
        y2 = o.forward(lay2, x, ids2, w2_, mode)
        assert np.array_equal(f32_bits(y), f32_bits(y2))
        sel = np.array([4, 1], np.int32)
        ys = o.forward_rows(lay, x, ids, w, sel, mode)
        assert np.array_equal(f32_bits(ys), f32_bits(y[sel]))
        p = RNG.permutation(5)
        yp = o.forward(lay, x[p], ids[p], w[p], mode)
        assert np.array_equal(f32_bits(yp), f32_bits(y[p]))


def pin_topp(o):
    """Adaptive top-p pruning of the top-k selection, checked by properties
    in exact rational arithmetic: the kept experts are the shortest prefix of
    the selection whose weights reach p, and the kept weights are the
    original ones rescaled to sum to one."""
    for (T, k, E, wid) in ((6, 8, 32, 100), (5, 4, 9, 101), (4, 16, 64, 102)):
        A, lay = tiny_layer(H=64, I=64, E=E, k=k, wid=wid)
        A["router_w"] *= 40.0  # spread the scores so that prefixes differ
        x = RNG.standard_normal((T, 64)).astype(np.float32)
        ids, w, _, sc = o.route(lay, x)
        for p in (1e-9, 0.2, 0.5, 0.7, 0.9, 0.99):
            pi, pw = o.prune_topp(ids, w, sc, p)
            for t in range(T):
                kp = int((pi[t] >= 0).sum())
                assert 1 <= kp <= k
                assert np.array_equal(pi[t, :kp], ids[t, :kp]), (p, t)
                assert np.all(pi[t, kp:] == -1) and np.all(pw[t, kp:] == 0.0)
                csum = [Fraction(0)]
                for j in range(k):
                    csum.append(csum[-1] + Fraction(float(w[t, j])))
                pf = Fraction(float(np.float32(p)))
                eps = Fraction(1, 10 ** 6)
                # reaches p with kp experts, not with kp - 1 (away from rounding)
                if kp < k or csum[k] >= pf + eps:
                    assert csum[kp] >= pf - eps, (p, t, kp)
                if kp > 1:
                    assert csum[kp - 1] < pf + eps, (p, t, kp)
                tot = sum(Fraction(float(v)) for v in pw[t, :kp])
                assert abs(tot - 1) < Fraction(1, 10 ** 6)
                for j in range(kp):
                    r_new = Fraction(float(pw[t, j])) / Fraction(float(pw[t, 0]))
                    r_old = Fraction(float(w[t, j])) / Fraction(float(w[t, 0]))
                    assert abs(r_new - r_old) <= Fraction(1, 10 ** 5) * r_old
            if p == 1e-9:
                assert np.all((pi >= 0).sum(axis=1) == 1) and np.all(pw[:, 0] == 1.0)
        # p >= 1: the selection is unchanged, bit for bit
        for p in (1.0, 1.5):
            pi, pw = o.prune_topp(ids, w, sc, p)
            assert np.array_equal(pi, ids) and np.array_equal(f32_bits(pw), f32_bits(w))
    # union of a pruned selection: brute force over the kept slots only
    ids = np.array([[4, 2, -1, -1], [2, -1, -1, -1], [7, 4, 1, -1]], np.int32)
    u, off, slots, nu = o.union(ids, 8)
    flat = ids.reshape(-1)
    kept = [s_ for s_ in range(flat.size) if flat[s_] >= 0]
    assert nu == 4 and list(u[:nu]) == [1, 2, 4, 7]
    assert off[nu] == len(kept) and all(v == len(kept) for v in off[nu:])
    for i, e in enumerate(u[:nu]):
        assert list(slots[off[i]:off[i + 1]]) == [s_ for s_ in kept if flat[s_] == e]
    # forward: a dropped slot contributes exactly nothing (same bits as the
    # same expert list with that slot's weight set to zero)
    for mode in (oracle_mod.ACT_F32, oracle_mod.ACT_I8):
        A, lay = tiny_layer(H=128, I=64, E=6, k=3, wid=103)
        x = RNG.standard_normal((2, 128)).astype(np.float32)
        ids, w, _, sc = o.route(lay, x)
        pi, pw = o.prune_topp(ids, w, sc, 0.3)
        z = np.where(pi >= 0, pi, ids).astype(np.int32)
        y1 = o.forward(lay, x, pi, pw, mode)
        y2 = o.forward(lay, x, z, pw, mode)
        assert np.array_equal(f32_bits(y1), f32_bits(y2)), mode


# ----------------------------------------------------------------------------
# compressed-KV (MLA) decode attention


def _ulps(a, b):
    ai = np.asarray(a, np.float32).view(np.int32).astype(np.int64)
    bi = np.asarray(b, np.float32).view(np.int32).astype(np.int64)
    ai = np.where(ai < 0, -(ai & 0x7FFFFFFF), ai)
    bi = np.where(bi < 0, -(bi & 0x7FFFFFFF), bi)
    return np.abs(ai - bi)


def _mla_ref(q, kv, scale, keys):
    """Library routines only: scipy's softmax over numpy float64 scores."""
    from scipy.special import softmax
    q64, kv64 = q.astype(np.float64), kv.astype(np.float64)
    scale = float(np.float32(scale))  # the oracle takes the scale as a float
    out = np.zeros(q.shape[:2] + (512,), np.float64)
    for b in range(q.shape[0]):
        rows = keys[b]
        if len(rows) == 0:
            continue
        s = scale * (q64[b] @ kv64[rows].T)          # [heads][keys]
        out[b] = softmax(s, axis=1) @ kv64[rows, :512]
    return out


def pin_mla_brute(o):
    for B, nh, T, scale in ((2, 3, 37, 0.07), (1, 16, 5, 0.3), (3, 2, 64, 0.0417)):
        q = RNG.standard_normal((B, nh, 576)).astype(np.float32)
        kv = RNG.standard_normal((T, 576)).astype(np.float32)
        lens = RNG.integers(1, T + 1, B).astype(np.int32)
        lens[0] = T
        got = o.mla_decode(q, kv, scale, lens=lens)
        ref = _mla_ref(q, kv, scale, [list(range(l)) for l in lens])
        assert _ulps(got, ref.astype(np.float32)).max() <= 1
    # large scores: the exponentials must stay finite
    q = (RNG.standard_normal((1, 4, 576)) * 30).astype(np.float32)
    kv = RNG.standard_normal((50, 576)).astype(np.float32)
    got = o.mla_decode(q, kv, 1.0, lens=np.array([50], np.int32))
    ref = _mla_ref(q, kv, 1.0, [list(range(50))])
    assert np.isfinite(got).all() and _ulps(got, ref.astype(np.float32)).max() <= 1


def pin_mla_closed_forms(o):
    T = 40
    kv = RNG.standard_normal((T, 576)).astype(np.float32)
    q = RNG.standard_normal((2, 8, 576)).astype(np.float32)
    # scale 0: every key weighs the same, o is the mean of the value rows
    lens = np.array([T, 13], np.int32)
    got = o.mla_decode(q, kv, 0.0, lens=lens)
    for b, l in enumerate(lens):
        mean = kv[:l, :512].astype(np.float64).mean(axis=0).astype(np.float32)
        assert _ulps(got[b], np.broadcast_to(mean, got[b].shape)).max() <= 1
    # one dominant key through the last rotary dimension: o is its value row
    qd = np.zeros((1, 3, 576), np.float32)
    qd[..., 575] = 1.0
    for target, l in ((7, 20), (19, 20), (20, 20)):
        kd = kv.copy()
        kd[:, 575] = 0.0
        kd[target, 575] = 1.0
        got = o.mla_decode(qd, kd, 80.0, lens=np.array([l], np.int32))
        if target < l:
            want = kd[target, :512]
        else:  # outside the prefix: every kept key scores 0
            want = kd[:l, :512].astype(np.float64).mean(axis=0).astype(np.float32)
        assert _ulps(got[0], np.broadcast_to(want, got[0].shape)).max() <= 1, (target, l)
    # a constant added to every score changes nothing
    qs = q.copy()
    qs[..., 575] = 1.0
    k0 = kv.copy()
    k0[:, 575] = 0.0
    base = o.mla_decode(qs, k0, 0.05, lens=lens)
    ks = k0.copy()
    ks[:, 575] = np.float32(37.0)  # every score moves by exactly 0.05 * 37
    assert _ulps(o.mla_decode(qs, ks, 0.05, lens=lens), base).max() <= 2
    # values use the latent part only
    qz = q.copy()
    qz[..., 512:] = 0.0
    kz = kv.copy()
    kz[:, 512:] = 1e6
    a = o.mla_decode(qz, kz, 0.05, lens=lens)
    kz[:, 512:] = 0.0
    assert np.array_equal(a, o.mla_decode(qz, kz, 0.05, lens=lens))
    # a query without keys gets zeros
    z = o.mla_decode(q[:1], kv, 0.05, lens=np.array([0], np.int32))
    assert not z.any()
    z = o.mla_decode(q[:1], kv, 0.05, idx=np.full((1, 5), -1, np.int32))
    assert not z.any()


def pin_mla_key_lists(o):
    T = 70
    kv = RNG.standard_normal((T, 576)).astype(np.float32)
    q = RNG.standard_normal((3, 4, 576)).astype(np.float32)
    lens = np.array([70, 33, 1], np.int32)
    dense = o.mla_decode(q, kv, 0.06, lens=lens)
    # the prefix as an explicit list, padded with -1 and out-of-range rows
    idx = np.full((3, 90), -1, np.int32)
    for b, l in enumerate(lens):
        idx[b, :l] = np.arange(l)
    idx[1, 50] = T
    idx[2, 7] = 10 ** 6
    assert np.array_equal(o.mla_decode(q, kv, 0.06, idx=idx), dense)
    # any order of the listed keys (only rounding differs)
    perm = idx.copy()
    for b, l in enumerate(lens):
        perm[b, :l] = RNG.permutation(l)
    assert _ulps(o.mla_decode(q, kv, 0.06, idx=perm), dense).max() <= 1
    # a sparse selection equals attention over those rows alone
    sel = np.sort(RNG.choice(T, 24, replace=False)).astype(np.int32)
    got = o.mla_decode(q[:1], kv, 0.06, idx=sel[None])
    ref = _mla_ref(q[:1], kv, 0.06, [sel.tolist()])
    assert _ulps(got, ref.astype(np.float32)).max() <= 1


PINS = [pin_f16, pin_int4, pin_logits, pin_sigmoid, pin_select_brute, pin_select_special,
        pin_union, pin_quant, pin_swiglu, pin_f32_expert_exact, pin_i8_expert, pin_combine,
        pin_rmsnorm, pin_relabel_and_independence, pin_topp, pin_mla_brute,
        pin_mla_closed_forms, pin_mla_key_lists]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(orc, pin):
    pin(orc)


def test_size_identities():
    """The layer shape reproduces the sizes the pages print."""
    golden = {}
    path = os.path.join(os.path.dirname(__file__), "golden", "size_identities.txt")
    for line in open(path, encoding="utf-8"):
        if line.startswith("#") or not line.strip():
            continue
        name, value, unit, tol, cite = [c.strip() for c in line.split("|")]
        golden[name] = (float(value), float(tol))
    w = synth.WORKLOADS["decode"]
    eb = synth.expert_bytes(w.H, w.I)
    assert eb == 20054016
    derived = {
        "expert_bytes": eb,
        "routed_experts_total": 76 * w.E,          # 75 MoE layers + the MTP layer
        "experts_on_disk_bytes": 76 * w.E * eb,
        "routed_bytes_per_token": 75 * w.k * eb,
        "experts_per_layer": w.E,
        "top_k": w.k,
        "moe_layers": 75,
    }
    for name, (value, tol) in golden.items():
        assert abs(derived[name] - value) <= tol * value, (name, derived[name], value)


# ----------------------------------------------------------------------------
# planted mistakes: each must be caught by at least one pin

MUTANTS = [
    ("int4 sign", "return nib < 8 ? nib : nib - 16;", "return nib < 8 ? nib : nib - 15;"),
    ("nibble order", "int nib = (kk & 1) ? (byte >> 4) & 0xF : byte & 0xF;",
     "int nib = (kk & 1) ? byte & 0xF : (byte >> 4) & 0xF;"),
    ("scale group", "return (float)orc_int4(row, kk) * fsrow[kk / 64];",
     "return (float)orc_int4(row, kk) * fsrow[0];"),
    ("f16 exponent", "v = ldexp((double)(man + 1024), exp - 25);",
     "v = ldexp((double)(man + 1024), exp - 24);"),
    ("dropped logit term", "acc += (double)xr[h] * (double)wr[h];",
     "acc += (double)xr[h] * (double)wr[h] * (h > 0);"),
    ("sigmoid sign", "s[e] = (float)(1.0 / (1.0 + exp(-l)));", "s[e] = (float)(1.0 / (1.0 + exp(l)));"),
    ("bias dropped", "c[e].key = s[e] + bias[e];", "c[e].key = s[e];"),
    ("tie order", "return (a->e > b->e) - (a->e < b->e);", "return (a->e < b->e) - (a->e > b->e);"),
    ("weights from biased key", "for (int32_t j = 0; j < k; ++j) sum += s[c[j].e];",
     "for (int32_t j = 0; j < k; ++j) sum += c[j].key;"),
    ("union offsets", "offsets[U] = run;", "offsets[U] = run + count[e];"),
    ("quant divisor", "float sc = amax / 127.0f;", "float sc = amax / 128.0f;"),
    ("quant rounding", "float r = rintf(xg[i] / sc);", "float r = truncf(xg[i] / sc);"),
    ("swiglu sign", "return g / (1.0f + expf(-g)) * u;", "return g / (1.0f + expf(g)) * u;"),
    ("group dot short", "for (int64_t kk = g * 64; kk < g * 64 + 64; ++kk)",
     "for (int64_t kk = g * 64; kk < g * 64 + 63; ++kk)"),
    ("down scale", "acc += (double)a * (double)shv[gg] * (double)orc_f16_to_f32(srow[gg]);",
     "acc += (double)a * (double)shv[0] * (double)orc_f16_to_f32(srow[gg]);"),
    ("down from codes scale", "acc += (double)group_dot(qh, row, gg) * (double)sh[gg] *",
     "acc += (double)group_dot(qh, row, gg) * (double)sh[0] *"),
    ("shared dropped", "if (!L->n_shared) break;", "break;"),
    ("weight index", "wj = (double)w_t[j];", "wj = (double)w_t[0];"),
    ("rms divisor", "double inv = 1.0 / sqrt(ss / (double)H + 1e-6);",
     "double inv = 1.0 / sqrt(ss / (double)(H - 1) + 1e-6);"),
    ("down input", "for (int64_t kk = 0; kk < I; ++kk) acc += (double)wdeq(r, sd, kk) * (double)hv[kk];",
     "for (int64_t kk = 0; kk < I; ++kk) acc += (double)wdeq(r, sd, kk) * (double)x[kk];"),
    ("gate/up swapped", "float gf = (float)ag, uf = (float)au;", "float gf = (float)au, uf = (float)ag;"),
    ("i8 gate/up swapped", "float gf = (float)val[0], uf = (float)val[1];",
     "float gf = (float)val[1], uf = (float)val[0];"),
    ("topp keeps one more", "                kp = m;\n", "                kp = m < k ? m + 1 : m;\n"),
    ("topp not renormalised", "wt[j] = scores[(size_t)t * E + it[j]] / sum;", "wt[j] = wt[j];"),
    ("topp drops from the front", "if (j < kp) {\n                wt[j]", "if (j >= k - kp) {\n                wt[j]"),
    ("union counts dropped slots", "    for (int32_t u = U; u <= cap; ++u) offsets[u] = run;",
     "    for (int32_t u = U; u <= cap; ++u) offsets[u] = n;"),
    ("mla no max shift", "double p = exp(s[j] - m);", "double p = exp(s[j]);"),
    ("mla value offset", "for (int32_t d = 0; d < DV; ++d) o[d] += p * (double)vr[d];",
     "for (int32_t d = 0; d < DV; ++d) o[d] += p * (double)vr[d + 64];"),
    ("mla prefix short", "for (int32_t t = 0; t < len; ++t) row[nk++] = t;",
     "for (int32_t t = 0; t + 1 < len; ++t) row[nk++] = t;"),
    ("mla scale dropped", "s[j] = (double)scale * acc;", "s[j] = acc;"),
    ("mla rotary part dropped", "for (int32_t d = 0; d < D; ++d) acc += (double)qv[d] * (double)kr[d];",
     "for (int32_t d = 0; d < DV; ++d) acc += (double)qv[d] * (double)kr[d];"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistakes(name, old, new):
    src = open(os.path.join(os.path.dirname(oracle_mod.__file__), "coli_oracle.c")).read()
    assert src.count(old) == 1, f"mutation anchor not unique/found: {name}"
    with tempfile.TemporaryDirectory() as d:
        import shutil
        shutil.copy(os.path.join(os.path.dirname(oracle_mod.__file__), "coli_oracle.h"), d)
        cpath = os.path.join(d, "coli_oracle.c")
        open(cpath, "w").write(src.replace(old, new))
        so = os.path.join(d, "libmut.so")
        subprocess.run(["gcc"] + oracle_mod.CFLAGS + ["-w", "-fPIC", "-shared", "-o", so, cpath, "-lm"],
                       check=True)
        mut = oracle_mod.Oracle(oracle_mod.load(so))
        caught = []
        for pin in PINS:
            try:
                pin(mut)
            except AssertionError:
                caught.append(pin.__name__)
        assert caught, f"planted mistake '{name}' passed every pin"
