"""GPU tests of the cases the method defines at its edges, against the CPU
oracle: exact key ties in the router (the lower expert index wins), a bias
that forces a set, all-zero tokens, the fp32 family on inputs where every
summation order is exact (the output must equal the oracle's exactly), and
the int8 activation quantiser on about a million groups including exact
round-half cases.

Every path that selects experts is exercised: the single-launch route and
union of up to 4 tokens, the router GEMM with the top-k and union kernels
(40 tokens), and the one-call step whose gate/up kernel routes the tokens
itself (up to 4 tokens in the fp32 family, one in the int8 family).
"""
import numpy as np
import pytest

from conftest import gpu_available

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]

import int4_routed_expert_bias_amd as coli  # noqa: E402
import oracle as oracle_mod  # noqa: E402
import synth  # noqa: E402
from gpu_util import GpuLayer, assert_close, check_route, orc_y_rows, pool_map  # noqa: E402

ORC = None


def orc():
    global ORC
    if ORC is None:
        ORC = oracle_mod.default()
    return ORC


def run_paths(lay: GpuLayer, x: np.ndarray, mode: int):
    """The layer on x through route_union + forward, and through the
    one-call step when it routes inside the gate/up kernel; returns a list
    of (path name, outputs)."""
    import torch
    T = x.shape[0]
    xd = torch.from_numpy(np.ascontiguousarray(x)).cuda()
    outs = []
    paths = ["route_union"] + (["step"] if coli.route_forward_fused(lay.dev, T, mode) else [])
    for path in paths:
        b = coli.Buffers(lay.dev, T, mode)
        coli.run_layer(lay.dev, xd, b, fused="step" if path == "step" else True)
        torch.cuda.synchronize()
        nu = int(b.n_union[0].item())
        outs.append((path, dict(ids=b.ids[:T].cpu().numpy(), w=b.w[:T].cpu().numpy(),
                                y=b.y[:T].cpu().numpy(), union_ids=b.union_ids.cpu().numpy(),
                                offsets=b.offsets.cpu().numpy(),
                                slots=b.slots[:T * lay.k].cpu().numpy(), n_union=nu)))
    return outs


def check_against_oracle(lay: GpuLayer, x, mode, out, what):
    ids, w, _, _ = orc().route(lay.orc, x)
    check_route(out["ids"], out["w"], ids, w)
    u, off, slots, nu = orc().union(ids, lay.E)
    assert out["n_union"] == nu, what
    assert np.array_equal(out["union_ids"], u), what
    assert np.array_equal(out["offsets"], off), what
    assert np.array_equal(out["slots"], slots), what
    ref = orc_y_rows(orc(), lay.orc, x, ids, w, mode)
    assert_close(out["y"], ref, f"{what}: y")
    return ids, w


# ---------------------------------------------------------------------------
# router ties and forced selections

def tie_layer(E, k, case, wid):
    """A small layer (H 256, I 128) whose router is set up for one tie case."""
    A = synth.layer_arrays(256, 128, E, k, wid=wid)
    e = np.arange(E)
    if case == "zero_router_equal_bias":
        A["router_w"][:] = 0.0
        A["router_b"][:] = 0.0
    elif case == "zero_router_partial_ties":
        A["router_w"][:] = 0.0
        A["router_b"][:] = (np.float32(0.05) * ((7 * e) % 5)).astype(np.float32)
    elif case == "forced_set":
        A["router_b"][:] = 0.0
        forced = np.array(sorted({E - 1, 3 % E, E // 2, 1, E // 3, E - 4, 5 % E, E // 5}))[:k]
        assert forced.size == k
        A["router_b"][forced] = 10.0
        A["forced"] = forced
    elif case == "duplicate_rows":
        # experts 2m and 2m+1 share their router row and bias: their keys
        # are equal bit for bit whatever the token
        A["router_w"][1::2] = A["router_w"][0::2][:E // 2]
        A["router_b"][1::2] = A["router_b"][0::2][:E // 2]
    else:
        raise ValueError(case)
    return A


@pytest.mark.parametrize("E,k", [(16, 2), (256, 8)])
@pytest.mark.parametrize("case", ["zero_router_equal_bias", "zero_router_partial_ties",
                                  "forced_set", "duplicate_rows"])
def test_router_ties(E, k, case):
    A = tie_layer(E, k, case, wid=200 + E)
    lay = GpuLayer(A, k)
    for T in (1, 4, 40):
        x = synth.activations(256, T, wid=201, layer=T)
        for mode in (coli.ACT_F32, coli.ACT_I8):
            for path, out in run_paths(lay, x, mode):
                what = f"{case} E={E} T={T} mode={mode} {path}"
                print(what, flush=True)
                ids, w = check_against_oracle(lay, x, mode, out, what)
                if case == "zero_router_equal_bias":
                    # every key is 0.5: the k lowest expert indices, in order,
                    # each with weight 0.5 / (k * 0.5) = 1/k exactly
                    assert np.array_equal(out["ids"], np.tile(np.arange(k), (T, 1))), what
                    assert np.all(out["w"] == np.float32(1.0 / k)), what
                elif case == "forced_set":
                    assert all(set(r) == set(A["forced"].tolist()) for r in out["ids"]), what
                elif case == "duplicate_rows":
                    # a tied pair is selected lower index first, or only its
                    # lower index when the k-th place splits it
                    for r in out["ids"]:
                        pos = {e: j for j, e in enumerate(r.tolist())}
                        for e in r.tolist():
                            if e % 2 == 1:
                                assert pos.get(e - 1, 99) < pos[e], (what, r)


# ---------------------------------------------------------------------------
# all-zero tokens

@pytest.mark.parametrize("mode", [coli.ACT_F32, coli.ACT_I8])
def test_zero_tokens(mode):
    """An all-zero token: its int8 scale is 0 and its codes 0, and in both
    families every expert output is 0, so its y row is exactly zero; the
    other tokens of the batch are unaffected."""
    lay = GpuLayer(synth.layer_arrays(512, 256, 16, 4, wid=210), 4)
    for T, zero in ((1, [0]), (3, [1]), (4, [0, 3]), (40, [0, 17, 39])):
        x = synth.activations(512, T, wid=211, layer=T)
        x[zero] = 0.0
        for path, out in run_paths(lay, x, mode):
            what = f"zero tokens T={T} mode={mode} {path}"
            check_against_oracle(lay, x, mode, out, what)
            assert np.all(out["y"][zero] == 0.0), what
            assert np.all(np.isfinite(out["y"])), what


# ---------------------------------------------------------------------------
# fp32 family: an input on which every summation order is exact

def exact_case_layer(H, I, E, k, wid):
    """Weights for which, with one-hot tokens of value 256, the whole fp32
    family is exact arithmetic:
      - router weights 0 (every score 0.5; the weights are 1/k exactly for k
        a power of two), distinct random biases pick the experts;
      - gate scales 2^-4 and gate codes outside {-5..-1, 1}, so
        g = 256 * code / 16 is 0, >= 32 or <= -96: 1 + exp(-g) rounds to 1
        or exp(-g) overflows, and SwiGLU gives g * u or a signed zero
        exactly, whatever the exp implementation;
      - up scales 2^-7: u = 2 * code, so h = 32 * gate code * up code;
      - down scales powers of two in 2^-4..2^-7: every product is a
        multiple of 1/4 and every partial sum of o stays below 2^24 / 4."""
    A = synth.layer_arrays(H, I, E, k, wid=wid)
    rng = np.random.default_rng(wid)
    A["router_w"][:] = 0.0
    A["router_b"][:] = rng.permutation(E).astype(np.float32) * np.float32(0.01)
    # gate codes: nibble -> code, remapped away from {-5..-1, 1}
    remap = np.arange(16, dtype=np.uint8)
    for nib, new in ((1, 2), (11, 8), (12, 9), (13, 10), (14, 8), (15, 9)):  # 1 -> 2, -5.. -1 -> -8..-6
        remap[nib] = new
    for wn, sn in (("w13", "s13"), ("sh_w13", "sh_s13")):
        w, s = A[wn], A[sn]
        gate = w[..., :I, :]
        lo, hi = remap[gate & 0xF], remap[gate >> 4]
        gate[...] = lo | (hi << 4)
        s[..., :I, :] = 0x2C00                     # 2^-4
        s[..., I:, :] = 0x2000                     # 2^-7
    for sn in ("s2", "sh_s2"):
        p = rng.integers(4, 8, size=A[sn].shape)   # 2^-4 .. 2^-7
        A[sn][...] = ((15 - p) << 10).astype(np.uint16)
    return A


def one_hot_tokens(T, H):
    """T tokens, each 256 at one position (spread over groups and both
    nibbles of a byte), 0 elsewhere."""
    x = np.zeros((T, H), np.float32)
    x[np.arange(T), (np.arange(T) * 97 + 5) % H] = 256.0
    return x


def exact_case_precondition(A, x, ids, k):
    """Checks, on the oracle's own double values, what makes every summation
    order exact: h is a multiple of 32 with |h| <= 1792, the expert outputs
    are multiples of 1/4, and each token's combine stays below 2^24 units
    of 1/(4k)."""
    T = x.shape[0]

    def experts(t):
        return [orc().expert_f32(A["w13"][e], A["s13"][e], A["w2"][e], A["s2"][e], x[t])
                for e in ids[t]] + [orc().expert_f32(A["sh_w13"], A["sh_s13"], A["sh_w2"],
                                                     A["sh_s2"], x[t])]
    for t, ex in enumerate(pool_map(experts, range(T))):
        for r in ex:
            assert np.abs(r["h"]).max() <= 1792 and np.all(np.mod(r["h"], 32) == 0), t
            assert np.all(np.mod(r["o"], 0.25) == 0), t
        bound = sum(np.abs(r["o"]) / k for r in ex[:k]) + np.abs(ex[k]["o"])
        assert bound.max() <= 2.0 ** 24 * 0.25 / k, t


@pytest.mark.parametrize("shape", [(256, 128, 16, 2), (6144, 2048, 32, 8)])
def test_fp32_exact_case(shape):
    """One-hot tokens (value 256) on exact_case_layer: g, u, h, the expert
    outputs and y are exact in any summation order, so the GPU's y must
    equal the oracle's exactly -- for the single-token, the few-token and
    the batched kernels and the one-call step."""
    H, I, E, k = shape
    A = exact_case_layer(H, I, E, k, wid=220 + H % 7)
    lay = GpuLayer(A, k)
    for T in ((1, 4, 40) if H <= 256 else (1, 4, 12)):
        x = one_hot_tokens(T, H)
        ids, w, _, _ = orc().route(lay.orc, x)
        assert np.all(w == np.float32(1.0 / k))
        exact_case_precondition(A, x, ids, k)
        ref = orc_y_rows(orc(), lay.orc, x, ids, w, coli.ACT_F32)
        for path, out in run_paths(lay, x, coli.ACT_F32):
            what = f"exact case {shape} T={T} {path}"
            print(what, flush=True)
            assert np.array_equal(out["ids"], ids), what
            bad = np.argwhere(out["y"] != ref)
            assert bad.size == 0, (what, bad[:4], out["y"][tuple(bad[0])], ref[tuple(bad[0])])


# ---------------------------------------------------------------------------
# the int8 activation quantiser on about a million groups

def quant_inputs(T, H, seed):
    """x [T, H] whose 64-groups cycle through kinds: normal values; exact
    round-half cases (amax 127 * 2^e, the other values (m + 1/2) * 2^e, so
    value / scale is exactly m + 1/2); all zeros with negative zeros; wide
    magnitudes (10^-15 .. 10^15, no subnormal scale); values placed at
    (m + 1/2) * scale for an arbitrary scale (near the rounding boundary)."""
    rng = np.random.default_rng(seed)
    G = T * H // 64
    x = rng.standard_normal((G, 64)).astype(np.float32)
    kind = np.arange(G) % 8
    # 3, 4: exact halves
    for kd, e in ((3, np.zeros(G, int)), (4, rng.integers(-10, 11, size=G))):
        sel = np.nonzero(kind == kd)[0]
        m = rng.integers(-127, 127, size=(sel.size, 64)).astype(np.float32) + np.float32(0.5)
        m[:, 0] = np.where(rng.random(sel.size) < 0.5, -127.0, 127.0)
        x[sel] = m * np.exp2(e[sel]).astype(np.float32)[:, None]
    # 5: zeros, some negative
    sel = np.nonzero(kind == 5)[0]
    x[sel] = np.where(rng.random((sel.size, 64)) < 0.5, np.float32(-0.0), np.float32(0.0))
    # 6: wide magnitudes
    sel = np.nonzero(kind == 6)[0]
    x[sel] *= (10.0 ** rng.uniform(-15, 15, size=(sel.size, 1))).astype(np.float32)
    # 7: (m + 1/2) * scale with the scale of the group's amax
    sel = np.nonzero(kind == 7)[0]
    amax = np.abs(x[sel]).max(axis=1)
    sc = (amax / np.float32(127.0)).astype(np.float32)
    m = rng.integers(-126, 126, size=(sel.size, 64)).astype(np.float32) + np.float32(0.5)
    y = (m * sc[:, None]).astype(np.float32)
    y[:, 0] = amax
    x[sel] = y
    return x.reshape(T, H)


def test_quantiser_million_groups():
    """The forward's own activation quantiser (its codes and scales from
    the accumulator dump) on 1,048,576 groups: bit-exact against the
    oracle's quantiser, exact round-half cases included."""
    import torch
    H, I, E, k, T = 8192, 64, 2, 1, 8192
    lay = GpuLayer(synth.layer_arrays(H, I, E, k, wid=230, n_shared=0), k, n_shared=0)
    x = quant_inputs(T, H, seed=231)
    # the exact round-half cases the data holds (float32 value / scale)
    g = x.reshape(-1, 64)
    sc = (np.abs(g).max(axis=1) / np.float32(127.0)).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = (g / sc[:, None]).astype(np.float32)
    ties = int(np.sum((sc[:, None] > 0) & (np.abs(r - np.trunc(r)) == 0.5)))
    assert g.shape[0] == 1 << 20 and ties > 100_000, ties
    b = coli.Buffers(lay.dev, T, coli.ACT_I8, dump=True)
    coli.run_layer(lay.dev, torch.from_numpy(x).cuda(), b)
    torch.cuda.synchronize()
    reg = coli.dump_regions(H, I, k, T, 0)
    (oq, _, sq), (os_, _, ss) = reg["qx"], reg["sx"]
    gq = b.dump[oq:oq + T * H].cpu().numpy().view(np.int8)
    gs = b.dump[os_:os_ + T * (H // 64) * 4].cpu().numpy().view(np.float32)
    rq, rs = orc().quant_i8(x)
    assert np.array_equal(gs.view(np.uint32), rs.view(np.uint32))
    bad = np.nonzero(gq != rq)[0]
    assert bad.size == 0, (bad.size, bad[:8], gq[bad[:8]], rq[bad[:8]])
    print(f"quantiser: {g.shape[0]} groups, {ties} exact half cases, all codes equal")
