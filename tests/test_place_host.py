"""Host-side tests of expert placement (no GPU needed).

The residency policy exists twice: the plain model in oracle/place_lru.py and
the library's planner (coli_moe_place_plan, host code in libcoli_moe.so).
Both are pinned to hand-worked sequences (tests/golden/place_lru.txt), then
compared on random call sequences, and every plan is checked for the safety
properties the overlap depends on.  Planted mistakes in the model must fail
these checks.  Argument errors of the placement entry points are checked
without touching a device."""
import ctypes
import os
import random

import pytest

import int4_routed_expert_bias_amd as coli
from conftest import ROOT
from oracle.place_lru import LRUPlacement

GOLDEN = os.path.join(ROOT, "tests", "golden", "place_lru.txt")


def read_golden():
    seqs, cur, call = [], None, None
    for line in open(GOLDEN):
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        key, *vals = line.split()
        if key == "config":
            cur = dict(E=int(vals[0]), n_slots=int(vals[1]), chunk=int(vals[2]), calls=[])
            seqs.append(cur)
        elif key == "call":
            call = dict(union=[int(v) for v in vals])
            cur["calls"].append(call)
        elif key in ("slot", "pass"):
            call["slot" if key == "slot" else "pass_"] = [int(v) for v in vals]
        elif key == "loads":
            call["loads"] = [tuple(int(x) for x in v.split(":")) for v in vals]
        elif key == "hits":
            call["hits"], call["passes"] = int(vals[0]), int(vals[2])
        elif key == "resident":
            call["resident"] = dict(tuple(int(x) for x in v.split(":")) for v in vals)
    return seqs


class CPlanner:
    """The library's planner behind the model's interface."""

    def __init__(self, E, n_slots, chunk):
        self.E = E
        self.p = coli.Placer(64, 64, E, 1, n_slots, 1, chunk)

    def plan(self, union):
        return self.p.plan(union)

    def resident(self):
        return {e: self.p.slot_of(e) for e in range(self.E) if self.p.slot_of(e) >= 0}


def model_resident(m):
    return {e: s for s, e in enumerate(m.content) if e is not None}


def check_plan(plan, union, before, n_slots, chunk):
    """Safety of one plan.  `before` maps expert -> slot before the call."""
    U = len(union)
    slot, pass_, loads = plan["slot"], plan["pass_"], plan["loads"]
    misses = [u for u in range(U) if union[u] not in before]
    assert plan["hits"] == U - len(misses)
    assert [u for u, _ in loads] == misses          # one copy per miss, union order
    assert plan["passes"] == 1 + -(-len(misses) // chunk)
    for i, u in enumerate(misses):
        assert pass_[u] == 1 + i // chunk
    for u in range(U):
        assert 0 <= slot[u] < n_slots
        if union[u] in before:
            assert pass_[u] == 0 and slot[u] == before[union[u]]
    # slot contents seen by each pass: a pass runs after every copy of
    # passes <= its own; a later copy into a slot it reads must wait for it
    for u in range(U):
        p, s = pass_[u], slot[u]
        writers = [(i, w) for i, (v, w) in enumerate(loads) if slot[v] == s]
        upto = [i for i, _ in writers if pass_[loads[i][0]] <= p]
        if union[u] in before:
            assert not upto, "a copy lands in a hit's slot before its pass"
        else:
            assert upto and loads[upto[-1]][0] == u
        for i, w in writers:
            if pass_[loads[i][0]] > p:
                assert w >= p, "a later copy overwrites a slot before its reader pass ends"
    # no two entries of one pass share a slot
    for p in set(pass_):
        ss = [slot[u] for u in range(U) if pass_[u] == p]
        assert len(ss) == len(set(ss))


def run_sequence(planner, resident_of, E, n_slots, chunk, calls, expect=None):
    for c, call in enumerate(calls):
        before = resident_of()
        plan = planner.plan(call if expect is None else call["union"])
        union = call if expect is None else call["union"]
        check_plan(plan, union, before, n_slots, chunk)
        after = resident_of()
        if len(union) <= n_slots:
            assert all(e in after for e in union)
        assert len(after) <= n_slots and len(set(after.values())) == len(after)
        if expect is not None:
            for key in ("slot", "pass_", "loads", "hits", "passes"):
                assert plan[key] == call[key], (c, key, plan[key], call[key])
            assert after == call["resident"], (c, after, call["resident"])


@pytest.mark.parametrize("impl", ["model", "library"])
def test_golden_sequences(impl):
    seqs = read_golden()
    assert len(seqs) == 2 and sum(len(s["calls"]) for s in seqs) == 8
    for sq in seqs:
        if impl == "model":
            m = LRUPlacement(sq["E"], sq["n_slots"], sq["chunk"])
            run_sequence(m, lambda: model_resident(m), sq["E"], sq["n_slots"], sq["chunk"],
                         sq["calls"], expect=True)
        else:
            c = CPlanner(sq["E"], sq["n_slots"], sq["chunk"])
            run_sequence(c, c.resident, sq["E"], sq["n_slots"], sq["chunk"], sq["calls"],
                         expect=True)


def random_unions(E, n_calls, max_u, rng, hot=None):
    out = []
    for _ in range(n_calls):
        U = rng.randint(1, max_u)
        pool = list(range(E)) if hot is None or rng.random() < 0.3 else hot
        out.append(sorted(rng.sample(pool, min(U, len(pool)))))
    return out


@pytest.mark.parametrize("E,n_slots,chunk,max_u", [
    (16, 6, 1, 8), (16, 6, 2, 12), (16, 16, 3, 16), (32, 4, 4, 20), (256, 192, 1, 9),
    (256, 64, 8, 130), (8, 1, 1, 5)])
def test_library_matches_model_on_random_sequences(E, n_slots, chunk, max_u):
    rng = random.Random(E * 1000 + n_slots * 10 + chunk)
    hot = rng.sample(range(E), max(1, E // 4))
    calls = random_unions(E, 60, max_u, rng, hot)
    m = LRUPlacement(E, n_slots, chunk)
    c = CPlanner(E, n_slots, chunk)
    for i, union in enumerate(calls):
        before = model_resident(m)
        pm, pc = m.plan(union), c.plan(union)
        assert pm == pc, (i, union)
        check_plan(pm, union, before, n_slots, chunk)
        assert model_resident(m) == c.resident()


def test_lru_order_when_cache_is_large_enough():
    # with n_slots >= U the evicted expert is always the least recently used
    # one outside the union (direct check of the LRU property)
    rng = random.Random(7)
    E, n = 20, 8
    m = LRUPlacement(E, n, 1)
    last = {}
    for t in range(1, 200):
        union = sorted(rng.sample(range(E), rng.randint(1, n)))
        before = model_resident(m)
        m.plan(union)
        after = model_resident(m)
        evicted = set(before) - set(after)
        kept_old = set(before) & set(after) - set(union)
        for e in evicted:
            assert e not in union
            assert all(last[e] <= last[k] for k in kept_old)
        for e in union:
            last[e] = t


# ---- planted mistakes: each must fail the golden sequences or the checks ----

class MRU(LRUPlacement):
    def plan(self, union):
        self.used_at = [-u for u in self.used_at]   # most recently used looks oldest
        try:
            return super().plan(union)
        finally:
            self.used_at = [abs(u) for u in self.used_at]


class HighTie(LRUPlacement):
    def plan(self, union):
        # ties broken towards the higher slot: reverse the slot order
        r = list(reversed(self.content)), list(reversed(self.used_at))
        self.content, self.used_at = r
        out = super().plan(union)
        self.content, self.used_at = list(reversed(self.content)), list(reversed(self.used_at))
        n = self.n_slots
        out["slot"] = [n - 1 - s for s in out["slot"]]
        return out


class NoWait(LRUPlacement):
    def plan(self, union):
        out = super().plan(union)
        out["loads"] = [(u, -1) for u, _ in out["loads"]]
        return out


class HitsIdle(LRUPlacement):
    """Forgets that a hit's slot is read in this call, so it may be evicted
    by a miss of the same call without waiting."""

    def plan(self, union):
        union = list(union)
        self.clock += 1
        U = len(union)
        slot, pass_ = [None] * U, [None] * U
        reader, misses = {}, []
        for u, e in enumerate(union):
            s = self.where(e)
            if s is None:
                misses.append(u)
            else:
                slot[u], pass_[u] = s, 0
                self.used_at[s] = self.clock
        loads = []
        for i, u in enumerate(misses):
            p = 1 + i // self.chunk
            empty = [s for s in range(self.n_slots) if self.content[s] is None]
            idle = [s for s in range(self.n_slots) if s not in reader]
            if empty:
                s, wait = min(empty), -1
            elif idle:
                s, wait = min(idle, key=lambda t: (self.used_at[t], t)), -1
            else:
                s = min(reader, key=lambda t: (reader[t], t))
                wait = reader[s]
            self.content[s] = union[u]
            self.used_at[s] = self.clock
            reader[s] = p
            slot[u], pass_[u] = s, p
            loads.append((u, wait))
        return dict(slot=slot, pass_=pass_, loads=loads, hits=U - len(misses),
                    passes=1 + -(-len(misses) // self.chunk))


@pytest.mark.parametrize("mutant", [MRU, HighTie, NoWait, HitsIdle])
def test_planted_mistakes_are_caught(mutant):
    caught = False
    for sq in read_golden():
        m = mutant(sq["E"], sq["n_slots"], sq["chunk"])
        try:
            run_sequence(m, lambda: model_resident(m), sq["E"], sq["n_slots"], sq["chunk"],
                         sq["calls"], expect=True)
        except AssertionError:
            caught = True
    assert caught


def test_plan_rejects_invalid_unions_and_keeps_state():
    p = coli.Placer(64, 64, 8, 2, 3, 4, 1)
    p.plan([1, 2])
    state = [p.slot_of(e) for e in range(8)]
    for bad in ([2, 1], [1, 1], [-1], [8], list(range(9))):
        with pytest.raises(coli.ColiError) as ei:
            p.plan(bad)
        assert ei.value.status == coli.COLI_E_ARG
        assert [p.slot_of(e) for e in range(8)] == state
    p.reset()
    assert all(p.slot_of(e) == -1 for e in range(8))
    assert p.slot_of(-1) == -1 and p.slot_of(8) == -1
    assert p.plan([]) == dict(slot=[], pass_=[], loads=[], hits=0, passes=1)


def test_placer_create_errors():
    L = coli.lib()
    h = ctypes.c_void_p()
    bad = [  # (H, I, E, k, n_slots, T_max, chunk), status
        ((100, 64, 8, 2, 3, 4, 1), coli.COLI_E_SHAPE),
        ((64, 64, 8, 9, 3, 4, 1), coli.COLI_E_SHAPE),
        ((64, 64, 8, 2, 9, 4, 1), coli.COLI_E_SHAPE),
        ((64, 64, 8, 2, 0, 4, 1), coli.COLI_E_SHAPE),
        ((64, 64, 8, 2, 3, 0, 1), coli.COLI_E_SHAPE),
        ((64, 64, 8, 2, 3, 4, 4), coli.COLI_E_ARG),
        ((64, 64, 8, 2, 3, 4, 0), coli.COLI_E_ARG),
    ]
    for args, st in bad:
        assert L.coli_moe_placer_create(*args, ctypes.byref(h)) == st, args
    assert L.coli_moe_placer_create(64, 64, 8, 2, 3, 4, 1, None) == coli.COLI_E_ARG
    assert L.coli_moe_placer_reset(None) == coli.COLI_E_ARG
    L.coli_moe_placer_destroy(None)


def test_place_ws_bytes():
    assert coli.place_ws_bytes(256, 8, 1) > 0
    assert coli.place_ws_bytes(256, 8, 4096) >= 4096 * 8 * 4 * 2
    assert coli.place_ws_bytes(256, 8, 4096) % 256 == 0
    assert coli.place_ws_bytes(4, 8, 1) == 0
    assert coli.place_ws_bytes(256, 8, -1) == 0


FAKE = 0x100000  # aligned, never dereferenced


def tiers(**kw):
    t = coli.ColiTiers()
    for n in ("host_w13", "host_s13", "host_w2", "host_s2", "slot_w13", "slot_s13", "slot_w2",
              "slot_s2", "slot_table"):
        setattr(t, n, kw.get(n, FAKE))
    return t


def test_forward_placed_argument_errors():
    L = coli.lib()
    P = coli.Placer(256, 128, 16, 2, 4, 8, 1)
    lay = coli.ColiLayer(256, 128, 16, 2, 1)
    for n in ("router_w", "router_bias", "sh_w13", "sh_s13", "sh_w2", "sh_s2"):
        setattr(lay, n, FAKE)

    def call(layer=lay, tr=None, T=4, mode=0, ws_nb=1 << 30, pws_nb=1 << 30, x=FAKE, pws=FAKE,
             placer=P.handle):
        tr = tr or tiers()
        return L.coli_moe_forward_placed(
            ctypes.byref(layer) if layer is not None else None, ctypes.byref(tr), placer, x, T,
            FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, mode, FAKE, FAKE, ws_nb, pws, pws_nb, None, None,
            None)

    assert call(layer=None) == coli.COLI_E_ARG
    assert call(placer=None) == coli.COLI_E_ARG
    assert call(T=9) == coli.COLI_E_SHAPE                      # T > T_max
    assert call(T=-1) == coli.COLI_E_SHAPE
    assert call(mode=2) == coli.COLI_E_UNSUPPORTED
    assert call(tr=tiers(host_w13=None)) == coli.COLI_E_ARG
    assert call(tr=tiers(slot_s2=FAKE + 4)) == coli.COLI_E_ALIGN
    assert call(tr=tiers(slot_table=None)) == coli.COLI_E_ARG
    assert call(x=None) == coli.COLI_E_ARG
    assert call(pws=None) == coli.COLI_E_ARG
    assert call(x=FAKE + 4) == coli.COLI_E_ALIGN
    assert call(ws_nb=16) == coli.COLI_E_WORKSPACE
    assert call(pws_nb=16) == coli.COLI_E_WORKSPACE
    other = coli.ColiLayer(256, 128, 16, 4, 1)
    assert call(layer=other) == coli.COLI_E_SHAPE              # k differs from the placer's
    no_sh = coli.ColiLayer(256, 128, 16, 2, 1)
    no_sh.router_w = no_sh.router_bias = FAKE
    assert call(layer=no_sh) == coli.COLI_E_ARG                # n_shared without weights
    assert call(T=0) == coli.COLI_OK                           # nothing to do
    # prefetch
    arr = (ctypes.c_int32 * 5)(1, 2, 2, 3, 4)
    assert L.coli_moe_place_prefetch(P.handle, ctypes.byref(tiers()), arr, 5, None, None) == \
        coli.COLI_E_ARG                                        # n > n_slots
    assert L.coli_moe_place_prefetch(P.handle, ctypes.byref(tiers()), arr, 3, None, None) == \
        coli.COLI_E_ARG                                        # duplicate expert
    arr2 = (ctypes.c_int32 * 2)(1, 16)
    assert L.coli_moe_place_prefetch(P.handle, ctypes.byref(tiers()), arr2, 2, None, None) == \
        coli.COLI_E_ARG                                        # out of range
    assert L.coli_moe_place_prefetch(P.handle, ctypes.byref(tiers()), arr, 0, None, None) == \
        coli.COLI_OK
    P.close()
