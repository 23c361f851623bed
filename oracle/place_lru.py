"""Plain model of the expert residency policy that places a layer's experts
in a pool of device slots (test infrastructure only: used by tests/; the
product path never imports it and it shares no code with the library).

Pages: the Colibri getting-started page (cti.vibequant.cc), section
"토큰당 처리 경로 (The Per-Token Path)" -- Place chooses where an expert is
fetched from and affects speed only, Overlap computes with resident experts
while missing ones load; hysenlabs.com "colibri: 744B MoEをストレージから推論
するCエンジン", section "なぜ744Bモデルが25GBのRAMで動くのか" -- a per-layer LRU
cache in front of the slower tier.

The pages fix only "per-layer LRU"; the rest is this library's reading:
  * one clock tick per call; every expert of the call's union counts as used
    at that tick;
  * hits are computed in pass 0; misses, in union order, form passes 1, 2,
    ... of at most `chunk` experts;
  * the slot for a miss of pass p is, in this order of preference,
      - the lowest-numbered empty slot,
      - the least recently used slot that no pass of this call reads
        (lowest number on ties),
      - the slot read by the earliest pass q < p of this call (lowest number
        on ties), whose copy must then wait for pass q to finish.

Parity: pinned by hand-worked sequences (tests/golden/place_lru.txt) and by
properties checked in tests (every union expert sits in its slot when its
pass runs, no copy overwrites a slot before its reader pass has finished,
LRU eviction order).
"""
from __future__ import annotations


class LRUPlacement:
    def __init__(self, E: int, n_slots: int, chunk: int = 1):
        assert 1 <= n_slots <= E and 1 <= chunk <= n_slots
        self.E, self.n_slots, self.chunk = E, n_slots, chunk
        self.content = [None] * n_slots   # expert held by each slot
        self.used_at = [0] * n_slots      # clock of the last call that used it
        self.clock = 0

    def where(self, e):
        """Slot holding expert e, or None."""
        for s, held in enumerate(self.content):
            if held == e:
                return s
        return None

    def plan(self, union):
        """Place one call's union (ascending distinct experts).

        Returns dict(slot=[...], pass_=[...], loads=[(u, wait), ...],
        hits=h, passes=P) with one slot and pass per union position."""
        union = list(union)
        assert union == sorted(set(union)) and all(0 <= e < self.E for e in union)
        self.clock += 1
        U = len(union)
        slot, pass_ = [None] * U, [None] * U
        reader = {}  # slot -> pass of this call that reads it
        misses = []
        for u, e in enumerate(union):
            s = self.where(e)
            if s is None:
                misses.append(u)
            else:
                slot[u], pass_[u] = s, 0
                self.used_at[s] = self.clock
                reader[s] = 0
        loads = []
        for i, u in enumerate(misses):
            p = 1 + i // self.chunk
            empty = [s for s in range(self.n_slots) if self.content[s] is None]
            idle = [s for s in range(self.n_slots) if s not in reader]
            done_earlier = [s for s in range(self.n_slots) if s in reader and reader[s] < p]
            if empty:
                s, wait = min(empty), -1
            elif idle:
                s, wait = min(idle, key=lambda t: (self.used_at[t], t)), -1
            else:
                s = min(done_earlier, key=lambda t: (reader[t], t))
                wait = reader[s]
            self.content[s] = union[u]
            self.used_at[s] = self.clock
            reader[s] = p
            slot[u], pass_[u] = s, p
            loads.append((u, wait))
        passes = 1 + -(-len(misses) // self.chunk)
        return dict(slot=slot, pass_=pass_, loads=loads, hits=U - len(misses), passes=passes)
