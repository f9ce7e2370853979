"""A model of the expert cache's slot policy, written from the rules that
include/qmoe.h states (not from the C++), used by the CPU policy test and the
GPU cache tests to predict every hit, miss and slot."""
from __future__ import annotations


class SlotModel:
    def __init__(self, n_experts: int, n_slots: int):
        self.E, self.S = n_experts, n_slots
        self.owner = [None] * n_slots        # expert in each slot
        self.used = [0] * n_slots            # request number that last used it
        self.pinned = set()                  # pinned slots
        self.requests = 0
        self.evictions = 0

    def slot_of(self, e):
        return self.owner.index(e) if e in self.owner else -1

    def request(self, experts, protect_from=None):
        """Returns (hits, [(expert, slot) loads]) or None if the misses do not
        fit (then nothing changes)."""
        need = sorted(set(int(e) for e in experts))
        keep = {self.slot_of(e) for e in need if self.slot_of(e) >= 0}
        hits = len(keep)
        loads = []
        for e in (e for e in need if self.slot_of(e) < 0):
            busy = keep | {s for _, s in loads}
            free = [s for s in range(self.S) if self.owner[s] is None and s not in busy]
            if free:
                loads.append((e, free[0]))
                continue
            ok = [s for s in range(self.S) if s not in busy and s not in self.pinned
                  and (protect_from is None or self.used[s] < protect_from)]
            if not ok:
                return None
            loads.append((e, min(ok, key=lambda s: (self.used[s], s))))
        self.requests += 1
        for e, s in loads:
            if self.owner[s] is not None:
                self.evictions += 1
            self.owner[s] = e
        for e in need:
            self.used[self.slot_of(e)] = self.requests
        return hits, loads

    def pin(self, experts):
        for e in experts:
            if self.slot_of(e) >= 0:
                self.pinned.add(self.slot_of(e))

    def unpin_all(self):
        self.pinned.clear()

    def table(self):
        return [self.slot_of(e) for e in range(self.E)]
