"""Brute-force list LRU: a second, independent formulation of the swap-in step.

It keeps no stamps for ranking. The hot buffer's slots sit in one Python list,
least recently used first; a step takes its victims from the front of that list
among the slots not hit, and moves every slot used in the step (hits and newly
filled ones) to the back in slot order. Unused slots start in slot order, so
empty slots are always taken first, lowest index first. Misses are paired with
victims in ascending token-id order. This is the LRU of the pages' swap-in
kernel ("HiSparse: Turbocharging Sparse Attention with Hierarchical Memory",
section 2) with the tie-breaks spelled out, written as list surgery rather than
as a sort, so a mistake in the oracle's sort keys or stamp handling shows up as
a disagreement.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence, Tuple

BAD_ID, DUP_ID = 1, 2


class ListLRU:
    """fifo=True: the same list, but a hit does not move its slot (FIFO replacement): only newly filled slots
    go to the back, and a slot's last-use step is the step it was filled."""

    def __init__(self, B: int, H: int, T: int = 0, fifo: bool = False):
        self.B, self.H, self.T, self.fifo = B, H, T, fifo
        self.reset()

    def reset(self) -> None:
        self.order: List[int] = list(range(self.B))   # least recently used first
        self.holder: Dict[int, int] = {}              # slot -> token
        self.where: Dict[int, int] = {}               # token -> slot
        self.last_used: Dict[int, int] = {}           # slot -> step it was last used
        self.t = 0

    def step(self, ids: Sequence[int], tail0: Optional[int] = None) -> Tuple[List[int], int, int]:
        out = [-1] * len(ids)
        status = 0
        seen = set()
        used_slots = set()
        missed: List[Tuple[int, int]] = []
        for i, x in enumerate(ids):
            if x == -1:
                continue
            if not (0 <= x < self.H):
                status |= BAD_ID
                continue
            in_tail = tail0 is not None and x >= tail0
            if in_tail and x - tail0 >= self.T:
                status |= BAD_ID
                continue
            if x in seen:
                status |= DUP_ID
                continue
            seen.add(x)
            if in_tail:
                out[i] = self.B + x % self.T
                continue
            if x in self.where:
                out[i] = self.where[x]
                used_slots.add(self.where[x])
            else:
                missed.append((x, i))
        missed.sort()
        free_order = [s for s in self.order if s not in used_slots]
        if len(missed) > len(free_order):
            raise RuntimeError("more misses than free slots")
        victims = free_order[:len(missed)]
        for (x, i), v in zip(missed, victims):
            old = self.holder.get(v)
            if old is not None:
                del self.where[old]
            self.holder[v] = x
            self.where[x] = v
            out[i] = v
        if self.fifo:
            moved = set(victims)
            self.order = [s for s in self.order if s not in moved] + sorted(moved)
        else:
            moved = used_slots | set(victims)
            self.order = free_order[len(missed):] + sorted(moved)
        for s in moved:
            self.last_used[s] = self.t
        self.t += 1
        return out, len(missed), status

    # views comparable with the oracle's arrays
    def slot_tok(self) -> List[int]:
        return [self.holder.get(s, -1) for s in range(self.B)]

    def stamps(self) -> List[int]:
        return [self.last_used.get(s, -1) for s in range(self.B)]

    def page(self) -> List[int]:
        p = [-1] * self.H
        for x, s in self.where.items():
            p[x] = s
        return p
