"""Host-side residency of adapters in a fixed number of GPU slots.

This is control plane and stays on the host.  It decides which adapter goes to
which slot; `lora_slot_load` does the upload.  The rules come from "Multi-LoRA
adapter cache in production" (oh-bug.com):

- section "GPU, CPU and disk form the adapter storage hierarchy":
  - vLLM's worker manager loads a new adapter when space is short, then drops
    the least recently used one;
  - a hit refreshes the entry's recency ("touch");
  - an adapter that in-flight work is using is never evicted;
- the parameter table: max_loras bounds the adapters one batch uses;
- the metrics section: the thrash ratio is reloads shortly after an eviction,
  divided by evictions;
- section "why pure LRU fails in multi-tenant settings": a burst of rarely used
  adapters must not push the hot ones out.  Two of its platform rules are here:
  a warm set of pinned adapters that are never evicted while resident, and a
  minimum residency (in steps) before a newly loaded adapter may be evicted.

One step is one batch.  Every adapter it uses must be resident before the batch
runs:

1. adapters already resident are hits and are touched;
2. the others are misses, loaded in order of first appearance;
3. a miss takes an empty slot (lowest index first), or else evicts the least
   recently used slot that the step itself does not use and that holds no
   pinned adapter.  Among those, slots whose adapter is younger than
   `min_residency` steps are taken only when no older one is left, and slots
   passed as `avoid` (read by batches still in flight, so a load into them has
   to wait for those batches) only when nothing else is.

A step with more distinct adapters than slots, or one that would have to evict
a pinned adapter, is refused.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Tuple

import numpy as np


@dataclass
class LruStats:
    steps: int = 0
    hits: int = 0
    misses: int = 0
    evictions: int = 0
    reloads_after_eviction: int = 0      # misses for an adapter evicted <= window steps before
    load_log: List[Tuple[int, int, int]] = field(default_factory=list)   # (step, slot, adapter)

    @property
    def thrash_ratio(self) -> float:
        return self.reloads_after_eviction / self.evictions if self.evictions else 0.0


class SlotLRU:
    def __init__(self, n_slots: int, thrash_window: int = 10, min_residency: int = 0):
        if n_slots < 1:
            raise ValueError("n_slots must be >= 1")
        if min_residency < 0:
            raise ValueError("min_residency must be >= 0")
        self.n_slots = n_slots
        self.thrash_window = thrash_window
        self.min_residency = min_residency
        self.pinned: set = set()
        self.loaded_at = [-1] * n_slots
        self.adapter_in: List[Optional[int]] = [None] * n_slots
        self.slot_of: Dict[int, int] = {}
        self.last_use = [-1] * n_slots
        self.tick = 0
        self.step_no = 0
        self.evicted_at: Dict[int, int] = {}
        self.stats = LruStats()

    def resident(self) -> Dict[int, int]:
        """adapter id -> slot for every resident adapter."""
        return dict(self.slot_of)

    def pin(self, adapter_ids) -> None:
        """Add adapters to the warm set: once resident they are never evicted.
        At least one slot must stay free of pinned adapters."""
        new = self.pinned | {int(a) for a in adapter_ids}
        if len(new) >= self.n_slots:
            raise ValueError(f"{len(new)} pinned adapters leave no evictable slot of {self.n_slots}")
        self.pinned = new

    def unpin(self, adapter_ids) -> None:
        self.pinned -= {int(a) for a in adapter_ids}

    def _touch(self, slot: int) -> None:
        self.tick += 1
        self.last_use[slot] = self.tick

    def plan_step(self, adapter_ids: np.ndarray, avoid=()) -> Tuple[np.ndarray, List[Tuple[int, int]]]:
        """Map one batch's per-token adapter ids (-1 = base only) to slots.

        Returns (slot per token, int32 with -1 kept) and the loads to issue
        before the batch, as (slot, adapter id) in order of first appearance.
        `avoid`: slots to evict only as a last resort.
        """
        avoid = set(avoid)
        ids = np.asarray(adapter_ids)
        act = ids >= 0
        uniq, first = np.unique(ids[act], return_index=True)
        distinct = [int(a) for a in uniq[np.argsort(first, kind="stable")]]
        if len(distinct) > self.n_slots:
            raise ValueError(f"step uses {len(distinct)} adapters but only {self.n_slots} slots exist")
        protected = {self.slot_of[a] for a in distinct if a in self.slot_of}
        n_miss = sum(1 for a in distinct if a not in self.slot_of)
        usable = sum(1 for s in range(self.n_slots)
                     if s not in protected and self.adapter_in[s] not in self.pinned)
        if n_miss > usable:
            raise ValueError(f"step needs {n_miss} slots but only {usable} hold no pinned "
                             "adapter and no adapter of the step")
        loads: List[Tuple[int, int]] = []
        for a in distinct:
            if a in self.slot_of:
                self.stats.hits += 1
                self._touch(self.slot_of[a])
                continue
            self.stats.misses += 1
            if a in self.evicted_at and self.step_no - self.evicted_at[a] <= self.thrash_window:
                self.stats.reloads_after_eviction += 1
            empty = [s for s in range(self.n_slots) if self.adapter_in[s] is None and s not in protected]
            if empty:
                slot = empty[0]
            else:
                cands = [s for s in range(self.n_slots)
                         if s not in protected and self.adapter_in[s] not in self.pinned]
                young = {s for s in cands if self.step_no - self.loaded_at[s] < self.min_residency}
                free = [s for s in cands if s not in avoid and s not in young]
                free = free or [s for s in cands if s not in avoid] or cands
                slot = min(free, key=lambda s: self.last_use[s])
                old = self.adapter_in[slot]
                del self.slot_of[old]
                self.evicted_at[old] = self.step_no
                self.stats.evictions += 1
            self.adapter_in[slot] = a
            self.slot_of[a] = slot
            self.loaded_at[slot] = self.step_no
            protected.add(slot)
            self._touch(slot)
            loads.append((slot, a))
            self.stats.load_log.append((self.step_no, slot, a))
        slots = np.full(ids.shape, -1, dtype=np.int32)
        if act.any():
            lut = {a: self.slot_of[a] for a in distinct}
            slots[act] = np.vectorize(lut.__getitem__, otypes=[np.int32])(ids[act])
        self.step_no += 1
        self.stats.steps += 1
        return slots, loads
