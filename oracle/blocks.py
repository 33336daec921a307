"""Plain reference of the paged-cache block bookkeeping and block copy.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  Written from the pages,
not from the library: a list of physical blocks per sequence, a reference
count per block, and copy-on-write of a shared block before a write into it.

* A request grows by taking the free blocks it needs when it needs them; the
  logical order lives in a per-sequence table of physical block ids: page
  "x321.org/?p=939", section "PagedAttention borrows an operating-system trick";
  page "chenhuiyu.github.io/blog/llm-infra-vllm-en", section "Logical
  continuity, physical flexibility".
* Blocks holding a common prefix are named by several tables and counted; a
  shared block is copied before one of its holders writes into it: page
  "praveentn.live/architecture/quiz/pagedattention-kv-cache-constraint",
  section "What the change bought".

Readings where the pages are silent: a new block is the lowest free id; the
holders of one partly filled shared block that append in one step are served
in the order given, the last remaining holder keeps the block; a failing step
changes nothing.
"""

from __future__ import annotations

from typing import Dict, List, Sequence, Tuple

import numpy as np


class NoBlocks(Exception):
    pass


class RefBlockManager:
    def __init__(self, num_blocks: int, block_size: int):
        self.B = block_size
        self.ref = [0] * num_blocks
        self.tables: Dict[int, List[int]] = {}
        self.lens: Dict[int, int] = {}

    def free_ids(self) -> List[int]:
        return [b for b, r in enumerate(self.ref) if r == 0]

    def _take(self) -> int:
        free = self.free_ids()
        if not free:
            raise NoBlocks()
        self.ref[free[0]] = 1
        return free[0]

    def add(self, sid: int, n: int) -> None:
        assert sid not in self.tables
        need = -(-n // self.B)
        if need > len(self.free_ids()):
            raise NoBlocks()
        self.tables[sid] = [self._take() for _ in range(need)]
        self.lens[sid] = n

    def fork(self, parent: int, child: int) -> None:
        assert parent in self.tables and child not in self.tables
        self.tables[child] = list(self.tables[parent])
        self.lens[child] = self.lens[parent]
        for b in self.tables[child]:
            self.ref[b] += 1

    def free(self, sid: int) -> None:
        for b in self.tables.pop(sid):
            self.ref[b] -= 1
        del self.lens[sid]

    def append(self, sids: Sequence[int]) -> Tuple[List[int], List[Tuple[int, int]]]:
        """One new token per sequence: the slot of each token and the block copies to make first."""
        saved = ([*self.ref], {k: list(v) for k, v in self.tables.items()}, dict(self.lens))
        slots, copies = [], []
        try:
            for sid in sids:
                n = self.lens[sid]
                table = self.tables[sid]
                pos = n % self.B
                if pos == 0:                        # every allocated slot is used: a new block
                    table.append(self._take())
                elif self.ref[table[-1]] > 1:       # last block shared: copy it, then write the copy
                    fresh = self._take()
                    copies.append((table[-1], fresh))
                    self.ref[table[-1]] -= 1
                    table[-1] = fresh
                slots.append(table[-1] * self.B + pos)
                self.lens[sid] = n + 1
        except NoBlocks:
            self.ref, self.tables, self.lens = saved
            raise
        return slots, copies

    def block_table(self, sid: int, max_blocks: int) -> List[int]:
        t = self.tables[sid]
        return t + [-1] * (max_blocks - len(t))


def copy_blocks(k_cache: np.ndarray, v_cache: np.ndarray, pairs: Sequence[Tuple[int, int]]) -> None:
    """Block dst becomes a bit copy of block src in both pools (in place, in pair order)."""
    for src, dst in pairs:
        k_cache[dst] = k_cache[src]
        v_cache[dst] = v_cache[src]
