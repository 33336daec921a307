"""Host block manager of the paged KV cache (binding of ``include/pagedkv_blocks.h``).

The manager lives in libpagedkv.so (C++); this class only marshals arguments.
It hands out blocks from a pool of ``num_blocks`` blocks of ``block_size``
tokens as sequences grow, shares blocks between forked sequences with
reference counts, and reports which shared, partly filled blocks must be
copied (``paged_block_copy``) before a step's tokens are written.
"""

from __future__ import annotations

import ctypes
from typing import List, Sequence, Tuple

import numpy as np

from . import _lib


class BlockManager:
    def __init__(self, num_blocks: int, block_size: int):
        self._L = _lib.lib()
        h = ctypes.c_void_p()
        _lib.check(self._L.pkv_bm_create(int(num_blocks), int(block_size), ctypes.byref(h)), "pkv_bm_create")
        self._h = h
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)

    def close(self) -> None:
        if self._h:
            self._L.pkv_bm_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def num_free(self) -> int:
        return int(self._L.pkv_bm_num_free(self._h))

    def refcount(self, block: int) -> int:
        return int(self._L.pkv_bm_refcount(self._h, int(block)))

    def seq_len(self, seq_id: int) -> int:
        return int(self._L.pkv_bm_seq_len(self._h, int(seq_id)))

    def add(self, seq_id: int, num_tokens: int) -> None:
        _lib.check(self._L.pkv_bm_add(self._h, int(seq_id), int(num_tokens)), "pkv_bm_add")

    def fork(self, parent: int, child: int) -> None:
        _lib.check(self._L.pkv_bm_fork(self._h, int(parent), int(child)), "pkv_bm_fork")

    def free(self, seq_id: int) -> None:
        _lib.check(self._L.pkv_bm_free(self._h, int(seq_id)), "pkv_bm_free")

    def append(self, seq_ids: Sequence[int]) -> Tuple[np.ndarray, np.ndarray]:
        """One token for each sequence: (slot_mapping int32 [n], copies int32 [c][2])."""
        ids = np.ascontiguousarray(np.asarray(seq_ids, dtype=np.int64))
        n = ids.size
        slots = np.empty(n, dtype=np.int32)
        copies = np.empty((max(n, 1), 2), dtype=np.int32)
        nc = ctypes.c_int32(0)
        st = self._L.pkv_bm_append(self._h, ids.ctypes.data_as(ctypes.c_void_p), n,
                                   slots.ctypes.data_as(ctypes.c_void_p), copies.ctypes.data_as(ctypes.c_void_p),
                                   copies.shape[0], ctypes.byref(nc))
        _lib.check(st, "pkv_bm_append")
        return slots, copies[: nc.value].copy()

    def slots(self, seq_id: int, first: int, count: int) -> np.ndarray:
        out = np.empty(count, dtype=np.int32)
        st = self._L.pkv_bm_slots(self._h, int(seq_id), int(first), int(count), out.ctypes.data_as(ctypes.c_void_p))
        _lib.check(st, "pkv_bm_slots")
        return out

    def block_tables(self, seq_ids: Sequence[int], max_blocks_per_seq: int) -> Tuple[np.ndarray, np.ndarray]:
        ids = np.ascontiguousarray(np.asarray(seq_ids, dtype=np.int64))
        n = ids.size
        tables = np.empty((n, max_blocks_per_seq), dtype=np.int32)
        lens = np.empty(n, dtype=np.int32)
        st = self._L.pkv_bm_block_tables(self._h, ids.ctypes.data_as(ctypes.c_void_p), n, int(max_blocks_per_seq),
                                         tables.ctypes.data_as(ctypes.c_void_p), lens.ctypes.data_as(ctypes.c_void_p))
        _lib.check(st, "pkv_bm_block_tables")
        return tables, lens
