"""CPU oracle for the paged decode step.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The product library
(``paged_kv_cache_276_amd``) never imports it, and it never imports the product
library: the two share nothing but the seeded inputs from ``workloads``.

``oracle.c`` is plain C in fp64 (built with gcc, OpenMP over output rows);
``arith.py`` holds the block and byte arithmetic; ``blocks.py`` the block
bookkeeping (allocation, sharing, copy-on-write) and the block copy.  Each function cites the
passage of the pages it follows.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass
from typing import Optional, Sequence, Tuple

import numpy as np

from . import arith  # noqa: F401
from . import blocks  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "oracle.c")
LIBRARY = os.path.join(_HERE, "liboracle.so")

ERRORS = {
    -1: "bad arguments",
    -2: "slot outside the pool",
    -3: "block table entry outside the pool",
    -4: "context length outside the table",
    -5: "out of host memory",
}


def build(source: str = SOURCE, output: str = LIBRARY) -> str:
    """Compile the oracle with gcc (plain -O2, IEEE arithmetic, OpenMP)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-Wall",
           "-o", output + ".tmp", source, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(output + ".tmp", output)
    return output


def _ptr(a) -> ctypes.c_void_p:
    if a is None:
        return ctypes.c_void_p(0)
    return ctypes.c_void_p(a.ctypes.data)


def _bits(t) -> np.ndarray:
    """Raw element bits of a CPU tensor or array as a contiguous numpy array."""
    try:
        import torch
    except ImportError:  # pragma: no cover
        torch = None
    if torch is not None and isinstance(t, torch.Tensor):
        t = t.detach().contiguous()
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).numpy()
        if t.dtype == torch.float32:
            return t.view(torch.int32).numpy()
        raise TypeError(f"unsupported dtype {t.dtype}")
    a = np.ascontiguousarray(t)
    if a.dtype == np.float32:
        return a.view(np.int32)
    if a.dtype in (np.int16, np.uint16, np.int32, np.uint32):
        return a
    raise TypeError(f"unsupported array dtype {a.dtype}")


class Oracle:
    """ctypes front end of one compiled ``oracle.c``."""

    def __init__(self, lib_path: str = LIBRARY):
        if not os.path.exists(lib_path):
            build(output=lib_path)
        self.lib = ctypes.CDLL(lib_path)
        i32, vp = ctypes.c_int32, ctypes.c_void_p
        self.lib.oracle_kv_write.restype = ctypes.c_int
        self.lib.oracle_kv_write.argtypes = [vp, vp, vp, i32, vp, vp, i32, i32, i32, i32, i32]
        self.lib.oracle_num_threads.restype = ctypes.c_int
        self.lib.oracle_num_threads.argtypes = []
        self.lib.oracle_attn_multi.restype = ctypes.c_int
        self.lib.oracle_attn_multi.argtypes = [
            vp, vp, vp, i32, vp, i32, vp, vp, i32, i32, i32, i32, i32, i32, ctypes.c_float, vp]
        self.lib.oracle_attn_decode.restype = ctypes.c_int
        self.lib.oracle_attn_decode.argtypes = [
            vp, vp, vp, i32, vp, i32, vp, i32, i32, i32, i32, i32, i32, ctypes.c_float, vp, i32, vp]

    def attn_multi(self, q, k_cache, v_cache, block_tables, context_lens, cu_q, scale: float,
                   num_kv_heads: Optional[int] = None) -> np.ndarray:
        """fp64 causal attention of several new tokens per sequence.  Returns [total_q][Hq][D]."""
        qb, kb, vb = _bits(q), _bits(k_cache), _bits(v_cache)
        tq, hq, d = qb.shape
        nb, hkv, b, d2 = kb.shape
        assert d2 == d and vb.shape == kb.shape and qb.dtype.itemsize == kb.dtype.itemsize
        if num_kv_heads is not None:
            assert num_kv_heads == hkv
        bt = np.ascontiguousarray(block_tables, dtype=np.int32)
        cl = np.ascontiguousarray(context_lens, dtype=np.int32)
        cu = np.ascontiguousarray(cu_q, dtype=np.int32)
        s = bt.shape[0]
        assert cl.shape == (s,) and cu.shape == (s + 1,) and int(cu[-1]) == tq
        out = np.zeros((tq, hq, d), dtype=np.float64)
        self._check(self.lib.oracle_attn_multi(
            _ptr(qb), _ptr(kb), _ptr(vb), qb.dtype.itemsize, _ptr(bt), bt.shape[1], _ptr(cl), _ptr(cu), s,
            hq, hkv, nb, b, d, ctypes.c_float(scale), _ptr(out)))
        return out

    def num_threads(self) -> int:
        return int(self.lib.oracle_num_threads())

    @staticmethod
    def _check(rc: int) -> None:
        if rc != 0:
            raise RuntimeError(f"oracle error {rc}: {ERRORS.get(rc, 'unknown')}")

    def kv_write(self, k_new, v_new, slot_mapping, k_cache_bits: np.ndarray,
                 v_cache_bits: np.ndarray, block_size: int) -> None:
        """Scatter new K/V rows into the pools given as raw-bit arrays (in place)."""
        kn, vn = _bits(k_new), _bits(v_new)
        sm = np.ascontiguousarray(slot_mapping, dtype=np.int32)
        assert k_cache_bits.flags.c_contiguous and v_cache_bits.flags.c_contiguous
        nb, hkv, b, d = k_cache_bits.shape
        assert b == block_size and kn.shape[1:] == (hkv, d) and kn.shape[0] == sm.shape[0]
        eb = k_cache_bits.dtype.itemsize
        self._check(self.lib.oracle_kv_write(
            _ptr(kn), _ptr(vn), _ptr(sm), int(sm.shape[0]), _ptr(k_cache_bits), _ptr(v_cache_bits),
            nb, hkv, b, d, eb))

    def attn_decode(self, q, k_cache, v_cache, block_tables, context_lens, scale: float,
                    num_kv_heads: Optional[int] = None,
                    rows: Optional[Sequence[Tuple[int, int]]] = None) -> np.ndarray:
        """fp64 decode attention.  Returns [S][Hq][D] (or [len(rows)][D] for a row sample)."""
        qb, kb, vb = _bits(q), _bits(k_cache), _bits(v_cache)
        s, hq, d = qb.shape
        nb, hkv, b, d2 = kb.shape
        assert d2 == d and vb.shape == kb.shape and qb.dtype.itemsize == kb.dtype.itemsize
        if num_kv_heads is not None:
            assert num_kv_heads == hkv
        bt = np.ascontiguousarray(block_tables, dtype=np.int32)
        cl = np.ascontiguousarray(context_lens, dtype=np.int32)
        assert bt.shape[0] == s and cl.shape == (s,)
        if rows is None:
            out = np.zeros((s, hq, d), dtype=np.float64)
            rr, nr = None, 0
        else:
            rr = np.ascontiguousarray(np.asarray(rows, dtype=np.int32).reshape(-1, 2))
            nr = rr.shape[0]
            out = np.zeros((nr, d), dtype=np.float64)
        self._check(self.lib.oracle_attn_decode(
            _ptr(qb), _ptr(kb), _ptr(vb), qb.dtype.itemsize, _ptr(bt), bt.shape[1], _ptr(cl), s,
            hq, hkv, nb, b, d, ctypes.c_float(scale), _ptr(rr), nr, _ptr(out)))
        return out


@dataclass
class StepResult:
    k_cache_bits: np.ndarray  # post-write pool, raw bits
    v_cache_bits: np.ndarray
    out: Optional[np.ndarray]  # fp64 attention output ([S][Hq][D] or sampled rows)


_default: Optional[Oracle] = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def decode_step(w, rows=None, attention: bool = True, oracle: Optional[Oracle] = None) -> StepResult:
    """The whole step on a workload: write the new tokens, then attend over the written pool."""
    o = oracle or default()
    kc = _bits(w.k_cache).copy()
    vc = _bits(w.v_cache).copy()
    o.kv_write(w.k_new, w.v_new, w.slot_mapping, kc, vc, w.block_size)
    out = None
    if attention:
        out = o.attn_decode(w.q, kc, vc, w.block_tables, w.context_lens, w.scale,
                            num_kv_heads=w.num_kv_heads, rows=rows)
    return StepResult(kc, vc, out)
