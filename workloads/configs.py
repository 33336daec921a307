"""The five synthetic decode workloads and a builder for custom test cases.

Structure (lengths, block placement) is drawn from ``numpy`` PCG64 seeded with
the workload's seed; values from a ``torch.Generator('cpu')`` seeded with the
same number: standard normal in fp32, cast to bf16 (round to nearest even) for
the bf16 workloads.

Layout of what is returned (all contiguous, row-major):

* ``k_cache``, ``v_cache``: ``[num_blocks][num_kv_heads][block_size][head_dim]``
  -- the cache *before* the step's write.  It holds ``ctx - 1`` tokens of every
  sequence; the step writes token ``ctx - 1``.
* ``block_tables``: int32 ``[num_seqs][max_blocks_per_seq]``, logical block
  ``b`` of sequence ``i`` at ``block_tables[i][b]``, unused entries ``-1``.
* ``context_lens``: int32 ``[num_seqs]``, tokens of each sequence *including*
  the one written this step.
* ``slot_mapping``: int32 ``[num_tokens]``, ``physical_block * block_size +
  offset`` of each new token, ``-1`` = skip.
* ``q``: ``[num_seqs][num_q_heads][head_dim]``; ``k_new``, ``v_new``:
  ``[num_tokens][num_kv_heads][head_dim]``.

Poison: with ``poison=True`` every free block and every slot at or past
position ``ctx - 1`` of a sequence's last block holds a quiet NaN, so a kernel
that reads outside the valid tokens, or misses the write, yields NaN.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np
import torch

CONFIG_NAMES = ("tiny", "llama8b_b64", "hc_b256", "long32k", "shared_prefix")

_SEEDS = {name: i for i, name in enumerate(CONFIG_NAMES)}

# Quiet NaNs with a recognisable payload.
_POISON_BITS = {torch.float32: 0x7FC0BEEF, torch.bfloat16: 0x7FC5}


def poison_value_bits(dtype: torch.dtype) -> int:
    return _POISON_BITS[dtype]


@dataclass
class Workload:
    name: str
    seed: int
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    dtype: torch.dtype
    num_blocks: int
    max_blocks_per_seq: int
    context_lens: np.ndarray
    block_tables: np.ndarray
    slot_mapping: np.ndarray
    q: torch.Tensor
    k_new: torch.Tensor
    v_new: torch.Tensor
    k_cache: torch.Tensor
    v_cache: torch.Tensor
    scale: float
    meta: Dict[str, object] = field(default_factory=dict)

    @property
    def num_tokens(self) -> int:
        return int(self.slot_mapping.shape[0])

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == torch.float32 else 2


def _int_bits_view(t: torch.Tensor) -> torch.Tensor:
    return t.view(torch.int32 if t.dtype == torch.float32 else torch.int16)


def _fill_normal(t: torch.Tensor, gen: torch.Generator, chunk: int = 1 << 25) -> None:
    flat = t.view(-1)
    n = flat.numel()
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        flat[s:e] = torch.randn(e - s, generator=gen, dtype=torch.float32).to(t.dtype)


def _poison(t: torch.Tensor, dtype: torch.dtype) -> None:
    bits = poison_value_bits(dtype)
    if dtype == torch.bfloat16 and bits >= 0x8000:
        bits -= 0x10000
    _int_bits_view(t).fill_(bits)


def _build(
    name: str,
    seed: int,
    lengths: Sequence[int],
    num_q_heads: int,
    num_kv_heads: int,
    head_dim: int,
    block_size: int,
    dtype: torch.dtype,
    max_blocks_per_seq: Optional[int] = None,
    prefix_groups: Optional[List[Tuple[int, List[int]]]] = None,
    pool_fill: float = 1.0,
    pool_blocks: Optional[int] = None,
    poison: bool = True,
    rng: Optional[np.random.Generator] = None,
    meta: Optional[Dict[str, object]] = None,
    values: bool = True,
) -> Workload:
    if rng is None:
        rng = np.random.Generator(np.random.PCG64(seed))
    S = len(lengths)
    B = block_size
    lengths = np.asarray(lengths, dtype=np.int64)
    nblk = [(int(n) + B - 1) // B for n in lengths]
    if max_blocks_per_seq is None:
        max_blocks_per_seq = max([1] + nblk)
    assert max(nblk + [0]) <= max_blocks_per_seq

    # Unique logical blocks: shared prefix blocks first, then private ones.
    owner_prefix = [None] * S  # (first unique id, count) of the shared prefix
    unique = 0
    if prefix_groups:
        for prefix_tokens, members in prefix_groups:
            assert prefix_tokens % B == 0, "shared prefixes are whole blocks"
            cnt = prefix_tokens // B
            for i in members:
                assert owner_prefix[i] is None
                assert lengths[i] > prefix_tokens, "the new token lands past the prefix"
                owner_prefix[i] = (unique, cnt)
            unique += cnt
    logical = []  # per sequence: list of unique ids
    for i in range(S):
        ids = []
        if owner_prefix[i] is not None:
            first, cnt = owner_prefix[i]
            ids.extend(range(first, first + cnt))
        while len(ids) < nblk[i]:
            ids.append(unique)
            unique += 1
        logical.append(ids)
    used = unique
    if pool_blocks is None:
        pool_blocks = max(1, int(math.ceil(used / pool_fill)))
    assert pool_blocks >= used
    phys = rng.permutation(pool_blocks)[:used].astype(np.int64)

    tables = np.full((S, max_blocks_per_seq), -1, dtype=np.int32)
    for i in range(S):
        if logical[i]:
            tables[i, : len(logical[i])] = phys[np.asarray(logical[i])]

    slots = np.full((S,), -1, dtype=np.int32)
    for i in range(S):
        n = int(lengths[i])
        if n > 0:
            pos = n - 1
            slots[i] = int(tables[i, pos // B]) * B + pos % B

    gen = torch.Generator().manual_seed(seed)
    D, Hkv, Hq = head_dim, num_kv_heads, num_q_heads
    if values:
        q = torch.empty((S, Hq, D), dtype=dtype)
        k_new = torch.empty((S, Hkv, D), dtype=dtype)
        v_new = torch.empty((S, Hkv, D), dtype=dtype)
        k_cache = torch.empty((pool_blocks, Hkv, B, D), dtype=dtype)
        v_cache = torch.empty((pool_blocks, Hkv, B, D), dtype=dtype)
        for t in (q, k_new, v_new, k_cache, v_cache):
            _fill_normal(t, gen)
    else:  # structure only: lengths, tables and slots, no values
        q = k_new = v_new = k_cache = v_cache = None

    if poison and values:
        free = np.ones(pool_blocks, dtype=bool)
        free[phys] = False
        free_ids = torch.from_numpy(np.nonzero(free)[0])
        if free_ids.numel():
            for c in (k_cache, v_cache):
                tmp = c[free_ids]  # advanced indexing copies; poison the copy and put it back
                _poison(tmp, dtype)
                c[free_ids] = tmp
        for i in range(S):
            n = int(lengths[i])
            if n == 0:
                continue
            last = int(tables[i, nblk[i] - 1])
            first_bad = (n - 1) - (nblk[i] - 1) * B
            for c in (k_cache, v_cache):
                _poison(c[last, :, first_bad:, :], dtype)

    scale = float(np.float32(1.0 / math.sqrt(D)))
    m = {"used_blocks": used, "pool_fill": used / pool_blocks}
    if prefix_groups:
        m["prefix_groups"] = [(int(p), [int(i) for i in members]) for p, members in prefix_groups]
    if meta:
        m.update(meta)
    return Workload(
        name=name,
        seed=seed,
        num_seqs=S,
        num_q_heads=Hq,
        num_kv_heads=Hkv,
        head_dim=D,
        block_size=B,
        dtype=dtype,
        num_blocks=pool_blocks,
        max_blocks_per_seq=max_blocks_per_seq,
        context_lens=lengths.astype(np.int32),
        block_tables=tables,
        slot_mapping=slots,
        q=q,
        k_new=k_new,
        v_new=v_new,
        k_cache=k_cache,
        v_cache=v_cache,
        scale=scale,
        meta=m,
    )


def make_config(name: str, poison: bool = True, num_seqs: Optional[int] = None,
                values: bool = True, block_size: Optional[int] = None,
                heads: Optional[Tuple[int, int, int]] = None) -> Workload:
    """One of the five named workloads.

    ``num_seqs`` trims the batch (used only to draw a bounded sample of a
    workload; the full configuration is ``num_seqs=None``).  The lengths of the
    first ``num_seqs`` sequences are the same as in the full draw.
    ``block_size`` redraws the same lengths into blocks of that many tokens (the
    block-size sweep); the table width is scaled to keep the same token
    capacity, and shared prefixes must stay whole blocks.
    ``heads`` = (query heads, KV heads, head dim) replaces the workload's head
    layout over the same lengths and tables (other shapes of the same batch).
    """
    seed = _SEEDS[name]
    rng = np.random.Generator(np.random.PCG64(seed))
    bf16 = torch.bfloat16
    if name == "tiny":
        lengths = [17, 33, 35, 64]
        kw = dict(num_q_heads=2, num_kv_heads=1, head_dim=64, block_size=16,
                  dtype=torch.float32, max_blocks_per_seq=4, pool_blocks=32)
        meta = {}
    elif name == "llama8b_b64":
        lengths = rng.integers(128, 4096, size=64, endpoint=True).tolist()
        kw = dict(num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                  dtype=bf16, max_blocks_per_seq=256)
        meta = {"lengths": "uniform [128,4096]"}
    elif name == "hc_b256":
        sigma = 1.0
        raw = np.exp(rng.normal(math.log(1024.0), sigma, size=256))
        lengths = np.clip(np.rint(raw), 1, 8192).astype(np.int64).tolist()
        kw = dict(num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                  dtype=bf16, max_blocks_per_seq=512, pool_fill=0.9)
        meta = {"lengths": "lognormal median 1024 sigma 1.0, clamp [1,8192]", "sigma": sigma}
    elif name == "long32k":
        lengths = [32768] * 8
        kw = dict(num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                  dtype=bf16, max_blocks_per_seq=2048)
        meta = {"lengths": "8 x 32768"}
    elif name == "shared_prefix":
        prompts, samples, prefix, B = 32, 8, 2048, 32
        suffix = rng.integers(1, 512, size=prompts * samples, endpoint=True)
        lengths = (prefix + suffix).tolist()
        groups = [(prefix, list(range(p * samples, (p + 1) * samples))) for p in range(prompts)]
        kw = dict(num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=B,
                  dtype=bf16, max_blocks_per_seq=(prefix + 512) // B, prefix_groups=groups)
        meta = {"lengths": "2048 shared + uniform [1,512]", "prompts": prompts, "samples": samples}
    else:
        raise KeyError(name)
    if heads is not None:
        kw["num_q_heads"], kw["num_kv_heads"], kw["head_dim"] = (int(x) for x in heads)
        meta = dict(meta, heads=f"{kw['num_q_heads']}/{kw['num_kv_heads']}/{kw['head_dim']}")
    if block_size is not None and block_size != kw["block_size"]:
        cap = kw["max_blocks_per_seq"] * kw["block_size"]
        kw["block_size"] = block_size
        kw["max_blocks_per_seq"] = -(-cap // block_size)
        kw.pop("pool_blocks", None)
        meta = dict(meta, block_size_sweep=block_size)
    if num_seqs is not None and num_seqs < len(lengths):
        lengths = lengths[:num_seqs]
        if "prefix_groups" in kw:
            kw["prefix_groups"] = [(p, [i for i in m if i < num_seqs]) for p, m in kw["prefix_groups"]]
            kw["prefix_groups"] = [g for g in kw["prefix_groups"] if g[1]]
        kw.pop("pool_blocks", None)
    return _build(name, seed, lengths, poison=poison, rng=rng, meta=meta, values=values, **kw)


def make_custom(
    lengths: Sequence[int],
    num_q_heads: int = 4,
    num_kv_heads: int = 1,
    head_dim: int = 128,
    block_size: int = 16,
    dtype: torch.dtype = torch.bfloat16,
    seed: int = 1234,
    max_blocks_per_seq: Optional[int] = None,
    prefix_groups: Optional[List[Tuple[int, List[int]]]] = None,
    pool_fill: float = 1.0,
    pool_blocks: Optional[int] = None,
    poison: bool = True,
    values: bool = True,
) -> Workload:
    """A test workload with explicit lengths and shapes (same recipe as the named ones)."""
    return _build(
        "custom", seed, list(lengths), num_q_heads, num_kv_heads, head_dim, block_size, dtype,
        max_blocks_per_seq=max_blocks_per_seq, prefix_groups=prefix_groups,
        pool_fill=pool_fill, pool_blocks=pool_blocks, poison=poison, values=values,
    )


@dataclass
class MultiWorkload:
    """Several new tokens per sequence: the cache holds ctx - q_len tokens of each
    sequence before the step; the step writes the q_len new tokens (slots in
    ``slot_mapping``, rows ``k_new``/``v_new`` in sequence order) and attends from
    each of them.  ``cu_q`` [S + 1] are the offsets of each sequence's rows in
    ``q``/``k_new``/``v_new``/``slot_mapping``."""

    base: Workload
    q_lens: np.ndarray
    cu_q: np.ndarray
    q: torch.Tensor
    k_new: torch.Tensor
    v_new: torch.Tensor
    slot_mapping: np.ndarray

    def __getattr__(self, name):  # everything else (pools, tables, shapes) comes from the base workload
        return getattr(self.base, name)


def make_multi(lengths: Sequence[int], q_lens: Sequence[int], num_q_heads: int = 8, num_kv_heads: int = 2,
               head_dim: int = 128, block_size: int = 16, dtype: torch.dtype = torch.bfloat16, seed: int = 0,
               max_blocks_per_seq: Optional[int] = None, pool_fill: float = 1.0, poison: bool = True,
               name: str = "custom_multi", meta: Optional[Dict[str, object]] = None) -> MultiWorkload:
    assert len(lengths) == len(q_lens) and all(0 < ql <= n for n, ql in zip(lengths, q_lens))
    base = _build(name, seed, lengths, num_q_heads, num_kv_heads, head_dim, block_size, dtype,
                  max_blocks_per_seq=max_blocks_per_seq, pool_fill=pool_fill, poison=False, meta=meta)
    B = block_size
    S = len(lengths)
    q_lens = np.asarray(q_lens, dtype=np.int32)
    cu = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    slots = np.empty(int(cu[-1]), dtype=np.int32)
    for i, n in enumerate(lengths):
        for j in range(int(q_lens[i])):
            pos = int(n) - int(q_lens[i]) + j
            slots[cu[i] + j] = int(base.block_tables[i, pos // B]) * B + pos % B
    gen = torch.Generator().manual_seed(seed + 7919)
    T = int(cu[-1])
    q = torch.empty((T, num_q_heads, head_dim), dtype=dtype)
    k_new = torch.empty((T, num_kv_heads, head_dim), dtype=dtype)
    v_new = torch.empty((T, num_kv_heads, head_dim), dtype=dtype)
    for t in (q, k_new, v_new):
        _fill_normal(t, gen)
    if poison:
        used = set(int(p) for p in base.block_tables.reshape(-1) if p >= 0)
        free = torch.tensor([b for b in range(base.num_blocks) if b not in used], dtype=torch.long)
        for c in (base.k_cache, base.v_cache):
            if free.numel():
                tmp = c[free]
                _poison(tmp, dtype)
                c[free] = tmp
            for i, n in enumerate(lengths):  # the slots the step writes, and the tail of each last block
                first = int(n) - int(q_lens[i])
                nblk = -(-int(n) // B)
                for blk in range(first // B, nblk):
                    lo = max(first - blk * B, 0)
                    _poison(c[int(base.block_tables[i, blk]), :, lo:, :], dtype)
    return MultiWorkload(base=base, q_lens=q_lens, cu_q=cu, q=q, k_new=k_new, v_new=v_new, slot_mapping=slots)


MULTI_CONFIG_NAMES = ("multi_spec4", "multi_chunk64")


def make_multi_config(name: str, poison: bool = True) -> MultiWorkload:
    """Multi-token steps: speculative verification of 4 draft tokens on the batch-64 lengths, and
    chunks of 64 prompt tokens appended to long contexts."""
    if name == "multi_spec4":
        rng = np.random.Generator(np.random.PCG64(11))
        lengths = rng.integers(128, 4096, size=64, endpoint=True).tolist()
        return make_multi(lengths, [4] * 64, 32, 8, 128, 16, torch.bfloat16, seed=11, max_blocks_per_seq=256,
                          poison=poison, name=name, meta={"lengths": "uniform [128,4096]", "q_len": 4})
    if name == "multi_chunk64":
        lengths = [4096] * 16
        return make_multi(lengths, [64] * 16, 32, 8, 128, 16, torch.bfloat16, seed=12, max_blocks_per_seq=256,
                          poison=poison, name=name, meta={"lengths": "16 x 4096", "q_len": 64})
    raise KeyError(name)
