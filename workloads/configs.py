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
                values: bool = True, block_size: Optional[int] = None) -> Workload:
    """One of the five named workloads.

    ``num_seqs`` trims the batch (used only to draw a bounded sample of a
    workload; the full configuration is ``num_seqs=None``).  The lengths of the
    first ``num_seqs`` sequences are the same as in the full draw.
    ``block_size`` redraws the same lengths into blocks of that many tokens (the
    block-size sweep); the table width is scaled to keep the same token
    capacity, and shared prefixes must stay whole blocks.
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
