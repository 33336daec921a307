"""Integer arithmetic of paged KV storage, as the pages state it.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

* Block count of an n-token sequence with B-token blocks is ceil(n / B); the
  unused slots are blocks * B - n: page "chenhuiyu.github.io/blog/llm-infra-vllm-en",
  section "Calculate a block-allocation example" (35 tokens at B = 16: three
  blocks, thirteen unused slots).
* Allocated tokens and total slack of a batch: same page, section "Logical
  continuity, physical flexibility" ([17, 33, 64] at B = 16 -> [32, 48, 64],
  slack 30).
* KV bytes per token = layers x 2 x KV heads x head dim x bytes per element;
  bytes per request = bytes per token x active length; cache-limited
  concurrency = available bytes / bytes per request: page "x321.org/?p=939",
  sections "First understand what the KV cache is storing" and "A useful
  calculation before deploying any model".
"""

from __future__ import annotations

from typing import Iterable, List


def blocks_needed(n_tokens: int, block_size: int) -> int:
    if n_tokens < 0 or block_size <= 0:
        raise ValueError("n_tokens >= 0 and block_size > 0 required")
    return -(-n_tokens // block_size)


def unused_slots(n_tokens: int, block_size: int) -> int:
    return blocks_needed(n_tokens, block_size) * block_size - n_tokens


def used_in_last_block(n_tokens: int, block_size: int) -> int:
    """Positions occupied in the sequence's final block (0 for an empty sequence)."""
    if n_tokens == 0:
        return 0
    return n_tokens - (blocks_needed(n_tokens, block_size) - 1) * block_size


def allocated_tokens(lengths: Iterable[int], block_size: int) -> List[int]:
    return [blocks_needed(n, block_size) * block_size for n in lengths]


def slack_tokens(lengths: Iterable[int], block_size: int) -> int:
    lengths = list(lengths)
    return sum(allocated_tokens(lengths, block_size)) - sum(lengths)


def kv_bytes_per_token(layers: int, kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    return layers * 2 * kv_heads * head_dim * elem_bytes


def kv_bytes_per_request(bytes_per_token: int, active_tokens: int) -> int:
    return bytes_per_token * active_tokens


def cache_limited_concurrency(available_bytes: int, bytes_per_request: int) -> int:
    return available_bytes // bytes_per_request


def slot_to_block_offset(slot: int, block_size: int):
    """Slot encoding read as slot = physical_block * block_size + offset (the pages give the
    block table, not a slot number): physical block and offset of a slot."""
    if slot < 0 or block_size <= 0:
        raise ValueError("slot >= 0 and block_size > 0 required")
    return slot // block_size, slot % block_size
