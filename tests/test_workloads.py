"""The seeded input generator: structure checked against the oracle's block arithmetic."""

import numpy as np
import pytest
import torch

from oracle import arith
from workloads import CONFIG_NAMES, make_config, make_custom


def _check_structure(w):
    B = w.block_size
    tables, ctx = w.block_tables, w.context_lens
    assert tables.dtype == np.int32 and ctx.dtype == np.int32 and w.slot_mapping.dtype == np.int32
    assert tables.shape == (w.num_seqs, w.max_blocks_per_seq)
    owners = {}
    for i in range(w.num_seqs):
        nb = arith.blocks_needed(int(ctx[i]), B)
        row = tables[i]
        assert np.all(row[:nb] >= 0) and np.all(row[:nb] < w.num_blocks)
        assert np.all(row[nb:] == -1)
        assert len(set(row[:nb].tolist())) == nb
        for b, p in enumerate(row[:nb].tolist()):
            owners.setdefault(p, set()).add((i, b))
        if ctx[i] > 0:
            blk, off = arith.slot_to_block_offset(int(w.slot_mapping[i]), B)
            assert blk == row[(ctx[i] - 1) // B] and off == (ctx[i] - 1) % B
        else:
            assert w.slot_mapping[i] == -1
    # a physical block is either private, or the same logical block index in every table naming it
    for p, refs in owners.items():
        assert len({b for _, b in refs}) == 1, p
    return owners


@pytest.mark.parametrize("name", CONFIG_NAMES)
def test_config_structure(name):
    w = make_config(name, values=False)
    owners = _check_structure(w)
    used = len(owners)
    assert used == w.meta["used_blocks"]
    if name == "tiny":
        assert w.num_blocks == 32 and used == 12
        assert w.context_lens.tolist() == [17, 33, 35, 64]
        assert arith.slack_tokens(w.context_lens.tolist(), 16) == 43
        assert (w.num_q_heads, w.num_kv_heads, w.head_dim, w.dtype) == (2, 1, 64, torch.float32)
    elif name == "llama8b_b64":
        assert w.num_seqs == 64 and w.num_blocks == used
        assert w.context_lens.min() >= 128 and w.context_lens.max() <= 4096
    elif name == "hc_b256":
        assert w.num_seqs == 256 and 0.89 < used / w.num_blocks <= 0.9
        assert w.context_lens.min() >= 1 and w.context_lens.max() <= 8192
        assert 700 < np.median(w.context_lens) < 1400
    elif name == "long32k":
        assert w.context_lens.tolist() == [32768] * 8 and w.num_blocks == 16384
    elif name == "shared_prefix":
        assert w.block_size == 32 and w.num_seqs == 256
        suffix = w.context_lens - 2048
        assert suffix.min() >= 1 and suffix.max() <= 512
        shared = [p for p, refs in owners.items() if len(refs) > 1]
        assert len(shared) == 32 * 64
        for p in range(32):
            rows = w.block_tables[p * 8:(p + 1) * 8, :64]
            assert np.all(rows == rows[0])
    if name != "tiny":
        assert (w.num_q_heads, w.num_kv_heads, w.head_dim, w.dtype) == (32, 8, 128, torch.bfloat16)


def test_determinism_and_poison():
    a = make_config("tiny")
    b = make_config("tiny")
    assert np.array_equal(a.block_tables, b.block_tables)
    for x, y in ((a.q, b.q), (a.k_cache, b.k_cache), (a.v_new, b.v_new)):
        assert torch.equal(x.view(torch.int32), y.view(torch.int32))
    B = a.block_size
    valid = np.zeros((a.num_blocks, B), dtype=bool)
    for i, n in enumerate(a.context_lens.tolist()):
        for j in range(n - 1):  # the cache holds ctx - 1 tokens before the write
            valid[a.block_tables[i, j // B], j % B] = True
    kc = a.k_cache.permute(0, 2, 1, 3).numpy()
    assert np.all(np.isfinite(kc[valid])) and np.all(np.isnan(kc[~valid]))


def test_custom_sharing_and_empty():
    w = make_custom([0, 20, 25, 9], num_q_heads=4, num_kv_heads=2, head_dim=16, block_size=8,
                    prefix_groups=[(16, [1, 2])], pool_fill=0.5)
    owners = _check_structure(w)
    assert w.block_tables[1, 0] == w.block_tables[2, 0] and w.block_tables[1, 1] == w.block_tables[2, 1]
    assert w.slot_mapping[0] == -1
    assert len(owners) * 2 == w.num_blocks
