"""GPU tests of the copy-on-write path: paged_block_copy bit for bit, and decode steps driven by the block manager.

The multi-step test runs parallel sampling the way the pages describe it
(page "praveentn.live/architecture/quiz/pagedattention-kv-cache-constraint",
section "What the change bought"): prompts written once, each forked into
several samples that share the prompt's blocks, then decode steps in which the
manager hands out slots and copy-on-write pairs, the GPU copies blocks, writes
the new tokens and decodes.  Every step is compared with the oracle on its own
host copy of the pools (oracle block copy, oracle write, oracle attention).
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_util import assert_parity, bits, device, say
from oracle.blocks import copy_blocks

pytestmark = pytest.mark.gpu


def _pools(nb, hkv, B, D, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    k = torch.randn((nb, hkv, B, D), generator=g).to(dtype)
    v = torch.randn((nb, hkv, B, D), generator=g).to(dtype)
    return k, v


@pytest.mark.parametrize("dtype,hkv,B,D", [(torch.bfloat16, 8, 16, 128), (torch.float32, 2, 32, 64),
                                           (torch.bfloat16, 1, 64, 256)])
def test_block_copy_bit_exact(dtype, hkv, B, D):
    import paged_kv_cache_276_amd as pkv

    say(f"block copy {dtype} hkv={hkv} B={B} D={D}")
    nb = 64
    k, v = _pools(nb, hkv, B, D, dtype, 11)
    k.view(torch.int16 if dtype == torch.bfloat16 else torch.int32)[3, 0, 0, :4] = torch.tensor(
        [0x7FC1, -0x8000, 0x0001, 0x7F80] if dtype == torch.bfloat16 else [0x7FC00001, -(2**31), 1, 0x7F800000],
        dtype=torch.int16 if dtype == torch.bfloat16 else torch.int32)  # NaN payload, -0, subnormal, inf
    pairs = [(3, 40), (7, 41), (0, 62), (63, 5), (2, 99), (-1, 6), (10, -3)]  # the last three are skipped
    dk, dv = k.to(device()), v.to(device())
    pkv.paged_block_copy(dk, dv, torch.tensor(pairs, dtype=torch.int32, device=device()))
    torch.cuda.synchronize()
    ek, ev = bits(k).copy(), bits(v).copy()
    copy_blocks(ek, ev, [p for p in pairs if 0 <= p[0] < nb and 0 <= p[1] < nb])
    assert np.array_equal(bits(dk), ek) and np.array_equal(bits(dv), ev)
    pkv.paged_block_copy(dk, dv, torch.zeros((0, 2), dtype=torch.int32, device=device()))  # no work


@pytest.mark.parametrize("dtype,hq,hkv,B,D", [(torch.bfloat16, 8, 2, 16, 128), (torch.float32, 4, 2, 8, 64),
                                              (torch.bfloat16, 16, 2, 32, 128)])
def test_parallel_sampling_steps(dtype, hq, hkv, B, D):
    import paged_kv_cache_276_amd as pkv
    from paged_kv_cache_276_amd import BlockManager

    say(f"parallel sampling {dtype} hq={hq} hkv={hkv} B={B} D={D}")
    rng = np.random.default_rng(5)
    gen = torch.Generator().manual_seed(5)
    nb, prompts, samples, steps = 160, 3, 4, 2 * B + 3
    bm = BlockManager(nb, B)
    o = oracle.Oracle()
    kc, vc = torch.zeros((nb, hkv, B, D), dtype=dtype), torch.zeros((nb, hkv, B, D), dtype=dtype)
    hk, hv = bits(kc).copy(), bits(vc).copy()           # oracle's pools
    dk, dv = kc.to(device()), vc.to(device())            # GPU pools
    seqs = []
    partial_prompts = 0
    for p in range(prompts):
        n = int(rng.integers(1, 3 * B))
        partial_prompts += n % B != 0
        sid = 100 * p
        bm.add(sid, n)
        kn = torch.randn((n, hkv, D), generator=gen).to(dtype)
        vn = torch.randn((n, hkv, D), generator=gen).to(dtype)
        slots = bm.slots(sid, 0, n)
        o.kv_write(kn, vn, slots, hk, hv, B)
        pkv.paged_kv_write(kn.to(device()), vn.to(device()), torch.from_numpy(slots).to(device()), dk, dv)
        seqs.append(sid)
        for s in range(1, samples):
            bm.fork(sid, sid + s)
            seqs.append(sid + s)
    maxb = nb
    scale = float(D) ** -0.5
    for step in range(steps):
        order = [int(x) for x in rng.permutation(seqs)]
        slots, copies = bm.append(order)
        if step == 0:  # every sample but the last served of a prompt with a partly filled block copies it
            assert len(copies) == partial_prompts * (samples - 1)
        kn = torch.randn((len(order), hkv, D), generator=gen).to(dtype)
        vn = torch.randn((len(order), hkv, D), generator=gen).to(dtype)
        q = torch.randn((len(order), hq, D), generator=gen).to(dtype)
        copy_blocks(hk, hv, [tuple(c) for c in copies])
        o.kv_write(kn, vn, slots, hk, hv, B)
        if len(copies):
            pkv.paged_block_copy(dk, dv, torch.from_numpy(np.ascontiguousarray(copies)).to(device()))
        pkv.paged_kv_write(kn.to(device()), vn.to(device()), torch.from_numpy(slots).to(device()), dk, dv)
        tables, lens = bm.block_tables(order, maxb)
        out = pkv.paged_attn_decode(q.to(device()), dk, dv, torch.from_numpy(tables).to(device()),
                                    torch.from_numpy(lens).to(device()), scale)
        torch.cuda.synchronize()
        assert np.array_equal(bits(dk), hk) and np.array_equal(bits(dv), hv), f"pools differ at step {step}"
        ref = o.attn_decode(q, hk, hv, tables, lens, scale, num_kv_heads=hkv)
        assert_parity(out, ref, f"step {step}")
