"""Pins of the CPU oracle to facts that do not come from the oracle itself.

Each ``pin_*`` takes an ``oracle.Oracle`` (or the arithmetic module) and raises
``AssertionError`` when the oracle disagrees with:

* numbers the pages print (tests/golden/*.json, each entry with its source),
* a library routine on a special case: torch's scaled_dot_product_attention in
  fp64 over the *contiguous* K/V that the test itself scattered into blocks,
* closed forms (one token; flat attention; a single dominant key),
* invariances the pages state (physical placement is arbitrary; shared blocks
  read the same as private copies), and
* byte-level facts of the append (placement, skipped slots, bit patterns).

The pins are plain functions so the mutation test can run them against
deliberately broken copies of the oracle.
"""

from __future__ import annotations

import json
import math
import os
from typing import List, Optional, Tuple

import numpy as np
import torch
import torch.nn.functional as F

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
NAN32 = np.array([0x7FC0BEEF], dtype=np.uint32).view(np.float32)[0]


def _golden(name: str):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# --------------------------------------------------------------------------
# Test-side data: contiguous logical K/V first, then scattered into a pool.
# --------------------------------------------------------------------------

class Case:
    """Contiguous per-sequence K/V (fp32) scattered into a paged pool by the test."""

    def __init__(self, rng: np.random.Generator, lengths: List[int], hq: int, hkv: int, d: int,
                 b: int, extra_blocks: int = 3, scale: Optional[float] = None,
                 tables_width: Optional[int] = None, placement: Optional[np.ndarray] = None):
        self.lengths = list(lengths)
        self.hq, self.hkv, self.d, self.b = hq, hkv, d, b
        nblk = [-(-n // b) for n in lengths]
        used = sum(nblk)
        self.num_blocks = used + extra_blocks
        width = tables_width or max([1] + nblk)
        self.q = rng.standard_normal((len(lengths), hq, d)).astype(np.float32)
        self.K = [rng.standard_normal((n, hkv, d)).astype(np.float32) for n in lengths]
        self.V = [rng.standard_normal((n, hkv, d)).astype(np.float32) for n in lengths]
        self.scale = float(np.float32(scale if scale is not None else 1.0 / math.sqrt(d)))
        if placement is None:
            placement = rng.permutation(self.num_blocks)[:used]
        self.placement = np.asarray(placement)
        self.width = width
        self.scatter()

    def scatter(self) -> None:
        """Build pool and tables from the logical data and self.placement."""
        S, b = len(self.lengths), self.b
        pool_k = np.full((self.num_blocks, self.hkv, b, self.d), NAN32, dtype=np.float32)
        pool_v = np.full_like(pool_k, NAN32)
        tables = np.full((S, self.width), -1, dtype=np.int32)
        u = 0
        for i, n in enumerate(self.lengths):
            for blk in range(-(-n // b)):
                phys = int(self.placement[u])
                u += 1
                tables[i, blk] = phys
                lo, hi = blk * b, min(n, (blk + 1) * b)
                # logical rows [lo, hi) of sequence i -> physical block phys, offsets 0..hi-lo
                pool_k[phys, :, : hi - lo, :] = self.K[i][lo:hi].transpose(1, 0, 2)
                pool_v[phys, :, : hi - lo, :] = self.V[i][lo:hi].transpose(1, 0, 2)
        self.pool_k, self.pool_v, self.tables = pool_k, pool_v, tables
        self.ctx = np.asarray(self.lengths, dtype=np.int32)

    def run(self, o) -> np.ndarray:
        return o.attn_decode(self.q, self.pool_k, self.pool_v, self.tables, self.ctx, self.scale)


def sdpa(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """torch's scaled_dot_product_attention in fp64 on contiguous K/V.

    q [Hq][D]; K, V [n][Hkv][D].  Grouped-query heads are expanded the usual
    way (each KV head repeated Hq/Hkv times, so query head h uses KV head
    h // (Hq/Hkv)).
    """
    hq, d = q.shape
    n, hkv, _ = K.shape
    if n == 0:
        return np.zeros((hq, d))
    g = hq // hkv
    qt = torch.from_numpy(q.astype(np.float64))[:, None, :]
    kt = torch.from_numpy(K.astype(np.float64)).permute(1, 0, 2).repeat_interleave(g, dim=0)
    vt = torch.from_numpy(V.astype(np.float64)).permute(1, 0, 2).repeat_interleave(g, dim=0)
    out = F.scaled_dot_product_attention(qt, kt.contiguous(), vt.contiguous(), scale=float(scale))
    return out[:, 0, :].numpy()


# --------------------------------------------------------------------------
# Pins
# --------------------------------------------------------------------------

def pin_block_arithmetic(arith) -> None:
    g = _golden("block_arithmetic.json")
    for e in g["single"]:
        B, n = e["block_size"], e["n_tokens"]
        assert arith.blocks_needed(n, B) == e["blocks"], e
        if "unused_slots" in e:
            assert arith.unused_slots(n, B) == e["unused_slots"], e
        if "capacity" in e:
            assert arith.blocks_needed(n, B) * B == e["capacity"], e
        if "used_in_last_block" in e:
            assert arith.used_in_last_block(n, B) == e["used_in_last_block"], e
    for e in g["batch"]:
        assert arith.allocated_tokens(e["lengths"], e["block_size"]) == e["allocated"], e
        assert arith.slack_tokens(e["lengths"], e["block_size"]) == e["slack_tokens"], e
    for B in (1, 2, 8, 16, 32):
        for n in range(1, 200):
            assert 0 <= arith.unused_slots(n, B) <= B - 1
            assert arith.blocks_needed(n, B) * B >= n > (arith.blocks_needed(n, B) - 1) * B


def pin_kv_bytes(arith) -> None:
    g = _golden("kv_bytes.json")
    for e in g["per_token"] + g["one_layer"]:
        assert arith.kv_bytes_per_token(e["layers"], e["kv_heads"], e["head_dim"], e["elem_bytes"]) == e["bytes"]
    e = g["per_token"][0]
    assert e["bytes"] == e["kib"] * 1024
    for e in g["per_sequence"]:
        per_tok = arith.kv_bytes_per_token(e["layers"], e["kv_heads"], e["head_dim"], e["elem_bytes"])
        assert arith.kv_bytes_per_request(per_tok, e["tokens"]) == e["bytes"] == 1 << 30
    for e in g["capacity"]:
        assert arith.cache_limited_concurrency(e["available_bytes"], e["bytes_per_request"]) == e["concurrency"]


def pin_block_map(o) -> None:
    """The pages' seven-slot example: request A at physical [3, 6, 5, 1], decoys NaN."""
    g = _golden("block_map.json")
    slots = g["pool_slots"]
    table = [slots.index(name) for name in g["logical_blocks"]]
    assert table == g["block_table"]
    rng = np.random.default_rng(7)
    b, d, hq, hkv = 4, 8, 2, 1
    for n in (16, 14, 13):  # full last block, and a partial one
        case = Case(rng, [n], hq, hkv, d, b, extra_blocks=7 - 4,
                    placement=np.asarray(g["block_table"]))
        assert case.tables[0, :4].tolist() == g["block_table"]
        out = case.run(o)
        assert np.all(np.isfinite(out)), "decoy blocks (B1, C2, free) or A3's tail were read"
        ref = sdpa(case.q[0], case.K[0], case.V[0], case.scale)
        np.testing.assert_allclose(out[0], ref, rtol=1e-12, atol=1e-12)


def pin_slot_encoding(arith) -> None:
    """The seven-slot example with slots numbered physical block * B + offset: logical token j
    of request A is in pool block table[j // B] at offset j % B, so A2 (pool block 5) holds
    token 2B + 3 in slot 5B + 3, which decodes to (5, 3).  Every token of A decodes to the
    block the diagram names for it, never to a decoy (B1, C2, free), at its own offset."""
    g = _golden("block_map.json")
    table = g["block_table"]
    for b in (4, 16):
        assert arith.slot_to_block_offset(5 * b + 3, b) == (5, 3)
        seen = set()
        for j in range(4 * b):
            blk, off = arith.slot_to_block_offset(table[j // b] * b + j % b, b)
            assert g["pool_slots"][blk] == g["logical_blocks"][j // b] and off == j % b
            seen.add((blk, off))
        assert len(seen) == 4 * b


def pin_brute_force(o) -> None:
    """Oracle on scattered blocks == SDPA on the contiguous data, many shapes."""
    rng = np.random.default_rng(11)
    shapes = [  # (lengths, hq, hkv, d, b)
        ([1, 2, 3, 4, 5], 1, 1, 8, 4),
        ([7, 8, 9, 16, 17], 4, 2, 16, 8),
        ([17, 33, 35, 64], 2, 1, 64, 16),
        ([31, 32, 33, 1, 100], 8, 2, 32, 32),
        ([5, 40, 63], 8, 8, 16, 16),
        ([129, 3], 4, 1, 128, 16),
    ]
    for lengths, hq, hkv, d, b in shapes:
        scale = float(rng.uniform(0.05, 0.5))
        case = Case(rng, lengths, hq, hkv, d, b, extra_blocks=5, scale=scale)
        out = case.run(o)
        for i in range(len(lengths)):
            ref = sdpa(case.q[i], case.K[i], case.V[i], case.scale)
            np.testing.assert_allclose(out[i], ref, rtol=1e-11, atol=1e-12,
                                       err_msg=f"seq {i} of {lengths} hq={hq} hkv={hkv} d={d} b={b}")


def pin_bf16_widening(o) -> None:
    """bf16 storage: the oracle must read exactly the bf16 values (vs SDPA on them in fp64)."""
    rng = np.random.default_rng(5)
    case = Case(rng, [9, 20], 4, 2, 16, 8, extra_blocks=2)
    q16 = torch.from_numpy(case.q).to(torch.bfloat16)
    k16 = torch.from_numpy(case.pool_k).to(torch.bfloat16)
    v16 = torch.from_numpy(case.pool_v).to(torch.bfloat16)
    out = o.attn_decode(q16, k16, v16, case.tables, case.ctx, case.scale)
    for i, n in enumerate(case.lengths):
        Kb = torch.from_numpy(case.K[i]).to(torch.bfloat16).to(torch.float64).numpy()
        Vb = torch.from_numpy(case.V[i]).to(torch.bfloat16).to(torch.float64).numpy()
        qb = q16[i].to(torch.float64).numpy()
        ref = sdpa(qb, Kb, Vb, case.scale)
        np.testing.assert_allclose(out[i], ref, rtol=1e-11, atol=1e-12)


def pin_single_token(o) -> None:
    """n = 1: softmax of one score is 1, so out = v_0 exactly, whatever q, K and scale."""
    rng = np.random.default_rng(3)
    case = Case(rng, [1, 1, 1], 4, 2, 16, 8, extra_blocks=2, scale=3.7)
    out = case.run(o)
    for i in range(3):
        for h in range(4):
            g = h // 2
            assert np.array_equal(out[i, h], case.V[i][0, g].astype(np.float64)), (i, h)


def pin_flat_attention(o) -> None:
    """q = 0, or all keys equal: every weight is 1/n, out = mean of V (closed form)."""
    rng = np.random.default_rng(4)
    case = Case(rng, [1, 5, 16, 37], 2, 1, 8, 8, extra_blocks=2)
    case.q[:] = 0.0
    out = case.run(o)
    for i, n in enumerate(case.lengths):
        mean = case.V[i][:, 0, :].astype(np.float64).mean(axis=0)
        np.testing.assert_allclose(out[i, 0], mean, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(out[i, 1], mean, rtol=1e-12, atol=1e-13)
    case = Case(rng, [3, 29], 2, 1, 8, 8, extra_blocks=2)
    for i in range(2):
        case.K[i][:] = case.K[i][0]
    case.scatter()
    out = case.run(o)
    for i in range(2):
        mean = case.V[i][:, 0, :].astype(np.float64).mean(axis=0)
        np.testing.assert_allclose(out[i, 0], mean, rtol=1e-12, atol=1e-13)


def needle_expected(V: np.ndarray, jstar: int, big: float) -> np.ndarray:
    """All scores 0 except one equal to `big`: out = (e^big v* + sum_{j!=j*} v_j) / (e^big + n - 1)."""
    n = V.shape[0]
    vstar = V[jstar].astype(np.float64)
    rest = V.astype(np.float64).sum(axis=0) - vstar
    eb = math.exp(big)
    return (eb * vstar + rest) / (eb + n - 1)


def pin_needle(o) -> None:
    """One key aligned with q (score 20), all others zero: closed form above, for several j*."""
    rng = np.random.default_rng(9)
    b, d, n = 8, 16, 45
    for jstar in (0, b - 1, b, 2 * b + 3, n - 1):
        case = Case(rng, [n], 1, 1, d, b, extra_blocks=3)
        q = case.q[0, 0].astype(np.float64)
        c = 20.0 / (case.scale * float(q @ q))
        case.K[0][:] = 0.0
        case.K[0][jstar, 0] = (c * q).astype(np.float32)
        case.scatter()
        big = case.scale * float(case.K[0][jstar, 0].astype(np.float64) @ case.q[0, 0].astype(np.float64))
        out = case.run(o)
        np.testing.assert_allclose(out[0, 0], needle_expected(case.V[0][:, 0], jstar, big),
                                   rtol=1e-11, atol=1e-12)


def pin_identical_queries(o) -> None:
    """Query heads of one group with equal q give equal rows; different groups differ."""
    rng = np.random.default_rng(12)
    case = Case(rng, [10, 21], 4, 2, 16, 8, extra_blocks=2)
    case.q[:, 1] = case.q[:, 0]
    case.q[:, 3] = case.q[:, 2]
    out = case.run(o)
    assert np.array_equal(out[:, 0], out[:, 1]) and np.array_equal(out[:, 2], out[:, 3])
    assert not np.allclose(out[:, 0], out[:, 2])


def pin_placement_invariance(o) -> None:
    """Same logical data, two physical placements (and pool sizes): identical bits out."""
    rng = np.random.default_rng(13)
    case = Case(rng, [3, 16, 17, 50], 4, 2, 16, 8, extra_blocks=6)
    a = case.run(o)
    used = len(case.placement)
    case.placement = np.random.default_rng(99).permutation(case.num_blocks)[:used]
    case.scatter()
    b = case.run(o)
    assert np.array_equal(a, b)


def pin_shared_blocks(o) -> None:
    """Several tables naming one physical prefix block read the same as private copies."""
    rng = np.random.default_rng(14)
    b, d, prefix = 8, 16, 16
    lengths = [prefix + 3, prefix + 9, prefix + 1]
    case = Case(rng, lengths, 2, 1, d, b, extra_blocks=4)
    for i in (1, 2):  # identical prefix tokens for every sequence
        case.K[i][:prefix] = case.K[0][:prefix]
        case.V[i][:prefix] = case.V[0][:prefix]
    case.scatter()
    private = case.run(o)
    shared_tables = case.tables.copy()
    for i in (1, 2):
        shared_tables[i, : prefix // b] = case.tables[0, : prefix // b]
    pk, pv = case.pool_k.copy(), case.pool_v.copy()
    for i in (1, 2):  # the private prefix copies become free (poisoned) blocks
        for blk in case.tables[i, : prefix // b]:
            pk[blk] = NAN32
            pv[blk] = NAN32
    shared = o.attn_decode(case.q, pk, pv, shared_tables, case.ctx, case.scale)
    assert np.array_equal(private, shared)


def pin_empty_sequence(o) -> None:
    rng = np.random.default_rng(15)
    case = Case(rng, [0, 5, 0], 2, 1, 8, 4, extra_blocks=1)
    out = case.run(o)
    assert np.array_equal(out[0], np.zeros_like(out[0])) and np.array_equal(out[2], np.zeros_like(out[2]))
    np.testing.assert_allclose(out[1], np.stack([sdpa(case.q[1], case.K[1], case.V[1], case.scale)[h]
                                                for h in range(2)]), rtol=1e-12, atol=1e-12)


def pin_row_sample(o) -> None:
    """Sampled rows equal the same rows of the full batch."""
    rng = np.random.default_rng(16)
    case = Case(rng, [4, 19, 33], 4, 2, 8, 8, extra_blocks=2)
    full = case.run(o)
    rows = [(2, 3), (0, 0), (1, 2), (2, 0)]
    part = o.attn_decode(case.q, case.pool_k, case.pool_v, case.tables, case.ctx, case.scale, rows=rows)
    for r, (i, h) in enumerate(rows):
        assert np.array_equal(part[r], full[i, h])


def pin_write(o) -> None:
    """Append: rows land at (slot // B, slot % B), -1 skipped, bits preserved, nothing else touched."""
    rng = np.random.default_rng(17)
    nb, hkv, b, d = 6, 3, 4, 8
    base_k = rng.integers(0, 2**32, size=(nb, hkv, b, d), dtype=np.uint64).astype(np.uint32).view(np.int32)
    base_v = rng.integers(0, 2**32, size=(nb, hkv, b, d), dtype=np.uint64).astype(np.uint32).view(np.int32)
    slots = np.array([0, b - 1, 2 * b + 1, -1, nb * b - 1, 3 * b], dtype=np.int32)
    T = slots.shape[0]
    kn = rng.standard_normal((T, hkv, d)).astype(np.float32)
    vn = rng.standard_normal((T, hkv, d)).astype(np.float32)
    special = np.array([0x80000000, 0x7FC0BEEF, 0xFFC00001, 0x00000001, 0x7F800000, 0xFF800000,
                        0x007FFFFF, 0x7FA00000], dtype=np.uint32).view(np.float32)
    kn[0, 0, :] = special
    vn[1, 2, :] = special[::-1]
    kc, vc = base_k.copy(), base_v.copy()
    o.kv_write(kn, vn, slots, kc, vc, b)
    ek, ev = base_k.copy(), base_v.copy()
    for t, s in enumerate(slots):
        if s < 0:
            continue
        ek[s // b, :, s % b, :] = kn[t].view(np.int32)
        ev[s // b, :, s % b, :] = vn[t].view(np.int32)
    assert np.array_equal(kc, ek) and np.array_equal(vc, ev)
    assert np.array_equal(kc[0, 0, 0].view(np.uint32), special.view(np.uint32))
    # the skipped token (slot -1) wrote nothing: every byte it could have reached is unchanged
    mask = np.ones((nb, b), dtype=bool)
    for s in slots[slots >= 0]:
        mask[s // b, s % b] = False
    assert np.array_equal(kc.transpose(0, 2, 1, 3)[mask], base_k.transpose(0, 2, 1, 3)[mask])
    # bf16 rows too
    kn16 = torch.from_numpy(kn).to(torch.bfloat16)
    vn16 = torch.from_numpy(vn).to(torch.bfloat16)
    kc16 = base_k.view(np.int16)[..., :d].copy()
    vc16 = base_v.view(np.int16)[..., :d].copy()
    o.kv_write(kn16, vn16, slots, kc16, vc16, b)
    for t, s in enumerate(slots):
        if s < 0:
            continue
        assert np.array_equal(kc16[s // b, :, s % b], kn16[t].view(torch.int16).numpy())
        assert np.array_equal(vc16[s // b, :, s % b], vn16[t].view(torch.int16).numpy())


def pin_errors(o) -> None:
    """Bad tables, lengths and slots are reported, not silently read."""
    rng = np.random.default_rng(18)
    case = Case(rng, [9], 2, 1, 8, 4, extra_blocks=1)
    bad = case.tables.copy()
    bad[0, 1] = case.num_blocks
    for tables, ctx in ((bad, case.ctx), (case.tables, np.array([case.tables.shape[1] * 4 + 1], np.int32))):
        try:
            o.attn_decode(case.q, case.pool_k, case.pool_v, tables, ctx, case.scale)
        except RuntimeError:
            pass
        else:
            raise AssertionError("oracle accepted an invalid table or length")
    kc = np.zeros((2, 1, 4, 8), np.int32)
    try:
        o.kv_write(np.zeros((1, 1, 8), np.float32), np.zeros((1, 1, 8), np.float32),
                   np.array([8], np.int32), kc, kc.copy(), 4)
    except RuntimeError:
        pass
    else:
        raise AssertionError("oracle accepted a slot outside the pool")


# --------------------------------------------------------------------------
# Several new tokens per sequence (causal)
# --------------------------------------------------------------------------

def _multi_case(seed: int, lengths: List[int], q_lens: List[int], hq: int, hkv: int, d: int, b: int):
    rng = np.random.default_rng(seed)
    case = Case(rng, lengths, hq, hkv, d, b)
    cu = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    qm = rng.standard_normal((int(cu[-1]), hq, d)).astype(np.float32)
    return case, cu, qm


def sdpa_causal(q_rows: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """SDPA in fp64 for the last len(q_rows) tokens of a contiguous sequence, each seeing itself and
    every earlier token (an explicit boolean mask; torch's own is_causal aligns the other corner)."""
    ql, hq, d = q_rows.shape
    n, hkv, _ = K.shape
    g = hq // hkv
    qt = torch.from_numpy(q_rows.astype(np.float64)).permute(1, 0, 2)                 # [hq][ql][d]
    kt = torch.from_numpy(K.astype(np.float64)).permute(1, 0, 2).repeat_interleave(g, dim=0)
    vt = torch.from_numpy(V.astype(np.float64)).permute(1, 0, 2).repeat_interleave(g, dim=0)
    pos = torch.arange(n - ql, n)[:, None]
    mask = torch.arange(n)[None, :] <= pos                                                # [ql][n]
    out = F.scaled_dot_product_attention(qt, kt.contiguous(), vt.contiguous(), attn_mask=mask, scale=float(scale))
    return out.permute(1, 0, 2).numpy()                                                   # [ql][hq][d]


def pin_multi_one_token_is_decode(o) -> None:
    """One new token per sequence: the causal multi-token attention is plain decode attention."""
    case, cu, _ = _multi_case(30, [1, 5, 16, 17, 40], [1, 1, 1, 1, 1], 4, 2, 16, 4)
    got = o.attn_multi(case.q, case.pool_k, case.pool_v, case.tables, case.ctx, cu, case.scale)
    ref = case.run(o)
    assert np.max(np.abs(got - ref)) <= 1e-12


def pin_multi_sdpa_causal(o) -> None:
    """Against fp64 SDPA with an explicit causal mask on the contiguous K/V, for GQA shapes and q_len up to n."""
    for seed, lengths, q_lens, hq, hkv in ((31, [7, 20, 33], [3, 1, 8], 4, 2), (32, [9, 12], [9, 5], 8, 8),
                                           (33, [64, 3], [16, 2], 2, 1)):
        case, cu, qm = _multi_case(seed, lengths, q_lens, hq, hkv, 16, 4)
        got = o.attn_multi(qm, case.pool_k, case.pool_v, case.tables, case.ctx, cu, case.scale)
        for i, (n, ql) in enumerate(zip(lengths, q_lens)):
            ref = sdpa_causal(qm[cu[i]:cu[i + 1]], case.K[i], case.V[i], case.scale)
            assert np.max(np.abs(got[cu[i]:cu[i + 1]] - ref)) <= 1e-12, (seed, i)


def pin_multi_rows_are_truncated_decodes(o) -> None:
    """Query row j of a sequence equals decode attention over the sequence cut after position n - q_len + j."""
    case, cu, qm = _multi_case(34, [13, 26], [4, 6], 4, 1, 8, 4)
    got = o.attn_multi(qm, case.pool_k, case.pool_v, case.tables, case.ctx, cu, case.scale)
    for i, n in enumerate(case.lengths):
        ql = int(cu[i + 1] - cu[i])
        for j in range(ql):
            ctx = np.zeros_like(case.ctx)
            ctx[i] = n - ql + j + 1
            q = np.zeros_like(case.q)
            q[i] = qm[cu[i] + j]
            ref = o.attn_decode(q, case.pool_k, case.pool_v, case.tables, ctx, case.scale)[i]
            assert np.max(np.abs(got[cu[i] + j] - ref)) <= 1e-12, (i, j)


def pin_multi_errors(o) -> None:
    """More new tokens than the sequence holds is reported."""
    case, _, qm = _multi_case(35, [3], [3], 2, 1, 8, 4)
    try:
        o.attn_multi(np.concatenate([qm, qm[:1]]), case.pool_k, case.pool_v, case.tables, case.ctx,
                     np.array([0, 4], np.int32), case.scale)
    except RuntimeError:
        return
    raise AssertionError("oracle accepted q_len > context length")


ORACLE_PINS = [
    pin_block_map, pin_brute_force, pin_bf16_widening, pin_single_token, pin_flat_attention,
    pin_needle, pin_identical_queries, pin_placement_invariance, pin_shared_blocks,
    pin_empty_sequence, pin_row_sample, pin_write, pin_errors,
    pin_multi_one_token_is_decode, pin_multi_sdpa_causal, pin_multi_rows_are_truncated_decodes,
    pin_multi_errors,
]
ARITH_PINS = [pin_block_arithmetic, pin_kv_bytes, pin_slot_encoding]
