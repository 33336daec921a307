"""Host model of the fast decode kernel's work split (its integer arithmetic, step by step).

The kernel gives wave w the tiles [start(w), start(w+1)) of all (sequence, KV head,
16-token tile) triples -- equal shares, or shares weighted by the wave's XCD -- finds its first sequence with a two-level prefix sum
(8 sequences per lane, 64 lanes, ballot), walks the tiles with a cursor, keeps
partial results at slot unit + w, and the wave that sees a unit's first tile
records (first slot, count) with count = wave_of(last tile) - w + 1.  This model
replays exactly that arithmetic and checks, for many length mixes and wave
counts, that every tile is visited once, every index stays in range, slots never
collide, and the recorded counts equal the number of waves that touch the unit.
"""

import numpy as np
import pytest

TOK = 16
MAX_WAVES = 8192
SEG_TILES = 128


def tiles_of(ctx, table_tokens):
    return 0 if (ctx < 0 or ctx > table_tokens) else (ctx + TOK - 1) // TOK


def locate(ctx, table_tokens, hkv, c0):
    """The kernel's second pass: lane l holds sequences base + 8l .. base + 8l + 7."""
    S = len(ctx)
    acc = 0
    for base in range(0, S, 64 * 8):
        nv = [[tiles_of(ctx[base + l * 8 + k], table_tokens) if base + l * 8 + k < S else 0
               for k in range(8)] for l in range(64)]
        s = [sum(x) for x in nv]
        incl = list(np.cumsum(s))
        chunk = int(incl[63]) * hkv
        if c0 < acc + chunk:
            mask = [acc + int(incl[l]) * hkv > c0 for l in range(64)]
            L = mask.index(True)
            b0 = acc + (int(incl[L]) - s[L]) * hkv
            for k in range(8):
                n = nv[L][k]
                if c0 < b0 + n * hkv:
                    return base + L * 8 + k, b0
                b0 += n * hkv
            raise AssertionError("lane L does not hold c0")
        acc += chunk
    return -1, 0


def segment_walk(ctx, hkv, block_size, max_blocks, c0, c1, cur, seg_runs):
    """The kernel's segment set-up: runs of <= seg_runs pieces and <= SEG_TILES tiles.

    Yields, per segment, the (sequence, KV head, tile) of every tile with its
    block-table index, as the per-tile records would hold them."""
    table_tokens = max_blocks * block_size
    P = dict(cur)
    seg0 = c0
    while seg0 < c1:
        room = min(SEG_TILES, c1 - seg0)
        runs, k = [], 0
        while k < room and len(runs) < seg_runs:
            ln = min(P["n"] - P["b"], room - k)
            assert ln > 0
            runs.append((P["i"], P["g"], P["n"], P["b"], k, P["ctx"]))
            k += ln
            P["b"] += ln
            if P["b"] == P["n"] and seg0 + k < c1:
                P["b"] = 0
                P["g"] += 1
                if P["g"] == hkv:
                    P["g"] = 0
                    while True:
                        P["i"] += 1
                        assert P["i"] < len(ctx)
                        P["ctx"] = ctx[P["i"]]
                        P["n"] = tiles_of(P["ctx"], table_tokens)
                        if P["n"]:
                            break
        seg_len = k
        tiles = []
        for j in range(seg_len):
            r = max(q for q in range(len(runs)) if j >= runs[q][4])
            i, g, n, b0, k0, c = runs[r]
            b = b0 + (j - k0)
            assert 0 <= b < n and (b * TOK) // block_size < max_blocks
            assert 1 <= min(TOK, c - b * TOK) <= TOK
            tiles.append((i, g, b))
        yield tiles
        seg0 += seg_len


FIRST_HALF_SHARE = 20  # tile_math.h kFirstHalfShare


class Split:
    """The kernel's work split (tile_math.h, Split and make_split), integer for integer."""

    def __init__(self, Nt, W, grid_waves, balance):
        lo = min(balance, 128 - balance)
        W8 = grid_waves // 8
        d = FIRST_HALF_SHARE if W8 % 2 == 0 else 0
        per_xcd = (W == grid_waves and grid_waves % 8 == 0 and balance != 64 and 0 < balance < 128
                   and Nt * lo * (64 - d) >= 4096 * W)
        self.Nt, self.W = Nt, W
        self.W8 = W8 if per_xcd else 0
        self.b = balance if per_xcd else 64
        self.d = d if per_xcd else 0

    def wt(self, x):
        return self.b if x & 1 else 128 - self.b

    def wh(self, j):
        return 64 + self.d if j < self.W8 // 2 else 64 - self.d

    def base(self, x):
        return (x >> 1) * 128 + ((128 - self.b) if x & 1 else 0)

    def halves(self, j):
        H = self.W8 // 2
        return j * (64 + self.d) if j < H else H * (64 + self.d) + (j - H) * (64 - self.d)

    def S(self, w):
        if self.W8 == 0:
            return 4096 * w
        x = w // self.W8
        return 64 * self.W8 * self.base(x) + self.wt(x) * self.halves(w - x * self.W8)

    def start(self, w):
        return (self.Nt * self.S(w)) // (4096 * self.W)

    def wave_of(self, t):
        T = ((t + 1) * 4096 * self.W - 1) // self.Nt
        if self.W8 == 0:
            return min(self.W - 1, T // 4096)
        x = 7
        while x > 0 and 64 * self.W8 * self.base(x) > T:
            x -= 1
        R = T - 64 * self.W8 * self.base(x)
        H = self.W8 // 2
        first = self.wt(x) * H * (64 + self.d)
        j = R // (self.wt(x) * (64 + self.d)) if R < first else H + (R - first) // (self.wt(x) * (64 - self.d))
        return x * self.W8 + min(self.W8 - 1, j)


def test_split_inverse_and_nonempty_waves():
    """wave_of inverts start, every wave below W owns a tile, and the shares follow the XCDs."""
    rng = np.random.default_rng(3)
    for _ in range(400):
        grid = int(rng.choice([8, 16, 64, 256, 2048, 2056, 24, 7]))
        Nt = int(rng.integers(1, 40 * grid))
        W = min(Nt, grid)
        b = int(rng.choice([1, 10, 40, 61, 62, 64, 70, 100, 127]))
        sp = Split(Nt, W, grid, b)
        starts = [sp.start(w) for w in range(W + 1)]
        assert starts[0] == 0 and starts[W] == Nt
        assert all(starts[w + 1] > starts[w] for w in range(W)), (grid, Nt, b)
        for t in rng.integers(0, Nt, 50):
            w = sp.wave_of(int(t))
            assert starts[w] <= t < starts[w + 1]
        if sp.W8 and Nt >= 100 * W:  # shares come out as asked, to within a tile
            for w in (0, sp.W8, 2 * sp.W8 + 1, 3 * sp.W8, sp.W8 - 1, sp.W8 // 2, 5 * sp.W8 + sp.W8 // 2 - 1):
                x = w // sp.W8
                want = Nt * sp.wt(x) * sp.wh(w - x * sp.W8) / (4096 * W)
                assert abs((starts[w + 1] - starts[w]) - want) <= 1
    # equal shares reduce to floor(Nt w / W)
    sp = Split(202792, 2048, 2048, 64)
    assert [sp.start(w) for w in range(0, 2049, 97)] == [w * 202792 // 2048 for w in range(0, 2049, 97)]


def run_schedule(ctx, hkv, block_size, max_blocks, nwaves, seg_runs=8, balance=64):
    table_tokens = max_blocks * block_size
    S = len(ctx)
    n = [tiles_of(c, table_tokens) for c in ctx]
    Nt = sum(n) * hkv
    units = S * hkv
    visits = {}
    slots = {}
    records = {}
    if Nt == 0:
        return Nt, visits, slots, records
    W = min(Nt, nwaves)
    seen_w = set()
    for bid in range(nwaves):
        w = (bid % 8) * (nwaves // 8) + bid // 8 if nwaves % 8 == 0 else bid
        assert w not in seen_w
        seen_w.add(w)
        if w >= W:
            continue
        sp = Split(Nt, W, nwaves, balance)
        c0, c1 = sp.start(w), sp.start(w + 1)
        assert c1 > c0, "every wave below W owns at least one tile"
        i, base = locate(ctx, table_tokens, hkv, c0)
        assert 0 <= i < S
        cur = dict(i=i, ctx=ctx[i], n=n[i], seq_base=base)
        off = c0 - base
        cur["g"], cur["b"] = off // cur["n"], off % cur["n"]
        start_cursor = dict(cur)
        walked = [x for seg in segment_walk(ctx, hkv, block_size, max_blocks, c0, c1, start_cursor, seg_runs)
                  for x in seg]
        assert len(walked) == c1 - c0
        from_start = False
        for t in range(c0, c1):
            assert walked[t - c0] == (cur["i"], cur["g"], cur["b"]), "segment walk and cursor disagree"
            first = t == c0 or cur["b"] == 0
            if first:
                from_start = cur["b"] == 0
            i, g, b = cur["i"], cur["g"], cur["b"]
            assert 0 <= i < S and 0 <= g < hkv and 0 <= b < cur["n"]
            tok0 = b * TOK
            blk = tok0 // block_size
            assert blk < max_blocks and tok0 % block_size + TOK <= block_size
            valid = min(TOK, cur["ctx"] - tok0)
            assert 1 <= valid <= TOK
            assert cur["seq_base"] + g * cur["n"] + b == t, "cursor and tile index agree"
            visits[t] = visits.get(t, 0) + 1
            unit_end = b == cur["n"] - 1
            if unit_end or t + 1 == c1:
                u = i * hkv + g
                complete = from_start and unit_end
                if not complete:
                    slot = u + w
                    assert slot < units + MAX_WAVES
                    assert slot not in slots, "partial slots collide"
                    slots[slot] = (u, w)
                if from_start:
                    last_tile = cur["seq_base"] + g * cur["n"] + cur["n"] - 1
                    w_last = sp.wave_of(last_tile)
                    records[u] = (u + w, w_last - w + 1)
                    assert (records[u][1] == 1) == complete
            # advance
            if t + 1 < c1:
                cur["b"] += 1
                if cur["b"] == cur["n"]:
                    cur["b"] = 0
                    cur["g"] += 1
                    if cur["g"] == hkv:
                        cur["g"] = 0
                        cur["seq_base"] += hkv * cur["n"]
                        while True:
                            cur["i"] += 1
                            assert cur["i"] < S
                            cur["ctx"] = ctx[cur["i"]]
                            cur["n"] = tiles_of(cur["ctx"], table_tokens)
                            if cur["n"]:
                                break
    return Nt, visits, slots, records


def _cases():
    rng = np.random.default_rng(0)
    cases = [
        ([17, 33, 35, 64], 1, 16, 4, 2048),
        ([0, 0, 5, 0], 8, 16, 4, 64),
        ([32768] * 8, 8, 16, 2048, 2048),
        ([1] * 300, 8, 16, 1, 1000),
        ([0, 1, 15, 16, 17, 100, 2000, 7, 4100, 33], 4, 16, 257, 3),
        ([31, 32, 33, 64, 999], 1, 32, 32, 8192),
        ([70, -3, 10**9, 5], 2, 64, 2, 24),  # bad lengths count as empty
    ]
    lens = np.clip(np.rint(np.exp(rng.normal(np.log(1024), 1.0, 256))), 1, 8192).astype(int).tolist()
    cases.append((lens, 8, 16, 512, 2048))
    cases.append((lens, 8, 16, 512, 2056))
    cases.append((rng.integers(0, 3000, 700).tolist(), 2, 32, 94, 1536))  # S > 512: two chunks
    for k in range(10):
        S = int(rng.integers(1, 40))
        B = int(rng.choice([16, 32, 64]))
        maxb = int(rng.integers(1, 20))
        lens = rng.integers(0, maxb * B + 1, S).tolist()
        cases.append((lens, int(rng.choice([1, 2, 8])), B, maxb, int(rng.integers(1, 300))))
    return cases


@pytest.mark.parametrize("seg_runs", [8, 4])
@pytest.mark.parametrize("case", range(len(_cases())))
def test_schedule_covers_every_tile_once(case, seg_runs):
    _check_case(case, seg_runs, 64)


@pytest.mark.parametrize("balance", [62, 20, 110])
@pytest.mark.parametrize("case", range(len(_cases())))
def test_schedule_with_xcd_shares(case, balance):
    _check_case(case, 8, balance)


def _check_case(case, seg_runs, balance):
    ctx, hkv, B, maxb, nwaves = _cases()[case]
    Nt, visits, slots, records = run_schedule(ctx, hkv, B, maxb, nwaves, seg_runs, balance)
    assert len(visits) == Nt and all(v == 1 for v in visits.values())
    table_tokens = maxb * B
    touched = {}
    for slot, (u, w) in slots.items():
        touched.setdefault(u, []).append(w)
    for i, c in enumerate(ctx):
        for g in range(hkv):
            u = i * hkv + g
            if tiles_of(c, table_tokens) == 0:
                assert u not in records
                continue
            first, count = records[u]
            if count == 1:
                assert u not in touched
            else:
                ws = sorted(touched[u])
                assert ws == list(range(ws[0], ws[0] + count)) and first == u + ws[0]
