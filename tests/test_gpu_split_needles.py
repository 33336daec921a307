"""Needles at long context (8 x 32,768 tokens) for the split-run decode kernel: 16 query heads
per KV head at head dim 128, and head dims 64 and 256 with 4 query heads per KV head.

The same construction as the needle test of decode_fast_kernel (key = c q_h with
scale c |q_h|^2 = 20, so head h's output is the softmax mix of its needles' value rows), placed
on both sides of every tile where this kernel hands a (sequence, KV head) unit over from one wave
to the next and every tile where a wave's piece of a unit starts a new LDS segment.  Attention is
the softmax formula of page "x321.org/?p=939", section "First understand what the KV cache is
storing"; the walk follows the block table in the context's logical order (page
"chenhuiyu.github.io/blog/llm-infra-vllm-en", section "Why naive KV allocation wastes memory").

The kernel's split: all units' tiles end to end, equal runs over the waves (wave w starts at
tile Nt w / W, rounded down); a run is cut at unit ends into pieces, and each piece is walked in
segments of 64 tiles from its own first tile.
"""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_276_amd as pkv
from gpu_util import run_step, say, to_device
from test_fast_schedule import TOK, Split
from test_gpu_long_needles import _check, _plant
from workloads import make_custom

pytestmark = pytest.mark.gpu

S, HKV, B, N = 8, 8, 16, 32768
TILES = N // TOK  # tiles per (sequence, KV head) unit
SEG = 64  # tiles per LDS segment of a piece

SHAPES = [(128, 128), (32, 64), (32, 256)]  # (query heads, head dim)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible AMD GPU"
    pkv.version()


def _default_grid(hq, d):
    """The wave count the library launches for this shape (the split-run kernel's resident waves)."""
    w = make_custom([40] * S, hq, HKV, d, B, torch.bfloat16, seed=310)
    run_step(w)
    info = pkv.last_launch_info()
    assert info["kernel"] == "fast" and info["xcd_balance"] == 64, info
    assert info["k_stream"] == (d == 256 or S * HKV * 16 <= info["grid"]), info  # few units: K streamed
    return info["grid"]


def _boundary_tiles(grid):
    """Global tile indices (tiles laid out (sequence, KV head, tile)) where a wave's run or a
    later segment of one of its pieces starts."""
    Nt = S * HKV * TILES
    W = min(Nt, grid)
    sp = Split(Nt, W, grid, 64)  # share 64: equal runs
    starts = [sp.start(w) for w in range(W + 1)]
    assert starts == [Nt * w // W for w in range(W + 1)]
    waves, segs = set(starts[:-1]), set()
    for w in range(W):
        t, c1 = starts[w], starts[w + 1]
        while t < c1:
            end = min(c1, (t // TILES + 1) * TILES)  # the piece ends at its unit's end
            segs.update(range(t + SEG, end, SEG))
            t = end
    return waves, segs


def _positions(unit, boundaries, rng):
    lo = unit * TILES
    pos = {0, B - 1, B, N - 1, int(rng.integers(1, N - 1))}
    for t in boundaries:
        if lo < t < lo + TILES:  # the last token before the boundary and the first after it
            b = t - lo
            pos |= {TOK * b - 1, TOK * b}
    return sorted(pos)


@pytest.mark.parametrize("hq,d", SHAPES, ids=[f"G{h // HKV}-d{d}" for h, d in SHAPES])
def test_split_run_needles(oracle_impl, hq, d):
    """The library's own launch, then 7 waves (runs of 18,724 or 18,725 tiles: every hand-over
    inside a unit, and segments that start off the 64-tile grid of the unit)."""
    grid = _default_grid(hq, d)
    waves, segs = _boundary_tiles(grid)
    w7, s7 = _boundary_tiles(7)
    assert all(t % TILES for t in w7 if t), "7 waves should hand over inside units"
    assert any((t % TILES) % SEG for t in s7), "7 waves should start segments off the unit's grid"
    say(f"[gpu] split-run needles G={hq // HKV} d={d}: default grid {grid} ({len(waves)} wave "
        f"starts, {len(segs)} segment starts); 7 waves ({len(s7)} segment starts)")
    w = make_custom([N] * S, hq, HKV, d, B, torch.bfloat16, seed=43 + d)
    rng = np.random.default_rng(43 + d)
    marks = waves | segs | w7 | s7
    planted = _plant(w, {(i, g): _positions(i * HKV + g, marks, rng) for i in range(S) for g in range(HKV)})
    say(f"[gpu] {sum(len(p) for p in planted.values())} needles in {S * HKV} units")
    ref = oracle.decode_step(w, oracle=oracle_impl)
    d0 = to_device(w)  # the second call repeats the write into the same slots: same pool
    _, out = run_step(w, d=d0)
    info = pkv.last_launch_info()
    assert info["kernel"] == "fast" and info["grid"] == grid
    _check(w, planted, out, ref, f"split-run needles G={hq // HKV} d={d}, {grid} waves")
    _, out = run_step(w, d=d0, kernel=pkv.PKV_KERNEL_FAST, grid_waves=7)
    assert pkv.last_launch_info()["grid"] == 7
    _check(w, planted, out, ref, f"split-run needles G={hq // HKV} d={d}, 7 waves")
