"""The allocation-free decode entry point (paged_attn_decode_noalloc) against paged_attn_decode.

Two calls in a row on one GPU, the second with a smaller batch than the first (the device scratch
keeps the first call's contents), then a call on the generic kernel (fp32, partitions of 64 tokens,
so its partials also go through the scratch).  Each output must be bit-identical to
paged_attn_decode's on the same inputs (the same kernels and wave split run) and within the
oracle's tolerance.
"""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_276_amd as pkv
from gpu_util import assert_parity, say, to_device
from workloads import make_custom

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible AMD GPU"
    pkv.version()


def _against_decode(w, oracle_impl, what, **kw):
    say(f"[gpu] noalloc {what}: S={w.num_seqs} Hq={w.num_q_heads} Hkv={w.num_kv_heads} {w.dtype} {kw}")
    d = to_device(w)
    pkv.paged_kv_write(d["k_new"], d["v_new"], d["slot_mapping"], d["k_cache"], d["v_cache"])
    want = pkv.paged_attn_decode(d["q"], d["k_cache"], d["v_cache"], d["block_tables"], d["context_lens"],
                                 w.scale, **kw)
    torch.cuda.synchronize()
    kind = pkv.last_launch_info()["kernel"]
    out = torch.full_like(want, float("nan"))
    pkv.paged_attn_decode_noalloc(d["q"], d["k_cache"], d["v_cache"], d["block_tables"], d["context_lens"],
                                  w.scale, out, **kw)
    torch.cuda.synchronize()
    assert pkv.last_launch_info()["kernel"] == kind
    assert torch.equal(out, want), f"{what}: differs from paged_attn_decode"
    ratio = assert_parity(out, oracle.decode_step(w, oracle=oracle_impl).out, what)
    say(f"[gpu] noalloc {what}: {kind} kernel, equal to paged_attn_decode, err/allowed {ratio:.4f}")


def test_noalloc_matches_decode(oracle_impl):
    rng = np.random.Generator(np.random.PCG64(401))
    lengths = np.clip(np.rint(np.exp(rng.normal(np.log(1024.0), 1.0, size=160))), 1, 8192).astype(int).tolist()
    big = make_custom(lengths, 32, 8, 128, 16, torch.bfloat16, seed=401, pool_fill=0.9)
    small = make_custom([1, 17, 300, 2000, 33], 32, 8, 128, 16, torch.bfloat16, seed=402)
    _against_decode(big, oracle_impl, "first call, 160 sequences")
    _against_decode(small, oracle_impl, "second call, 5 sequences")
    fp32 = make_custom([5, 200, 700], 4, 2, 128, 16, torch.float32, seed=403)
    _against_decode(fp32, oracle_impl, "generic kernel", partition_tokens=64)
    _against_decode(small, oracle_impl, "fast kernel after the generic one, 64 waves", grid_waves=64)


def test_noalloc_falls_back_to_generic_when_the_fast_plan_is_too_large(oracle_impl):
    """16 query heads per KV head (and head dim 256) run on the split-run kernel, whose workspace
    (16 rows for each of up to PKV_MAX_GRID_WAVES partial slots) exceeds the scratch array: with
    the kernel left to the library the call runs the generic kernel, bit-identical to
    paged_attn_decode with the generic kernel forced; forcing the fast kernel is refused."""
    for hq, hkv, d, seed in ((32, 2, 128, 404), (16, 4, 256, 405)):
        w = make_custom([1, 17, 300, 2000, 33], hq, hkv, d, 16, torch.bfloat16, seed=seed)
        desc = pkv.CacheDesc(w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim, 1)
        plan = pkv.paged_attn_plan(w.num_seqs, w.num_q_heads, w.max_blocks_per_seq, desc)
        assert plan["kernel"] == "fast" and plan["workspace_bytes"] > pkv.NOALLOC_SCRATCH_BYTES
        say(f"[gpu] noalloc fallback: Hq={hq} Hkv={hkv} d={d}")
        dd = to_device(w)
        pkv.paged_kv_write(dd["k_new"], dd["v_new"], dd["slot_mapping"], dd["k_cache"], dd["v_cache"])
        want = pkv.paged_attn_decode(dd["q"], dd["k_cache"], dd["v_cache"], dd["block_tables"], dd["context_lens"],
                                     w.scale, kernel=pkv.PKV_KERNEL_GENERIC)
        out = torch.full_like(want, float("nan"))
        pkv.paged_attn_decode_noalloc(dd["q"], dd["k_cache"], dd["v_cache"], dd["block_tables"],
                                      dd["context_lens"], w.scale, out)
        torch.cuda.synchronize()
        assert pkv.last_launch_info()["kernel"] == "generic"
        assert torch.equal(out, want)
        assert_parity(out, oracle.decode_step(w, oracle=oracle_impl).out, f"noalloc fallback d{d}")
        with pytest.raises(pkv.PkvError):
            pkv.paged_attn_decode_noalloc(dd["q"], dd["k_cache"], dd["v_cache"], dd["block_tables"],
                                          dd["context_lens"], w.scale, out, kernel=pkv.PKV_KERNEL_FAST)

