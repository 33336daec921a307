"""The benchmark's byte accounting and contract, on the CPU.

The roofline's `achieved` figure divides algorithmic bytes by the call's
duration, so the bytes must be the method's own: every cached token's K and V
once (the per-token formula of page x321.org/?p=939, section "First
understand what the KV cache is storing", at one layer), plus q, the fp32
output, the block table entries the call needs and the lengths.  Shared prefix blocks count once
per physical block in the unique figure.
"""

import json
import os
import subprocess
import sys

import numpy as np
import torch

import bench
from oracle.arith import kv_bytes_per_token
from workloads import make_custom

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_algorithmic_bytes_follow_the_per_token_formula():
    lengths = [17, 33, 64, 1, 0]
    w = make_custom(lengths, 32, 8, 128, 16, torch.bfloat16, seed=5, values=False)
    b = bench.algorithmic_bytes(w)
    per_token = kv_bytes_per_token(1, 8, 128, 2)
    assert per_token == 4096
    assert b["kv"] == sum(lengths) * per_token
    assert b["kv_unique"] == b["kv"]  # no block is shared
    assert b["q"] == 5 * 32 * 128 * 2 and b["out"] == 5 * 32 * 128 * 4
    assert b["tables"] == (2 + 3 + 4 + 1 + 0) * 4 + 5 * 4
    assert b["total"] == b["kv"] + b["q"] + b["out"] + b["tables"]


def test_unique_bytes_count_a_shared_prefix_once():
    # three sequences share a 32-token prefix (two blocks of 16); a fourth has no prefix
    lengths = [40, 50, 60, 20]
    w = make_custom(lengths, 8, 2, 64, 16, torch.float32, seed=6, values=False,
                    prefix_groups=[(32, [0, 1, 2])])
    b = bench.algorithmic_bytes(w)
    per_token = kv_bytes_per_token(1, 2, 64, 4)
    assert b["kv"] == sum(lengths) * per_token
    assert b["kv_unique"] == (32 + (40 - 32) + (50 - 32) + (60 - 32) + 20) * per_token
    assert b["total"] - b["total_unique"] == b["kv"] - b["kv_unique"]


def test_several_gpus_are_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, cwd=ROOT, timeout=300)
    assert p.returncode == 2
    line = json.loads(p.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"]


def test_source_stamp_ignores_comments_and_layout(tmp_path):
    a, b, c = (tmp_path / n for n in ("a", "b", "c"))
    for d in (a, b, c):
        d.mkdir()
    (a / "k.hip").write_text("int f(int x) {\n    return x + 1;  // one more\n}\n")
    (b / "k.hip").write_text("/* the successor */\nint f(int x) { return x + 1; }\n")
    (c / "k.hip").write_text("int f(int x) {\n    return x + 2;\n}\n")
    sa, sb, sc = (bench._kernel_source_sha(str(d)) for d in (a, b, c))
    assert sa == sb and sa != sc
    assert len(np.unique([sa, sc])) == 2


def test_heads_override_keeps_the_batch():
    """bench --heads reruns a workload's batch with another head layout: the same lengths, tables and
    slots, the new head counts and dim, and bytes priced on the new layout."""
    from workloads import make_config

    base = make_config("llama8b_b64", values=False)
    other = make_config("llama8b_b64", values=False, heads=(128, 8, 256))
    assert (other.num_q_heads, other.num_kv_heads, other.head_dim) == (128, 8, 256)
    assert np.array_equal(base.context_lens, other.context_lens)
    assert np.array_equal(base.block_tables, other.block_tables)
    assert np.array_equal(base.slot_mapping, other.slot_mapping)
    assert bench.algorithmic_bytes(other)["kv"] == 2 * bench.algorithmic_bytes(base)["kv"]
