"""Plant plausible mistakes in copies of the oracle and check that a pin catches each one.

Every mutant is a one-spot text change of ``oracle/oracle.c`` (a dropped term, a
wrong sign or index, a transposed operand, ...).  It is compiled into a
temporary library and the pins run against it in a child process (a mutant may
crash).  The test fails if any mutant passes every pin.
"""

import os
import subprocess
import sys
import tempfile

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTANTS = {
    "gqa_interleaved": ("const int32_t g = h / group;", "const int32_t g = h % num_kv_heads;"),
    "scale_dropped": ("s[j] = scale * acc;", "s[j] = acc;"),
    "scale_squared": ("s[j] = scale * acc;", "s[j] = scale * scale * acc;"),
    "table_index_mod": ("block_tables[(int64_t)i * max_blocks_per_seq + j / block_size]",
                        "block_tables[(int64_t)i * max_blocks_per_seq + j % max_blocks_per_seq]"),
    "offset_reversed": ("int64_t off = j % block_size;", "int64_t off = block_size - 1 - j % block_size;"),
    "last_token_dropped": ("for (j = 0; j < n; ++j) {\n        int64_t phys",
                           "for (j = 0; j + 1 < n; ++j) {\n        int64_t phys"),
    "k_v_swapped": ("kh[j * D + x] = load_elem(k_cache, base + x, elem_bytes);",
                    "kh[j * D + x] = load_elem(v_cache, base + x, elem_bytes);"),
    "no_normalisation": ("out_row[x] /= denom;", "out_row[x] /= 1.0;"),
    "exp_sign": ("s[j] = exp(s[j] - m);", "s[j] = exp(m - s[j]);"),
    "bf16_shift": ("u = ((uint32_t)b) << 16;", "u = ((uint32_t)b) << 15;"),
    "query_head_is_kv_head": ("qv[x] = load_elem(q, ((int64_t)i * num_q_heads + h) * D + x, elem_bytes);",
                              "qv[x] = load_elem(q, ((int64_t)i * num_q_heads + g) * D + x, elem_bytes);"),
    "layout_token_major": ("base = ((phys * num_kv_heads + g) * block_size + off) * D;",
                           "base = ((phys * block_size + off) * num_kv_heads + g) * D;"),
    "wrong_sequence_row": ("qv[x] = load_elem(q, ((int64_t)i * num_q_heads + h) * D + x, elem_bytes);",
                           "qv[x] = load_elem(q, ((int64_t)(i == 0 ? 0 : i - 1) * num_q_heads + h) * D + x, elem_bytes);"),
    "write_block_offset_swapped": ("blk = slot / block_size;\n        off = slot % block_size;",
                                   "blk = slot % block_size;\n        off = slot / block_size;"),
    "write_v_dropped": ("memcpy((char *)v_cache + dst, (const char *)v_new + src, (size_t)row_bytes);", ""),
    "write_skip_ignored": ("if (slot < 0)\n            continue;", "if (slot < -1)\n            continue;"),
    "write_head_fixed": ("int64_t dst = ((blk * num_kv_heads + h) * block_size + off) * row_bytes;",
                         "int64_t dst = ((blk * num_kv_heads + 0) * block_size + off) * row_bytes;"),
    "multi_sees_next_token": ("const int64_t visible = pos + 1;", "const int64_t visible = pos + 2 < n ? pos + 2 : n;"),
    "multi_mask_top_left": ("const int64_t pos = n - ql + (qrow - cu_q[s]);", "const int64_t pos = qrow - cu_q[s];"),
    "multi_previous_query_row": ("qv[x] = load_elem(q, (qrow * num_q_heads + h) * D + x, elem_bytes);",
                                 "qv[x] = load_elem(q, ((qrow > 0 ? qrow - 1 : 0) * num_q_heads + h) * D + x, elem_bytes);"),
    "multi_value_is_key": ("out_row[x] += s[t] * load_elem(v_cache, base + x, elem_bytes);",
                           "out_row[x] += s[t] * load_elem(k_cache, base + x, elem_bytes);"),
}

CHILD = r"""
import sys
sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})
import oracle, pins
o = oracle.Oracle({lib!r})
caught = []
for pin in pins.ORACLE_PINS:
    try:
        pin(o)
    except Exception as e:  # AssertionError or an oracle error report
        caught.append(pin.__name__)
print("CAUGHT", ",".join(caught))
"""


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    before, after = MUTANTS[name]
    with open(oracle.SOURCE) as f:
        src = f.read()
    assert src.count(before) >= 1, f"mutation site for {name} not found"
    mutated = src.replace(before, after, 1)
    cfile = tmp_path / "oracle_mut.c"
    cfile.write_text(mutated)
    lib = str(tmp_path / "liboracle_mut.so")
    oracle.build(str(cfile), lib)
    code = CHILD.format(root=ROOT, tests=os.path.join(ROOT, "tests"), lib=lib)
    p = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    if p.returncode != 0:
        return  # the mutant crashed the pins: caught
    line = [l for l in p.stdout.splitlines() if l.startswith("CAUGHT")][-1]
    caught = [c for c in line.split(" ", 1)[1].split(",") if c]
    assert caught, f"mutant {name} passed every pin"
