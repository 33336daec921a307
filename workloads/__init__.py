"""Seeded synthetic inputs for one paged decode step.

This module builds inputs only: context lengths, a block pool with its
per-sequence block tables, the new token's slot, and N(0,1) values for q, the
cached K/V and the new K/V.  It computes no attention and copies no K/V into
slots; both the CPU oracle (``oracle/``) and the GPU path consume what it
returns, and neither imports the other.

Building a block table needs the block count of a sequence, ceil(n / B); this
is the allocator's job on the pages (page "x321.org/?p=939", section
"PagedAttention borrows an operating-system trick": a sequence asks how many
free blocks it needs and grows by whole blocks).  The oracle carries its own
copy of that arithmetic, pinned to the pages' worked numbers.
"""

from .configs import (  # noqa: F401
    CONFIG_NAMES,
    MULTI_CONFIG_NAMES,
    MultiWorkload,
    Workload,
    make_config,
    make_custom,
    make_multi,
    make_multi_config,
    poison_value_bits,
)
