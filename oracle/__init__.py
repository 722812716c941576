"""CPU float64 oracle for paged KV-cache writes and paged attention.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU
baseline, never by the product path.  It shares no code with the HIP library.

Pins: every function here is checked in ``tests/test_oracle.py`` against things other than itself: the
pages' worked example (indices), brute-force scalar loops, closed forms, a library routine
(``torch.nn.functional.scaled_dot_product_attention`` in float64 on the CPU), and invariances;
``tests/test_oracle_mutants.py`` plants mistakes in it and checks that a pin catches each one.
"""

from .paged_kv import (  # noqa: F401
    BF16,
    FP32,
    attend_head,
    attend_sequence,
    causal_mask,
    default_scale,
    gather_sequence,
    head_scores,
    kv_head_of,
    kv_write,
    last_visible_key,
    logical_block_count,
    paged_attention,
    run_step,
    slot_to_block_offset,
    softmax_rows,
    to_float64,
)
from .block_manager import BlockManagerOracle, CacheError, copy_blocks  # noqa: F401,E402
