"""CPU oracle for EAGLE-3 mixed attention. Test infrastructure only: imported
by the tests, the smoke check and the benchmark's CPU-baseline leg, never by
the product path. See eagle3_oracle.py."""
from .eagle3_oracle import (  # noqa: F401
    LAYOUTS, query_positions, doc_start, visible_mask, pair_count, ring_steps,
    forward_head, forward, backward_head, backward, block_attention, lse_merge,
)
