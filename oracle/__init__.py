"""fp64 CPU oracle of the FlashPrefill block-sparse prefill path.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this package:
only the tests, `__graft_entry__.smoke()` and the `cpu_baseline` leg of
`bench.py` may call it.  It shares no code with the HIP library.
"""

from .flashprefill import (  # noqa: F401
    BAND_REL,
    OracleProblem,
    attend_block,
    bf16_round,
    block_scores,
    csr_from_results,
    decode_bf16,
    decode_e4m3,
    decode_storage,
    forced_blocks,
    pool_blocks,
    pooled_all,
    run_pipeline,
    rank_order,
    select_row,
    select_row_topk,
    select_row_topp,
)
