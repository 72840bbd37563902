"""Float64 CPU oracle (test infrastructure only; never used by the product path)."""

from .sla_oracle import (  # noqa: F401
    BLOCK, OracleResult, block_counts, classify, compressed_scores, forward,
    compressed_map, linear_branch, num_blocks, phi, phi_elu1, router_pool, soft_topk, sparse_branch,
    token_mask, token_rows,
)
