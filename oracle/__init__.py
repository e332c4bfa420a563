"""fp64 CPU oracle for column-sparse masked attention (test infrastructure only)."""
from .oracle import (  # noqa: F401
    FULL, PARTIAL, SKIP, attention, backward, classify, classify_tile, column_gradients, decode_e4m3,
    dense_mask,
    exact_tile_classes, forward, forward_fp8, head_backward, head_forward, key_block_summary,
    localize_bounds,
    mask_head, rows_seeing, upcast_bf16,
)
