"""CPU oracle (test infrastructure only): plain NumPy definition of the
tile-hybrid dense / 2:4 (and 4:8) pruning, the HYB1 stream format and the float64
reference product.  Never imported by the product path."""
from .hyb_oracle import (  # noqa: F401
    DTYPES, META_KINDS, PATTERNS, check_shape, dense_index, group_shape, kept_positions,
    kept_positions_nm, magnitude_key, mask8, meta_word_index, nibble, pack, plan,
    positions_from_mask8, positions_from_nibble, prune, ref_lowrank, ref_matmul, ref_rows,
    sparsity, unpack, value_index, value_index8, widen, within_bound,
)
