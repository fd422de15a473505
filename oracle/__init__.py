"""fp64 CPU oracle for training-free Dual Chunk Attention (DCA).

TEST INFRASTRUCTURE ONLY.  Nothing in the product library imports, calls or
links anything in this package; only the tests, the smoke check and the CPU
baseline leg of the benchmark use it.  It shares no code with the HIP path.
"""
from .dca_ref import (  # noqa: F401
    chunk_size,
    rope_inv_freq,
    rope_rotate,
    key_position,
    query_positions,
    relation,
    relative_position_table,
    remap_positions,
    rope_remap_ref,
    dca_prefill_ref,
    dca_prefill_formB,
    dca_decode_ref,
    dca_prefill_chunk_ref,
    paged_rows,
    dca_decode_paged_ref,
    dca_prefill_chunk_paged_ref,
    MAP_KEY,
    MAP_Q_INTRA,
    MAP_Q_SUCC,
    MAP_Q_INTER,
    MAP_PLAIN,
)
from .selfextend_ref import (  # noqa: F401
    MAP_SE_KEY_GROUPED,
    MAP_SE_Q_GROUPED,
    NEIGHBOR,
    GROUPED,
    se_relation,
    se_key_position,
    se_query_position,
    se_relative_position_table,
    se_remap_positions,
    se_rope_remap_ref,
    selfextend_prefill_ref,
    selfextend_prefill_formB,
    selfextend_decode_ref,
)
from .coarse_fine_ref import (  # noqa: F401
    coarse_fine_distance_table,
    coarse_fine_positions,
    coarse_fine_key_positions,
    coarse_fine_prefill_ref,
    coarse_fine_prefill_formB,
    coarse_fine_key_remap_ref,
    coarse_fine_decode_ref,
)
