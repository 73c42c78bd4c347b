"""Plain fp64 CPU oracle for permuted block-sparse attention prefill.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg
of ``bench.py`` may import or call anything in this package.  The GPU library never does, and
nothing here imports the GPU library: the two share no code.

``pbsa_oracle`` follows the pages' definitions step by step in NumPy fp64 (library matmul,
sort and exp as primitives).  ``brute`` re-derives every stage with pure-Python loops and
``math.fsum`` for tiny shapes.  Every function is pinned by the CPU tests (closed forms,
invariants, the brute force and a hand-derived example); none is marked "parity unpinned".
"""
from .pbsa_oracle import (  # noqa: F401
    block_mask,
    block_range,
    block_sparse_attention,
    calibrate_thresholds,
    dense_attention,
    default_scale,
    kept_bitmap,
    key_importance,
    key_rows_of_block,
    mask_from_patterns,
    mass_cut,
    num_blocks,
    num_segments,
    pool_blocks,
    pool_permuted_blocks,
    pooled_block_logits,
    query_guide_scores,
    query_permutation,
    prefix_kv_ranking,
    prefix_offset,
    prefix_ranking_length,
    ranked_blocks,
    s2o_attention,
    s2o_gain_ratios,
    s2o_prefix_attention,
    s2o_prefix_gain_ratios,
    sample_attention_mask,
    sampled_masses,
    segment_of_block,
    segment_permutation,
    segment_representatives,
    tile_max,
    tri_offset,
    trunk_rows,
    two_pass_attention_on,
)
