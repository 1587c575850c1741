"""CPU oracle (test infrastructure only; see ``oracle.collectives``)."""
from .collectives import *  # noqa: F401,F403
from .collectives import (  # noqa: F401
    all_gather, all_reduce, block_at_step, block_vs_step_table, bf16_to_f32,
    bucketed_all_reduce, f16_to_f32, f32_to_bf16, f32_to_f16, fold, fuse_offsets, fuse_pack, fuse_unpack,
    fused_all_reduce, fusion_groups, grouped_all_reduce, half_wire_all_reduce, naive_all_reduce, naive_fold_order, reduce_scatter,
    ring_fold_order, segment_bounds,
)
from .sparse import (  # noqa: F401,E402
    sparse_all_reduce, sparse_combine, sparsify_threshold, sparsify_topk, topk_count,
)
