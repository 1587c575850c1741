"""rsx: ring reduce-scatter, all-gather and all-reduce for one MI355X (gfx950).

W virtual ranks are W buffers in one GPU's HBM.  The kernels live in the HIP
library ``librsx.so`` (C ABI in ``include/rsx.h``), loaded on first use; the
Python layer only marshals tensors into pointers and counts.
"""
from .api import (  # noqa: F401
    ALGOS, DTYPES, OPS, AllReduce, AllReduceBucketed, BucketedAllReduce, FusedAllReduce, FusePack, FuseUnpack, ReduceScatter,
    GroupedAllReduce, TensorFusionAllReduce, fusion_groups, fusion_threshold,
    all_gather, all_reduce,
    all_reduce_bucketed, bucket_count, fuse_pack, fuse_unpack, fused_all_reduce, reduce_scatter,
    segment_begin, version, SparseAllReduce, sparse_all_reduce, topk_count, SPARSE_MODES,
    occupancy_caps,
)
from ._lib import RsxError  # noqa: F401
