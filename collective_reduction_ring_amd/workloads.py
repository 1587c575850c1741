"""Seeded synthetic inputs for the five reduce-scatter / all-reduce workloads.

This module only draws numbers.  It holds none of the collective's arithmetic
(no reduction, no ordering, no rounding rule of its own), so that both the CPU
oracle side and the HIP side of every test can be fed from it without sharing
any of the method.  The one type conversion it performs, fp32 -> bf16 for the
bf16 workload's inputs, is delegated to PyTorch's CPU cast (a library routine).

Every rank ``r`` of workload ``cfg`` draws from ``numpy.random.default_rng((cfg, r))``
so any element can be regenerated on any machine.  Sizes can be scaled down for
quick tests; the value distribution and the structure (W, segment divisibility,
bucket size) are kept.

The workloads follow the gradient-reduction setting of the pages: a ring
reduce-scatter (NCCL 1.x ``src/reduce_scatter.cu``) over W ranks, the
all-reduce = reduce-scatter + all-gather decomposition ("Distributed
primitives", *In practice*), bucketed all-reduce on one stream (same page),
Horovod/SINGA tensor fusion, and the MLX JACCL note on a naive all-reduce for
messages of at most 32 KB ("Add scatter reduce for JACCL#3901").
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

# ---------------------------------------------------------------- constants --
# bf16 all-reduce buckets: 25 MiB of bf16 input bytes per rank.
BUCKET_BYTES = 25 * 1024 * 1024
BF16_BUCKET_ELEMS = BUCKET_BYTES // 2  # 13,107,200 elements

# Message-size sweep of the fused small-tensor workload, KiB per rank.
SWEEP_KIB = (1, 2, 4, 8, 16, 32)


@dataclass(frozen=True)
class Workload:
    """One named workload: W ranks, ``n`` elements per rank, a dtype and ops."""

    cfg: int
    name: str
    world: int          # W, number of (virtual) ranks
    n: int              # elements per rank (reduce-scatter input length)
    dtype: str          # "f32" | "bf16" | "i32"
    dist: str           # value distribution, see ``draw``
    ops: tuple = ("sum",)
    collectives: tuple = ("reduce_scatter",)
    extra: dict = field(default_factory=dict)


WORKLOADS = {
    1: Workload(1, "rs+ar sum fp32, W=4, 4096 elements/rank, uniform[-1,1]",
                4, 4096, "f32", "uniform", ("sum",), ("reduce_scatter", "all_reduce")),
    2: Workload(2, "rs sum fp32, W=8, 67,108,864 elements/rank (256 MiB), N(0, 1e-3)",
                8, 67_108_864, "f32", "normal_1e-3", ("sum",), ("reduce_scatter",)),
    3: Workload(3, "ar avg bf16 (fp32 accumulate), W=8, 134,217,728 elements/rank, "
                   "25 MiB buckets on one stream",
                8, 134_217_728, "bf16", "normal_bf16", ("avg",), ("all_reduce",),
                {"bucket_elems": BF16_BUCKET_ELEMS}),
    4: Workload(4, "rs+ar sum/max int32, W=16, 33,554,432 elements/rank, uniform[-2^20, 2^20]",
                16, 33_554_432, "i32", "int_2e20", ("sum", "max"),
                ("reduce_scatter", "all_reduce")),
    5: Workload(5, "fused pack->ar->unpack fp32, W=4, 200 tensors log-uniform in "
                   "[256, 1,048,576] elements, N(0,1); 1-32 KiB naive-vs-ring sweep",
                4, 0, "f32", "normal", ("sum",), ("fuse_pack", "all_reduce", "fuse_unpack")),
}


def rng_for(cfg: int, rank: int) -> np.random.Generator:
    """The generator of rank ``rank`` in workload ``cfg``."""
    return np.random.default_rng((cfg, rank))


def draw(dist: str, rng: np.random.Generator, n: int) -> np.ndarray:
    """Draw ``n`` values of distribution ``dist``.

    Returns float32 for the fp32 distributions, float64 for ``normal_f64``,
    int32 for ``int_2e20`` and ``int_full``, int64 / uint64 / int8 over their
    whole range for ``int64_full`` / ``uint64_full`` / ``int8_full`` (so sums
    and products wrap), and uint16 bit patterns for ``normal_bf16`` (bf16)
    and ``normal_f16`` (IEEE half).
    """
    if dist == "uniform":
        return rng.uniform(-1.0, 1.0, n).astype(np.float32)
    if dist == "normal_1e-3":
        return rng.standard_normal(n, dtype=np.float32) * np.float32(1e-3)
    if dist == "normal":
        return rng.standard_normal(n, dtype=np.float32)
    if dist == "int_2e20":
        return rng.integers(-(2 ** 20), 2 ** 20, n, dtype=np.int32, endpoint=True)
    if dist == "int_full":
        return rng.integers(-(2 ** 31), 2 ** 31, n, dtype=np.int64).astype(np.int32)
    if dist == "int64_full":
        return rng.integers(np.iinfo(np.int64).min, np.iinfo(np.int64).max, n, dtype=np.int64,
                            endpoint=True)
    if dist == "uint64_full":
        return rng.integers(0, np.iinfo(np.uint64).max, n, dtype=np.uint64, endpoint=True)
    if dist == "int8_full":
        return rng.integers(-128, 127, n, dtype=np.int8, endpoint=True)
    if dist == "normal_f64":
        return rng.standard_normal(n)
    if dist == "normal_f16":
        return to_f16_bits_torch(rng.standard_normal(n, dtype=np.float32))
    if dist == "normal_bf16":
        return to_bf16_bits_torch(rng.standard_normal(n, dtype=np.float32))
    raise ValueError(f"unknown distribution {dist!r}")


def to_bf16_bits_torch(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns through PyTorch's CPU cast (input generation only)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def to_f16_bits_torch(x: np.ndarray) -> np.ndarray:
    """fp32 -> IEEE half bit patterns through PyTorch's CPU cast (input generation only)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.float16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def rank_inputs(cfg: int, n: int | None = None, world: int | None = None,
                dist: str | None = None) -> list[np.ndarray]:
    """Per-rank inputs of workload ``cfg``; ``n``/``world``/``dist`` override its shape."""
    w = WORKLOADS[cfg]
    n = w.n if n is None else n
    world = w.world if world is None else world
    dist = w.dist if dist is None else dist
    # Each rank has its own generator, so drawing them on threads (NumPy
    # releases the GIL for bulk draws) gives the same values as a loop.
    workers = max(1, min(world, 16, os.cpu_count() or 1))
    with ThreadPoolExecutor(workers) as ex:
        return list(ex.map(lambda r: draw(dist, rng_for(cfg, r), n), range(world)))


# ------------------------------------------------------ fused-tensor inputs --
FUSED_SIZE_SEED = (5, 1_000)      # generator of the 200 tensor sizes
FUSED_COUNT = 200
FUSED_MIN, FUSED_MAX = 256, 1_048_576


def fused_sizes(count: int = FUSED_COUNT, lo: int = FUSED_MIN, hi: int = FUSED_MAX) -> np.ndarray:
    """Tensor sizes log-uniform in [lo, hi], rounded to integers and clipped."""
    rng = np.random.default_rng(FUSED_SIZE_SEED)
    s = np.rint(np.exp(rng.uniform(np.log(lo), np.log(hi), count)))
    return np.clip(s, lo, hi).astype(np.int64)


def fused_tensors(world: int = 4, sizes: np.ndarray | None = None) -> list[list[np.ndarray]]:
    """``out[r][i]`` = tensor ``i`` of rank ``r``, N(0,1) fp32."""
    sizes = fused_sizes() if sizes is None else sizes
    out = []
    for r in range(world):
        rng = rng_for(5, r)
        out.append([rng.standard_normal(int(s), dtype=np.float32) for s in sizes])
    return out


# ------------------------------------------------ sparsified all-reduce --
# Gradients of the reduce-scatter headline's shape (W = 8, 64 Mi fp32 per
# rank, N(0, 1e-3)) with an error-feedback residual of the same spread; top-K
# keeps 1 % of the entries, the threshold about 1 % (|g + acc| >= 3.6e-3 for
# g + acc ~ N(0, 1.41e-3)).  The pages give no sizes for this path.
SPARSE_CFG = 6
SPARSE_WORLD = 8
SPARSE_N = 67_108_864
SPARSE_TOPK_FRACTION = 0.01
SPARSE_THRESHOLD = 3.6e-3


def sparse_inputs(n: int = SPARSE_N, world: int = SPARSE_WORLD):
    """(grads, accums): per rank N(0, 1e-3) fp32 from (6, r) and (6, 100 + r)."""
    def one(seed):
        return rng_for(SPARSE_CFG, seed).standard_normal(n, dtype=np.float32) * np.float32(1e-3)
    workers = max(1, min(2 * world, 16, os.cpu_count() or 1))
    with ThreadPoolExecutor(workers) as ex:
        grads = list(ex.map(one, range(world)))
        accums = list(ex.map(one, range(100, 100 + world)))
    return grads, accums


def sweep_inputs(kib: int, world: int = 4) -> list[np.ndarray]:
    """Sweep point of ``kib`` KiB of fp32 per rank, N(0,1)."""
    n = kib * 1024 // 4
    return [rng_for(5, 100 + kib * 16 + r).standard_normal(n, dtype=np.float32)
            for r in range(world)]

