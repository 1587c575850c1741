"""CPU oracle of the ring reduce-scatter, all-gather and all-reduce.

TEST INFRASTRUCTURE.  Only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run this module.  The HIP
library never calls it, and it shares no code with the HIP library: no
kernels, headers, helpers, tables or constants.  It is deliberately plain and
slow: NumPy arrays, one Python loop per ring step, nothing blocked, fused or
reordered beyond what the definitions state.

Sources (web pages this follows):

* [NC] NCCL 1.x ``src/reduce_scatter.cu`` (pytorch mirror, "Git at Google"):
  the ``GetBlock`` schedule function, the reduce-scatter kernel's step 0
  (copy own block to the next GPU), steps 1..W-2 (reduce received partial
  with local input, pass on) and step W-1 (reduce into the output), and the
  host launcher's 4-GPU block-vs-step table for ``userFromRing = {1,2,0,3}``.
  Its op set is sum/prod/max/min and its ``recvcount`` is the per-rank output
  length; the per-rank input is ``W * recvcount``.
* [DP] "Distributed primitives" (notes): all-reduce is a reduction (sum, max
  or average) followed by a broadcast; reduce-scatter reduces, then splits the
  result so each node gets one segment; all-gather concatenates every node's
  piece onto every node; Ring AllReduce = ReduceScatter + AllGather.
* [SG] Apache SINGA ``src/io/communicator.cc``, ``fusedSynch``: tensors are
  copied back to back into one fusion buffer, all-reduced, and copied out at
  the same running offsets.  [HV] Horovod ``operations.cc``,
  ``PerformOperation``: the same memcpy-in / all-reduce / memcpy-out on the
  fused buffer.
* [MX] "Add scatter reduce for JACCL#3901": a naive all-reduce is kept for
  messages of at most 32 KB.
* [SG] ``synchHalf`` / ``fusedSynchHalf``: fp32 gradients are converted to
  half (``float2half``), all-reduced as ``ncclHalf``, and converted back
  (``half2float``) into the fp32 tensors: fp16 as the wire format of an fp32
  all-reduce (dtype ``"f32h"`` here).

Precision.  The pages fix it: the NCCL kernel reduces in the element type.
Its ring buffers (``ThisBuffer`` / ``NextBuffer`` of
``ReduceScatterKernelArgs<T>``) hold ``T``, and every step from 1 on reduces
the partial it received with its own input into one of them, so the partial
is stored as ``T`` after every step.  Hence fp32, fp64 and fp16 (the page's
``half``) are folded with IEEE round-to-nearest-even operations in their own
type, one per ring step, and int8 / int32 / int64 / uint64 with wrapping
integer arithmetic.  bf16 is not on the page's type list; its workload defines
it as bf16 in, fp32 accumulate, bf16 out: widened exactly to fp32, folded in
fp32 and rounded once to bf16 at the end.

Readings where the pages are silent:

* ring = identity (``userFromRing[i] = i``): rank ``r`` is ring position ``r``;
* the segment of a rank that does not divide evenly in an all-reduce is the
  ceil split ``S = ceil(count / W)``, segment ``k = [min(kS,count), min((k+1)S,count))``;
* max/min fold by compare-and-select, ``acc = x if x > acc else acc`` (``<``
  for min): the earlier of two equal values (``+0``/``-0``) is kept, a NaN in
  ``acc`` is kept, a later NaN is ignored;
* ``avg`` = the sum fold, then one division by W in the accumulation type
  (IEEE division for floats; signed integers truncate toward zero, uint64
  floors);
* ``prod`` multiplies in the accumulation type (integers wrap);
* fp16 (the page's ``half``; its functors are off-page): each step's result
  is the exact result of the operation rounded to nearest-even half (NumPy's
  float16 arithmetic), so a half partial enters the next step; ``avg``
  divides the half fold by W and rounds the quotient to half; the naive fold
  rounds the same way, in rank order;
* ``"f32h"`` (fp32 data, half on the wire): each fp32 input is rounded to
  half (``float2half``), the halves are folded as fp16 is, and the half
  result is widened to fp32 for the output (``half2float``);
* bf16 rounding: round-to-nearest-even on the fp32 bits, NaN -> quiet NaN
  with the sign kept (``sign | 0x7FC0``), overflow to +-inf as RNE gives;
* the naive all-reduce folds in rank order 0..W-1;
* fusion offsets are back to back in list order, with no padding.
"""
from __future__ import annotations

import numpy as np

OPS = ("sum", "prod", "max", "min", "avg")
DTYPES = ("f32", "bf16", "i32", "f64", "f16", "i64", "u64", "i8", "f32h")

# storage type of each dtype (bf16 and f16 as their 16-bit patterns)
STORAGE = {"f32": np.float32, "bf16": np.uint16, "i32": np.int32, "f64": np.float64,
           "f16": np.uint16, "i64": np.int64, "u64": np.uint64, "i8": np.int8,
           "f32h": np.float32}
# integer types and the unsigned type of the same width (wrap-around arithmetic)
_UNSIGNED = {np.dtype(np.int8): np.uint8, np.dtype(np.int32): np.uint32,
             np.dtype(np.int64): np.uint64, np.dtype(np.uint64): np.uint64}

# --------------------------------------------------------------- schedule ----


def block_at_step(index: int, step: int, user_from_ring) -> int:
    """Block that ring position ``index`` works on at ``step`` [NC ``GetBlock``].

    The position ``index - 1 - step`` (mod W) of ``user_from_ring``: at the last
    step a position holds its own block, and each earlier step holds the block
    the next position will hold one step later.
    """
    w = len(user_from_ring)
    return int(user_from_ring[(w + index - 1 - step) % w])


def block_vs_step_table(user_from_ring) -> np.ndarray:
    """Rows = steps 0..W-1, columns = ring positions 0..W-1 [NC host-launcher table]."""
    w = len(user_from_ring)
    return np.array([[block_at_step(i, s, user_from_ring) for i in range(w)]
                     for s in range(w)], dtype=np.int64)


def ring_fold_order(k: int, world: int) -> list[int]:
    """Ranks whose inputs enter block ``k``, in the order the ring folds them.

    Walk the schedule with the identity ring: at step 0 the position whose block
    is ``k`` copies its input to the next position; at every later step the
    position holding block ``k`` folds its own input into the partial it received.
    """
    ident = list(range(world))
    order = []
    for step in range(world):
        holders = [i for i in range(world) if block_at_step(i, step, ident) == k]
        assert len(holders) == 1
        order.append(holders[0])
    return order


def naive_fold_order(world: int) -> list[int]:
    """Rank order 0..W-1 for the naive (direct-sum) all-reduce [MX]."""
    return list(range(world))


def segment_bounds(count: int, world: int) -> list[tuple[int, int]]:
    """All-reduce split of ``count`` elements into W segments (ceil split)."""
    s = -(-count // world) if world > 0 else 0
    return [(min(k * s, count), min((k + 1) * s, count)) for k in range(world)]


# ------------------------------------------------------------- bf16 bits -----


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 exactly (they are the top 16 fp32 bits)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 bit patterns, to nearest, ties to even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    keep_lsb = (u >> np.uint64(16)) & np.uint64(1)
    out = ((u + np.uint64(0x7FFF) + keep_lsb) >> np.uint64(16)) & np.uint64(0xFFFF)
    nan = np.isnan(x)
    out[nan] = ((u[nan] >> np.uint64(16)) & np.uint64(0x8000)) | np.uint64(0x7FC0)
    return out.astype(np.uint16)


# ------------------------------------------------------------------ folds ----


def f16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen IEEE half bit patterns to fp32 (exact)."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float32)


def f32_to_f16(x: np.ndarray) -> np.ndarray:
    """Round fp32 to IEEE half bit patterns, to nearest, ties to even (NumPy's conversion)."""
    with np.errstate(over="ignore"):    # beyond the half range is +-inf, as RNE gives
        return np.asarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def _widen(x: np.ndarray, dtype: str) -> np.ndarray:
    """Storage -> accumulation type: bf16 bits -> fp32; f16 bits -> float16 values
    (the ring partial stays half); fp32 -> half for ``"f32h"`` (``float2half`` on
    the sender); every other type as is."""
    if dtype == "bf16":
        return bf16_to_f32(x)
    if dtype == "f16":
        return np.asarray(x, dtype=np.uint16).view(np.float16)
    if dtype == "f32h":
        return np.asarray(x, dtype=np.float32).astype(np.float16)
    if dtype in STORAGE:
        return np.asarray(x, dtype=STORAGE[dtype])
    raise ValueError(dtype)


def _combine(op: str, acc: np.ndarray, x: np.ndarray) -> np.ndarray:
    """One ring step: partial received so far, combined with the local input.

    Integer sums and products wrap modulo 2^bits: they are computed in the
    unsigned type of the same width, whose low bits equal the two's-complement
    result.
    """
    if op in ("sum", "avg", "prod"):
        u = _UNSIGNED.get(acc.dtype)
        if u is not None:
            a, b = acc.view(u), x.astype(acc.dtype).view(u)
            return (a * b if op == "prod" else a + b).astype(u).view(acc.dtype)
        return acc * x if op == "prod" else acc + x
    if op == "max":
        return np.where(x > acc, x, acc)
    if op == "min":
        return np.where(x < acc, x, acc)
    raise ValueError(op)


def _finish(op: str, acc: np.ndarray, world: int, dtype: str) -> np.ndarray:
    """Average (if asked) in the accumulation type, then back to the storage type."""
    if op == "avg":
        if acc.dtype.kind == "i":          # signed: truncate toward zero
            q = acc // acc.dtype.type(world)
            fix = (acc < 0) & (acc % acc.dtype.type(world) != 0)
            acc = (q + fix.astype(acc.dtype)).astype(acc.dtype)
        elif acc.dtype.kind == "u":
            acc = acc // acc.dtype.type(world)
        else:
            acc = (acc / acc.dtype.type(world)).astype(acc.dtype)
    if dtype == "bf16":
        return f32_to_bf16(acc)
    if dtype == "f16":                      # the half result, as bits
        return np.ascontiguousarray(acc, dtype=np.float16).view(np.uint16)
    if dtype == "f32h":                     # the half result, then half2float
        return np.asarray(acc, dtype=np.float16).astype(np.float32)
    return acc


def fold(inputs, order, op: str, dtype: str, lo: int = 0, hi: int | None = None) -> np.ndarray:
    """Fold ``inputs[order[0]][lo:hi]``, then each later rank of ``order``, then finish."""
    if op not in OPS:
        raise ValueError(f"op {op!r}")
    hi = len(inputs[0]) if hi is None else hi
    # overflow to +-inf and inf - inf = NaN are the IEEE results, not errors
    with np.errstate(over="ignore", invalid="ignore"):
        acc = _widen(inputs[order[0]][lo:hi], dtype).copy()
        for r in order[1:]:
            acc = _combine(op, acc, _widen(inputs[r][lo:hi], dtype))
        return _finish(op, acc, len(inputs), dtype)


# ------------------------------------------------------------ collectives ----


def reduce_scatter(inputs, op: str = "sum", dtype: str = "f32") -> list[np.ndarray]:
    """Reduce-scatter: rank ``k`` receives block ``k`` of the reduction [NC, DP].

    Every rank holds ``N = W * recvcount`` elements; block ``k`` is elements
    ``[k*recvcount, (k+1)*recvcount)`` of every rank, folded in ring order.
    """
    w = len(inputs)
    n = len(inputs[0])
    if any(len(x) != n for x in inputs):
        raise ValueError("ranks differ in length")
    if n % w:
        raise ValueError("reduce-scatter needs a per-rank length divisible by W")
    s = n // w
    return [fold(inputs, ring_fold_order(k, w), op, dtype, k * s, (k + 1) * s)
            for k in range(w)]


def all_gather(segments) -> list[np.ndarray]:
    """All-gather: every rank receives the concatenation of all ranks' pieces [DP]."""
    full = np.concatenate([np.asarray(s) for s in segments])
    return [full.copy() for _ in segments]


def all_reduce(inputs, op: str = "sum", dtype: str = "f32") -> list[np.ndarray]:
    """Ring all-reduce = reduce-scatter, then all-gather [DP *In practice*].

    Segment ``k`` of the ceil split is folded in ring order from rank
    ``(k+1) % W`` round to rank ``k``; every rank then receives all segments.
    """
    w = len(inputs)
    n = len(inputs[0])
    segs = [fold(inputs, ring_fold_order(k, w), op, dtype, lo, hi)
            for k, (lo, hi) in enumerate(segment_bounds(n, w))]
    return all_gather(segs)


def naive_all_reduce(inputs, op: str = "sum", dtype: str = "f32") -> list[np.ndarray]:
    """Naive all-reduce: every element folded in rank order, result on every rank [MX]."""
    out = fold(inputs, naive_fold_order(len(inputs)), op, dtype)
    return [out.copy() for _ in inputs]


def bucketed_all_reduce(inputs, bucket: int, op: str = "sum", dtype: str = "f32") -> list[np.ndarray]:
    """All-reduce of consecutive buckets of ``bucket`` elements, one after another.

    Each bucket is an all-reduce of its own, with its own segments ["Distributed
    primitives", bucketed ring all-reduce].
    """
    n = len(inputs[0])
    outs = [np.empty_like(np.asarray(x)) for x in inputs]
    start = 0
    while start < n:
        stop = min(start + bucket, n)
        part = all_reduce([x[start:stop] for x in inputs], op, dtype)
        for r in range(len(inputs)):
            outs[r][start:stop] = part[r]
        start = stop
    return outs


def half_wire_all_reduce(inputs, op: str = "sum", algo: str = "ring") -> list[np.ndarray]:
    """fp32 all-reduce with half on the wire [SG ``synchHalf``].

    Each rank converts its fp32 data to half, the half buffers are all-reduced
    as fp16, and each rank converts the half result back to fp32.
    """
    halves = [f32_to_f16(x) for x in inputs]
    red = all_reduce(halves, op, "f16") if algo == "ring" else naive_all_reduce(halves, op, "f16")
    return [f16_to_f32(h) for h in red]


# ------------------------------------------------------------------ fusion ---


def fuse_offsets(counts) -> list[int]:
    """Element offset of each tensor in the fusion buffer: running sum, no padding [SG, HV]."""
    offs, run = [], 0
    for c in counts:
        offs.append(run)
        run += int(c)
    return offs


def fuse_pack(tensors) -> np.ndarray:
    """Copy tensors back to back, in list order, into one buffer [SG ``fusedSynch``]."""
    return np.concatenate([np.asarray(t).ravel() for t in tensors]) if len(tensors) else np.empty(0)


def fuse_unpack(fused: np.ndarray, counts) -> list[np.ndarray]:
    """Split a fusion buffer back into tensors of ``counts`` elements at the same offsets."""
    return [np.asarray(fused)[o:o + int(c)].copy() for o, c in zip(fuse_offsets(counts), counts)]


def fusion_groups(sizes_bytes, dtypes, threshold: int) -> list[tuple[int, int]]:
    """Horovod's fusion of consecutive all-reduce requests [HV BackgroundThreadLoop].

    Walk the tensors in order.  A group starts at the first tensor not yet
    grouped and keeps taking the next tensor while it has the same dtype and
    the group's bytes plus the next tensor's bytes stay at or below
    ``threshold``; at the first tensor that does not fit, the group ends (no
    tensor is skipped to fill a group).  Returns [start, end) index ranges.
    """
    groups = []
    i, n = 0, len(sizes_bytes)
    while i < n:
        total = int(sizes_bytes[i])
        j = i + 1
        while j < n and dtypes[j] == dtypes[i] and total + int(sizes_bytes[j]) <= threshold:
            total += int(sizes_bytes[j])
            j += 1
        groups.append((i, j))
        i = j
    return groups


def fused_all_reduce(tensors_per_rank, op: str = "sum", dtype: str = "f32") -> list[list[np.ndarray]]:
    """pack -> all-reduce of the fusion buffers -> unpack, per rank [HV ``PerformOperation``]."""
    counts = [len(t) for t in tensors_per_rank[0]]
    fused = [fuse_pack(ts) for ts in tensors_per_rank]
    red = all_reduce(fused, op, dtype)
    return [fuse_unpack(f, counts) for f in red]


def grouped_all_reduce(tensors_per_rank, threshold: int, op: str = "sum",
                       dtype: str = "f32") -> list[list[np.ndarray]]:
    """Fusion groups of the tensor list, each all-reduced as one fusion buffer."""
    sizes = [np.asarray(t).nbytes for t in tensors_per_rank[0]]
    out = [[None] * len(sizes) for _ in tensors_per_rank]
    for lo, hi in fusion_groups(sizes, [dtype] * len(sizes), threshold):
        part = fused_all_reduce([ts[lo:hi] for ts in tensors_per_rank], op, dtype)
        for r in range(len(tensors_per_rank)):
            out[r][lo:hi] = part[r]
    return out
