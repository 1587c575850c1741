"""PyTorch-facing wrappers of librsx: lists of device tensors in, kernels out.

PyTorch supplies device memory and the current HIP stream; every element is
computed by the library's HIP kernels.  The wrappers check what the C ABI
cannot see (tensor sizes, dtypes, devices, contiguity) so that a wrong shape
is a Python error and never an out-of-bounds kernel access, then pass raw
pointers and counts.

Semantics (see include/rsx.h): W virtual ranks are W tensors on one GPU.
``reduce_scatter`` folds block k of every rank in ring order (k+1)%W, ..., k
(NCCL 1.x ring reduce-scatter, GetBlock); ``all_reduce`` is reduce-scatter then
all-gather ("Distributed primitives", Ring AllReduce), in one pass unless
``algo="ring_split"``.
"""
from __future__ import annotations

import ctypes
import os
from typing import Sequence

import torch

from . import _lib as L

DTYPES = {torch.float32: L.RSX_FLOAT32, torch.bfloat16: L.RSX_BFLOAT16, torch.int32: L.RSX_INT32,
          torch.float64: L.RSX_FLOAT64, torch.float16: L.RSX_FLOAT16, torch.int64: L.RSX_INT64,
          torch.uint64: L.RSX_UINT64, torch.int8: L.RSX_INT8}
OPS = {"sum": L.RSX_SUM, "max": L.RSX_MAX, "min": L.RSX_MIN, "avg": L.RSX_AVG, "prod": L.RSX_PROD}
ALGOS = {"ring": L.RSX_ALGO_RING, "naive": L.RSX_ALGO_NAIVE, "auto": L.RSX_ALGO_AUTO,
         "ring_fused": L.RSX_ALGO_RING_FUSED, "ring_split": L.RSX_ALGO_RING_SPLIT}


def _launch(plan, name: str, stream) -> None:
    """Call a prepared entry point on the plan's device and the given (or current) stream."""
    if torch.cuda.current_device() == plan.device.index:
        L.check(name, plan.fn(*plan.args, _stream_handle(stream)))
    else:
        with torch.cuda.device(plan.device):
            L.check(name, plan.fn(*plan.args, _stream_handle(stream)))


def _stream_handle(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(ts: Sequence[torch.Tensor], numel: int, what: str, dtype=None, device=None):
    for i, t in enumerate(ts):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{what}[{i}] is not a tensor")
        if t.device.type != "cuda":
            raise ValueError(f"{what}[{i}] is not on a GPU")
        if device is not None and t.device != device:
            raise ValueError(f"{what}[{i}] is on {t.device}, expected {device}")
        if dtype is not None and t.dtype != dtype:
            raise ValueError(f"{what}[{i}] has dtype {t.dtype}, expected {dtype}")
        if not t.is_contiguous():
            raise ValueError(f"{what}[{i}] is not contiguous")
        if t.numel() != numel:
            raise ValueError(f"{what}[{i}] has {t.numel()} elements, expected {numel}")


WIRES = ("f16",)


def _dtype_code(t: torch.Tensor, wire: str | None = None) -> int:
    """Library dtype of ``t``; ``wire="f16"`` selects fp32 data with half on the
    wire (SINGA synchHalf: float2half, half all-reduce, half2float)."""
    if wire is not None:
        if wire not in WIRES:
            raise ValueError(f"unknown wire format {wire!r}; one of {WIRES}")
        if t.dtype != torch.float32:
            raise ValueError(f"the f16 wire format is for float32 tensors, got {t.dtype}")
        return L.RSX_FLOAT32_HALF_WIRE
    try:
        return DTYPES[t.dtype]
    except KeyError:
        raise ValueError(f"unsupported dtype {t.dtype}; one of {sorted(str(d) for d in DTYPES)}") from None


def _op_code(op: str) -> int:
    try:
        return OPS[op]
    except KeyError:
        raise ValueError(f"unknown op {op!r}; one of {sorted(OPS)}") from None


def _ranks(inputs) -> int:
    w = len(inputs)
    if not 1 <= w <= L.RSX_MAX_RANKS:
        raise ValueError(f"need 1..{L.RSX_MAX_RANKS} ranks, got {w}")
    return w


class ReduceScatter:
    """A prepared reduce-scatter over fixed tensors; calling it enqueues one launch.

    ``inputs[r]`` has W*recvcount elements, ``outputs[k]`` recvcount.
    """

    def __init__(self, inputs, outputs, op: str = "sum", wire: str | None = None):
        w = _ranks(inputs)
        if len(outputs) != w:
            raise ValueError("need one output per rank")
        recvcount = outputs[0].numel()
        dev, dt = inputs[0].device, inputs[0].dtype
        _check(inputs, w * recvcount, "inputs", dt, dev)
        _check(outputs, recvcount, "outputs", dt, dev)
        self.device = dev
        self.args = (L.ptr_array([t.data_ptr() for t in inputs]),
                     L.ptr_array([t.data_ptr() for t in outputs]),
                     w, recvcount, _dtype_code(inputs[0], wire), _op_code(op))
        self.fn = L.lib().rsx_reduce_scatter
        self.keep = (list(inputs), list(outputs))

    def __call__(self, stream=None) -> None:
        _launch(self, "rsx_reduce_scatter", stream)


class AllReduce:
    """A prepared all-reduce; every tensor has ``count`` elements.

    ``algo``: "ring" (ring order, one pass), "ring_fused" (the same, named
    by its form), "ring_split" (ring order as a reduce-scatter, then an
    all-gather; W must divide count), "naive" (rank order) or "auto" (naive
    up to RSX_NAIVE_MAX_BYTES per rank, else ring)."""

    def __init__(self, inputs, outputs=None, op: str = "sum", algo: str = "ring",
                 wire: str | None = None):
        w = _ranks(inputs)
        outputs = inputs if outputs is None else outputs
        if len(outputs) != w:
            raise ValueError("need one output per rank")
        count = inputs[0].numel()
        dev, dt = inputs[0].device, inputs[0].dtype
        _check(inputs, count, "inputs", dt, dev)
        _check(outputs, count, "outputs", dt, dev)
        if algo not in ALGOS:
            raise ValueError(f"unknown algo {algo!r}")
        self.device = dev
        self.args = (L.ptr_array([t.data_ptr() for t in inputs]),
                     L.ptr_array([t.data_ptr() for t in outputs]),
                     w, count, _dtype_code(inputs[0], wire), _op_code(op), ALGOS[algo])
        self.fn = L.lib().rsx_all_reduce
        self.keep = (list(inputs), list(outputs))

    def __call__(self, stream=None) -> None:
        _launch(self, "rsx_all_reduce", stream)


def reduce_scatter(inputs, outputs, op: str = "sum", stream=None, wire: str | None = None) -> None:
    """Reduce-scatter ``inputs`` (W tensors of W*n) into ``outputs`` (W tensors of n)."""
    ReduceScatter(inputs, outputs, op, wire)(stream)


def all_gather(inputs, outputs, stream=None) -> None:
    """All-gather: ``outputs[r][k*n:(k+1)*n] = inputs[k]`` for every r, k."""
    w = _ranks(inputs)
    if len(outputs) != w:
        raise ValueError("need one output per rank")
    n = inputs[0].numel()
    dev, dt = inputs[0].device, inputs[0].dtype
    _check(inputs, n, "inputs", dt, dev)
    _check(outputs, w * n, "outputs", dt, dev)
    with torch.cuda.device(dev):
        st = L.lib().rsx_all_gather(L.ptr_array([t.data_ptr() for t in inputs]),
                                    L.ptr_array([t.data_ptr() for t in outputs]),
                                    w, n, _dtype_code(inputs[0]), _stream_handle(stream))
    L.check("rsx_all_gather", st)


def all_reduce(inputs, outputs=None, op: str = "sum", algo: str = "ring", stream=None,
               wire: str | None = None) -> None:
    """All-reduce; ``outputs=None`` reduces in place.  ``wire="f16"``: float32
    tensors reduced with half as the wire format (SINGA synchHalf)."""
    AllReduce(inputs, outputs, op, algo, wire)(stream)


class AllReduceBucketed(AllReduce):
    """A prepared bucketed all-reduce (``rsx_all_reduce_bucketed``): consecutive
    buckets of ``bucket_elems`` elements, each an all-reduce of its own with its
    own segments, in order on one stream ("Distributed primitives", bucketed
    ring all-reduce).  When W divides the bucket the full buckets share one
    launch per pass; the result is the same."""

    def __init__(self, inputs, outputs=None, bucket_elems: int = 13_107_200, op: str = "sum",
                 algo: str = "ring", wire: str | None = None):
        super().__init__(inputs, outputs, op, algo, wire)
        if bucket_elems <= 0:
            raise ValueError("bucket_elems must be positive")
        self.args = self.args[:4] + (int(bucket_elems),) + self.args[4:]
        self.fn = L.lib().rsx_all_reduce_bucketed

    def __call__(self, stream=None) -> None:
        _launch(self, "rsx_all_reduce_bucketed", stream)


class _OneBucket(AllReduce):
    """A prepared ``rsx_all_reduce_bucket``: bucket b of a bucketed all-reduce."""

    def __init__(self, inputs, outputs, bucket_elems: int, bucket: int, op: str, algo: str,
                 wire: str | None):
        super().__init__(inputs, outputs, op, algo, wire)
        self.args = self.args[:4] + (int(bucket_elems), int(bucket)) + self.args[4:]
        self.fn = L.lib().rsx_all_reduce_bucket

    def __call__(self, stream=None) -> None:
        _launch(self, "rsx_all_reduce_bucket", stream)


def bucket_count(count: int, bucket_elems: int) -> int:
    """Buckets of a bucketed all-reduce of ``count`` elements (``rsx_bucket_count``)."""
    return int(L.lib().rsx_bucket_count(int(count), int(bucket_elems)))


def all_reduce_bucketed(inputs, outputs=None, bucket_elems: int = 13_107_200, op: str = "sum",
                        algo: str = "ring", stream=None, wire: str | None = None) -> None:
    """All-reduce consecutive buckets of ``bucket_elems`` elements in order on one
    stream ("Distributed primitives", bucketed ring all-reduce).

    Each bucket is an all-reduce of its own with its own segment split.
    """
    AllReduceBucketed(inputs, outputs, bucket_elems, op, algo, wire)(stream)


class occupancy_caps:
    """Context manager: the library's occupancy caps on (True) or off (False)
    for the launches this thread makes inside it (rsx_set_occupancy_caps);
    the previous setting comes back on exit.  Off suits launches that overlap
    other kernels; the results are the same either way."""

    def __init__(self, enabled: bool):
        self.enabled = bool(enabled)

    def __enter__(self):
        self.prev = L.lib().rsx_set_occupancy_caps(1 if self.enabled else 0)
        return self

    def __exit__(self, *exc):
        L.lib().rsx_set_occupancy_caps(self.prev)
        return False


class BucketedAllReduce:
    """Bucketed all-reduce that overlaps with whatever produces the gradients
    ("Distributed primitives", In practice: the gradient is all-reduced in
    buckets on a separate stream while the backward pass goes on).

    Consecutive buckets of ``bucket_elems`` elements, each its own all-reduce
    (its own segments), as ``all_reduce_bucketed``.  ``ready(b)`` is called
    by the producer once bucket b's inputs are enqueued on its stream: it
    records an event there, makes the reduction stream wait for it and
    enqueues bucket b's all-reduce on the reduction stream, so the producer's
    later work and the reduction run side by side.  ``wait()`` makes a stream
    wait for every enqueued reduction.  The reduction stream is created here
    with the default priority unless one is given.

    ``occupancy_caps`` (default False): the reductions launched by ``ready``
    and ``__call__`` run without the library's occupancy caps, so that the
    producer's kernels still find LDS free on the CUs they share.
    """

    def __init__(self, inputs, outputs=None, bucket_elems: int = 13_107_200, op: str = "sum",
                 algo: str = "ring", wire: str | None = None, stream=None,
                 occupancy_caps: bool = False):
        if bucket_elems <= 0:
            raise ValueError("bucket_elems must be positive")
        outputs = inputs if outputs is None else outputs
        nb = L.lib().rsx_bucket_count(inputs[0].numel(), bucket_elems)
        self.plans = [_OneBucket(inputs, outputs, bucket_elems, b, op, algo, wire) for b in range(nb)]
        self.serial = AllReduceBucketed(inputs, outputs, bucket_elems, op, algo, wire)
        self.device = inputs[0].device
        self.stream = stream if stream is not None else torch.cuda.Stream(device=self.device)
        self.events = [torch.cuda.Event() for _ in self.plans]
        self.occupancy_caps = occupancy_caps

    def __len__(self) -> int:
        return len(self.plans)

    def ready(self, b: int, stream=None) -> None:
        """Bucket b's inputs are enqueued on `stream` (default: current): reduce it on the side."""
        src = torch.cuda.current_stream(self.device) if stream is None else stream
        self.events[b].record(src)
        self.stream.wait_event(self.events[b])
        with occupancy_caps(self.occupancy_caps):
            self.plans[b](self.stream)

    def wait(self, stream=None) -> None:
        """Make `stream` (default: current) wait for every reduction enqueued so far."""
        dst = torch.cuda.current_stream(self.device) if stream is None else stream
        dst.wait_stream(self.stream)

    def __call__(self, stream=None) -> None:
        """Every bucket at once, on `stream` (no overlap): the serial reference,
        one rsx_all_reduce_bucketed call."""
        with occupancy_caps(self.occupancy_caps):
            self.serial(stream)


class _FuseCopy:
    """A prepared pack (tensors -> fused) or unpack (fused -> tensors)."""

    def __init__(self, tensors, fused: torch.Tensor, pack: bool):
        counts = [t.numel() for t in tensors]
        _check([fused], sum(counts), "fused", None, None)
        for i, t in enumerate(tensors):
            _check([t], counts[i], f"tensors[{i}]", fused.dtype, fused.device)
        self.device = fused.device
        self.pack = pack
        lib = L.lib()
        ptrs = L.ptr_array([t.data_ptr() for t in tensors])
        sizes = L.size_array(counts)
        code = _dtype_code(fused)
        if pack:
            self.fn, self.name = lib.rsx_fuse_pack, "rsx_fuse_pack"
            self.args = (ptrs, sizes, len(tensors), fused.data_ptr(), code)
        else:
            self.fn, self.name = lib.rsx_fuse_unpack, "rsx_fuse_unpack"
            self.args = (fused.data_ptr(), ptrs, sizes, len(tensors), code)
        self.keep = (list(tensors), fused)

    def __call__(self, stream=None) -> None:
        _launch(self, self.name, stream)


class FusePack(_FuseCopy):
    """Prepared copy of ``tensors`` back to back into ``fused`` (SINGA fusedSynch /
    Horovod memcpy into the fusion buffer)."""

    def __init__(self, tensors, fused):
        super().__init__(tensors, fused, True)


class FuseUnpack(_FuseCopy):
    """Prepared copy of ``fused`` out into ``tensors`` at the same running offsets."""

    def __init__(self, fused, tensors):
        super().__init__(tensors, fused, False)


class FusedAllReduce:
    """Prepared pack -> in-place all-reduce of the fusion buffers -> unpack
    (Horovod PerformOperation).  ``outputs_per_rank=None`` writes the results
    back into the input tensors."""

    def __init__(self, tensors_per_rank, fused_per_rank, outputs_per_rank=None, op: str = "sum",
                 algo: str = "ring", wire: str | None = None):
        outputs_per_rank = tensors_per_rank if outputs_per_rank is None else outputs_per_rank
        self.packs = [FusePack(ts, f) for ts, f in zip(tensors_per_rank, fused_per_rank)]
        self.reduce = AllReduce(list(fused_per_rank), None, op, algo, wire)
        self.unpacks = [FuseUnpack(f, ts) for f, ts in zip(fused_per_rank, outputs_per_rank)]

    def __call__(self, stream=None) -> None:
        for p in self.packs:
            p(stream)
        self.reduce(stream)
        for u in self.unpacks:
            u(stream)


class TensorFusionAllReduce:
    """Prepared all-reduce of every rank's tensor list with tensor-fusion
    semantics, without a fusion buffer (``rsx_fused_all_reduce``).

    ``tensors_per_rank[r][i]`` is rank r's tensor i; every rank lists tensors of
    the same sizes.  The result equals, bit for bit, packing each rank's list
    back to back, all-reducing the W fused buffers with ``algo`` and unpacking
    (SINGA fusedSynch / Horovod PerformOperation), but only the tensors
    themselves are read and written.  ``outputs_per_rank=None`` is in place.
    """

    def __init__(self, tensors_per_rank, outputs_per_rank=None, op: str = "sum", algo: str = "ring",
                 wire: str | None = None):
        w = _ranks(tensors_per_rank)
        outputs_per_rank = tensors_per_rank if outputs_per_rank is None else outputs_per_rank
        if len(outputs_per_rank) != w:
            raise ValueError("need one output list per rank")
        counts = [t.numel() for t in tensors_per_rank[0]]
        first = next((t for ts in tensors_per_rank for t in ts), None)
        if first is None:
            raise ValueError("empty tensor lists")
        dev, dt = first.device, first.dtype
        for r in range(w):
            if len(tensors_per_rank[r]) != len(counts) or len(outputs_per_rank[r]) != len(counts):
                raise ValueError("every rank needs the same number of tensors")
            for i, c in enumerate(counts):
                _check([tensors_per_rank[r][i]], c, f"tensors[{r}][{i}]", dt, dev)
                _check([outputs_per_rank[r][i]], c, f"outputs[{r}][{i}]", dt, dev)
        if algo not in ALGOS:
            raise ValueError(f"unknown algo {algo!r}")
        self.device = dev
        self.args = (L.ptr_array([t.data_ptr() for ts in tensors_per_rank for t in ts]),
                     L.ptr_array([t.data_ptr() for ts in outputs_per_rank for t in ts]),
                     L.size_array(counts), len(counts), w, _dtype_code(first, wire), _op_code(op),
                     ALGOS[algo])
        self.fn = L.lib().rsx_fused_all_reduce
        self.keep = (tensors_per_rank, outputs_per_rank)

    def __call__(self, stream=None) -> None:
        _launch(self, "rsx_fused_all_reduce", stream)


def fusion_threshold() -> int:
    """Fusion threshold in bytes: ``RSX_FUSION_THRESHOLD`` if set, else 64 MiB
    (Horovod's default, overridable from the environment in the same way)."""
    v = os.environ.get("RSX_FUSION_THRESHOLD")
    return int(v) if v is not None else L.RSX_FUSION_THRESHOLD_DEFAULT


def fusion_groups(tensors, threshold: int | None = None) -> list[tuple[int, int]]:
    """Horovod's grouping of consecutive same-dtype tensors under a byte threshold,
    computed by ``rsx_fusion_plan``; returns [start, end) index ranges."""
    threshold = fusion_threshold() if threshold is None else int(threshold)
    n = len(tensors)
    if n == 0:
        return []
    counts = L.size_array([t.numel() for t in tensors])
    dts = (ctypes.c_int * n)(*[_dtype_code(t) for t in tensors])
    ends = (ctypes.c_int * n)()
    g = L.lib().rsx_fusion_plan(counts, dts, n, threshold, ends)
    if g < 0:
        raise ValueError("rsx_fusion_plan rejected its arguments")
    starts = [0] + [ends[k] for k in range(g - 1)]
    return [(starts[k], ends[k]) for k in range(g)]


class GroupedAllReduce:
    """Prepared all-reduce of tensor lists in Horovod fusion groups: each group of
    consecutive same-dtype tensors under the byte threshold is all-reduced as one
    fusion buffer would be (one ``rsx_fused_all_reduce`` per group)."""

    def __init__(self, tensors_per_rank, outputs_per_rank=None, op: str = "sum", algo: str = "ring",
                 threshold: int | None = None, wire: str | None = None):
        outputs_per_rank = tensors_per_rank if outputs_per_rank is None else outputs_per_rank
        self.groups = fusion_groups(tensors_per_rank[0], threshold)
        self.plans = [TensorFusionAllReduce([ts[lo:hi] for ts in tensors_per_rank],
                                            [os_[lo:hi] for os_ in outputs_per_rank], op, algo, wire)
                      for lo, hi in self.groups]

    def __call__(self, stream=None) -> None:
        for p in self.plans:
            p(stream)


def fuse_pack(tensors, fused: torch.Tensor, stream=None) -> None:
    """Copy ``tensors`` back to back into ``fused``."""
    FusePack(tensors, fused)(stream)


def fuse_unpack(fused: torch.Tensor, tensors, stream=None) -> None:
    """Copy ``fused`` back out into ``tensors`` at the same running offsets."""
    FuseUnpack(fused, tensors)(stream)


def fused_all_reduce(tensors_per_rank, fused_per_rank, outputs_per_rank=None, op: str = "sum",
                     algo: str = "ring", stream=None, wire: str | None = None) -> None:
    """pack -> in-place all-reduce of the fusion buffers -> unpack (SINGA fusedSynch;
    with ``wire="f16"``, fusedSynchHalf)."""
    FusedAllReduce(tensors_per_rank, fused_per_rank, outputs_per_rank, op, algo, wire)(stream)


SPARSE_MODES = {"threshold": L.RSX_SPARSE_THRESHOLD, "topk": L.RSX_SPARSE_TOPK}


def topk_count(count: int, fraction: float) -> int:
    """K of the top-K mode: ceil(fraction * count) in fp32 arithmetic (SINGA topKSparsAllReduce)."""
    return int(L.lib().rsx_sparse_topk_count(count, fraction))


class SparseAllReduce:
    """Prepared sparsified all-reduce with error feedback (SINGA communicator.cc,
    sparsification -> valSparsAllReduce / topKSparsAllReduce).

    ``grads``: W float32 tensors of ``count`` elements.  ``accums``: None, or W
    float32 tensors that are added to the gradients first and receive what was
    not sent.  ``outs``: None writes the result into ``grads`` (as the page
    does); otherwise W tensors.  ``mode="threshold"`` sends entries with
    ``|g| >= threshold``; ``mode="topk"`` sends the ``k`` largest values (or
    ``topk_count(count, fraction)``).  After a call, rank r's message is
    ``msg_idx[r][:n]`` / ``msg_val[r][:n]`` with ``n = nnz_host()[r]``.
    The message buffers, the lengths and the workspace are allocated here,
    once, by PyTorch; calls allocate nothing.  ``noalloc=True`` allocates no
    workspace and calls ``rsx_sparse_all_reduce_noalloc``, which uses the
    library's per-GPU scratch array (calls on one GPU must not overlap).
    """

    def __init__(self, grads, accums=None, outs=None, mode: str = "threshold",
                 threshold: float = 0.0, k: int | None = None, fraction: float | None = None,
                 noalloc: bool = False):
        w = _ranks(grads)
        count = grads[0].numel()
        dev = grads[0].device
        _check(grads, count, "grads", torch.float32, dev)
        outs = grads if outs is None else outs
        if len(outs) != w or (accums is not None and len(accums) != w):
            raise ValueError("need one output and one accumulation buffer per rank")
        _check(outs, count, "outs", torch.float32, dev)
        if accums is not None:
            _check(accums, count, "accums", torch.float32, dev)
        for t in list(grads) + list(outs) + list(accums or []):
            if t.data_ptr() % 16:
                raise ValueError("sparse all-reduce buffers must be 16-byte aligned")
        if mode not in SPARSE_MODES:
            raise ValueError(f"unknown mode {mode!r}; one of {sorted(SPARSE_MODES)}")
        if mode == "topk":
            if k is None:
                if fraction is None:
                    raise ValueError("top-K needs k or fraction")
                k = topk_count(count, fraction)
            if not 0 <= k <= count:
                raise ValueError(f"k={k} outside [0, {count}]")
            cap = k
        else:
            k, cap = 0, count
        lib = L.lib()
        self.device, self.count, self.world, self.k = dev, count, w, k
        self.msg_idx = [torch.empty(max(cap, 1), dtype=torch.int32, device=dev) for _ in range(w)]
        self.msg_val = [torch.empty(max(cap, 1), dtype=torch.float32, device=dev) for _ in range(w)]
        self.nnz = torch.zeros(w, dtype=torch.int32, device=dev)
        ws = lib.rsx_sparse_workspace_size(w, count, SPARSE_MODES[mode], int(accums is not None))
        if ws == 0:
            raise ValueError("rsx_sparse_workspace_size rejected the sizes")
        self.args = (L.ptr_array([t.data_ptr() for t in grads]),
                     L.ptr_array([t.data_ptr() for t in accums]) if accums is not None else None,
                     L.ptr_array([t.data_ptr() for t in outs]),
                     w, count, SPARSE_MODES[mode], float(threshold), k,
                     L.ptr_array([t.data_ptr() for t in self.msg_idx]),
                     L.ptr_array([t.data_ptr() for t in self.msg_val]),
                     cap, self.nnz.data_ptr())
        if noalloc:
            self._ws = None
            self.name = "rsx_sparse_all_reduce_noalloc"
        else:
            self._ws = torch.empty(ws + 256, dtype=torch.uint8, device=dev)
            self.args += (self._ws.data_ptr() + (-self._ws.data_ptr()) % 256, ws)
            self.name = "rsx_sparse_all_reduce"
        self.fn = getattr(lib, self.name)
        self.keep = (list(grads), accums, list(outs))

    def __call__(self, stream=None) -> None:
        _launch(self, self.name, stream)

    def nnz_host(self) -> list[int]:
        """Message lengths (synchronises with the device)."""
        return [int(v) & 0xFFFFFFFF for v in self.nnz.cpu().tolist()]

    def message(self, r: int):
        """Rank r's (indices, values) message as device tensors (synchronises)."""
        n = self.nnz_host()[r]
        return self.msg_idx[r][:n], self.msg_val[r][:n]


def sparse_all_reduce(grads, accums=None, outs=None, mode: str = "threshold", threshold: float = 0.0,
                      k: int | None = None, fraction: float | None = None, stream=None,
                      noalloc: bool = False) -> SparseAllReduce:
    """One sparsified all-reduce; returns the plan, whose buffers hold the messages."""
    p = SparseAllReduce(grads, accums, outs, mode, threshold, k, fraction, noalloc)
    p(stream)
    return p


def segment_begin(count: int, nranks: int, k: int) -> int:
    """First element of segment k of a ring all-reduce of ``count`` elements."""
    return int(L.lib().rsx_segment_begin(count, nranks, k))


def version() -> int:
    return int(L.lib().rsx_version())
