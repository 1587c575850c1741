"""CPU oracle of the sparsified all-reduce (gradient sparsification with error feedback).

TEST INFRASTRUCTURE.  Only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run this module.  It shares
no code with the HIP library.  Plain NumPy, one rank at a time, in the order
of the page's steps.

Source: Apache SINGA ``src/io/communicator.cc`` (the web page of that title),
``valSparsAllReduce`` and ``topKSparsAllReduce``, reached from
``sparsification`` / ``fusedSparsification``.  Per rank, with gradient ``t``
and an optional accumulation buffer ``acc`` (error feedback):

1. with ``acc``: ``g = t + acc`` (fp32 add) and a backup copy of ``g``;
2. threshold mode: ``sparsabs`` zeroes the entries of small magnitude;
   top-K mode: the entries are sorted from large to small values (with their
   one-based indices as the payload) and the first ``K = ceil(threshold *
   num)`` are kept;
3. with ``acc``: the new accumulation is the backup minus what is sent
   (threshold mode: minus the sparsified array; top-K mode: minus a zeroed
   buffer into which the K kept values were scatter-added);
4. the message is the kept entries' indices and values (threshold mode: the
   nonzero entries, compacted in index order);
5. the messages of all ranks are all-gathered, and every rank zeroes a dense
   buffer and scatter-adds rank 0's message, then rank 1's, ... (``saxpyi``
   with ``alpha = 1``): the result, the same on every rank, replaces ``t``.

Readings where the page is silent (the kernels ``sparsabs``, ``sortbykey`` and
the type of ``threshold`` are off-page):

* ``sparsabs`` keeps ``x`` when ``|x| >= threshold`` and writes 0 otherwise;
  ``sparsindex`` then keeps only nonzero entries, so a kept ``+-0`` is not
  sent;
* the top-K sort is by value, largest first, as the page's comment says (not
  by magnitude); equal values keep index order (a stable sort), ``-0`` equals
  ``+0``, and a NaN sorts below every number;
* ``threshold`` is a ``float``, so ``threshold * num`` is an fp32 product
  (``num`` converted to fp32 first) and K is its ceiling;
* indices in messages are zero-based here (the page's are one-based for its
  sparse BLAS call); top-K messages are returned in the page's order (by
  value), threshold messages in index order.
"""
from __future__ import annotations

import math

import numpy as np


def topk_count(num: int, fraction: float) -> int:
    """K = ceil(threshold * num) with ``threshold`` an fp32 and the product in fp32."""
    return int(math.ceil(float(np.float32(fraction) * np.float32(num))))


def _with_feedback(grad, accum):
    g = np.asarray(grad, dtype=np.float32)
    if accum is None:
        return g.copy(), None
    g = g + np.asarray(accum, dtype=np.float32)
    return g, g.copy()


def sparsify_threshold(grad, accum, threshold: float):
    """One rank of ``valSparsAllReduce`` up to the all-gather.

    Returns ``(idx, val, new_accum)``: zero-based indices in increasing order,
    their values, and the new accumulation (``None`` without ``accum``).
    """
    g, backup = _with_feedback(grad, accum)
    thr = np.float32(threshold)
    s = np.where(np.abs(g) >= thr, g, np.float32(0)).astype(np.float32)    # sparsabs
    new_accum = None if backup is None else (backup - s).astype(np.float32)
    one_based = np.where(s != 0, np.arange(1, len(s) + 1), 0)              # sparsindex
    idx = one_based[one_based != 0] - 1                                     # removezeroidx
    val = s[s != 0]                                                         # removezeroval
    return idx.astype(np.int64), val, new_accum


def sparsify_topk(grad, accum, k: int):
    """One rank of ``topKSparsAllReduce`` up to the all-gather.

    Returns ``(idx, val, new_accum)`` with the K kept entries in the page's
    order (values from large to small, equal values by index).
    """
    g, backup = _with_feedback(grad, accum)
    if not 0 <= k <= len(g):
        raise ValueError("K out of range")
    index = np.arange(1, len(g) + 1)                                        # generateindex
    order = np.argsort(-g, kind="stable")                                   # sortbykey, large to small
    keys, index = g[order], index[order]
    new_accum = None
    if backup is not None:
        a = np.zeros(len(g), np.float32)
        a[index[:k] - 1] = a[index[:k] - 1] + keys[:k]                      # saxpyi into zeros
        new_accum = (backup - a).astype(np.float32)
    return (index[:k] - 1).astype(np.int64), keys[:k].copy(), new_accum


def sparse_combine(messages, count: int) -> np.ndarray:
    """Zeroed dense buffer, then each rank's (idx, val) scatter-added in rank order."""
    out = np.zeros(count, np.float32)
    for idx, val in messages:
        out[idx] = out[idx] + np.float32(1) * np.asarray(val, np.float32)
    return out


def sparse_all_reduce(grads, accums=None, mode: str = "threshold", threshold: float = 0.0,
                      k: int | None = None):
    """Every rank's sparsification, the all-gather of the messages and the combine.

    Returns ``(outs, new_accums, messages)``: the result on every rank, each
    rank's new accumulation (``None`` without ``accums``), and each rank's
    (idx, val) message.
    """
    w = len(grads)
    accums = [None] * w if accums is None else accums
    msgs, new_acc = [], []
    for r in range(w):
        if mode == "threshold":
            i, v, a = sparsify_threshold(grads[r], accums[r], threshold)
        elif mode == "topk":
            i, v, a = sparsify_topk(grads[r], accums[r], k)
        else:
            raise ValueError(mode)
        msgs.append((i, v))
        new_acc.append(a)
    res = sparse_combine(msgs, len(grads[0]))
    return [res.copy() for _ in range(w)], new_acc, msgs
