"""Pins of the sparsified all-reduce oracle (Apache SINGA communicator.cc,
valSparsAllReduce / topKSparsAllReduce), each independent of its formulas:
hand-derived cases, brute-force scalar loops, and invariants."""
import numpy as np
import pytest

import oracle

f32 = np.float32


def test_topk_count_is_fp32_arithmetic():
    # 0.1f * 10 = 1.0000000149 rounds to 1.0f: K = 1 (double arithmetic would give 2)
    assert oracle.topk_count(10, 0.1) == 1
    # num is converted to fp32 first: 2^24 + 1 becomes 2^24
    assert oracle.topk_count(2 ** 24 + 1, 1.0) == 2 ** 24
    assert oracle.topk_count(1000, 0.5) == 500
    assert oracle.topk_count(7, 0.0) == 0
    assert oracle.topk_count(3, 1.0) == 3
    # 0.3f * 10 = 3 + 2^-23 exactly, halfway between 3 and the next fp32: ties to even, K = 3
    assert oracle.topk_count(10, 0.3) == 3


def test_threshold_hand_case():
    g = np.array([0.5, -0.25, 0.25, 0.125, -0.0, 0.375, 0.0, -1.0], f32)
    idx, val, acc = oracle.sparsify_threshold(g, np.zeros(8, f32), 0.25)
    # |x| >= 0.25 kept; the zeros are never sent
    assert idx.tolist() == [0, 1, 2, 5, 7]
    assert val.tolist() == [0.5, -0.25, 0.25, 0.375, -1.0]
    # residual: what was not sent (the -0 input plus +0 accumulation is +0)
    assert acc.tolist() == [0, 0, 0, 0.125, 0, 0, 0, 0]
    # threshold 0 sends every nonzero entry, never a zero
    idx, _, _ = oracle.sparsify_threshold(np.array([0.0, -0.0, 1e-30], f32), None, 0.0)
    assert idx.tolist() == [2]


def test_threshold_nan_and_negative():
    # the comparison |g| >= threshold decides: a NaN threshold sends nothing, a
    # negative one keeps everything but a NaN entry (|NaN| >= t is false) and
    # sends what is nonzero
    g = np.array([1.0, -2.0, 0.0, -0.0, np.nan, np.inf], f32)
    acc = np.zeros(6, f32)
    idx, val, res = oracle.sparsify_threshold(g, acc, float("nan"))
    assert idx.tolist() == [] and val.tolist() == []
    bits = res.view(np.uint32).tolist()
    assert bits[:4] == [0x3F800000, 0xC0000000, 0, 0] and np.isnan(res[4]) and res[5] == np.inf
    idx, val, res = oracle.sparsify_threshold(g, acc, -1.0)
    assert idx.tolist() == [0, 1, 5] and val.tolist() == [1.0, -2.0, np.inf]
    # sent entries leave x - x: 0 for finite, NaN for inf; the kept -0 leaves
    # (-0 + 0) - (-0 + 0) = +0; the NaN entry stays
    assert res[:4].view(np.uint32).tolist() == [0, 0, 0, 0]
    assert np.isnan(res[4]) and np.isnan(res[5])


def test_threshold_error_feedback_two_steps():
    # step 1: 1.0 is sent, 0.25 is kept back; step 2: 0.25 + 0.375 = 0.625 >= 0.5 is sent
    acc = np.zeros(2, f32)
    i1, v1, acc = oracle.sparsify_threshold(np.array([1.0, 0.25], f32), acc, 0.5)
    assert (i1.tolist(), v1.tolist(), acc.tolist()) == ([0], [1.0], [0.0, 0.25])
    i2, v2, acc = oracle.sparsify_threshold(np.array([0.0, 0.375], f32), acc, 0.5)
    assert (i2.tolist(), v2.tolist(), acc.tolist()) == ([1], [0.625], [0.0, 0.0])


def test_topk_hand_case_ties_by_index():
    g = np.array([3, -5, 3, 7, 0, 3], f32)
    idx, val, acc = oracle.sparsify_topk(g, np.zeros(6, f32), 3)
    # sorted large to small: 7 (3), 3 (0), 3 (2), 3 (5), 0 (4), -5 (1)
    assert idx.tolist() == [3, 0, 2] and val.tolist() == [7, 3, 3]
    assert acc.tolist() == [0, -5, 0, 0, 0, 3]
    # by value, not magnitude: -5 is the smallest
    idx, _, _ = oracle.sparsify_topk(g, None, 5)
    assert sorted(idx.tolist()) == [0, 2, 3, 4, 5]


def test_topk_signed_zero_nan_and_inf():
    g = np.array([np.nan, -0.0, 0.0, -np.inf, np.inf, 1.0], f32)
    # a -0 accumulation keeps -0 inputs -0 (a +0 one would turn them into +0)
    idx, val, acc = oracle.sparsify_topk(g, np.full(6, -0.0, f32), 4)
    # order: inf (4), 1 (3... index 5), -0 (1) and +0 (2) equal, by index; -inf; NaN last
    assert idx.tolist() == [4, 5, 1, 2]
    assert np.isnan(acc[0]) and acc[3] == -np.inf
    # a sent inf leaves inf - inf = NaN behind; a sent -0 leaves -0 - (0 + -0) = -0
    assert np.isnan(acc[4]) and acc[5] == 0
    assert np.signbit(acc[1]) and acc[1] == 0
    # the combine starts from +0: a single -0 contribution gives +0
    out = oracle.sparse_combine([(np.array([0]), np.array([-0.0], f32))], 1)
    assert out[0] == 0 and not np.signbit(out[0])


def test_combine_adds_ranks_in_rank_order():
    big = f32(2 ** 24)
    msgs = [(np.array([0]), np.array([big], f32)), (np.array([0]), np.array([1], f32)),
            (np.array([0]), np.array([1], f32)), (np.array([0]), np.array([-big], f32))]
    # ((2^24 + 1) -> 2^24) + 1 -> 2^24, - 2^24 = 0; another order would give 1 or 2
    assert oracle.sparse_combine(msgs, 3).tolist() == [0, 0, 0]


def _brute_threshold(g, thr):
    sent = []
    for i, x in enumerate(g):
        if abs(float(x)) >= float(f32(thr)) and float(x) != 0.0:
            sent.append((i, float(x)))
    return sent


def _brute_topk(g, k):
    # repeated selection of the largest remaining value, lowest index first; NaN never wins
    left = list(range(len(g)))
    sent = []
    for _ in range(k):
        best = None
        for i in left:
            x = float(g[i])
            if best is None:
                best = i
                continue
            b = float(g[best])
            if np.isnan(b) and not np.isnan(x):
                best = i
            elif not np.isnan(x) and x > b:
                best = i
        sent.append(best)
        left.remove(best)
    return sent


@pytest.mark.parametrize("w", [1, 2, 3, 5])
def test_brute_force_small(w):
    rng = np.random.default_rng(40 + w)
    n = 37
    grads = [rng.integers(-6, 7, n).astype(f32) * f32(0.25) for _ in range(w)]
    accs = [rng.integers(-2, 3, n).astype(f32) * f32(0.125) for _ in range(w)]
    gp = [g + a for g, a in zip(grads, accs)]
    for mode, param in (("threshold", 0.5), ("topk", 9)):
        outs, new_acc, msgs = oracle.sparse_all_reduce(
            grads, accs, mode, threshold=param if mode == "threshold" else 0.0,
            k=param if mode == "topk" else None)
        dense = [0.0] * n
        for r in range(w):
            if mode == "threshold":
                sent = _brute_threshold(gp[r], param)
            else:
                sent = [(i, float(gp[r][i])) for i in _brute_topk(gp[r], param)]
            assert sorted(msgs[r][0].tolist()) == sorted(i for i, _ in sent)
            got = dict(zip(msgs[r][0].tolist(), msgs[r][1].tolist()))
            assert got == dict(sent)
            for i in range(n):
                want_res = float(gp[r][i]) - (dict(sent)[i] if i in dict(sent) else 0.0)
                assert float(new_acc[r][i]) == want_res
            for i, v in sent:
                dense[i] = float(f32(dense[i]) + f32(v))
        for r in range(w):
            assert outs[r].tolist() == dense


def test_invariants_random():
    rng = np.random.default_rng(50)
    n, w = 5000, 4
    grads = [(rng.standard_normal(n) * 1e-3).astype(f32) for _ in range(w)]
    accs = [(rng.standard_normal(n) * 1e-3).astype(f32) for _ in range(w)]
    k = oracle.topk_count(n, 0.01)
    outs, new_acc, msgs = oracle.sparse_all_reduce(grads, accs, "topk", k=k)
    for r in range(w):
        gp = grads[r] + accs[r]
        idx, val = msgs[r]
        assert len(idx) == k == 50
        rest = np.delete(gp, idx)
        assert val.min() >= rest.max()                         # the K largest values
        sent = np.zeros(n, f32)
        sent[idx] = val
        assert np.array_equal(sent + new_acc[r], gp)            # nothing lost (finite data)
    # K = n sends everything: small-integer data sums exactly
    gi = [rng.integers(-100, 100, 64).astype(f32) for _ in range(3)]
    outs, acc, _ = oracle.sparse_all_reduce(gi, [np.zeros(64, f32)] * 3, "topk", k=64)
    assert np.array_equal(outs[0], np.sum(gi, axis=0)) and all(not a.any() for a in acc)
    # K = 0 sends nothing: the result is zero and the residual is everything
    outs, acc, msgs = oracle.sparse_all_reduce(gi, [np.zeros(64, f32)] * 3, "topk", k=0)
    assert not outs[0].any() and all(np.array_equal(a, g) for a, g in zip(acc, gi))
    # threshold mode: the result is the rank-order sum of the kept entries
    outs, acc, msgs = oracle.sparse_all_reduce(grads, None, "threshold", threshold=2e-3)
    kept = [np.where(np.abs(g) >= f32(2e-3), g, 0).astype(f32) for g in grads]
    want = np.zeros(n, f32)
    for kk in kept:
        want = want + kk
    assert np.array_equal(outs[1], want) and acc == [None] * w
