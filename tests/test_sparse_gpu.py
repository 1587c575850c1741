"""Parity of the sparsified all-reduce (HIP, through the C ABI) with the CPU oracle.

Bit-exact on everything: the results on every rank, the residual in every
accumulation buffer, the message lengths, and every message entry.  The
oracle's top-K message is in the page's order (by value); the library sends
the same pairs in index order, so the oracle's pairs are compared sorted by
index (indices are unique within a message).  Sizes span several 4096-element
tiles with a ragged tail; W from 1 to 16; both modes, with and without error
feedback; ties at the cut, signed zeros, infinities and NaNs; K = 0 and K =
count; in place.
"""
import numpy as np
import pytest
import torch

import collective_reduction_ring_amd as rsx
import oracle
from parity_util import say

pytestmark = pytest.mark.gpu

f32 = np.float32


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x, f32)).to("cuda:0")


def host(t):
    return t.cpu().numpy()


def same_bits(got, want, what):
    got, want = np.asarray(got, f32), np.asarray(want, f32)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    bad = np.flatnonzero(got.view(np.uint32) != want.view(np.uint32))
    bad = bad[~(np.isnan(got[bad]) & np.isnan(want[bad]))]
    assert bad.size == 0, (f"{what}: {bad.size} of {got.size} differ; first at {bad[:5].tolist()}: "
                           f"got {got[bad[:5]].tolist()} want {want[bad[:5]].tolist()}")


def run_case(grads, accs, mode, threshold=0.0, k=None, in_place=False):
    w = len(grads)
    g = [dev(x) for x in grads]
    a = [dev(x) for x in accs] if accs is not None else None
    outs = None if in_place else [torch.full((len(grads[0]),), 7.0, device="cuda:0") for _ in range(w)]
    plan = rsx.SparseAllReduce(g, a, outs, mode, threshold, k)
    plan()
    torch.cuda.synchronize()
    res = [host(t) for t in (g if in_place else outs)]
    acc_out = [host(t) for t in a] if a is not None else None
    nnz = plan.nnz_host()
    msgs = [(host(plan.msg_idx[r][:nnz[r]]).view(np.uint32).astype(np.int64),
             host(plan.msg_val[r][:nnz[r]])) for r in range(w)]
    return res, acc_out, nnz, msgs


def check(grads, accs, mode, threshold=0.0, k=None, in_place=False, what=""):
    say(f"sparse {what} mode={mode} w={len(grads)} n={len(grads[0])} thr={threshold} k={k}")
    res, acc_out, nnz, msgs = run_case(grads, accs, mode, threshold, k, in_place)
    want_res, want_acc, want_msgs = oracle.sparse_all_reduce(grads, accs, mode, threshold, k)
    for r in range(len(grads)):
        wi, wv = want_msgs[r]
        order = np.argsort(wi, kind="stable")
        assert nnz[r] == len(wi), (what, r, nnz[r], len(wi))
        assert np.array_equal(msgs[r][0], wi[order]), f"{what}: rank {r} message indices"
        same_bits(msgs[r][1], wv[order], f"{what}: rank {r} message values")
        same_bits(res[r], want_res[r], f"{what}: rank {r} result")
        if accs is not None:
            same_bits(acc_out[r], want_acc[r], f"{what}: rank {r} residual")


def normal_case(seed, w, n, scale=1e-3):
    rng = np.random.default_rng(seed)
    grads = [(rng.standard_normal(n) * scale).astype(f32) for _ in range(w)]
    accs = [(rng.standard_normal(n) * scale).astype(f32) for _ in range(w)]
    return grads, accs


SIZES = [1, 5, 4096, 3 * 4096 + 777]


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("w", [1, 2, 3, 8, 16])
@pytest.mark.parametrize("feedback", [True, False])
def test_threshold(w, n, feedback):
    grads, accs = normal_case((60, w, n), w, n)
    check(grads, accs if feedback else None, "threshold", threshold=2e-3, what="threshold")


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("w", [1, 2, 3, 8, 16])
@pytest.mark.parametrize("feedback", [True, False])
def test_topk(w, n, feedback):
    grads, accs = normal_case((61, w, n), w, n)
    k = rsx.topk_count(n, 0.05)
    assert k == oracle.topk_count(n, 0.05)
    check(grads, accs if feedback else None, "topk", k=k, what="topk")


@pytest.mark.parametrize("mode", ["threshold", "topk"])
def test_ties_at_the_cut_and_specials(mode):
    # values on a coarse grid, so the cut falls inside long runs of equal values
    rng = np.random.default_rng(62)
    w, n = 4, 5 * 4096 + 100
    grads = [(rng.integers(-4, 5, n) * 0.5).astype(f32) for _ in range(w)]
    accs = [(rng.integers(-1, 2, n) * 0.25).astype(f32) for _ in range(w)]
    special = np.array([np.nan, np.inf, -np.inf, -0.0, 0.0, 2.0 ** -149, -(2.0 ** -149)], f32)
    for r in range(w):
        pos = rng.choice(n, 300, replace=False)
        grads[r][pos] = special[rng.integers(0, len(special), 300)]
        accs[r][pos[:40]] = -0.0
    if mode == "threshold":
        for thr in (1.0, 0.0, 2.0 ** -149, np.inf, -1.0, np.nan):  # NaN sends nothing; <= 0 every nonzero
            check(grads, accs, mode, threshold=thr, what=f"ties thr={thr}")
    else:
        for k in (1, 7, 1000, 4096, n // 2, n - 1):
            check(grads, accs, mode, k=k, what=f"ties k={k}")


def test_topk_k_zero_and_all_in_place():
    grads, accs = normal_case(63, 3, 2 * 4096 + 9)
    check(grads, accs, "topk", k=0, what="k=0")
    check(grads, accs, "topk", k=len(grads[0]), what="k=n")
    check(grads, None, "topk", k=321, in_place=True, what="in place")
    check(grads, accs, "threshold", threshold=1e-3, in_place=True, what="in place")


def test_error_feedback_over_steps():
    # three steps on fixed gradients: each step's residual feeds the next
    w, n = 4, 4096 + 3
    rng = np.random.default_rng(64)
    grads = [(rng.standard_normal(n) * 1e-3).astype(f32) for _ in range(w)]
    acc_host = [np.zeros(n, f32) for _ in range(w)]
    acc_dev = [dev(a) for a in acc_host]
    g_dev = [dev(g) for g in grads]
    outs = [torch.empty(n, device="cuda:0") for _ in range(w)]
    plan = rsx.SparseAllReduce(g_dev, acc_dev, outs, "topk", fraction=0.01)
    for step in range(3):
        say(f"error feedback step {step}")
        plan()
        torch.cuda.synchronize()
        want_res, acc_host, _ = oracle.sparse_all_reduce(grads, acc_host, "topk", k=plan.k)
        for r in range(w):
            same_bits(host(outs[r]), want_res[r], f"step {step} rank {r}")
            same_bits(host(acc_dev[r]), acc_host[r], f"step {step} rank {r} residual")


def test_count_zero_zeroes_nnz():
    g = [torch.empty(0, device="cuda:0") for _ in range(2)]
    plan = rsx.SparseAllReduce(g, None, None, "topk", k=0)
    plan.nnz.fill_(5)
    plan()
    assert plan.nnz_host() == [0, 0]


def test_errors_with_real_tensors():
    x = [torch.zeros(64, device="cuda:0") for _ in range(2)]
    with pytest.raises(ValueError):
        rsx.SparseAllReduce(x, None, None, "topk", k=65)
    with pytest.raises(ValueError):
        rsx.SparseAllReduce(x, None, None, "bogus")
    with pytest.raises(ValueError):
        rsx.SparseAllReduce([t[1:] for t in x], None, None, "threshold")   # misaligned
    with pytest.raises(rsx.RsxError) as e:   # accumulation = gradient of another rank
        rsx.SparseAllReduce(x, [x[1], torch.zeros(64, device="cuda:0")], None, "threshold")()
    assert e.value.status == 5


def test_mid_size_w8():
    # the bench's shape scaled down: W = 8, N(0, 1e-3) gradients and residuals
    grads, accs = normal_case(65, 8, 1 << 20)
    check(grads, accs, "topk", k=rsx.topk_count(1 << 20, 0.01), what="w8 topk 1%")
    check(grads, accs, "threshold", threshold=3.6e-3, what="w8 threshold")


# keys per rank the top-K gather bound is sampled from: runs of 16
# consecutive elements, one every 16 * (n // SAMPLE) elements
SAMPLE = 65536


def sampled_positions(n):
    s = np.arange(min(n, SAMPLE))
    return (s >> 4) * (16 * max(1, n // SAMPLE)) + (s & 15)


@pytest.mark.parametrize("n", [SAMPLE + 3 * 4096 + 5, 2 * SAMPLE + 4096 + 3])
@pytest.mark.parametrize("fraction", [0.001, 0.01, 0.3, 0.97, 1.0])
def test_topk_past_the_sample_size(fraction, n):
    # more elements than the keys the top-K bound is sampled from; a large K
    # makes the sampled rank exceed the sample (the bound is then 0)
    grads, accs = normal_case((66, int(fraction * 1000), n), 3, n)
    check(grads, accs, "topk", k=rsx.topk_count(n, fraction), what=f"topk {fraction}")


@pytest.mark.parametrize("feedback", [True, False])
@pytest.mark.parametrize("fraction", [0.05, 0.5])
def test_topk_sample_misled(feedback, fraction):
    # White-box: the top-K bound is drawn from the keys at sampled_positions.
    # Large values at exactly those positions make the sample claim that
    # few keys reach the bound's level, so the gather holds fewer than K
    # keys and the exact fallback must take over.  Rank 1 keeps ordinary
    # values, so one call mixes ranks with and without the fallback.
    n = 3 * SAMPLE + 777
    w = 3
    grads, accs = normal_case((67, int(fraction * 1000)), w, n)
    rng = np.random.default_rng(68)
    sampled = sampled_positions(n)
    assert sampled[-1] < n and len(np.unique(sampled)) == SAMPLE
    for r in (0, 2):
        grads[r][sampled] = (1.0 + rng.random(SAMPLE)).astype(f32)
    check(grads, accs if feedback else None, "topk", k=rsx.topk_count(n, fraction),
          what=f"misled sample {fraction}")


@pytest.mark.parametrize("feedback", [True, False])
def test_topk_sample_misled_low(feedback):
    # The other direction: the sampled positions hold tiny values, so the
    # bound and the guessed cut are far too low.  Most elements are then
    # gathered, most guessed sent, and the combine corrects the residual of
    # every candidate that is not.
    n = 2 * SAMPLE + 4096 + 3
    grads, accs = normal_case(69, 3, n)
    sampled = sampled_positions(n)
    for r in (0, 1):
        grads[r][sampled] = f32(1e-9)
        accs[r][sampled] = f32(0.0)
    check(grads, accs if feedback else None, "topk", k=rsx.topk_count(n, 0.01),
          what="sample misled low")


@pytest.mark.timeout(600)
def test_more_tiles_than_the_bench_shape():
    # 16386 tiles per rank with a ragged tail: more than the bench shape's
    # 16384, so the per-rank offset scan's last pass is a partial one; the
    # top-K sample's runs are 1024 runs of 16 apart
    n = 16384 * 4096 + 4096 + 5
    grads, accs = normal_case(70, 2, n)
    check(grads, accs, "threshold", threshold=3.6e-3, what="16386 tiles, threshold")
    check(grads, accs, "topk", k=rsx.topk_count(n, 0.001), what="16386 tiles, top-K")


@pytest.mark.parametrize("case", range(40))
def test_random_configurations(case):
    # Seeded random mixes: rank count, size (some past the sampled 65536
    # keys), mode, K or threshold, error feedback, a coarse value grid (ties at
    # the cut) and planted specials.
    rng = np.random.default_rng((71, case))
    w = int(rng.choice([1, 2, 3, 5, 8, 16]))
    n = int(rng.choice([int(rng.integers(1, 3 * 4096)), int(rng.integers(SAMPLE, 2 * SAMPLE + 9000))]))
    coarse = rng.random() < 0.3
    grads, accs = [], []
    for _ in range(w):
        if coarse:
            g = (rng.integers(-6, 7, n) * 0.125).astype(f32)
            a = (rng.integers(-2, 3, n) * 0.0625).astype(f32)
        else:
            g = (rng.standard_normal(n) * 1e-3).astype(f32)
            a = (rng.standard_normal(n) * 1e-3).astype(f32)
        m = int(rng.integers(0, max(1, n // 50)))
        if m:
            pos = rng.choice(n, m, replace=False)
            g[pos] = np.array([np.nan, np.inf, -np.inf, -0.0, 0.0, 2.0 ** -149], f32)[rng.integers(0, 6, m)]
        grads.append(g)
        accs.append(a)
    feedback = rng.random() < 0.7
    if rng.random() < 0.5:
        frac = float(rng.choice([0.0, 0.0005, 0.01, 0.05, 0.3, 0.9, 1.0]))
        check(grads, accs if feedback else None, "topk", k=rsx.topk_count(n, frac),
              what=f"random {case} topk w={w} n={n} frac={frac} coarse={coarse}")
    else:
        thr = float(rng.choice([1e-3, 2e-3, 0.25, 0.0]))
        check(grads, accs if feedback else None, "threshold", threshold=thr,
              what=f"random {case} threshold w={w} n={n} thr={thr} coarse={coarse}")


@pytest.mark.parametrize("mode", ["topk", "threshold"])
def test_graph_capture_replays(mode):
    # The whole sparse call (all its kernels) captured in a HIP graph: every
    # replay starts from the same residual (restored eagerly between
    # replays, with synchronisation) and must equal the oracle bit for bit.
    w, n = 4, 3 * 4096 + 500
    grads, accs = normal_case(66, w, n)
    g = [dev(x) for x in grads]
    a = [dev(x) for x in accs]
    a0 = [t.clone() for t in a]
    outs = [torch.empty(n, device="cuda:0") for _ in range(w)]
    kw = {"k": 150} if mode == "topk" else {"threshold": 2e-3}
    plan = rsx.SparseAllReduce(g, a, outs, mode, **kw)
    want_res, want_acc, want_msgs = oracle.sparse_all_reduce(
        grads, accs, mode, kw.get("threshold", 0.0), kw.get("k"))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        plan()                                 # warm-up outside the graph
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    say(f"sparse graph capture mode={mode}")
    with torch.cuda.graph(graph):
        plan()
    for rep in range(4):
        for d, s0 in zip(a, a0):
            d.copy_(s0)                        # eager work between replays
        for o in outs:
            o.fill_(-7.0)
        plan.nnz.fill_(12345)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        nnz = plan.nnz_host()
        for r in range(w):
            wi, wv = want_msgs[r]
            order = np.argsort(wi, kind="stable")
            assert nnz[r] == len(wi), (rep, r)
            assert np.array_equal(host(plan.msg_idx[r][:nnz[r]]).view(np.uint32), wi[order].astype(np.uint32))
            same_bits(host(plan.msg_val[r][:nnz[r]]), wv[order], f"replay {rep} rank {r} message")
            same_bits(host(outs[r]), want_res[r], f"replay {rep} rank {r} result")
            same_bits(host(a[r]), want_acc[r], f"replay {rep} rank {r} residual")


def _oracle_per_rank(fn, grads, accs, arg):
    """The oracle's per-rank sparsification of every rank, ranks in parallel
    threads (NumPy releases the GIL in its sorts and element-wise passes)."""
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(max_workers=len(grads)) as ex:
        return list(ex.map(lambda r: fn(grads[r], accs[r], arg), range(len(grads))))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("mode", ["threshold", "topk"])
def test_full_size_bench_shape_against_oracle(mode):
    # W = 8, 64 Mi fp32 per rank, the timed configuration, compared with the
    # oracle bit for bit: every rank's message (indices and values), every
    # residual, and the result on every rank.
    from collective_reduction_ring_amd import workloads as wl
    w, n = wl.SPARSE_WORLD, wl.SPARSE_N
    say(f"full-size sparse {mode}: generating")
    grads, accs = wl.sparse_inputs()
    g = [dev(x) for x in grads]
    a = [dev(x) for x in accs]
    outs = [torch.empty(n, device="cuda:0") for _ in range(w)]
    kw = {"fraction": wl.SPARSE_TOPK_FRACTION} if mode == "topk" else {"threshold": wl.SPARSE_THRESHOLD}
    plan = rsx.SparseAllReduce(g, a, outs, mode, **kw)
    say(f"full-size sparse {mode}: launching")
    plan()
    torch.cuda.synchronize()
    nnz = plan.nnz_host()
    del g
    say(f"full-size sparse {mode}: oracle, {w} ranks in parallel")
    if mode == "topk":
        k = oracle.topk_count(n, wl.SPARSE_TOPK_FRACTION)
        assert plan.k == k
        per_rank = _oracle_per_rank(oracle.sparsify_topk, grads, accs, k)
    else:
        per_rank = _oracle_per_rank(oracle.sparsify_threshold, grads, accs, wl.SPARSE_THRESHOLD)
    msgs = [(i, v) for i, v, _ in per_rank]
    for r, (wi, wv, wacc) in enumerate(per_rank):
        order = np.argsort(wi, kind="stable")    # top-K: the page's value order -> index order
        assert nnz[r] == len(wi), (mode, r, nnz[r], len(wi))
        assert np.array_equal(host(plan.msg_idx[r][:nnz[r]]).view(np.uint32), wi[order].astype(np.uint32))
        same_bits(host(plan.msg_val[r][:nnz[r]]), wv[order], f"{mode} rank {r} message values")
        same_bits(host(a[r]), wacc, f"{mode} rank {r} residual")
    del per_rank
    say(f"full-size sparse {mode}: oracle combine")
    want = oracle.sparse_combine(msgs, n)
    for r in range(w):
        same_bits(host(outs[r]), want, f"{mode} rank {r} result")


