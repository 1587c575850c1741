"""Pins of the CPU oracle against what the pages and plain mathematics fix.

None of these checks re-types the oracle's own formula: each compares it with a
value printed on a page (the block-vs-step table), an order-free library
reduction, a closed-form error bound, exact small-integer arithmetic, a hand-
derived value that only one summation order produces, or a library rounding
routine.
"""
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _f32(*v):
    return np.array(v, dtype=np.float32)


# ----------------------------------------------------------- schedule (P2) --

def _read_table(name):
    rows, ufr = [], None
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, vals = line.split(":")
            vals = [int(v) for v in vals.split()]
            if key == "user_from_ring":
                ufr = vals
            else:
                rows.append(vals)
    return ufr, np.array(rows)


def test_schedule_reproduces_printed_table():
    ufr, table = _read_table("ring_schedule_user_from_ring_1_2_0_3.txt")
    assert np.array_equal(oracle.block_vs_step_table(ufr), table)


def test_schedule_last_step_is_own_block_and_rows_rotate():
    # The page's two remarks on its table: the last row is userFromRing itself,
    # and each earlier row is the next one rotated left by one.
    for ufr in ([1, 2, 0, 3], [0, 1, 2, 3, 4, 5, 6, 7], [4, 0, 3, 1, 2]):
        t = oracle.block_vs_step_table(ufr)
        assert list(t[-1]) == ufr
        for s in range(len(ufr) - 1):
            assert list(t[s]) == list(t[s + 1][1:]) + [t[s + 1][0]]


def test_ring_fold_order_identity_ring_w4():
    # Read off the identity-ring table by hand: block k is copied out by
    # position k+1 at step 0 and ends on position k.
    assert oracle.ring_fold_order(0, 4) == [1, 2, 3, 0]
    assert oracle.ring_fold_order(1, 4) == [2, 3, 0, 1]
    assert oracle.ring_fold_order(3, 4) == [0, 1, 2, 3]
    assert oracle.ring_fold_order(0, 1) == [0]


# --------------------------------------------------- ring-order probe (P6) --

BIG = np.float32(2.0 ** 24)


def _probe_inputs(w, k, s, order_vals):
    """Rank inputs of length w*s where segment k, element 0 of rank r is order_vals[r]."""
    xs = [np.zeros(w * s, np.float32) for _ in range(w)]
    for r, v in enumerate(order_vals):
        xs[r][k * s] = v
    return xs


def test_ring_order_probe_sum():
    # Segment 0 of W=4, inputs x0=1, x1=2^24, x2=1, x3=-2^24 at the same index.
    # Ring order 1,2,3,0: 2^24+1 rounds (tie to even) to 2^24, -2^24 gives 0, +1 gives 1.
    # Rank order 0..3: 1+2^24 -> 2^24, +1 -> 2^24, -2^24 -> 0.
    # Reverse ring 3,2,1,0: -2^24+1 is exact, +2^24 -> 1, +1 -> 2.
    xs = _probe_inputs(4, 0, 8, [1.0, BIG, 1.0, -BIG])
    rs = oracle.reduce_scatter(xs, "sum", "f32")
    assert rs[0][0] == np.float32(1.0)
    ar = oracle.all_reduce(xs, "sum", "f32")
    assert all(a[0] == np.float32(1.0) for a in ar)
    nv = oracle.naive_all_reduce(xs, "sum", "f32")
    assert all(a[0] == np.float32(0.0) for a in nv)


@pytest.mark.parametrize("k", [0, 1, 2, 3])
def test_ring_order_probe_every_segment(k):
    # Same probe placed in segment k: ranks k+1, k+2, k+3, k (mod 4) get 2^24, 1, -2^24, 1.
    w, s = 4, 4
    vals = [0.0] * w
    vals[(k + 1) % w] = BIG
    vals[(k + 2) % w] = 1.0
    vals[(k + 3) % w] = -BIG
    vals[k] = 1.0
    xs = _probe_inputs(w, k, s, vals)
    assert oracle.reduce_scatter(xs, "sum", "f32")[k][0] == np.float32(1.0)


# ---------------------------------------- order-free reductions (P3, P5) ----

@pytest.mark.parametrize("w", [1, 2, 3, 4, 8, 16])
def test_int32_matches_order_free_reductions(w):
    rng = np.random.default_rng(7)
    s = 37
    xs = [rng.integers(-(2 ** 31), 2 ** 31, w * s, dtype=np.int64).astype(np.int32) for _ in range(w)]
    stack = np.stack(xs).astype(np.int64)
    want_sum = ((stack.sum(0) + 2 ** 31) % 2 ** 32 - 2 ** 31).astype(np.int32)   # wraps
    got = np.concatenate(oracle.reduce_scatter(xs, "sum", "i32"))
    assert np.array_equal(got, want_sum)
    assert np.array_equal(np.concatenate(oracle.reduce_scatter(xs, "max", "i32")),
                          np.maximum.reduce(xs))
    assert np.array_equal(np.concatenate(oracle.reduce_scatter(xs, "min", "i32")),
                          np.minimum.reduce(xs))


def test_int32_avg_truncates_toward_zero():
    # sums 7, -7, 6, -6, 0 over W=4 -> 1, -1, 1, -1, 0 (C division, not floor)
    xs = [np.array(v, np.int32) for v in ([7, -7, 6, -6, 0, 0, 0, 0],
                                           [0] * 8, [0] * 8, [0] * 8)]
    got = oracle.all_reduce(xs, "avg", "i32")[0]
    assert list(got[:5]) == [1, -1, 1, -1, 0]


@pytest.mark.parametrize("w", [2, 4, 8, 16])
def test_fp32_small_integers_sum_exactly(w):
    # |x| <= 2^10 and W <= 16: every partial sum is an integer below 2^24, so
    # every fp32 add is exact and the ring fold equals the integer sum.
    rng = np.random.default_rng(11)
    xi = [rng.integers(-1024, 1025, w * 64).astype(np.int32) for _ in range(w)]
    xf = [x.astype(np.float32) for x in xi]
    got = np.concatenate(oracle.reduce_scatter(xf, "sum", "f32"))
    assert np.array_equal(got, np.stack(xi).astype(np.int64).sum(0).astype(np.float32))


@pytest.mark.parametrize("w", [2, 3, 4, 8, 16])
def test_fp32_within_recursive_summation_bound(w):
    # |fl(sum) - sum| <= (W-1) u sum|x| + O(u^2), u = 2^-24 (Higham, recursive summation).
    rng = np.random.default_rng(3)
    xs = [rng.standard_normal(w * 257).astype(np.float32) for _ in range(w)]
    got = np.concatenate(oracle.reduce_scatter(xs, "sum", "f32")).astype(np.float64)
    st = np.stack(xs).astype(np.float64)
    exact, absum = st.sum(0), np.abs(st).sum(0)
    bound = (w - 1) * 2.0 ** -24 * absum * (1 + 1e-6)
    assert np.all(np.abs(got - exact) <= bound)


def test_fp32_avg_is_one_ieee_division():
    xs = [_f32(1.0, 2.0, 1.0), _f32(1.0, 2.0, 0.5), _f32(2.0, 3.0, 0.25)]
    got = oracle.naive_all_reduce(xs, "avg", "f32")[0]
    # sums 4, 7, 1.75 divided by 3, rounded once from the exact quotient
    assert np.array_equal(got, _f32(4.0 / 3.0, 7.0 / 3.0, 1.75 / 3.0))
    xs4 = [_f32(1.0, 3.0)] * 4
    assert np.array_equal(oracle.naive_all_reduce(xs4, "avg", "f32")[0], _f32(1.0, 3.0))


# ------------------------------------------------ max / min reading (c7) ----

def test_max_min_compare_select_rule():
    nan = np.float32("nan")
    # ring order for segment 0 at W=2 is rank 1, then rank 0.
    x0 = _f32(-0.0, 0.0, nan, 1.0)
    x1 = _f32(0.0, -0.0, 1.0, nan)
    mx = oracle.reduce_scatter([np.concatenate([x0, x0]), np.concatenate([x1, x1])], "max")[0]
    # +0 then -0 -> keeps +0 (first); -0 then +0 -> keeps -0; acc=1 then NaN -> 1;
    # acc=NaN then 1 -> NaN.
    assert np.signbit(mx[0]) == False and mx[0] == 0  # noqa: E712
    assert np.signbit(mx[1]) == True and mx[1] == 0   # noqa: E712
    assert mx[2] == 1.0
    assert np.isnan(mx[3])
    mn = oracle.reduce_scatter([np.concatenate([x0, x0]), np.concatenate([x1, x1])], "min")[0]
    assert np.signbit(mn[0]) == False and np.signbit(mn[1]) == True  # noqa: E712
    assert mn[2] == 1.0 and np.isnan(mn[3])


# ----------------------------------------------------------- bf16 (P7) ------

def test_bf16_rounding_matches_torch_cast():
    rng = np.random.default_rng(5)
    x = np.concatenate([
        rng.standard_normal(500_000).astype(np.float32),
        (rng.standard_normal(250_000) * 1e30).astype(np.float32),
        rng.integers(0, 2 ** 32, 250_000, dtype=np.uint64).astype(np.uint32).view(np.float32),
        _f32(0.0, -0.0, np.inf, -np.inf, 3.3895314e38, -3.3895314e38, 1e-45, -1e-45),
    ])
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.f32_to_bf16(x)
    ok = ~np.isnan(x)
    assert np.array_equal(got[ok], want[ok])
    # NaN stays NaN after widening back
    assert np.all(np.isnan(oracle.bf16_to_f32(got[~ok])))


def test_bf16_hand_ties_and_widening():
    # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7: ties to the even 1.0.
    # 1 + 3*2^-8 lies halfway between 1+2^-7 and 1+2^-6: ties to the even 1 + 2^-6.
    got = oracle.f32_to_bf16(_f32(1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8)))
    assert list(got) == [0x3F80, 0x3F82, 0xBF80]
    assert np.array_equal(oracle.bf16_to_f32(np.array([0x3F80, 0xC000, 0x0001], np.uint16)),
                          _f32(1.0, -2.0, 2.0 ** -133))


def test_bf16_accumulates_in_fp32_and_rounds_once():
    # Rank order: 1 + 2^-8 + 2^-8 = 1 + 2^-7 exactly in fp32 -> bf16 0x3F81.
    # Rounding each partial to bf16 would give 1.0 (0x3F80): 1+2^-8 ties to 1.
    xs = [np.array([0x3F80], np.uint16), np.array([0x3B80], np.uint16),
          np.array([0x3B80], np.uint16)]
    assert oracle.naive_all_reduce(xs, "sum", "bf16")[0][0] == 0x3F81
    # avg divides the fp32 sum before the one rounding: (1+2^-7)/... with W=3
    got = oracle.naive_all_reduce(xs, "avg", "bf16")[0][0]
    q = np.float32(np.float32(1 + 2 ** -7) / np.float32(3))
    assert got == torch.tensor([float(q)]).to(torch.bfloat16).view(torch.int16).item() & 0xFFFF


# ------------------------------------------------------ invariants (P4) -----

@pytest.mark.parametrize("dtype,op", [("f32", "sum"), ("f32", "max"), ("i32", "sum"),
                                      ("i32", "max"), ("bf16", "avg"), ("f32", "avg")])
@pytest.mark.parametrize("w", [1, 2, 3, 4, 8])
def test_all_gather_of_reduce_scatter_is_all_reduce(dtype, op, w):
    rng = np.random.default_rng(w)
    n = w * 19
    if dtype == "i32":
        xs = [rng.integers(-1000, 1000, n).astype(np.int32) for _ in range(w)]
    elif dtype == "bf16":
        xs = [torch.from_numpy(rng.standard_normal(n).astype(np.float32)).to(torch.bfloat16)
              .view(torch.int16).numpy().view(np.uint16) for _ in range(w)]
    else:
        xs = [rng.standard_normal(n).astype(np.float32) for _ in range(w)]
    ag = oracle.all_gather(oracle.reduce_scatter(xs, op, dtype))
    ar = oracle.all_reduce(xs, op, dtype)
    for a, b in zip(ag, ar):
        assert a.tobytes() == b.tobytes()
    assert all(a.tobytes() == ar[0].tobytes() for a in ar)


def test_single_rank_is_identity():
    x = np.random.default_rng(0).standard_normal(33).astype(np.float32)
    assert oracle.reduce_scatter([x], "sum")[0].tobytes() == x.tobytes()
    assert oracle.all_reduce([x], "max")[0].tobytes() == x.tobytes()
    assert oracle.naive_all_reduce([x], "sum")[0].tobytes() == x.tobytes()


def test_empty_inputs():
    xs = [np.zeros(0, np.float32)] * 4
    assert all(len(s) == 0 for s in oracle.reduce_scatter(xs))
    assert all(len(s) == 0 for s in oracle.all_reduce(xs))


def test_reduce_scatter_needs_divisible_length():
    with pytest.raises(ValueError):
        oracle.reduce_scatter([np.zeros(10, np.float32)] * 4)


# --------------------------------------------- segment split (c3) -----------

def test_segment_bounds_hand_cases():
    assert oracle.segment_bounds(10, 4) == [(0, 3), (3, 6), (6, 9), (9, 10)]
    assert oracle.segment_bounds(2, 4) == [(0, 1), (1, 2), (2, 2), (2, 2)]
    assert oracle.segment_bounds(8, 4) == [(0, 2), (2, 4), (4, 6), (6, 8)]
    assert oracle.segment_bounds(0, 3) == [(0, 0)] * 3


def test_all_reduce_ragged_uses_each_segments_ring_order():
    # count = 10, W = 4, ceil split: [0,3) [3,6) [6,9) [9,10).  Probe element 3
    # (segment 1: order 2,3,0,1) and element 8 (segment 2: order 3,0,1,2).
    # A floor split ([6,10) last) or numpy.array_split ([8,10) last) would put
    # element 8 in segment 3, whose order 0,1,2,3 turns the same values into 2.
    w, n = 4, 10
    xs = [np.zeros(n, np.float32) for _ in range(w)]
    for e, k in ((3, 1), (8, 2)):
        xs[(k + 1) % w][e], xs[(k + 2) % w][e] = BIG, 1.0
        xs[(k + 3) % w][e], xs[k][e] = -BIG, 1.0
    ar = oracle.all_reduce(xs, "sum")
    assert ar[0][3] == 1.0 and ar[0][8] == 1.0
    assert oracle.naive_all_reduce(xs, "sum")[0][8] == 2.0


# -------------------------------------------------- buckets (c10) -----------

def test_buckets_restart_segmentation():
    # N = 16, bucket = 8, W = 4: each bucket has 2-element segments.  Element 8
    # is element 0 of bucket 1 -> segment 0 -> order 1,2,3,0 -> probe gives 1.
    # Without buckets element 8 is in segment 2 (order 3,0,1,2), where the same
    # values give 1 + (-2^24) ... = 2 (exact -2^24+1, +2^24, +1).
    w, n = 4, 16
    xs = [np.zeros(n, np.float32) for _ in range(w)]
    xs[1][8], xs[2][8], xs[3][8], xs[0][8] = BIG, 1.0, -BIG, 1.0
    assert oracle.bucketed_all_reduce(xs, 8, "sum")[0][8] == 1.0
    assert oracle.all_reduce(xs, "sum")[0][8] == 2.0
    # integer sums do not depend on the bucketing
    rng = np.random.default_rng(1)
    xi = [rng.integers(-9, 9, 23).astype(np.int32) for _ in range(w)]
    want = np.stack(xi).sum(0).astype(np.int32)
    for b in (1, 5, 8, 23, 100):
        assert all(np.array_equal(o, want) for o in oracle.bucketed_all_reduce(xi, b, "sum", "i32"))


# ----------------------------------------------------- fusion (c8) ----------

def test_fusion_offsets_and_round_trip():
    assert oracle.fuse_offsets([2, 3, 1]) == [0, 2, 5]
    ts = [_f32(1, 2), _f32(3, 4, 5), _f32(6)]
    fused = oracle.fuse_pack(ts)
    assert list(fused) == [1, 2, 3, 4, 5, 6]
    back = oracle.fuse_unpack(fused, [2, 3, 1])
    assert all(a.tobytes() == b.tobytes() for a, b in zip(back, ts))


def test_fused_all_reduce_int_sum_per_tensor():
    rng = np.random.default_rng(2)
    counts = [3, 1, 7, 2]
    per_rank = [[rng.integers(-50, 50, c).astype(np.int32) for c in counts] for _ in range(4)]
    out = oracle.fused_all_reduce(per_rank, "sum", "i32")
    for i, c in enumerate(counts):
        want = np.sum([per_rank[r][i] for r in range(4)], axis=0).astype(np.int32)
        for r in range(4):
            assert np.array_equal(out[r][i], want)


# ------------------------------------------------------ brute force (P1) ----

@pytest.mark.parametrize("w", [1, 2, 3, 4])
def test_brute_force_scalar_loop(w):
    # Scalar loop with the closed-form ring index (k+1+j) mod W, element by element.
    rng = np.random.default_rng(40 + w)
    s = 5
    xs = [rng.standard_normal(w * s).astype(np.float32) for _ in range(w)]
    rs = oracle.reduce_scatter(xs, "sum")
    for k in range(w):
        for i in range(s):
            acc = xs[(k + 1) % w][k * s + i]
            for j in range(2, w + 1):
                acc = np.float32(acc + xs[(k + j) % w][k * s + i])
            assert rs[k][i] == acc


# --------------------------------------------- fusion planner (Horovod) ----

def test_fusion_groups_hand_cases():
    f32 = "f32"
    # equality with the threshold still fuses: 10 + 20 + 30 = 60 <= 60
    assert oracle.fusion_groups([10, 20, 30, 40], [f32] * 4, 60) == [(0, 3), (3, 4)]
    assert oracle.fusion_groups([10, 20, 30, 40], [f32] * 4, 59) == [(0, 2), (2, 3), (3, 4)]
    # a tensor above the threshold is a group of its own
    assert oracle.fusion_groups([100, 1, 1], [f32] * 3, 50) == [(0, 1), (1, 3)]
    # a dtype change ends a group
    assert oracle.fusion_groups([1, 1, 1], [f32, "i32", f32], 10 ** 9) == [(0, 1), (1, 2), (2, 3)]
    # no tensor is skipped to fill a group
    assert oracle.fusion_groups([10, 100, 10], [f32] * 3, 50) == [(0, 1), (1, 2), (2, 3)]
    # threshold 0: only zero-byte tensors fuse
    assert oracle.fusion_groups([4, 4], [f32] * 2, 0) == [(0, 1), (1, 2)]
    assert oracle.fusion_groups([0, 0, 5], [f32] * 3, 4) == [(0, 2), (2, 3)]
    assert oracle.fusion_groups([], [], 64) == []


def test_grouped_all_reduce_int_sum_is_per_tensor_sum():
    rng = np.random.default_rng(4)
    counts = [5, 17, 3, 40, 1, 9]
    per_rank = [[rng.integers(-100, 100, c).astype(np.int32) for c in counts] for _ in range(3)]
    out = oracle.grouped_all_reduce(per_rank, threshold=4 * 30, op="sum", dtype="i32")
    for i in range(len(counts)):
        want = np.sum([per_rank[r][i] for r in range(3)], axis=0).astype(np.int32)
        for r in range(3):
            assert np.array_equal(out[r][i], want)


# ------------------------------------- wider types and prod (next rows) ----

INT_TYPES = {"i8": (np.int8, 8, True), "i32": (np.int32, 32, True),
             "i64": (np.int64, 64, True), "u64": (np.uint64, 64, False)}


def _wrap(v, bits, signed):
    v %= 2 ** bits
    return v - 2 ** bits if signed and v >= 2 ** (bits - 1) else v


@pytest.mark.parametrize("dt", list(INT_TYPES))
@pytest.mark.parametrize("op", ["sum", "prod"])
def test_integer_sum_prod_wrap_like_python_ints(dt, op):
    # Big-integer sum / product, reduced mod 2^bits: order-free and exact.
    np_t, bits, signed = INT_TYPES[dt]
    info = np.iinfo(np_t)
    rng = np.random.default_rng(bits)
    w, s = 5, 11
    xs = [rng.integers(info.min, info.max, w * s, dtype=np_t, endpoint=True) for _ in range(w)]
    got = np.concatenate(oracle.reduce_scatter(xs, op, dt))
    for e in range(w * s):
        vals = [int(x[e]) for x in xs]
        acc = 0 if op == "sum" else 1
        for v in vals:
            acc = acc + v if op == "sum" else acc * v
        assert int(got[e]) == _wrap(acc, bits, signed)


@pytest.mark.parametrize("dt", list(INT_TYPES))
def test_integer_max_min_avg(dt):
    np_t, bits, signed = INT_TYPES[dt]
    info = np.iinfo(np_t)
    rng = np.random.default_rng(100 + bits)
    xs = [rng.integers(info.min, info.max, 36, dtype=np_t, endpoint=True) for _ in range(4)]
    assert np.array_equal(np.concatenate(oracle.reduce_scatter(xs, "max", dt)), np.maximum.reduce(xs))
    assert np.array_equal(np.concatenate(oracle.reduce_scatter(xs, "min", dt)), np.minimum.reduce(xs))
    # avg: wrapped sum, then division toward zero (floor for unsigned)
    got = np.concatenate(oracle.reduce_scatter(xs, "avg", dt))
    for e in range(36):
        tot = _wrap(sum(int(x[e]) for x in xs), bits, signed)
        q = abs(tot) // 4
        assert int(got[e]) == (q if tot >= 0 else -q)


def test_signed_avg_hand_cases():
    xs = [np.array([-7, 7, -8, -128], np.int8), np.zeros(4, np.int8),
          np.zeros(4, np.int8), np.zeros(4, np.int8)]
    assert list(oracle.naive_all_reduce(xs, "avg", "i8")[0]) == [-1, 1, -2, -32]
    big = np.array([np.iinfo(np.int64).min], np.int64)
    assert oracle.naive_all_reduce([big, np.zeros(1, np.int64)], "avg", "i64")[0][0] == -(2 ** 62)
    u = [np.array([7], np.uint64), np.zeros(1, np.uint64), np.zeros(1, np.uint64), np.zeros(1, np.uint64)]
    assert oracle.naive_all_reduce(u, "avg", "u64")[0][0] == 1


def test_f64_probe_and_exact_sums():
    big = 2.0 ** 53
    # segment 0 at W=4: ring 1,2,3,0 over (x0..x3) = (1, 2^53, 1, -2^53) gives 1, rank order 0
    xs = [np.zeros(8) for _ in range(4)]
    for r, v in enumerate([1.0, big, 1.0, -big]):
        xs[r][0] = v
    assert oracle.reduce_scatter(xs, "sum", "f64")[0][0] == 1.0
    assert oracle.naive_all_reduce(xs, "sum", "f64")[0][0] == 0.0
    rng = np.random.default_rng(9)
    xi = [rng.integers(-2 ** 40, 2 ** 40, 64) for _ in range(8)]
    got = np.concatenate(oracle.reduce_scatter([x.astype(np.float64) for x in xi], "sum", "f64"))
    assert np.array_equal(got, np.sum(xi, axis=0).astype(np.float64))


def test_float_prod_powers_of_two_exact_and_bounded():
    rng = np.random.default_rng(12)
    e = [rng.integers(-20, 20, 42) for _ in range(6)]
    xs = [np.ldexp(np.float32(1), ei).astype(np.float32) * np.where(ei % 3 == 0, -1, 1).astype(np.float32)
          for ei in e]
    got = np.concatenate(oracle.reduce_scatter(xs, "prod", "f32"))
    want = np.prod(np.stack(xs).astype(np.float64), axis=0)
    assert np.array_equal(got.astype(np.float64), want)
    xs = [rng.standard_normal(60).astype(np.float32) for _ in range(6)]
    got = np.concatenate(oracle.reduce_scatter(xs, "prod", "f32")).astype(np.float64)
    exact = np.prod(np.stack(xs).astype(np.float64), axis=0)
    assert np.all(np.abs(got - exact) <= ((1 + 2.0 ** -24) ** 5 - 1) * np.abs(exact) * (1 + 1e-9))


def test_f16_rounding_hand_ties_and_torch_cast():
    f = np.float32
    got = oracle.f32_to_f16(np.array([1 + 2 ** -11, 1 + 3 * 2 ** -11, 65520.0, 65519.0,
                                      2.0 ** -25, 3 * 2.0 ** -25, -0.0], f))
    # 1+2^-11 ties to 1.0; 1+3*2^-11 ties to 1+2^-9; 65520 ties to inf (65504 has an
    # odd significand); 65519 rounds down to 65504; 2^-25 ties to 0; 1.5*2^-24 ties to 2^-23
    assert list(got) == [0x3C00, 0x3C02, 0x7C00, 0x7BFF, 0x0000, 0x0002, 0x8000]
    rng = np.random.default_rng(13)
    x = np.concatenate([rng.standard_normal(100_000).astype(f),
                        (rng.standard_normal(50_000) * 1e5).astype(f),
                        (rng.standard_normal(50_000) * 1e-6).astype(f)])
    want = torch.from_numpy(x).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.f32_to_f16(x), want)
    assert np.array_equal(oracle.f16_to_f32(want), torch.from_numpy(want.view(np.int16)).view(torch.float16).float().numpy())


H1, H_EPS = 0x3C00, 0x1000          # half 1.0 and 2^-11


def _h(*bits):
    return np.array(bits, dtype=np.uint16)


def test_f16_partial_rounded_to_half_after_every_ring_step():
    # W = 3, one element per block; block 0 is folded in ring order 1, 2, 0.
    # x1 = 1, x2 = x0 = 2^-11: 1 + 2^-11 is a half tie and goes to the even 1.0
    # at step 1 and again at step 2 -> 0x3C00.  An fp32 partial rounded once
    # at the end would give 1 + 2^-10 = 0x3C01.
    assert oracle.f16_to_f32(_h(H_EPS))[0] == 2.0 ** -11
    xs = [_h(H_EPS, 0, 0), _h(H1, 0, 0), _h(H_EPS, 0, 0)]
    assert oracle.reduce_scatter(xs, "sum", "f16")[0][0] == 0x3C00
    assert oracle.all_reduce(xs, "sum", "f16")[1][0] == 0x3C00
    # naive (rank order 0, 1, 2): 2^-11 + 1 -> 1.0, then + 2^-11 -> 1.0
    assert oracle.naive_all_reduce(xs, "sum", "f16")[2][0] == 0x3C00


def test_f16_ring_order_probe():
    # W = 4, segment 0, (x0..x3) = (1, 2048, 1, -2048).  Half spacing at 2048
    # is 2.  Ring order 1, 2, 3, 0: 2048 + 1 ties to 2048, - 2048 = 0, + 1 = 1.
    # Rank order: 1 + 2048 -> 2048, + 1 -> 2048, - 2048 = 0.  (In exact or
    # fp32 arithmetic both orders give 1.)
    vals = [0x3C00, 0x6800, 0x3C00, 0xE800]       # 1, 2048, 1, -2048
    xs = [_h(v, 0, 0, 0) for v in vals]
    assert oracle.reduce_scatter(xs, "sum", "f16")[0][0] == 0x3C00
    assert oracle.naive_all_reduce(xs, "sum", "f16")[0][0] == 0x0000


def test_f16_overflow_inside_the_fold_sticks():
    # 65504 + 16 = 65520 lies halfway between 65504 (odd significand) and 2^16,
    # which is beyond the format: it rounds to +inf, and inf - 65504 stays inf.
    # fp32 accumulation would give 16.
    xs = [_h(0x7BFF), _h(0x4C00), _h(0xFBFF)]      # 65504, 16, -65504
    assert oracle.naive_all_reduce(xs, "sum", "f16")[0][0] == 0x7C00
    # prod: 256 * 256 = 65536 overflows to inf; inf * 2^-8 = inf (exact: 256)
    xs = [_h(0x5C00), _h(0x5C00), _h(0x1C00)]      # 256, 256, 2^-8
    assert oracle.naive_all_reduce(xs, "prod", "f16")[0][0] == 0x7C00


def test_f16_avg_divides_the_half_fold():
    # half fold of (1, 2^-11, 2^-11) in rank order is 1.0; 1/3 rounded to half:
    # spacing 2^-12 in [1/4, 1/2), 4096/3 = 1365.33 -> 1365 * 2^-12 = 0x3555.
    # The fp32 fold 1 + 2^-10 divided by 3 would round to 1367 * 2^-12 = 0x3557.
    xs = [_h(H1), _h(H_EPS), _h(H_EPS)]
    assert oracle.naive_all_reduce(xs, "avg", "f16")[0][0] == 0x3555


def _half_exact(bits):
    """Exact rational value of a finite IEEE half bit pattern."""
    from fractions import Fraction
    sign = -1 if bits & 0x8000 else 1
    e, m = (bits >> 10) & 0x1F, bits & 0x3FF
    mag = Fraction(m, 2 ** 24) if e == 0 else Fraction(1024 + m, 1024) * Fraction(2) ** (e - 15)
    return sign * mag


def _round_half(q):
    """Round an exact rational to IEEE binary16 by the definition: nearest value
    on the grid of the operand's binade (subnormal spacing 2^-24 below 2^-14),
    ties to the even significand, +-inf once the rounded magnitude reaches 2^16.
    Returns a float (every half is exactly a Python float)."""
    from fractions import Fraction
    if q == 0:
        return 0.0
    neg, a = q < 0, abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, -14)
    ulp = Fraction(2) ** (e - 10)
    n, rem = divmod(a, ulp)
    n = int(n)
    rem = rem / ulp
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    val = n * ulp
    out = float("inf") if val >= 2 ** 16 else float(val)
    return -out if neg else out


def _random_finite_halves(rng, n):
    """Finite, nonzero halves spread over the whole range, with many ties."""
    mags = rng.choice([1e-6, 1e-3, 1.0, 30.0, 2000.0, 30000.0], n)
    with np.errstate(over="ignore"):
        x = (rng.standard_normal(n) * mags).astype(np.float16)
    x[x == 0] = np.float16(1.0)
    x[~np.isfinite(x)] = np.float16(-3.0)
    return x.view(np.uint16)


@pytest.mark.parametrize("w", [1, 2, 3, 4])
@pytest.mark.parametrize("op", ["sum", "prod", "max", "min", "avg"])
def test_f16_brute_force_exact_rationals(w, op):
    # Every ring step in exact rational arithmetic, rounded to half by the
    # definition above; block k is folded from rank (k+1) mod W round to k.
    rng = np.random.default_rng(300 + 7 * w + len(op))
    s = 16
    xs = [_random_finite_halves(rng, w * s) for _ in range(w)]
    got = np.concatenate(oracle.reduce_scatter(xs, op, "f16")).view(np.float16).astype(np.float64)
    from fractions import Fraction
    for k in range(w):
        for i in range(s):
            e = k * s + i
            acc = None
            for j in range(w):
                v = float(_half_exact(int(xs[(k + 1 + j) % w][e])))
                if acc is None:
                    acc = v
                elif op == "sum" or op == "avg":
                    acc = acc + v if np.isinf(acc) else _round_half(Fraction(acc) + Fraction(v))
                elif op == "prod":
                    acc = acc * v if np.isinf(acc) else _round_half(Fraction(acc) * Fraction(v))
                elif op == "max":
                    acc = v if v > acc else acc
                else:
                    acc = v if v < acc else acc
            if op == "avg" and np.isfinite(acc):
                acc = _round_half(Fraction(acc) / w)
            elif op == "avg":
                acc = acc / w
            g = got[e]
            assert (np.isnan(g) and np.isnan(acc)) or g == acc, (op, w, k, i, g, acc)


@pytest.mark.parametrize("op", ["sum", "prod"])
def test_f16_fold_matches_torch_cpu_half_arithmetic(op):
    # PyTorch's CPU half add / multiply (a library routine, correctly rounded to
    # half per operation), applied in ring order segment by segment.
    rng = np.random.default_rng(17)
    w, s = 5, 4000
    xs = [(rng.standard_normal(w * s) * (30 if op == "sum" else 1.5)).astype(np.float16).view(np.uint16)
          for _ in range(w)]
    got = np.concatenate(oracle.reduce_scatter(xs, op, "f16"))
    th = [torch.from_numpy(x.view(np.int16)).view(torch.float16) for x in xs]
    want = []
    for k in range(w):
        acc = th[(k + 1) % w][k * s:(k + 1) * s].clone()
        for j in range(1, w):
            x = th[(k + 1 + j) % w][k * s:(k + 1) * s]
            acc = acc + x if op == "sum" else acc * x
        want.append(acc.view(torch.int16).numpy().view(np.uint16))
    want = np.concatenate(want)
    same = (got == want) | (np.isnan(got.view(np.float16)) & np.isnan(want.view(np.float16)))
    assert same.all()
    # and it is not the fp32-accumulated result on this data
    acc32 = [np.sum(np.stack([oracle.f16_to_f32(x[k * s:(k + 1) * s]) for x in xs]), 0) for k in range(w)]
    assert op == "prod" or not np.array_equal(got, oracle.f32_to_f16(np.concatenate(acc32)))


def test_half_wire_partial_is_half_at_every_step():
    f = np.float32
    # 1, 2^-11, 2^-11 are exact halves; the half fold in rank order gives 1.0
    # (each 1 + 2^-11 ties to 1.0); an fp32 fold rounded once would give 1 + 2^-10.
    xs = [np.array([1.0], f), np.array([2 ** -11], f), np.array([2 ** -11], f)]
    assert oracle.naive_all_reduce(xs, "sum", "f32h")[0][0] == f(1.0)


def test_half_wire_rounds_inputs_and_result_to_half():
    f = np.float32
    # inputs: 1 + 2^-11 is a half tie and goes to 1.0 before the fold; 2^-11 and
    # 3 are exact halves.  Half fold in rank order: 1 + 2^-11 ties to 1.0, and
    # 1 + 3 = 4; the output is fp32 4.0.
    xs = [np.array([1 + 2 ** -11], f), np.array([2 ** -11], f), np.array([3.0], f)]
    out = oracle.naive_all_reduce(xs, "sum", "f32h")
    assert out[0].dtype == np.float32 and out[0][0] == f(4.0)
    # without the wire rounding the fp32 sum would be 4 + 2^-10
    assert oracle.naive_all_reduce(xs, "sum", "f32")[0][0] == f(4 + 2 ** -10)
    # beyond half's range: 70000 is inf on the wire
    big = [np.array([70000.0, -70000.0], f), np.zeros(2, f)]
    assert list(oracle.naive_all_reduce(big, "sum", "f32h")[0]) == [np.inf, -np.inf]
    # every output is a half value widened: it survives another round trip unchanged
    rng = np.random.default_rng(14)
    ys = [rng.standard_normal(96).astype(f) for _ in range(4)]
    for o in oracle.all_reduce(ys, "sum", "f32h"):
        assert np.array_equal(oracle.f16_to_f32(oracle.f32_to_f16(o)), o)


@pytest.mark.parametrize("op", ["sum", "max", "avg"])
def test_half_wire_small_integers_exact(op):
    # small integers (|sum| <= 800) are exact in half at every step
    rng = np.random.default_rng(15)
    xi = [rng.integers(-200, 200, 48) for _ in range(4)]
    got = oracle.all_reduce([x.astype(np.float32) for x in xi], op, "f32h")[0]
    st = np.stack(xi).astype(np.float64)
    want = {"sum": st.sum(0), "max": st.max(0), "avg": st.sum(0) / 4}[op]
    want = want.astype(np.float16).astype(np.float32)   # avg: a quarter step may round
    assert np.array_equal(got, want)


def test_half_wire_is_singa_float2half_allreduce_half2float():
    rng = np.random.default_rng(16)
    xs = [(rng.standard_normal(77) * 10).astype(np.float32) for _ in range(5)]
    lit = oracle.half_wire_all_reduce(xs, "sum")
    assert all(np.array_equal(a, b) for a, b in zip(lit, oracle.all_reduce(xs, "sum", "f32h")))
    lit = oracle.half_wire_all_reduce(xs, "max", "naive")
    assert all(np.array_equal(a, b) for a, b in zip(lit, oracle.naive_all_reduce(xs, "max", "f32h")))
