"""Parity of the HIP path (through the C ABI) with the CPU oracle.

fp32 and int32 must match bit for bit, bf16 within one bf16 ulp (NaN where
NaN).  Sizes span several workgroup tiles plus a ragged tail; every rank
count 1..16 class, every op and dtype, both the dwordx4 and the unaligned
kernels, in-place forms, the naive algorithm, all-gather and the fusion path.
"""
import numpy as np
import pytest
import torch

import collective_reduction_ring_amd as rsx
import oracle
from collective_reduction_ring_amd import workloads as wl
from parity_util import assert_parity, empty, say, to_dev, to_host

pytestmark = pytest.mark.gpu

DIST = {"f32": "normal", "bf16": "normal_bf16", "i32": "int_full", "f64": "normal_f64",
        "f16": "normal_f16", "i64": "int64_full", "u64": "uint64_full", "i8": "int8_full",
        "f32h": "normal"}
VL = {"f32": 4, "bf16": 8, "i32": 4, "f64": 2, "f16": 8, "i64": 2, "u64": 2, "i8": 16, "f32h": 4}
ALL_DTYPES = list(DIST)
ES = {"f32": 4, "bf16": 2, "i32": 4, "f64": 8, "f16": 2, "i64": 8, "u64": 8, "i8": 1, "f32h": 4}
RSX_NAIVE_MAX_BYTES = 32768


def wire(dtype):
    """"f32h" = float32 tensors reduced with half as the wire format."""
    return "f16" if dtype == "f32h" else None


def units(w):  # dwordx4 per lane per source in the fold kernels
    return 1


def tile_elems(w, dtype):
    return units(w) * 256 * VL[dtype]


def inputs(seed, w, n, dtype, dist=None):
    return [wl.draw(dist or DIST[dtype], np.random.default_rng((seed, w, r)), n) for r in range(w)]


def run_rs(xs, dtype, op, recvcount):
    dev = [to_dev(x, dtype) for x in xs]
    out = [empty(recvcount, dtype, fill=0x55) for _ in xs]
    rsx.reduce_scatter(dev, out, op, wire=wire(dtype))
    torch.cuda.synchronize()
    return [to_host(o, dtype) for o in out]


def run_ar(xs, dtype, op, algo="ring", in_place=False):
    dev = [to_dev(x, dtype) for x in xs]
    out = None if in_place else [empty(len(xs[0]), dtype, fill=0x55) for _ in xs]
    rsx.all_reduce(dev, out, op, algo, wire=wire(dtype))
    torch.cuda.synchronize()
    return [to_host(o, dtype) for o in (dev if in_place else out)]


OPS = ["sum", "max", "min", "avg", "prod"]
WORLDS = [1, 2, 3, 4, 5, 8, 13, 16]


# ------------------------------------------------------- reduce-scatter ----

@pytest.mark.parametrize("dtype", ALL_DTYPES)
@pytest.mark.parametrize("op", OPS)
@pytest.mark.parametrize("w", WORLDS)
@pytest.mark.parametrize("aligned", [True, False])
def test_reduce_scatter(w, op, dtype, aligned):
    te = tile_elems(w, dtype)
    recvcount = 2 * te + te // 2 + 3 * VL[dtype] + (0 if aligned else 1)
    xs = inputs(1, w, w * recvcount, dtype)
    say(f"rs w={w} op={op} dtype={dtype} recvcount={recvcount}")
    got = run_rs(xs, dtype, op, recvcount)
    want = oracle.reduce_scatter(xs, op, dtype)
    for k in range(w):
        assert_parity(got[k], want[k], dtype, f"block {k}")


@pytest.mark.parametrize("dtype", ALL_DTYPES)
@pytest.mark.parametrize("op", OPS)
@pytest.mark.parametrize("w", WORLDS)
@pytest.mark.parametrize("algo", ["ring", "naive"])
def test_all_reduce(w, op, dtype, algo):
    te = tile_elems(w, dtype)
    count = w * (2 * te + te // 3) + 5   # divisible by neither W nor the vector width
    xs = inputs(2, w, count, dtype)
    say(f"ar w={w} op={op} dtype={dtype} algo={algo} count={count}")
    got = run_ar(xs, dtype, op, algo)
    want = (oracle.all_reduce if algo == "ring" else oracle.naive_all_reduce)(xs, op, dtype)
    for r in range(w):
        assert_parity(got[r], want[r], dtype, f"rank {r}")


@pytest.mark.parametrize("dtype", ALL_DTYPES)
@pytest.mark.parametrize("w", WORLDS)
@pytest.mark.parametrize("ragged", [False, True])
def test_all_reduce_two_pass_form(w, dtype, ragged):
    # Reduce-scatter into each output's own segment, then an in-place
    # all-gather: the same bits as the one-pass form and the oracle.  A
    # segment that is not a whole number of 16-byte vectors takes the
    # element-wise kernels.  Op and in-place vary with the case.
    te = tile_elems(w, dtype)
    seg = 2 * te + te // 2 + 3 * VL[dtype] + (1 if ragged else 0)
    i = WORLDS.index(w) + 3 * ALL_DTYPES.index(dtype) + int(ragged)
    op, in_place = OPS[i % len(OPS)], bool(i % 2)
    xs = inputs(21, w, w * seg, dtype)
    say(f"ar two-pass w={w} dtype={dtype} seg={seg} op={op} in_place={in_place}")
    got = run_ar(xs, dtype, op, "ring_split", in_place)
    fused = run_ar(xs, dtype, op, "ring_fused", in_place)
    want = oracle.all_reduce(xs, op, dtype)
    for r in range(w):
        assert_parity(got[r], want[r], dtype, f"two-pass rank {r}")
        assert_parity(fused[r], want[r], dtype, f"one-pass rank {r}")


@pytest.mark.parametrize("op", OPS)
@pytest.mark.parametrize("dtype", ["f32", "bf16", "i32", "f32h"])
def test_all_reduce_two_pass_every_op(op, dtype):
    w = 8
    seg = 3 * tile_elems(w, dtype) + 5 * VL[dtype]
    xs = inputs(22, w, w * seg, dtype)
    say(f"ar two-pass w={w} dtype={dtype} op={op}")
    got = run_ar(xs, dtype, op, "ring_split")
    want = oracle.all_reduce(xs, op, dtype)
    for r in range(w):
        assert_parity(got[r], want[r], dtype, f"rank {r}")


@pytest.mark.parametrize("w,dtype,count,in_place,algo", [
    (4, "f32", 1 << 20, False, "ring"),
    (4, "f32", 1 << 20, False, "ring_split"),
    (8, "bf16", 1 << 21, True, "ring"),
    (8, "bf16", 1 << 21, True, "ring_split"),
    (16, "i32", (1 << 20) + 8, False, "ring"),    # W does not divide count
    (3, "f32", 3 << 20, False, "ring_split"),
    (11, "f32", 11 << 18, False, "ring_split"),
    (2, "f32", 1 << 21, False, "ring_split"),
    # the shapes where the launch shape changes: the one-pass all-reduce runs
    # two tiles per 512-lane workgroup from W = 5; `ring` takes two passes
    # (its all-gather in place with pairs) from W = 7 and 4 MiB per rank
    (5, "f32", 5 << 18, False, "ring"),
    (6, "f32", 6 << 18, True, "ring"),
    (7, "f32", 7 << 18, False, "ring"),
    (7, "bf16", 7 << 19, True, "ring_fused"),
    (12, "i32", 12 << 18, False, "ring"),
    (16, "f32", 16 << 16, True, "ring"),           # exactly 4 MiB per rank
    (16, "f32", (16 << 16) - 16, False, "ring"),   # just below: one pass
])
@pytest.mark.parametrize("caps", [True, False])
def test_large_grids_with_occupancy_caps(w, dtype, count, in_place, algo, caps):
    # Grids of thousands of workgroups, far more than the capped number of
    # resident workgroups per CU (the caps depend on W and the kernel), with
    # the caps on and off: the all-reduce and, where W divides count, the
    # reduce-scatter give the oracle's bits.
    xs = inputs(23, w, count, dtype)
    say(f"large grid ar w={w} dtype={dtype} count={count} in_place={in_place} algo={algo} caps={caps}")
    with rsx.occupancy_caps(caps):
        got = run_ar(xs, dtype, "sum", algo, in_place)
    want = oracle.all_reduce(xs, "sum", dtype)
    for r in range(w):
        assert_parity(got[r], want[r], dtype, f"rank {r}")
    if count % w == 0:
        say(f"large grid rs w={w} dtype={dtype} recvcount={count // w} caps={caps}")
        with rsx.occupancy_caps(caps):
            got = run_rs(xs, dtype, "sum", count // w)
        want = oracle.reduce_scatter(xs, "sum", dtype)
        for k in range(w):
            assert_parity(got[k], want[k], dtype, f"block {k}")


@pytest.mark.parametrize("w,dtype,extra", [(3, "f32", 1), (8, "f32", 3), (16, "f32", 2), (8, "bf16", 5),
                                           (5, "i8", 11), (8, "f64", 1), (2, "f16", 7), (8, "i32", 2),
                                           (12, "f32", 1), (8, "bf16", 6), (4, "i8", 12), (11, "i64", 1)])
@pytest.mark.parametrize("caps", [True, False])
def test_reduce_scatter_blocks_of_partial_vectors(w, dtype, extra, caps):
    # Block length a whole number of vectors plus `extra` elements, on
    # 16-byte-aligned buffers: every block but the first starts mid-vector in
    # the sources, the last reaches the end of them; thousands of
    # workgroups.  Blocks whose byte length is a multiple of 4 take the
    # dwordx4 kernel (dword-aligned loads, a tail per block; W >= 10 in
    # pairs when capped), the others the element-wise kernel.
    recvcount = (1 << 17) + extra
    xs = inputs(27, w, w * recvcount, dtype)
    say(f"rs partial-vector blocks w={w} dtype={dtype} recvcount={recvcount} caps={caps}")
    with rsx.occupancy_caps(caps):
        got = run_rs(xs, dtype, "sum", recvcount)
    want = oracle.reduce_scatter(xs, "sum", dtype)
    for k in range(w):
        assert_parity(got[k], want[k], dtype, f"block {k}")


def test_two_pass_with_outputs_a_permutation_of_the_inputs():
    # recvbufs[r] == sendbufs[(r + 1) % W]: the reduce-scatter overwrites a
    # segment of another rank's input only in the lanes that already read it.
    for w, algo in ((8, "ring_split"), (8, "ring"), (5, "ring_split")):
        seg = (1 << 19) if algo == "ring" else 3000
        xs = inputs(24, w, w * seg, "f32")
        dev = [to_dev(x, "f32") for x in xs]
        say(f"ar permuted outputs w={w} algo={algo}")
        rsx.all_reduce(dev, [dev[(r + 1) % w] for r in range(w)], "sum", algo)
        torch.cuda.synchronize()
        want = oracle.all_reduce(xs, "sum", "f32")
        for r in range(w):
            assert_parity(to_host(dev[r], "f32"), want[r], "f32", f"rank {r}")


def test_two_pass_unaligned_and_refusals():
    w, s = 4, 3001
    xs = inputs(25, w, w * s, "f32")
    bases = [to_dev(np.concatenate([np.zeros(1, np.float32), x]), "f32") for x in xs]
    dev = [b[1:] for b in bases]                      # 4-byte offset: not 16-byte aligned
    outs = [empty(w * s + 3, "f32")[3:] for _ in range(w)]
    say("unaligned two-pass ar")
    rsx.all_reduce(dev, outs, "min", "ring_split")
    torch.cuda.synchronize()
    want = oracle.all_reduce(xs, "min", "f32")
    for r in range(w):
        assert_parity(to_host(outs[r], "f32"), want[r], "f32", f"rank {r}")
    with pytest.raises(rsx.RsxError) as e:           # W does not divide count
        rsx.all_reduce([d[:-1] for d in dev], None, "sum", "ring_split")
    assert e.value.status == 4
    tens = [[to_dev(x[:100], "f32")] for x in xs]
    with pytest.raises(rsx.RsxError) as e:           # the tensor-list kernel is one pass only
        rsx.TensorFusionAllReduce(tens, None, "sum", "ring_split")()
    assert e.value.status == 4


def test_two_pass_graph_capture_replays():
    w, n = 8, 8 * 4096
    xs = inputs(26, w, n, "bf16")
    dev = [to_dev(x, "bf16") for x in xs]
    out = [empty(n, "bf16") for _ in range(w)]
    ar = rsx.AllReduce(dev, out, "avg", "ring_split")
    want = oracle.all_reduce(xs, "avg", "bf16")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ar()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    say("graph capture two-pass ar")
    with torch.cuda.graph(g):
        ar()
    for rep in range(4):
        for o in out:
            o.fill_(3.0)                      # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for r in range(w):
            assert_parity(to_host(out[r], "bf16"), want[r], "bf16", f"replay {rep} rank {r}")


@pytest.mark.parametrize("kind", ["bucketed", "gather_dword"])
def test_graph_capture_replays_grouped_buckets_and_dword_gather(kind):
    # The grouped bucket launches (W divides the bucket: one launch per pass
    # over the full buckets, then the last bucket) and the all-gather of
    # pieces that are whole dwords but not whole vectors, captured in a HIP
    # graph and replayed with eager work in between.
    w = 8
    if kind == "bucketed":
        bucket = 8 * 5000
        n = 3 * bucket + 8 * 123
        xs = inputs(27, w, n, "bf16")
        dev = [to_dev(x, "bf16") for x in xs]
        out = [empty(n, "bf16") for _ in range(w)]
        plan = rsx.AllReduceBucketed(dev, out, bucket, "avg", "ring_split")
        want = oracle.bucketed_all_reduce(xs, bucket, "avg", "bf16")
        dt = "bf16"
    else:
        n = 4096 + 3
        pieces = inputs(28, w, n, "f32")
        src = [to_dev(p, "f32") for p in pieces]
        out = [empty(w * n, "f32") for _ in range(w)]
        plan = lambda: rsx.all_gather(src, out)  # noqa: E731
        want = oracle.all_gather(pieces)
        dt = "f32"
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        plan()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    say(f"graph capture {kind}")
    with torch.cuda.graph(g):
        plan()
    for rep in range(4):
        for o in out:
            o.fill_(3.0)                      # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for r in range(w):
            assert_parity(to_host(out[r], dt), want[r], dt, f"replay {rep} rank {r}")


def _with_ieee_specials(xs, dtype, seed):
    """Normal data with IEEE specials planted: +-inf, NaN, +-0, the smallest
    subnormal and values near the top of the range (sums and products then
    overflow, tiny products underflow)."""
    ft = np.float32 if dtype == "f32" else np.float64
    fi = np.finfo(ft)
    specials = np.array([np.inf, -np.inf, np.nan, 0.0, -0.0, fi.smallest_subnormal, -fi.smallest_subnormal,
                         fi.max / 2, -fi.max / 2, fi.tiny, 1e-30 if dtype == "f32" else 1e-300], ft)
    rng = np.random.default_rng(seed)
    out = []
    for x in xs:
        x = x.astype(ft).copy()
        pos = rng.choice(len(x), len(x) // 8, replace=False)
        x[pos] = specials[rng.integers(0, len(specials), len(pos))]
        out.append(x)
    return out


@pytest.mark.parametrize("dtype", ["f32", "f64"])
@pytest.mark.parametrize("op", ["sum", "prod", "avg"])
@pytest.mark.parametrize("w", [2, 3, 8])
def test_ieee_specials_rs_and_ar(w, op, dtype):
    # inf - inf and 0 * inf give NaN, overflow gives inf, subnormals are kept
    # (no flush to zero), -0 + -0 stays -0: bit for bit against the oracle
    te = tile_elems(w, dtype)
    recvcount = te + 7
    xs = _with_ieee_specials(inputs(4, w, w * recvcount, dtype), dtype, (40, w))
    say(f"ieee specials rs/ar w={w} op={op} dtype={dtype}")
    got = run_rs(xs, dtype, op, recvcount)
    want = oracle.reduce_scatter(xs, op, dtype)
    for k in range(w):
        assert_parity(got[k], want[k], dtype, f"rs block {k}")
    got = run_ar(xs, dtype, op, "ring")
    want = oracle.all_reduce(xs, op, dtype)
    for r in range(w):
        assert_parity(got[r], want[r], dtype, f"ar rank {r}")


@pytest.mark.parametrize("case", range(60))
def test_random_configurations(case):
    # Seeded random mixes of rank count, size, type, op, algorithm and
    # in-place form, for both collectives.
    rng = np.random.default_rng((72, case))
    w = int(rng.integers(1, 17))
    dtype = str(rng.choice(ALL_DTYPES))
    op = str(rng.choice(OPS))
    recvcount = int(rng.integers(1, 3 * tile_elems(w, dtype) // max(1, w // 4)))
    xs = inputs(5 + case, w, w * recvcount, dtype)
    say(f"random {case}: rs w={w} dtype={dtype} op={op} recvcount={recvcount}")
    got = run_rs(xs, dtype, op, recvcount)
    want = oracle.reduce_scatter(xs, op, dtype)
    for k in range(w):
        assert_parity(got[k], want[k], dtype, f"rs block {k}")
    count = int(rng.integers(1, 3 * tile_elems(w, dtype)))
    algo = str(rng.choice(["ring", "naive", "auto"]))
    in_place = bool(rng.random() < 0.5)
    xs = inputs(500 + case, w, count, dtype)
    say(f"random {case}: ar w={w} dtype={dtype} op={op} count={count} algo={algo} in_place={in_place}")
    got = run_ar(xs, dtype, op, algo, in_place)
    # auto: naive at or below RSX_NAIVE_MAX_BYTES of elements per rank (rsx.h)
    naive = algo == "naive" or (algo == "auto" and count * ES[dtype] <= RSX_NAIVE_MAX_BYTES)
    want = (oracle.naive_all_reduce if naive else oracle.all_reduce)(xs, op, dtype)
    for r in range(w):
        assert_parity(got[r], want[r], dtype, f"ar rank {r}")


def _offset_dev(x, dtype, off):
    # x on the device starting `off` elements into its allocation
    base = to_dev(np.concatenate([np.zeros(off, dtype=x.dtype), x]), dtype)
    return base[off:]


@pytest.mark.parametrize("case", range(30))
def test_random_bucketed_and_all_gather(case):
    # Seeded random mixes for the bucketed all-reduce (bucket sizes that W
    # divides or not, every algorithm, in place or not, buffers 0, 1 or 4
    # elements past an aligned address) and the all-gather (random piece
    # lengths and offsets).
    rng = np.random.default_rng((73, case))
    w = int(rng.integers(1, 17))
    dtype = str(rng.choice(ALL_DTYPES))
    op = str(rng.choice(OPS))
    te = tile_elems(w, dtype)
    bucket = int(rng.integers(1, 4 * te)) * (w if rng.random() < 0.5 else 1)
    count = int(rng.integers(1, 5)) * bucket + int(rng.integers(0, bucket))
    algo = str(rng.choice(["ring", "ring_fused", "naive", "auto"]))
    in_place = bool(rng.random() < 0.5)
    off = int(rng.choice([0, 1, 4]))
    xs = inputs(900 + case, w, count, dtype)
    dev = [_offset_dev(x, dtype, off) for x in xs]
    out = None if in_place else [_offset_dev(np.zeros_like(x), dtype, off) for x in xs]
    say(f"random {case}: bucketed w={w} dtype={dtype} op={op} count={count} bucket={bucket} algo={algo} "
        f"in_place={in_place} off={off}")
    rsx.all_reduce_bucketed(dev, out, bucket, op, algo, wire=wire(dtype))
    torch.cuda.synchronize()
    for r in range(w):
        got = to_host((dev if in_place else out)[r], dtype)
        for b0 in range(0, count, bucket):
            b1 = min(b0 + bucket, count)
            naive = algo == "naive" or (algo == "auto" and (b1 - b0) * ES[dtype] <= RSX_NAIVE_MAX_BYTES)
            want = (oracle.naive_all_reduce if naive else oracle.all_reduce)([x[b0:b1] for x in xs], op, dtype)
            assert_parity(got[b0:b1], want[r], dtype, f"rank {r} bucket at {b0}")
    n = int(rng.integers(1, 3 * te))
    pieces = inputs(950 + case, w, n, dtype)
    src = [_offset_dev(p, dtype, off) for p in pieces]
    dst = [_offset_dev(np.zeros(w * n, dtype=pieces[0].dtype), dtype, int(rng.choice([0, 1, 4]))) for _ in range(w)]
    say(f"random {case}: ag w={w} dtype={dtype} n={n} off={off}")
    rsx.all_gather(src, dst)
    torch.cuda.synchronize()
    want = oracle.all_gather(pieces)
    for r in range(w):
        assert_parity(to_host(dst[r], dtype), want[r], dtype, f"ag rank {r}")


@pytest.mark.parametrize("count", [1, 2, 3, 7, 8, 9, 15, 16, 17, 31, 33, 100, 1023])
@pytest.mark.parametrize("w", [2, 4, 16])
def test_all_reduce_small_and_ragged(w, count):
    for dtype in ("f32", "bf16"):
        xs = inputs(3, w, count, dtype)
        say(f"ar small w={w} count={count} dtype={dtype}")
        got = run_ar(xs, dtype, "sum", "ring")
        want = oracle.all_reduce(xs, "sum", dtype)
        for r in range(w):
            assert_parity(got[r], want[r], dtype, f"rank {r}")


def test_ring_order_probe():
    # Segment 0 at W=4 with x0=1, x1=2^24, x2=1, x3=-2^24: only ring order
    # 1,2,3,0 gives 1; rank order gives 0; reverse ring order gives 2.
    big = np.float32(2.0 ** 24)
    s = 1024
    xs = [np.zeros(4 * s, np.float32) for _ in range(4)]
    for k in range(4):  # same probe in every block k, at its element 5
        xs[(k + 1) % 4][k * s + 5], xs[(k + 2) % 4][k * s + 5] = big, 1.0
        xs[(k + 3) % 4][k * s + 5], xs[k][k * s + 5] = -big, 1.0
    say("ring-order probe")
    rs = run_rs(xs, "f32", "sum", s)
    assert [rs[k][5] for k in range(4)] == [1.0] * 4
    ar = run_ar(xs, "f32", "sum", "ring")
    assert all(ar[r][k * s + 5] == 1.0 for r in range(4) for k in range(4))
    nv = run_ar(xs, "f32", "sum", "naive")
    # rank order: block 0 gives 0 (as above); blocks 1..3 start elsewhere
    want = oracle.naive_all_reduce(xs, "sum", "f32")
    assert nv[0][5] == 0.0
    assert_parity(nv[0], want[0], "f32", "naive")


def test_max_min_ties_and_nans():
    nan = np.float32("nan")
    base0 = np.array([-0.0, 0.0, nan, 1.0, -np.inf, 3.0, nan, 0.0], np.float32)
    base1 = np.array([0.0, -0.0, 1.0, nan, np.inf, 3.0, nan, -0.0], np.float32)
    xs = [np.tile(base0, 128), np.tile(base1, 128)]   # 1024 elements, two ranks
    for op in ("max", "min"):
        say(f"ties/NaN op={op}")
        got = run_rs(xs, "f32", op, 512)
        want = oracle.reduce_scatter(xs, op, "f32")
        for k in range(2):
            assert_parity(got[k], want[k], "f32", f"{op} block {k}")
            assert np.array_equal(np.signbit(got[k]), np.signbit(want[k]))


def test_bf16_specials_and_rounding_ties():
    # Tie cases and specials: 1+2^-8 pairs (rounds to even), large values
    # overflowing to inf, NaN, +-0.
    vals = [0x3F80, 0x3B80, 0x3B80, 0x7F7F, 0x7F7F, 0x7FC0, 0x8000, 0x0000]
    xs = [np.tile(np.array(vals, np.uint16), 64) for _ in range(4)]
    xs[1] = np.roll(xs[1], 1)
    xs[2] = np.roll(xs[2], 2)
    for op in OPS:
        say(f"bf16 specials op={op}")
        got = run_ar(xs, "bf16", op, "ring")
        want = oracle.all_reduce(xs, op, "bf16")
        assert_parity(got[0], want[0], "bf16", op)


# ----------------------------------------------------------- in place -------

@pytest.mark.parametrize("algo", ["ring", "naive"])
def test_half_wire_ties_ranges_and_one_rank(algo):
    # half ties, values beyond half's range, half subnormals and fp32 values
    # below them, in fp32 tensors; W = 1 (also in place) still rounds.
    f = np.float32
    special = np.array([1 + 2 ** -11, 1 + 3 * 2 ** -11, 65519.0, 65520.0, 1e5, -1e5, 2.0 ** -25,
                        3 * 2.0 ** -25, 1e-9, -0.0, np.inf, np.nan, 4 + 2 ** -11, 2.0 ** -14], f)
    rng = np.random.default_rng(31)
    for w in (1, 3, 4):
        xs = [np.concatenate([np.tile(special, 40), (rng.standard_normal(3000) * 3e4).astype(f),
                              (rng.standard_normal(3000) * 1e-6).astype(f)]) for _ in range(w)]
        say(f"half wire specials w={w} algo={algo}")
        got = run_ar(xs, "f32h", "sum", algo)
        want = (oracle.all_reduce if algo == "ring" else oracle.naive_all_reduce)(xs, "sum", "f32h")
        lit = oracle.half_wire_all_reduce(xs, "sum", algo)
        for r in range(w):
            assert_parity(got[r], want[r], "f32h", f"rank {r}")
            assert_parity(got[r], lit[r], "f32h", f"rank {r} vs float2half-allreduce-half2float")
    say("half wire W=1 in place")
    got = run_ar([xs[0][:1000]], "f32h", "avg", algo, in_place=True)
    assert_parity(got[0], oracle.f16_to_f32(oracle.f32_to_f16(xs[0][:1000])), "f32h", "W=1")


@pytest.mark.parametrize("dtype", ALL_DTYPES)
@pytest.mark.parametrize("w", [1, 2, 4, 8])
def test_in_place(w, dtype):
    te = tile_elems(w, dtype)
    s = te + 2 * VL[dtype]
    xs = inputs(4, w, w * s, dtype)
    dev = [to_dev(x, dtype) for x in xs]
    say(f"in-place rs w={w} dtype={dtype}")
    rsx.reduce_scatter(dev, [dev[k][k * s:(k + 1) * s] for k in range(w)], "sum", wire=wire(dtype))
    torch.cuda.synchronize()
    want = oracle.reduce_scatter(xs, "sum", dtype)
    for k in range(w):
        assert_parity(to_host(dev[k][k * s:(k + 1) * s], dtype), want[k], dtype, f"rs block {k}")
    say(f"in-place ar w={w} dtype={dtype}")
    got = run_ar(xs, dtype, "avg", "ring", in_place=True)
    want = oracle.all_reduce(xs, "avg", dtype)
    for r in range(w):
        assert_parity(got[r], want[r], dtype, f"ar rank {r}")


def test_unaligned_pointers():
    w, s = 4, 3000
    xs = inputs(5, w, w * s, "f32")
    bases = [to_dev(np.concatenate([np.zeros(1, np.float32), x]), "f32") for x in xs]
    dev = [b[1:] for b in bases]                      # 4-byte offset: not 16-byte aligned
    outs = [empty(s + 3, "f32")[3:] for _ in range(w)]
    say("unaligned rs")
    rsx.reduce_scatter(dev, outs, "sum")
    torch.cuda.synchronize()
    want = oracle.reduce_scatter(xs, "sum", "f32")
    for k in range(w):
        assert_parity(to_host(outs[k], "f32"), want[k], "f32", f"block {k}")
    say("unaligned ar")
    outs = [empty(w * s + 1, "f32")[1:] for _ in range(w)]
    rsx.all_reduce(dev, outs, "max")
    torch.cuda.synchronize()
    want = oracle.all_reduce(xs, "max", "f32")
    for r in range(w):
        assert_parity(to_host(outs[r], "f32"), want[r], "f32", f"rank {r}")


def test_side_stream_and_repeat():
    w, s = 8, 8192
    xs = inputs(6, w, w * s, "f32")
    dev = [to_dev(x, "f32") for x in xs]
    out = [empty(s, "f32") for _ in range(w)]
    plan = rsx.ReduceScatter(dev, out, "sum")
    st = torch.cuda.Stream()
    say("side stream rs x5")
    with torch.cuda.stream(st):
        for _ in range(5):
            plan()
    st.synchronize()
    want = oracle.reduce_scatter(xs, "sum", "f32")
    for k in range(w):
        assert_parity(to_host(out[k], "f32"), want[k], "f32", f"block {k}")


def test_graph_capture_replays():
    # Library launches captured in a HIP graph: every replay, with eager work
    # and synchronisation in between, must equal the eager result.
    w, n = 4, 4 * 1024 + 12
    xs = inputs(10, w, n, "f32")
    dev = [to_dev(x, "f32") for x in xs]
    out_rs = [empty(n // w, "f32") for _ in range(w)]
    out_ar = [empty(n, "f32") for _ in range(w)]
    rs = rsx.ReduceScatter(dev, out_rs, "sum")
    ar = rsx.AllReduce(dev, out_ar, "max", "ring")
    want_rs = oracle.reduce_scatter(xs, "sum", "f32")
    want_ar = oracle.all_reduce(xs, "max", "f32")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        rs()
        ar()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    say("graph capture rs + ar")
    with torch.cuda.graph(g):
        rs()
        ar()
    for rep in range(4):
        for o in out_rs + out_ar:
            o.fill_(-7.0)                     # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in range(w):
            assert_parity(to_host(out_rs[k], "f32"), want_rs[k], "f32", f"replay {rep} rs {k}")
            assert_parity(to_host(out_ar[k], "f32"), want_ar[k], "f32", f"replay {rep} ar {k}")


# ---------------------------------------------------------- all-gather ------

@pytest.mark.parametrize("dtype", ["f32", "bf16", "f64", "i8"])
@pytest.mark.parametrize("w", [1, 2, 3, 8, 16])
@pytest.mark.parametrize("n", [1, 5, 8, 4096 + 8, 4096 + 3])
def test_all_gather(w, n, dtype):
    pieces = inputs(7, w, n, dtype)
    dev = [to_dev(p, dtype) for p in pieces]
    out = [empty(w * n, dtype, fill=0x11) for _ in range(w)]
    say(f"ag w={w} n={n} dtype={dtype}")
    rsx.all_gather(dev, out)
    torch.cuda.synchronize()
    want = oracle.all_gather(pieces)
    for r in range(w):
        assert_parity(to_host(out[r], dtype), want[r], dtype, f"rank {r}")


def test_all_gather_in_place_and_composition():
    w, n = 4, 10_000
    xs = inputs(8, w, w * n, "f32")
    dev = [to_dev(x, "f32") for x in xs]
    say("rs in place then ag in place")
    rsx.reduce_scatter(dev, [dev[k][k * n:(k + 1) * n] for k in range(w)], "sum")
    rsx.all_gather([dev[k][k * n:(k + 1) * n] for k in range(w)], dev)
    torch.cuda.synchronize()
    want = oracle.all_reduce(xs, "sum", "f32")   # AG(RS) == AR when W divides N
    for r in range(w):
        assert_parity(to_host(dev[r], "f32"), want[r], "f32", f"rank {r}")


@pytest.mark.parametrize("w", [2, 3, 4, 5, 6, 7, 8, 12, 16])
@pytest.mark.parametrize("in_place", [False, True])
@pytest.mark.parametrize("caps", [True, False])
@pytest.mark.parametrize("extra", [4, 3])
def test_all_gather_large_grids(w, in_place, caps, extra):
    # Pieces of 512 Ki + 4 fp32 (a ragged last tile), thousands of workgroups:
    # every occupancy cap the all-gather uses (in place and out of place,
    # W = 2..16), and none.  With 512 Ki + 3 the pieces sit at offsets that
    # are not 16-byte multiples in the outputs: an element head, dword-aligned
    # vector loads and an element tail per piece.
    n = (1 << 19) + extra
    pieces = inputs(9, w, n, "f32")
    out = [empty(w * n, "f32", fill=0x11) for _ in range(w)]
    if in_place:
        for k in range(w):
            out[k][k * n:(k + 1) * n].copy_(to_dev(pieces[k], "f32"))
        src = [out[k][k * n:(k + 1) * n] for k in range(w)]
    else:
        src = [to_dev(p, "f32") for p in pieces]
    say(f"ag large grid w={w} n={n} in_place={in_place} caps={caps}")
    with rsx.occupancy_caps(caps):
        rsx.all_gather(src, out)
    torch.cuda.synchronize()
    want = oracle.all_gather(pieces)
    for r in range(w):
        assert_parity(to_host(out[r], "f32"), want[r], "f32", f"rank {r}")


# --------------------------------------------------------------- fusion -----

@pytest.mark.parametrize("dtype", ["f32", "bf16", "f64", "i8", "f16", "f32h"])
def test_fused_pack_allreduce_unpack(dtype):
    w = 4
    sizes = wl.fused_sizes(count=70, lo=1, hi=70_000)
    per_rank = [[wl.draw(DIST[dtype], np.random.default_rng((9, r, i)), int(s))
                 for i, s in enumerate(sizes)] for r in range(w)]
    tens = [[to_dev(t, dtype) for t in ts] for ts in per_rank]
    total = int(sizes.sum())
    fused = [empty(total, dtype) for _ in range(w)]
    say(f"fused dtype={dtype} tensors={len(sizes)} total={total}")
    for r in range(w):
        rsx.fuse_pack(tens[r], fused[r])
    torch.cuda.synchronize()
    for r in range(w):
        assert_parity(to_host(fused[r], dtype), oracle.fuse_pack(per_rank[r]), dtype, "pack")
    outs = [[empty(int(s), dtype) for s in sizes] for _ in range(w)]
    rsx.fused_all_reduce(tens, fused, outs, "sum", wire=wire(dtype))
    torch.cuda.synchronize()
    want = oracle.fused_all_reduce(per_rank, "sum", dtype)
    for r in range(w):
        for i in range(len(sizes)):
            assert_parity(to_host(outs[r][i], dtype), want[r][i], dtype, f"rank {r} tensor {i}")


@pytest.mark.parametrize("dtype", ["i8", "bf16", "f32", "f64"])
def test_pack_unpack_many_tensors_every_alignment(dtype):
    # 600 tensors (three launches of at most RSX_FUSE_BATCH copies), sizes 0
    # to 20,000 elements, each a view at element offset 0..7 of a larger
    # buffer and the fusion buffer at an element offset too, so source and
    # destination meet at every relative alignment: 16-byte, dword, and
    # (2- and 1-byte types) odd ones.
    rng = np.random.default_rng(77)
    sizes = rng.integers(0, 20_000, 600)
    sizes[::37] = 0
    sizes[5::41] = rng.integers(1, 9, len(sizes[5::41]))
    host = [wl.draw(DIST[dtype], np.random.default_rng((78, i)), int(n)) for i, n in enumerate(sizes)]
    offs = rng.integers(0, 8, len(sizes))
    bases = [empty(int(n) + 8, dtype) for n in sizes]
    tens = []
    for b, o, h in zip(bases, offs, host):
        v = b[int(o):int(o) + len(h)]
        v.copy_(to_dev(h, dtype))
        tens.append(v)
    total = int(sizes.sum())
    for foff in (0, 1, 3, 5):
        fbase = empty(total + 8, dtype, fill=0x5A)
        fused = fbase[foff:foff + total]
        say(f"pack/unpack dtype={dtype} tensors={len(sizes)} fused offset={foff}")
        rsx.fuse_pack(tens, fused)
        torch.cuda.synchronize()
        assert_parity(to_host(fused, dtype), oracle.fuse_pack(host), dtype, f"pack, fused offset {foff}")
        outs = [b[int(o):int(o) + int(n)] for b, o, n in zip(
            [empty(int(n) + 8, dtype, fill=0x33) for n in sizes], offs[::-1], sizes)]
        rsx.fuse_unpack(fused, outs)
        torch.cuda.synchronize()
        want = oracle.fuse_unpack(oracle.fuse_pack(host), sizes)
        for i, (o, wv) in enumerate(zip(outs, want)):
            assert_parity(to_host(o, dtype), wv, dtype, f"unpack tensor {i}, fused offset {foff}")


def _list_case(seed, w, sizes, dtype):
    return [[wl.draw(DIST[dtype], np.random.default_rng((seed, r, i)), int(n))
             for i, n in enumerate(sizes)] for r in range(w)]


LIST_SIZES = [0, 1, 3, 4096 + 5, 7, 0, 20_000, 1, 1024, 33, 65_536 + 3, 2, 9_999]


@pytest.mark.parametrize("dtype", ALL_DTYPES)
@pytest.mark.parametrize("op", OPS)
@pytest.mark.parametrize("w", [1, 2, 3, 4, 8, 16])
@pytest.mark.parametrize("algo", ["ring", "naive"])
def test_tensor_fusion_all_reduce(w, op, dtype, algo):
    # Ring segments of the fused layout end inside tensors and inside vectors.
    per_rank = _list_case(20, w, LIST_SIZES, dtype)
    tens = [[to_dev(t, dtype) for t in ts] for ts in per_rank]
    outs = [[empty(len(t), dtype, fill=0x33) for t in ts] for ts in per_rank]
    say(f"tensor-fusion ar w={w} op={op} dtype={dtype} algo={algo}")
    rsx.TensorFusionAllReduce(tens, outs, op, algo, wire=wire(dtype))()
    torch.cuda.synchronize()
    want = oracle.fused_all_reduce(per_rank, op, dtype) if algo == "ring" else [
        oracle.fuse_unpack(f, LIST_SIZES) for f in oracle.naive_all_reduce(
            [oracle.fuse_pack(ts) for ts in per_rank], op, dtype)]
    for r in range(w):
        for i in range(len(LIST_SIZES)):
            assert_parity(to_host(outs[r][i], dtype), want[r][i], dtype, f"rank {r} tensor {i}")


def test_tensor_fusion_matches_pipeline_many_launches_in_place():
    # W=16: 2W pointers per tensor, so 120 tensors take several launches.
    w = 16
    sizes = wl.fused_sizes(count=120, lo=1, hi=30_000)
    per_rank = _list_case(21, w, sizes, "f32")
    a = [[to_dev(t, "f32") for t in ts] for ts in per_rank]
    b = [[to_dev(t, "f32") for t in ts] for ts in per_rank]
    fused = [empty(int(sizes.sum()), "f32") for _ in range(w)]
    say("tensor-fusion vs pipeline, W=16, 120 tensors")
    rsx.TensorFusionAllReduce(a, None, "sum", "ring")()                 # in place, no buffer
    rsx.FusedAllReduce(b, fused, None, "sum", "ring")()                 # pack -> ar -> unpack
    torch.cuda.synchronize()
    for r in range(w):
        for i in range(len(sizes)):
            assert to_host(a[r][i], "f32").tobytes() == to_host(b[r][i], "f32").tobytes()
    want = oracle.fused_all_reduce(per_rank, "sum", "f32")
    for r in (0, 9, 15):
        for i in range(len(sizes)):
            assert_parity(to_host(a[r][i], "f32"), want[r][i], "f32", f"rank {r} tensor {i}")


def test_tensor_fusion_unaligned_views():
    w = 4
    sizes = [5, 4096, 3, 777]
    per_rank = _list_case(22, w, sizes, "bf16")
    tens, outs = [], []
    for ts in per_rank:
        row, orow = [], []
        for t in ts:
            base = to_dev(np.concatenate([np.zeros(1, np.uint16), t]), "bf16")
            row.append(base[1:])                      # 2-byte offset
            orow.append(empty(len(t) + 3, "bf16")[3:])
        tens.append(row)
        outs.append(orow)
    say("tensor-fusion unaligned bf16")
    rsx.TensorFusionAllReduce(tens, outs, "avg", "ring")()
    torch.cuda.synchronize()
    want = oracle.fused_all_reduce(per_rank, "avg", "bf16")
    for r in range(w):
        for i in range(len(sizes)):
            assert_parity(to_host(outs[r][i], "bf16"), want[r][i], "bf16", f"rank {r} tensor {i}")


@pytest.mark.parametrize("threshold", [0, 4 * 5000, 4 * 60_000, 64 * 2 ** 20])
def test_grouped_all_reduce(threshold):
    w = 4
    sizes = wl.fused_sizes(count=40, lo=1, hi=50_000)
    per_rank = _list_case(23, w, sizes, "f32")
    tens = [[to_dev(t, "f32") for t in ts] for ts in per_rank]
    plan = rsx.GroupedAllReduce(tens, None, "sum", "ring", threshold)
    assert plan.groups == oracle.fusion_groups([4 * int(n) for n in sizes], ["f32"] * len(sizes),
                                               threshold)
    say(f"grouped all-reduce threshold={threshold}: {len(plan.groups)} groups")
    plan()
    torch.cuda.synchronize()
    want = oracle.grouped_all_reduce(per_rank, threshold, "sum", "f32")
    for r in range(w):
        for i in range(len(sizes)):
            assert_parity(to_host(tens[r][i], "f32"), want[r][i], "f32", f"rank {r} tensor {i}")


def test_full_c5_tensor_fusion_direct():
    w = 4
    sizes = wl.fused_sizes()
    per_rank = wl.fused_tensors(w, sizes)
    tens = [[to_dev(t, "f32") for t in ts] for ts in per_rank]
    say(f"full cfg=5 direct: {int(sizes.sum())} elements per rank")
    rsx.TensorFusionAllReduce(tens, None, "sum", "ring")()
    torch.cuda.synchronize()
    want = oracle.fused_all_reduce(per_rank, "sum", "f32")
    for r in range(w):
        for i in range(len(sizes)):
            assert_parity(to_host(tens[r][i], "f32"), want[r][i], "f32", f"rank {r} tensor {i}")


@pytest.mark.parametrize("kib", wl.SWEEP_KIB)
def test_sweep_naive_ring_auto(kib):
    xs = wl.sweep_inputs(kib)
    for algo, ref in (("naive", oracle.naive_all_reduce), ("ring", oracle.all_reduce),
                      ("auto", oracle.naive_all_reduce)):
        say(f"sweep {kib} KiB algo={algo}")
        got = run_ar(xs, "f32", "sum", algo)
        want = ref(xs, "sum", "f32")
        for r in range(4):
            assert_parity(got[r], want[r], "f32", f"{algo} rank {r}")


def test_auto_switches_to_ring_above_32k():
    xs = wl.sweep_inputs(64)   # 64 KiB per rank -> ring
    got = run_ar(xs, "f32", "sum", "auto")
    want = oracle.all_reduce(xs, "sum", "f32")
    assert_parity(got[0], want[0], "f32", "auto 64 KiB")


# --------------------------------------------------------- error paths ------

def test_errors_with_real_tensors():
    # Each case is refused by the binding or the library's validation, before
    # any kernel is launched.
    x = [torch.zeros(64, device="cuda:0") for _ in range(4)]
    big = torch.zeros(128, device="cuda:0")
    with pytest.raises(rsx.RsxError) as e:   # output shifted by 8 elements onto input 0
        rsx.all_reduce([big[:64], x[1]], [big[8:72], x[2]], "sum")
    assert e.value.status == 5
    with pytest.raises(rsx.RsxError) as e:   # two ranks share one output
        rsx.all_reduce([x[0], x[1]], [x[2], x[2]], "sum")
    assert e.value.status == 5
    with pytest.raises(rsx.RsxError) as e:   # block 1 written over rank 0's input
        rsx.reduce_scatter([big[:64], x[1]], [x[2][:32], big[32:64]], "sum")
    assert e.value.status == 5
    with pytest.raises(ValueError):
        rsx.reduce_scatter(x, [torch.zeros(15, device="cuda:0")] * 4)
    with pytest.raises(ValueError):
        rsx.all_reduce([torch.zeros(8, dtype=torch.int16, device="cuda:0")] * 2)
    with pytest.raises(ValueError):
        rsx.all_reduce(x, op="xor")
    with pytest.raises(ValueError):
        rsx.all_reduce([torch.zeros(8, device="cuda:0")] * 17)
    with pytest.raises(ValueError):
        rsx.all_reduce([x[0], torch.zeros(64, device="cuda:0", dtype=torch.int32)])


# ------------------------------------------------- full-size workloads ------

def _full_rs(cfg, op, dtype):
    w = wl.WORKLOADS[cfg]
    say(f"full cfg={cfg} rs op={op}: generating")
    xs = wl.rank_inputs(cfg)
    dev = [to_dev(x, dtype) for x in xs]
    s = w.n // w.world
    out = [empty(s, dtype) for _ in range(w.world)]
    say(f"full cfg={cfg} rs op={op}: launching")
    rsx.reduce_scatter(dev, out, op)
    torch.cuda.synchronize()
    got = [to_host(o, dtype) for o in out]
    del dev
    say(f"full cfg={cfg} rs op={op}: oracle")
    want = oracle.reduce_scatter(xs, op, dtype)
    for k in range(w.world):
        assert_parity(got[k], want[k], dtype, f"block {k}")
    return xs


def test_full_c1_rs_and_ar():
    xs = _full_rs(1, "sum", "f32")
    got = run_ar(xs, "f32", "sum", "ring")
    want = oracle.all_reduce(xs, "sum", "f32")
    for r in range(4):
        assert_parity(got[r], want[r], "f32", f"ar rank {r}")


def test_full_c2_rs_sum_fp32():
    _full_rs(2, "sum", "f32")


@pytest.mark.parametrize("op", ["sum", "max"])
def test_full_c4_int32(op):
    xs = _full_rs(4, op, "i32")
    w = wl.WORKLOADS[4]
    say(f"full cfg=4 ar op={op}")
    dev = [to_dev(x, "i32") for x in xs]
    rsx.all_reduce(dev, None, op, "ring")
    torch.cuda.synchronize()
    want = oracle.all_reduce(xs, op, "i32")
    # every rank, one host copy at a time (each rank's output has its own stores)
    for r in range(w.world):
        assert_parity(to_host(dev[r], "i32"), want[r], "i32", f"ar rank {r}")


@pytest.mark.parametrize("dtype,op,w,n,bucket,algo", [
    ("bf16", "avg", 8, 3 * 8192 + 4096 + 8, 8192, "ring"),       # ragged last bucket
    ("f32", "sum", 3, 100_003, 7 * 4096 + 1, "ring"),            # buckets not a multiple of W
    ("f32", "sum", 4, 4 * 30_000, 4 * 7_000, "ring_split"),      # W divides every bucket
    ("i32", "max", 16, 50_000, 3_000, "auto"),                    # small buckets: naive per bucket
    ("f16", "prod", 5, 20_000, 20_000, "naive"),                  # one bucket
    ("f32h", "sum", 2, 9_000, 2_500, "ring"),                    # half wire
    ("f32", "sum", 4, 1_000, 10 ** 9, "ring"),                    # bucket above count
    # W divides the bucket: the full buckets share one launch per pass
    ("f32", "sum", 8, 5 * 8 * 65536 + 1000, 8 * 65536, "ring"),   # two passes over 5 buckets, ragged last
    ("bf16", "avg", 8, 4 * 8 * 1001 + 8, 8 * 1001, "ring"),       # one pass, segments not 16-byte multiples
    ("i32", "max", 16, 3 * 16 * 70_000, 16 * 70_000, "ring_split"),  # two passes, no last bucket
    ("f32", "sum", 12, 4 * 12 * 40_000 + 12, 12 * 40_000, "ring"),   # two passes at W = 12
    ("f16", "sum", 7, 6 * 7 * 3000 + 5, 7 * 3000, "ring_fused"),  # one pass at W = 7
    ("f32", "prod", 5, 3 * 5 * 4096 + 77, 5 * 4096, "naive"),     # rank order over every bucket
    ("i32", "sum", 8, 4 * 8 * 512, 8 * 512, "auto"),              # small buckets: naive, shared launch
])
@pytest.mark.parametrize("in_place", [False, True])
def test_all_reduce_bucketed_entry(dtype, op, w, n, bucket, algo, in_place):
    # rsx_all_reduce_bucketed against the oracle's bucket-by-bucket all-reduce
    xs = inputs(60, w, n, dtype)
    dev = [to_dev(x, dtype) for x in xs]
    out = None if in_place else [empty(n, dtype, fill=0x55) for _ in range(w)]
    say(f"bucketed entry dtype={dtype} op={op} w={w} n={n} bucket={bucket} algo={algo} in_place={in_place}")
    rsx.all_reduce_bucketed(dev, out, bucket, op, algo, wire=wire(dtype))
    torch.cuda.synchronize()
    ref_algo = "naive" if algo == "naive" else "ring"
    want = [np.empty_like(x) for x in xs]
    for b0 in range(0, n, bucket):
        b1 = min(b0 + bucket, n)
        part = [x[b0:b1] for x in xs]
        nbytes = (b1 - b0) * ES[dtype]
        naive = ref_algo == "naive" or (algo == "auto" and nbytes <= RSX_NAIVE_MAX_BYTES)
        res = (oracle.naive_all_reduce if naive else oracle.all_reduce)(part, op, dtype)
        for r in range(w):
            want[r][b0:b1] = res[r]
    for r in range(w):
        assert_parity(to_host((dev if in_place else out)[r], dtype), want[r], dtype, f"rank {r}")


@pytest.mark.parametrize("dtype,op,w,n,bucket,algo", [
    ("f32", "sum", 8, 5 * 8 * 65536 + 1000, 8 * 65536, "ring"),
    ("bf16", "avg", 8, 3 * 8192 + 4096 + 8, 8192, "ring"),
    ("i32", "max", 16, 50_000, 3_000, "auto"),
    ("f16", "sum", 7, 6 * 7 * 3000 + 5, 7 * 3000, "ring_fused"),
])
def test_single_bucket_calls(dtype, op, w, n, bucket, algo):
    # rsx_all_reduce_bucket, one call per bucket in reverse order (each
    # bucket's result depends on nothing else), against the oracle's
    # bucket-by-bucket all-reduce
    xs = inputs(62, w, n, dtype)
    dev = [to_dev(x, dtype) for x in xs]
    out = [empty(n, dtype, fill=0x55) for _ in range(w)]
    plan = rsx.BucketedAllReduce(dev, out, bucket, op, algo, wire=wire(dtype),
                                 stream=torch.cuda.current_stream())
    say(f"single buckets dtype={dtype} op={op} w={w} n={n} bucket={bucket} algo={algo} buckets={len(plan)}")
    assert len(plan) == -(-n // bucket)
    for b in reversed(range(len(plan))):
        plan.ready(b)
    torch.cuda.synchronize()
    ref_algo = "naive" if algo == "naive" else "ring"
    for b0 in range(0, n, bucket):
        b1 = min(b0 + bucket, n)
        part = [x[b0:b1] for x in xs]
        naive = ref_algo == "naive" or (algo == "auto" and (b1 - b0) * ES[dtype] <= RSX_NAIVE_MAX_BYTES)
        res = (oracle.naive_all_reduce if naive else oracle.all_reduce)(part, op, dtype)
        for r in range(w):
            assert_parity(to_host(out[r], dtype)[b0:b1], res[r], dtype, f"rank {r} bucket at {b0}")


@pytest.mark.parametrize("algo", ["ring", "ring_split", "ring_fused"])
def test_all_reduce_bucketed_unaligned(algo):
    # 4-byte offsets: element kernels in both passes, several buckets per launch
    w, bucket = 8, 8 * 3001
    n = 4 * bucket + 8 * 17
    xs = inputs(61, w, n, "f32")
    bases = [to_dev(np.concatenate([np.zeros(1, np.float32), x]), "f32") for x in xs]
    dev = [b[1:] for b in bases]
    outs = [empty(n + 3, "f32", fill=0x55)[3:] for _ in range(w)]
    say(f"bucketed unaligned algo={algo}")
    rsx.all_reduce_bucketed(dev, outs, bucket, "sum", algo)
    torch.cuda.synchronize()
    want = oracle.bucketed_all_reduce(xs, bucket, "sum", "f32")
    for r in range(w):
        assert_parity(to_host(outs[r], "f32"), want[r], "f32", f"rank {r}")


def test_full_c3_bf16_bucketed_avg():
    w = wl.WORKLOADS[3]
    say("full cfg=3: generating")
    xs = wl.rank_inputs(3)
    dev = [to_dev(x, "bf16") for x in xs]
    out = [empty(w.n, "bf16") for _ in range(w.world)]
    say("full cfg=3: 11 bucketed all-reduces")
    rsx.all_reduce_bucketed(dev, out, w.extra["bucket_elems"], "avg")
    torch.cuda.synchronize()
    del dev
    say("full cfg=3: oracle")
    want = oracle.bucketed_all_reduce(xs, w.extra["bucket_elems"], "avg", "bf16")
    # every rank, one host copy at a time
    stats = [assert_parity(to_host(out[r], "bf16"), want[r], "bf16", f"rank {r}") for r in range(w.world)]
    say(f"bf16 exact fraction {stats[0]['exact'] / stats[0]['n']:.6f}")


@pytest.mark.parametrize("dtype,op", [("bf16", "avg"), ("f32", "sum")])
def test_bucket_overlap_on_a_side_stream(dtype, op):
    # The producer writes bucket b only after some unrelated work on its
    # stream and then calls ready(b); the inputs hold junk before that, so a
    # reduction that did not wait for the producer's event would show.
    w, bucket = 4, 3 * 4096 + 40
    n = 3 * bucket + 1000
    xs = inputs(40, w, n, dtype)
    staged = [to_dev(x, dtype) for x in xs]
    ins = [empty(n, dtype, fill=0x7F7F) for _ in range(w)]
    outs = [empty(n, dtype, fill=0x55) for _ in range(w)]
    plan = rsx.BucketedAllReduce(ins, outs, bucket, op)
    assert plan.stream != torch.cuda.current_stream() and len(plan) == 4
    a = torch.randn(1024, 1024, device="cuda:0")
    say(f"bucket overlap dtype={dtype} op={op} buckets={len(plan)}")
    for b in range(len(plan)):
        b0, b1 = b * bucket, min((b + 1) * bucket, n)
        for _ in range(4):
            a = torch.mm(a, a) * 1e-3         # producer busy before bucket b exists
        for r in range(w):
            ins[r][b0:b1].copy_(staged[r][b0:b1])
        plan.ready(b)
    plan.wait()
    torch.cuda.synchronize()
    want = oracle.bucketed_all_reduce(xs, bucket, op, dtype)
    for r in range(w):
        assert_parity(to_host(outs[r], dtype), want[r], dtype, f"rank {r}")


def test_full_c5_fused_200_tensors():
    w = 4
    sizes = wl.fused_sizes()
    per_rank = wl.fused_tensors(w, sizes)
    tens = [[to_dev(t, "f32") for t in ts] for ts in per_rank]
    total = int(sizes.sum())
    fused = [empty(total, "f32") for _ in range(w)]
    say(f"full cfg=5: total {total} elements per rank")
    rsx.fused_all_reduce(tens, fused, None, "sum")
    torch.cuda.synchronize()
    want = oracle.fused_all_reduce(per_rank, "sum", "f32")
    for r in range(w):
        for i in range(len(sizes)):
            assert_parity(to_host(tens[r][i], "f32"), want[r][i], "f32", f"rank {r} tensor {i}")


# ------------------------------------------------- beyond 32-bit offsets ----

def _sample_positions(rng, n, bounds, extra=20000):
    pos = set(rng.integers(0, n, extra).tolist())
    for b in bounds:
        for d in (-2, -1, 0, 1, 2):
            if 0 <= b + d < n:
                pos.add(b + d)
    for v in (2 ** 31 - 1, 2 ** 31, 2 ** 31 + 1, 2 ** 30 - 1, 2 ** 30, n - 1):
        if 0 <= v < n:
            pos.add(v)
    return np.array(sorted(pos), dtype=np.int64)


def test_rank_buffers_beyond_2_pow_31_elements():
    # W=2 ranks of 2^31 + 4096 fp32 (8 GiB each): element indices above 2^31,
    # byte offsets above 8 GiB, reduce-scatter segments above 4 GiB.  Inputs
    # from a seeded device generator; outputs checked at sampled positions,
    # including every segment boundary, against the oracle's fold.
    w, n = 2, 2 ** 31 + 4096
    s = n // w
    gen = torch.Generator(device="cuda:0")
    gen.manual_seed(2024)
    say("large: generating 2 x 8 GiB on the device")
    xs = [torch.randn(n, device="cuda:0", generator=gen) for _ in range(w)]
    rng = np.random.default_rng(11)

    out = [empty(s, "f32") for _ in range(w)]
    say("large: reduce-scatter")
    rsx.reduce_scatter(xs, out, "sum")
    torch.cuda.synchronize()
    pos = _sample_positions(rng, s, [0, s - 1])
    ti = torch.from_numpy(pos).to("cuda:0")
    for k in range(w):
        vals = [x[k * s + ti].cpu().numpy() for x in xs]
        want = oracle.fold(vals, oracle.ring_fold_order(k, w), "sum", "f32")
        assert_parity(out[k][ti].cpu().numpy(), want, "f32", f"rs block {k}")
    del out

    say("large: all-reduce in place")
    pos = _sample_positions(rng, n, [oracle.segment_bounds(n, w)[k][0] for k in range(w)])
    ti = torch.from_numpy(pos).to("cuda:0")
    before = [x[ti].cpu().numpy() for x in xs]
    rsx.all_reduce(xs, None, "max", "ring")
    torch.cuda.synchronize()
    segs = oracle.segment_bounds(n, w)
    for k, (lo, hi) in enumerate(segs):
        m = (pos >= lo) & (pos < hi)
        want = oracle.fold([b[m] for b in before], oracle.ring_fold_order(k, w), "max", "f32")
        for r in range(w):
            assert_parity(xs[r][ti[torch.from_numpy(m).to("cuda:0")]].cpu().numpy(), want, "f32",
                          f"ar segment {k} rank {r}")
