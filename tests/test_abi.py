"""C-ABI tests that need no GPU: symbols, enums, host-side validation.

The validation tests pass made-up device addresses: every such case must be
rejected before the library makes a HIP call.  They are skipped where a GPU
is visible, so a validation bug can never turn them into a real launch on
fake pointers; the GPU suite covers the same error paths with real tensors.
"""
import ctypes
import os
import re

import pytest

from collective_reduction_ring_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rsx.h")


def _gpu_visible():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


fake_ptrs = pytest.mark.skipif(_gpu_visible(), reason="fake device pointers only where no GPU exists")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L.LIB_PATH):
        pytest.fail("librsx.so is not built; run `python -m collective_reduction_ring_amd.build`")
    return L.lib()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rsx_[a-z_]+)\s*\(", text)))


def _header_int(name):
    m = re.search(rf"#define\s+{name}\s+(\d+)", open(HEADER).read())
    return int(m.group(1))


def test_exports_every_declared_symbol(lib):
    names = _declared_functions()
    assert "rsx_reduce_scatter" in names and len(names) >= 9
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(L.SIGNATURES)


def test_enum_and_macro_values_match_binding(lib):
    text = open(HEADER).read()
    for name, val in [("RSX_FLOAT32", L.RSX_FLOAT32), ("RSX_BFLOAT16", L.RSX_BFLOAT16),
                      ("RSX_INT32", L.RSX_INT32), ("RSX_FLOAT64", L.RSX_FLOAT64),
                      ("RSX_FLOAT16", L.RSX_FLOAT16), ("RSX_INT64", L.RSX_INT64),
                      ("RSX_UINT64", L.RSX_UINT64), ("RSX_INT8", L.RSX_INT8),
                      ("RSX_FLOAT32_HALF_WIRE", L.RSX_FLOAT32_HALF_WIRE),
                      ("RSX_SUM", L.RSX_SUM), ("RSX_MAX", L.RSX_MAX),
                      ("RSX_MIN", L.RSX_MIN), ("RSX_AVG", L.RSX_AVG), ("RSX_PROD", L.RSX_PROD),
                      ("RSX_ALGO_RING", L.RSX_ALGO_RING), ("RSX_ALGO_NAIVE", L.RSX_ALGO_NAIVE),
                      ("RSX_ALGO_AUTO", L.RSX_ALGO_AUTO), ("RSX_ALGO_RING_FUSED", L.RSX_ALGO_RING_FUSED),
                      ("RSX_ALGO_RING_SPLIT", L.RSX_ALGO_RING_SPLIT)]:
        assert re.search(rf"\b{name}\s*=\s*{val}\b", text), name
    for code, name in L.STATUS.items():
        assert re.search(rf"\b{name}\s*=\s*{code}\b", text), name
    assert _header_int("RSX_MAX_RANKS") == L.RSX_MAX_RANKS
    assert _header_int("RSX_NAIVE_MAX_BYTES") == L.RSX_NAIVE_MAX_BYTES
    assert _header_int("RSX_FUSE_BATCH") == L.RSX_FUSE_BATCH
    assert lib.rsx_version() == _header_int("RSX_VERSION")


def test_dtype_size_and_status_strings(lib):
    assert [lib.rsx_dtype_size(d) for d in (0, 1, 2, 3, 4, 5, 6, 7, 8, 9, -1)] == [4, 2, 4, 8, 2, 8, 8, 1, 4, 0, 0]
    for code in range(7):
        assert lib.rsx_status_string(code)
    assert lib.rsx_status_string(99) == b"unknown status"


def test_segment_begin_ceil_split(lib):
    import oracle
    for count in (0, 1, 2, 3, 10, 17, 4096, 25_165_823, 2 ** 40 + 3):
        for w in (1, 2, 3, 4, 7, 8, 16):
            bounds = oracle.segment_bounds(count, w) if count < 10 ** 6 else None
            for k in range(w + 1):
                got = lib.rsx_segment_begin(count, w, k)
                s = -(-count // w)
                assert got == min(k * s, count)
                if bounds is not None and k < w:
                    assert got == bounds[k][0]
    assert lib.rsx_segment_begin(10, 0, 1) == 0
    assert lib.rsx_segment_begin(10, 4, -1) == 0


# ------------------------------------------------------ validation paths --

A = 0x7F0000000000  # made-up, 16-byte aligned device addresses (never dereferenced)
MB = 1 << 20


def _arr(vals):
    return L.ptr_array(vals)


def _rs(lib, sends, recvs, w, n, dt=0, op=0):
    return lib.rsx_reduce_scatter(_arr(sends), _arr(recvs), w, n, dt, op, None)


def _ar(lib, sends, recvs, w, n, dt=0, op=0, algo=0):
    return lib.rsx_all_reduce(_arr(sends), _arr(recvs), w, n, dt, op, algo, None)


def _ag(lib, sends, recvs, w, n, dt=0):
    return lib.rsx_all_gather(_arr(sends), _arr(recvs), w, n, dt, None)


@fake_ptrs
def test_null_arrays_and_rank_range(lib):
    assert lib.rsx_reduce_scatter(None, _arr([A]), 1, 4, 0, 0, None) == 1
    assert lib.rsx_all_reduce(_arr([A]), None, 1, 4, 0, 0, 0, None) == 1
    assert lib.rsx_all_gather(None, None, 1, 4, 0, None) == 1
    s = [A + i * MB for i in range(17)]
    r = [A + 64 * MB + i * MB for i in range(17)]
    assert _rs(lib, s, r, 0, 4) == 1
    assert _rs(lib, s, r, 17, 4) == 1
    assert _ar(lib, s, r, -1, 4) == 1
    assert _ag(lib, s, r, 17, 4) == 1


@fake_ptrs
def test_bad_enums(lib):
    s, r = [A, A + MB], [A + 2 * MB, A + 3 * MB]
    assert _rs(lib, s, r, 2, 4, dt=9) == 2
    assert _rs(lib, s, r, 2, 4, dt=-1) == 2
    assert _rs(lib, s, r, 2, 4, op=5) == 3
    assert _ar(lib, s, r, 2, 4, op=-1) == 3
    assert _ar(lib, s, r, 2, 4, algo=5) == 1
    assert _ar(lib, s, r, 2, 4, algo=-1) == 1
    assert _ag(lib, s, r, 2, 4, dt=9) == 2
    # type is checked before op, as the page's dispatch switches on type first
    assert _rs(lib, s, r, 2, 4, dt=9, op=9) == 2


def test_occupancy_caps_setting_is_per_thread(lib):
    import threading
    assert lib.rsx_set_occupancy_caps(0) == 1           # on by default
    assert lib.rsx_set_occupancy_caps(5) == 0           # any nonzero value turns them on
    assert lib.rsx_set_occupancy_caps(0) == 1
    seen = []
    th = threading.Thread(target=lambda: seen.append(lib.rsx_set_occupancy_caps(1)))
    th.start()
    th.join()
    assert seen == [1]                                  # another thread still has its default
    assert lib.rsx_set_occupancy_caps(1) == 0           # this thread's setting was kept


@fake_ptrs
def test_ring_split_needs_rank_count_to_divide_count(lib):
    s = [A + i * MB for i in range(3)]
    r = [A + 8 * MB + i * MB for i in range(3)]
    assert _ar(lib, s, r, 3, 4, algo=L.RSX_ALGO_RING_SPLIT) == 4
    assert _ar(lib, s, r, 3, 7, algo=L.RSX_ALGO_RING_SPLIT) == 4
    assert _ar(lib, s, r, 3, 0, algo=L.RSX_ALGO_RING_SPLIT) == 0   # nothing to do
    # bad arguments are still reported as such
    assert _ar(lib, s, r, 3, 4, op=9, algo=L.RSX_ALGO_RING_SPLIT) == 3
    assert _ar(lib, s[:2] + [None], r, 3, 4, algo=L.RSX_ALGO_RING_SPLIT) == 1


@fake_ptrs
def test_zero_count_is_success_without_launch(lib):
    assert _rs(lib, [A, A], [None, None], 2, 0) == 0
    assert _ar(lib, [None] * 3, [None] * 3, 3, 0) == 0
    assert _ag(lib, [A], [A], 1, 0) == 0


@fake_ptrs
def test_null_device_pointer(lib):
    assert _rs(lib, [A, None], [A + 4 * MB, A + 5 * MB], 2, 4) == 1
    assert _ar(lib, [A, A + MB], [A + 2 * MB, None], 2, 4) == 1


def _arb(lib, sends, recvs, w, n, bucket, dt=0, op=0, algo=0):
    return lib.rsx_all_reduce_bucketed(_arr(sends), _arr(recvs), w, n, bucket, dt, op, algo, None)


@fake_ptrs
def test_bucketed_all_reduce_validation(lib):
    # The same checks as one all-reduce over the whole buffers, all before the
    # first bucket's launch; plus the bucket size and, for the two-pass form,
    # W dividing every bucket.
    s, r = [A, A + MB], [A + 2 * MB, A + 3 * MB]
    assert _arb(lib, s, r, 2, 1000, 0) == 1                               # no bucket size
    assert _arb(lib, s, r, 2, 0, 100) == 0                                # nothing to do
    assert lib.rsx_all_reduce_bucketed(None, _arr(r), 2, 1000, 100, 0, 0, 0, None) == 1
    assert _arb(lib, s, r, 0, 1000, 100) == 1 and _arb(lib, s, r, 17, 1000, 100) == 1
    assert _arb(lib, s, r, 2, 1000, 100, dt=9) == 2
    assert _arb(lib, s, r, 2, 1000, 100, op=7) == 3
    assert _arb(lib, s, r, 2, 1000, 100, algo=9) == 1
    assert _arb(lib, s, [A + 2 * MB, A + 2 * MB + 64], 2, 1000, 100) == 5  # outputs overlap
    assert _arb(lib, s, [A + 8, r[1]], 2, 1000, 100) == 5                 # output inside an input
    assert _arb(lib, [A + 2, A + MB], r, 2, 1000, 100) == 1               # misaligned fp32 input
    # two passes: W must divide every bucket (1000 = 3 * 300 + 100; 300 % 3 == 0, 100 % 3 != 0)
    s3, r3 = [A, A + MB, A + 2 * MB], [A + 3 * MB, A + 4 * MB, A + 5 * MB]
    assert _arb(lib, s3, r3, 3, 1000, 300, algo=L.RSX_ALGO_RING_SPLIT) == 4
    assert _arb(lib, s3, r3, 3, 900, 301, algo=L.RSX_ALGO_RING_SPLIT) == 4
    assert _arb(lib, s3, r3, 3, 1000, 10 ** 30 % 2 ** 60, algo=L.RSX_ALGO_RING_SPLIT) == 4
    # one rank in place: valid and nothing to launch, whatever the bucket size
    assert _arb(lib, [A], [A], 1, 1000, 7) == 0
    assert _arb(lib, [A], [A], 1, 1000, 2 ** 63) == 0


def test_bucket_count(lib):
    assert lib.rsx_bucket_count(1000, 100) == 10
    assert lib.rsx_bucket_count(1001, 100) == 11
    assert lib.rsx_bucket_count(99, 100) == 1
    assert lib.rsx_bucket_count(0, 100) == 0
    assert lib.rsx_bucket_count(1000, 0) == 0
    assert lib.rsx_bucket_count(2 ** 64 - 1, 2 ** 63) == 2


def _ar1(lib, sends, recvs, w, n, bucket_elems, bucket, dt=0, op=0, algo=0):
    return lib.rsx_all_reduce_bucket(_arr(sends), _arr(recvs), w, n, bucket_elems, bucket, dt, op, algo, None)


@fake_ptrs
def test_single_bucket_validation(lib):
    # rsx_all_reduce_bucket: the bucketed call's checks on the whole buffers,
    # then the bucket index (every check before any HIP call).
    s, r = [A, A + MB], [A + 2 * MB, A + 3 * MB]
    assert _ar1(lib, s, r, 2, 1000, 0, 0) == 1                             # no bucket size
    assert _ar1(lib, s, r, 2, 1000, 100, 10) == 1                          # past the last bucket
    assert _ar1(lib, s, r, 2, 1001, 100, 11) == 1
    assert _ar1(lib, s, r, 2, 0, 100, 0) == 0                              # nothing to do
    assert _ar1(lib, s, r, 2, 1000, 100, 3, dt=9) == 2
    assert _ar1(lib, s, r, 2, 1000, 100, 3, op=7) == 3
    assert _ar1(lib, s, [A + 2 * MB, A + 2 * MB + 64], 2, 1000, 100, 3) == 5
    s3, r3 = [A, A + MB, A + 2 * MB], [A + 3 * MB, A + 4 * MB, A + 5 * MB]
    assert _ar1(lib, s3, r3, 3, 1000, 300, 0, algo=L.RSX_ALGO_RING_SPLIT) == 4  # last bucket of 100
    assert _ar1(lib, [A], [A], 1, 1000, 7, 142) == 0                       # one rank in place: nothing
    assert _ar1(lib, [A], [A], 1, 1000, 7, 143) == 1                       # but the index is still checked


@fake_ptrs
def test_pointers_must_be_element_aligned(lib):
    # A buffer that does not start at a multiple of its element size is refused
    # before any HIP call (the kernels' element accesses are naturally aligned).
    s, r = [A, A + MB], [A + 2 * MB, A + 3 * MB]
    for i, dt, es in [(0, L.RSX_FLOAT32, 4), (1, L.RSX_BFLOAT16, 2), (2, L.RSX_FLOAT64, 8),
                      (3, L.RSX_INT64, 8), (4, L.RSX_FLOAT16, 2), (5, L.RSX_INT32, 4)]:
        for off in range(1, es):
            bad_s = list(s)
            bad_s[i % 2] += off
            bad_r = list(r)
            bad_r[(i + 1) % 2] += off
            assert _rs(lib, bad_s, r, 2, 64, dt=dt) == 1, (dt, off)
            assert _rs(lib, s, bad_r, 2, 64, dt=dt) == 1, (dt, off)
            assert _ar(lib, bad_s, r, 2, 64, dt=dt) == 1, (dt, off)
            assert _ar(lib, s, bad_r, 2, 64, dt=dt, algo=L.RSX_ALGO_NAIVE) == 1, (dt, off)
            assert _ag(lib, bad_s, r, 2, 64, dt=dt) == 1, (dt, off)
            counts = L.size_array([10, 7])
            assert lib.rsx_fuse_pack(_arr(bad_s), counts, 2, A + 8 * MB, dt, None) == 1
            assert lib.rsx_fuse_pack(_arr(s), counts, 2, A + 8 * MB + off, dt, None) == 1
            assert lib.rsx_fuse_unpack(A + 8 * MB + off, _arr(r), counts, 2, dt, None) == 1
            assert lib.rsx_fuse_unpack(A + 8 * MB, _arr(bad_r), counts, 2, dt, None) == 1
            assert _far(lib, bad_s + [A + 4 * MB, A + 5 * MB], r + [A + 6 * MB, A + 7 * MB],
                        [10, 7], 2, dt=dt) == 1, (dt, off)
    # int8 has no alignment requirement; such a call gets past the check (to the
    # aliasing rule here, which it breaks on purpose so that nothing launches)
    assert _rs(lib, [A + 1, A + 1 + MB], [A + 1, A + 2], 2, 64, dt=L.RSX_INT8) == 5


@fake_ptrs
def test_single_rank_in_place_is_a_no_op(lib):
    assert _rs(lib, [A], [A], 1, 100) == 0
    assert _ar(lib, [A], [A], 1, 100) == 0
    assert _ag(lib, [A], [A], 1, 100) == 0


@fake_ptrs
def test_half_wire_is_for_reductions_only(lib):
    # a gather reduces nothing, so the half wire type is refused before any HIP call
    assert _ag(lib, [A, A + MB], [A + 2 * MB, A + 3 * MB], 2, 4, dt=L.RSX_FLOAT32_HALF_WIRE) == 2


@fake_ptrs
def test_size_overflow(lib):
    s, r = [A, A + MB], [A + 2 * MB, A + 3 * MB]
    assert _rs(lib, s, r, 2, 2 ** 63) == 4
    assert _ar(lib, s, r, 2, 2 ** 62 + 1) == 4
    assert _ag(lib, s, r, 2, 2 ** 62) == 4


@fake_ptrs
def test_reduce_scatter_aliasing(lib):
    n = 1024  # recvcount; inputs are 4*n fp32 = 16 KiB
    s = [A + i * MB for i in range(4)]
    # output overlapping another rank's input
    assert _rs(lib, s, [A + 2 * MB + 64, A + 8 * MB, A + 9 * MB, A + 10 * MB], 4, n) == 5
    # outputs overlapping each other
    assert _rs(lib, s, [A + 8 * MB, A + 8 * MB + 16, A + 9 * MB, A + 10 * MB], 4, n) == 5
    # inputs partially overlapping
    s2 = [A, A + 64, A + 2 * MB, A + 3 * MB]
    assert _rs(lib, s2, [A + 8 * MB + i * MB for i in range(4)], 4, n) == 5
    # in place, but at the wrong block of rank 1
    r = [s[0], s[1] + 2 * n * 4, s[2] + 2 * n * 4, s[3] + 3 * n * 4]
    assert _rs(lib, s, r, 4, n) == 5


@fake_ptrs
def test_all_reduce_aliasing(lib):
    n = 1000
    s = [A + i * MB for i in range(3)]
    assert _ar(lib, s, [s[0] + 8, A + 8 * MB, A + 9 * MB], 3, n) == 5   # shifted onto input
    assert _ar(lib, s, [A + 8 * MB, A + 8 * MB, A + 9 * MB], 3, n) == 5  # shared output
    assert _ar(lib, [A, A + 4, A + 2 * MB], [A + 8 * MB + i * MB for i in range(3)], 3, n) == 5


@fake_ptrs
def test_all_gather_aliasing(lib):
    n = 256
    r = [A + i * MB for i in range(4)]
    # piece 1 inside rank 0's output
    assert _ag(lib, [A + 8 * MB, r[0] + 8, A + 9 * MB, A + 10 * MB], r, 4, n) == 5
    # overlapping outputs
    assert _ag(lib, [A + 8 * MB + i * MB for i in range(4)], [A, A + 16, A + 2 * MB, A + 3 * MB],
               4, n) == 5


@fake_ptrs
def test_fuse_validation(lib):
    counts = L.size_array([10, 0, 5])
    ts = _arr([A, None, A + MB])
    assert lib.rsx_fuse_pack(ts, None, 3, A + 4 * MB, 0, None) == 1       # counts missing
    assert lib.rsx_fuse_pack(ts, counts, -1, A + 4 * MB, 0, None) == 1
    assert lib.rsx_fuse_pack(ts, counts, 3, A + 4 * MB, 9, None) == 2     # bad dtype
    assert lib.rsx_fuse_pack(ts, counts, 3, None, 0, None) == 1           # no fused buffer
    assert lib.rsx_fuse_pack(ts, counts, 3, A + 36, 0, None) == 5         # fused overlaps t0
    assert lib.rsx_fuse_unpack(A + MB - 8, ts, counts, 3, 0, None) == 5   # fused overlaps t2
    assert lib.rsx_fuse_unpack(A + 4 * MB, _arr([A, None, A + 8]), counts, 3, 0, None) == 5
    zero = L.size_array([0, 0])
    assert lib.rsx_fuse_pack(_arr([None, None]), zero, 2, None, 0, None) == 0
    assert lib.rsx_fuse_unpack(None, _arr([None, None]), zero, 2, 0, None) == 0
    assert lib.rsx_fuse_pack(None, zero, 0, None, 0, None) == 0
    assert lib.rsx_fuse_pack(_arr([A]), L.size_array([2 ** 62]), 1, A + MB, 0, None) == 4
    # a fusion buffer of 2^40 bytes or more is refused (offsets are 40 bits)
    assert lib.rsx_fuse_pack(_arr([A]), L.size_array([2 ** 38]), 1, A + 2 ** 42, 0, None) == 4


def test_binding_refuses_missing_library(tmp_path, monkeypatch):
    monkeypatch.setattr(L, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(L, "_lib", None)
    with pytest.raises(RuntimeError, match="not found"):
        L.lib()


def _far(lib, sends, recvs, counts, w, dt=0, op=0, algo=0):
    n = len(counts)
    return lib.rsx_fused_all_reduce(_arr(sends), _arr(recvs), L.size_array(counts), n, w, dt, op,
                                    algo, None)


@fake_ptrs
def test_fused_all_reduce_validation(lib):
    c = [100, 0, 37]
    s = [A + i * MB for i in range(6)]               # rank-major: rank 0 tensors 0..2, rank 1 ...
    r = [A + 16 * MB + i * MB for i in range(6)]
    assert lib.rsx_fused_all_reduce(_arr(s), _arr(r), None, 3, 2, 0, 0, 0, None) == 1   # counts
    assert _far(lib, s, r, c, 0) == 1 and _far(lib, s, r, c, 17) == 1
    assert _far(lib, s, r, c, 2, dt=9) == 2
    assert _far(lib, s, r, c, 2, op=7) == 3
    assert _far(lib, s, r, c, 2, algo=9) == 1
    assert _far(lib, s, r, c, 2, algo=L.RSX_ALGO_RING_SPLIT) == 4   # the list kernel is one pass
    assert _far(lib, s, r, [0, 0, 0], 2) == 0                      # nothing to do, no launch
    assert lib.rsx_fused_all_reduce(None, None, L.size_array([0]), 1, 2, 0, 0, 0, None) == 0
    assert _far(lib, s, r, [2 ** 62, 1, 1], 2) == 4                 # bytes overflow
    s_null = list(s)
    s_null[3] = None                                                # rank 1 tensor 0 (count 100)
    assert _far(lib, s_null, r, c, 2) == 1


@fake_ptrs
def test_fused_all_reduce_aliasing(lib):
    c = [100, 50]
    s = [A, A + MB, A + 2 * MB, A + 3 * MB]
    r = [A + 8 * MB, A + 9 * MB, A + 10 * MB, A + 11 * MB]
    # destination overlapping a source partially
    assert _far(lib, s, [A + 8, r[1], r[2], r[3]], c, 2) == 5
    # two destinations overlapping
    assert _far(lib, s, [r[0], r[0] + 16, r[2], r[3]], c, 2) == 5
    # sources overlapping partially
    assert _far(lib, [A, A + 200, s[2], s[3]], r, c, 2) == 5
    # destination equal to a source of another tensor index
    assert _far(lib, s, [s[1], r[1], r[2], r[3]], [50, 50], 2) == 5
    # single rank, every destination its own source: nothing to do
    assert _far(lib, [A, A + MB], [A, A + MB], c, 1) == 0


@fake_ptrs
def test_buffers_wrapping_the_address_space(lib):
    top = 2 ** 64 - 4096
    assert _rs(lib, [top, A], [A + MB, A + 2 * MB], 2, 1024) == 1
    assert _ar(lib, [A, A + MB], [A + 2 * MB, top], 2, 4096) == 1
    assert _ag(lib, [A, A + MB], [top, A + 4 * MB], 2, 1024) == 1
    assert lib.rsx_fuse_pack(_arr([A]), L.size_array([4096]), 1, top, 0, None) == 1
    assert _far(lib, [top, A + MB], [A + 2 * MB, A + 3 * MB], [4096], 2) == 1


def _plan(lib, counts, dtypes, threshold):
    n = len(counts)
    ends = (ctypes.c_int * max(1, n))()
    dts = (ctypes.c_int * max(1, n))(*dtypes)
    g = lib.rsx_fusion_plan(L.size_array(counts), dts, n, threshold, ends)
    if g < 0:
        return None
    starts = [0] + [ends[k] for k in range(g - 1)]
    return [(starts[k], ends[k]) for k in range(g)]


def test_fusion_plan_matches_oracle(lib):
    import numpy as np

    import oracle
    es = {0: 4, 1: 2, 2: 4, 3: 8, 4: 2, 5: 8, 6: 8, 7: 1}
    rng = np.random.default_rng(8)
    for trial in range(400):
        n = int(rng.integers(0, 40))
        counts = [int(c) for c in rng.integers(0, 5000, n)]
        if trial % 5 == 0:
            counts = [int(c) for c in rng.integers(0, 3, n)]
        dts = [int(d) for d in rng.choice([0, 0, 0, 1, 2, 3, 7], n)]
        th = int(rng.choice([0, 1, 100, 4000, 16000, 64 * 2 ** 20]))
        got = _plan(lib, counts, dts, th)
        want = oracle.fusion_groups([c * es[d] for c, d in zip(counts, dts)], dts, th)
        assert got == want, (counts, dts, th)


def test_fusion_plan_validation(lib):
    assert lib.rsx_fusion_plan(None, None, 0, 10, None) == 0
    assert lib.rsx_fusion_plan(None, None, -1, 10, None) == -1
    ends = (ctypes.c_int * 2)()
    assert lib.rsx_fusion_plan(L.size_array([1, 2]), (ctypes.c_int * 2)(0, 9), 2, 10, ends) == -1
    assert lib.rsx_fusion_plan(L.size_array([1, 2]), None, 2, 10, ends) == -1
    # a tensor whose byte count overflows is a group of its own
    assert _plan(lib, [2 ** 63, 1, 1], [0, 0, 0], 2 ** 40) == [(0, 1), (1, 3)]


# ------------------------------------------------ sparsified all-reduce --

def test_sparse_topk_count_fp32_arithmetic(lib):
    import oracle
    for n, frac in [(10, 0.1), (2 ** 24 + 1, 1.0), (10, 0.3), (7, 0.0), (1000, 0.5),
                    (67_108_864, 0.01), (12345, 0.123)]:
        assert lib.rsx_sparse_topk_count(n, frac) == oracle.topk_count(n, frac), (n, frac)
    assert lib.rsx_sparse_topk_count(10, -0.5) == 0
    assert lib.rsx_sparse_topk_count(10, float("nan")) == 0


def test_sparse_workspace_size(lib):
    T, K = L.RSX_SPARSE_THRESHOLD, L.RSX_SPARSE_TOPK
    assert lib.rsx_sparse_workspace_size(0, 100, T, 0) == 0
    assert lib.rsx_sparse_workspace_size(17, 100, T, 0) == 0
    assert lib.rsx_sparse_workspace_size(2, 100, 2, 0) == 0
    assert lib.rsx_sparse_workspace_size(2, 2 ** 32, T, 0) == 0
    size = lib.rsx_sparse_workspace_size(4, 10_000, K, 0)
    assert size % 256 == 0
    # a slot of 4096 (index, value) entries per tile of every rank: 3 tiles of 4096
    assert size >= 4 * 3 * 4096 * 8
    assert all(lib.rsx_sparse_workspace_size(4, 10_000, m, acc) == size for m in (T, K) for acc in (0, 1))


def _sp(lib, grads, accs, outs, w, n, mode=0, thr=0.5, k=0, mi=None, mv=None, cap=None, nnz=None,
        ws=None, wsb=None):
    cap = n if cap is None else cap
    mi = mi if mi is not None else [A + (40 + 2 * r) * MB for r in range(w)]
    mv = mv if mv is not None else [A + (41 + 2 * r) * MB for r in range(w)]
    nnz = A + 90 * MB if nnz is None else nnz
    ws = A + 100 * MB if ws is None else ws
    wsb = lib.rsx_sparse_workspace_size(w, n, mode, int(accs is not None)) if wsb is None else wsb
    return lib.rsx_sparse_all_reduce(_arr(grads), _arr(accs) if accs is not None else None, _arr(outs),
                                     w, n, mode, thr, k, _arr(mi), _arr(mv), cap, nnz, ws, wsb, None)


@fake_ptrs
def test_sparse_validation(lib):
    g, o, a = [A, A + MB], [A + 2 * MB, A + 3 * MB], [A + 4 * MB, A + 5 * MB]
    n = 1000
    assert lib.rsx_sparse_all_reduce(None, None, _arr(o), 2, n, 0, 0.5, 0, _arr([A] * 2), _arr([A] * 2),
                                     n, A, A, 1 << 20, None) == 1
    assert _sp(lib, g, a, o, 0, n) == 1                       # no ranks
    assert _sp(lib, g * 9, a * 9, o * 9, 17, n) == 1          # too many ranks
    assert _sp(lib, g, a, o, 2, n, mode=2) == 1               # unknown mode
    assert _sp(lib, g, a, o, 2, 2 ** 32, wsb=1 << 40) == 4    # indices are uint32
    assert _sp(lib, g, a, o, 2, n, mode=1, k=n + 1) == 1      # k > count
    assert _sp(lib, g, a, o, 2, n, cap=n - 1) == 1            # threshold needs room for count
    assert _sp(lib, g, a, o, 2, n, mode=1, k=10, cap=9) == 1  # top-K needs room for k
    assert _sp(lib, [A + 4, A + MB], a, o, 2, n) == 1         # gradient not 16-byte aligned
    assert _sp(lib, g, [A + 4 * MB, A + 5 * MB + 8], o, 2, n) == 1
    assert _sp(lib, g, a, o, 2, n, nnz=A + 90 * MB + 2) == 1  # nnz not 4-byte aligned
    assert _sp(lib, g, a, o, 2, n, ws=A + 100 * MB + 64) == 1  # workspace not 256-byte aligned
    assert _sp(lib, g, a, o, 2, n, mode=1, k=5,
               wsb=lib.rsx_sparse_workspace_size(2, n, 1, 1) - 1) == 1   # workspace too small
    assert _sp(lib, g, a, [A + 2 * MB, None], 2, n) == 1      # null output


@fake_ptrs
def test_sparse_aliasing(lib):
    g, o, a = [A, A + MB], [A + 2 * MB, A + 3 * MB], [A + 4 * MB, A + 5 * MB]
    n = 1000
    assert _sp(lib, g, [A + MB, A + 5 * MB], o, 2, n) == 5                 # accumulation = a gradient
    assert _sp(lib, g, a, [A + 2 * MB, A + 2 * MB + 16], 2, n) == 5       # outputs overlap
    assert _sp(lib, g, a, [A + 4 * MB, A + 3 * MB], 2, n) == 5            # output = accumulation
    assert _sp(lib, g, a, o, 2, n, mi=[A + 3 * MB, A + 42 * MB]) == 5     # message over an output
    assert _sp(lib, g, a, o, 2, n, ws=A + 41 * MB) == 5                   # workspace over a message
    assert _sp(lib, g, a, o, 2, n, nnz=A + 8) == 5                        # nnz inside a gradient


def _spn(lib, grads, accs, outs, w, n, mode=0, thr=0.5, k=0, mi=None, mv=None, cap=None, nnz=None):
    cap = n if cap is None else cap
    mi = mi if mi is not None else [A + (2 * r) * (1 << 30) + (1 << 40) for r in range(w)]
    mv = mv if mv is not None else [A + (2 * r + 1) * (1 << 30) + (1 << 40) for r in range(w)]
    nnz = A + (1 << 41) if nnz is None else nnz
    return lib.rsx_sparse_all_reduce_noalloc(_arr(grads), _arr(accs) if accs is not None else None,
                                             _arr(outs), w, n, mode, thr, k, _arr(mi), _arr(mv), cap,
                                             nnz, None)


@fake_ptrs
def test_sparse_noalloc_validation_and_size_limit(lib):
    # The same checks as the workspace form, all before any HIP call; sizes
    # whose workspace exceeds the scratch array are refused with
    # RSX_ERR_UNSUPPORTED, also before any HIP call.
    g, o, a = [A, A + MB], [A + 2 * MB, A + 3 * MB], [A + 4 * MB, A + 5 * MB]
    n = 1000
    assert _spn(lib, g, a, o, 0, n) == 1
    assert _spn(lib, g, a, o, 2, n, mode=2) == 1
    assert _spn(lib, g, a, o, 2, n, mode=1, k=n + 1) == 1
    assert _spn(lib, g, a, o, 2, n, cap=n - 1) == 1
    assert _spn(lib, [A + 4, A + MB], a, o, 2, n) == 1
    assert _spn(lib, g, a, [A + 4 * MB, A + 3 * MB], 2, n) == 5            # output = accumulation
    assert _spn(lib, g, a, o, 2, n, nnz=A + 8) == 5                        # nnz inside a gradient
    assert _spn(lib, g, a, o, 2, 2 ** 32) == 4                             # indices are uint32
    assert lib.rsx_sparse_all_reduce_noalloc(None, None, _arr(o), 2, n, 0, 0.5, 0, _arr([A] * 2),
                                             _arr([A] * 2), n, A, None) == 1
    limit = _header_int("RSX_SPARSE_SCRATCH_BYTES")
    assert limit == 128 << 20
    # the largest W = 8 count that fits, and the next size up, which does not
    fits = max(c for c in range(0, 3 << 20, 4096)
               if lib.rsx_sparse_workspace_size(8, c, 1, 1) <= limit)
    assert fits >= 2_000_000
    assert lib.rsx_sparse_workspace_size(8, fits + 4096, 1, 1) > limit
    G = 1 << 30
    g8 = [A + r * G for r in range(8)]
    o8 = [A + (8 + r) * G for r in range(8)]
    a8 = [A + (16 + r) * G for r in range(8)]
    for mode, k in ((0, 0), (1, 100)):
        assert _spn(lib, g8, a8, o8, 8, fits + 4096, mode=mode, k=k) == 4


def test_occupancy_caps_context_manager_restores_the_setting(lib):
    import collective_reduction_ring_amd as rsx
    assert lib.rsx_set_occupancy_caps(1) in (0, 1)      # start from "on"
    with rsx.occupancy_caps(False):
        assert lib.rsx_set_occupancy_caps(0) == 0        # off inside
        with rsx.occupancy_caps(True):
            assert lib.rsx_set_occupancy_caps(1) == 1    # on in the nested block
        assert lib.rsx_set_occupancy_caps(0) == 0        # off again after it
    assert lib.rsx_set_occupancy_caps(1) == 1            # on after the outer block
    try:
        with rsx.occupancy_caps(False):
            raise RuntimeError("inside")
    except RuntimeError:
        pass
    assert lib.rsx_set_occupancy_caps(1) == 1            # restored on an exception too
