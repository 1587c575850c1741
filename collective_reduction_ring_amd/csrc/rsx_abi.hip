// C ABI of librsx.so (declared in include/rsx.h): argument validation,
// aliasing rules, launch geometry and dispatch to the kernel launchers.
//
// Every check runs before the first HIP call, so a rejected call has no side
// effect and the error paths can be exercised on a machine without a GPU.
#include <math.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include "rsx_internal.h"
#include "sparse_internal.h"

// The allocation-free sparsified all-reduce's workspace: one array per GPU,
// held until the process ends, shared by every such call on that GPU.  In
// host code `scratch` names a host-side stand-in, not the device memory: the
// device address comes from hipGetSymbolAddress, once per device (with that
// device current), and only that address is passed on.
static __device__ __align__(256) unsigned char scratch[RSX_SPARSE_SCRATCH_BYTES];

namespace rsx {
namespace {

thread_local char g_hip_error[256] = "HIP error";

rsx_status_t hip_status(hipError_t e) {
  if (e == hipSuccess) return RSX_SUCCESS;
  snprintf(g_hip_error, sizeof(g_hip_error), "HIP error %d: %s", static_cast<int>(e),
           hipGetErrorString(e));
  return RSX_ERR_HIP;
}

size_t esize_of(int dtype) {
  switch (dtype) {
    case RSX_FLOAT32:
    case RSX_INT32:
    case RSX_FLOAT32_HALF_WIRE:
      return 4;
    case RSX_BFLOAT16:
    case RSX_FLOAT16:
      return 2;
    case RSX_FLOAT64:
    case RSX_INT64:
    case RSX_UINT64:
      return 8;
    case RSX_INT8:
      return 1;
    default:
      return 0;
  }
}

bool valid_op(int op) { return op >= RSX_SUM && op <= RSX_PROD; }

// Occupancy caps.  Every lane of the dwordx4 fold and copy kernels keeps one
// 16-byte access per buffer in flight, so with all 8 workgroups per CU
// resident the chip keeps more HBM streams open than the memory system serves
// best.  Reserving LDS, which these kernels do not otherwise use, limits the
// workgroups resident per CU.  Measured best caps (fp32, 256 MiB per rank,
// W = 2..16; W = 8 reduce-scatter 381 -> 362-371 us, one-pass all-reduce
// 805 -> 725-732 us, all-gather 426 -> 380-383 us):
//   reduce-scatter (W+1 streams per workgroup): 8 at W <= 2, 5 up to W = 9
//     (from W = 10 it runs in pairs, two per CU: rs_pairs);
//   all-reduce, one pass (2W streams): 8 at W = 1, 5 at W = 2, 3 from W = 3;
//   all-gather, every piece in place (1 + (W-1)): 8 at W <= 2, 6 at W = 4, 6, 8,
//     otherwise 5 up to W = 9, 3 above;
//   all-gather, out of place (1 + W): 5 up to W = 5, 3 above (W = 2 164 -> 130 us,
//     W = 8 498 -> 459 us);
//   tensor-list all-reduce: 5 up to W = 4 (C5-like lists: 182 -> 177 us), 3 above.
// The element-wise kernels (unaligned buffers) run best uncapped: they keep
// less in flight per lane.
// The caps are per calling thread (rsx_set_occupancy_caps): launches meant to
// overlap other kernels go without them.
constexpr uint32_t kLdsPerCu = 160u * 1024u;
thread_local bool t_caps = true;
uint32_t lds_for_cap(uint32_t wg_per_cu) {
  if (!t_caps || wg_per_cu >= 8) return 0u;
  // One per CU: any reservation above half the CU's LDS does it.
  if (wg_per_cu == 1) return 96u * 1024u;
  return (kLdsPerCu / wg_per_cu) & ~1023u;
}
uint32_t ag_cap(int w, bool in_place) {
  if (!in_place) return w <= 5 ? 5u : 3u;
  if (w <= 2) return 8u;
  if (w == 4 || w == 6 || w == 8) return 6u;
  return w <= 9 ? 5u : 3u;
}
uint32_t list_cap(int w) { return w <= 1 ? 8u : w <= 4 ? 5u : 3u; }
// Write-heavy kernels (the one-pass all-reduce, the all-gather) run faster
// at larger W with fewer, larger workgroups: two 256-lane tiles per 512-lane
// workgroup, one workgroup per CU ("pairs").  Measured in one process, 256
// MiB per rank, one tile per workgroup at the caps above against pairs:
//   one-pass all-reduce fp32, W = 3..16: W = 3, 4 +0.9 / +0.8%; W = 5, 6, 7,
//     8 +3.0 / +5.0 / +5.2 / +1.4%; W = 10, 12, 14, 16 +1.6 / +2.3 / -0.7 /
//     +1.7% (W = 8 at 256 MiB per rank: 732 -> 722 us; other boxes 735 ->
//     682-715 us);
//   all-gather out of place, W = 6, 7, 8: +14.7 / +14.3 / +8.9% (W = 8:
//     448 -> 409 us); W = 10..16: -0.6 .. +3.7%; W <= 5: -3 .. -18%;
//   all-gather in place, W = 7, 8: +5.9 / +10.1%; W = 10..16: +2.1 .. +4.8%;
//     W = 6: -2.5%; W <= 5: -11 .. -47%.
// For these write-heavy kernels pairs at two workgroups per CU lose almost
// everywhere (up to -16%); the reduce-scatter is the other way round (below).
// Pairs are a form of the occupancy cap: with the caps off (launches that
// overlap other work) every kernel runs one tile per workgroup.
bool ar_pairs(int w) { return t_caps && w >= 5; }
// The reduce-scatter (dwordx4) in pairs at two workgroups per CU against one
// tile per workgroup at rs_cap, int32 sum, 128 MiB per rank, same process:
// W = 10 248 -> 245 us, 11 280 -> 264, 12 309 -> 294, 13 331 -> 321, 14 345
// -> 337, 15 362 -> 357, 16 375 -> 368; W = 9 229 -> 231.  At W = 8 it
// wins at 128 MiB per rank (199 -> 194 us) but loses at 256 MiB (366 -> 379
// us), so W = 8 keeps single tiles.
bool rs_pairs(int w) { return t_caps && w >= 10; }
// The ring all-reduce as two passes (a reduce-scatter, then an all-gather in
// place) against one pass, whole calls, same process (fp32 and bf16; ratio
// of two-pass to one-pass time): W = 8, 4 / 16 / 64 / 256 MiB per rank:
// 0.96 / 0.91 / 0.97 / 0.97 (256 MiB: 721 -> 699 us); W = 7, 10, 12 from 4
// MiB: 0.92 .. 1.0; W = 16: 0.93-0.95 at 4 MiB, 0.97 at 128 MiB (int32,
// 774 -> 752 us), 0.95-0.97 at 256 MiB, but 1.06 at 64 MiB; W <= 6: one
// pass ahead (up to 8%); below 4 MiB per rank the second launch costs more
// than it saves (1 MiB: 1.2-1.5).  Without the occupancy caps the
// all-gather has no pairs and one pass is kept.
// `count` is one bucket's elements; a launch may cover `groups` equal
// buckets, and its size is what the measurements above key on.
bool two_passes_pay(int w, size_t count, size_t groups, size_t es, bool vec) {
  const size_t seg = count / static_cast<size_t>(w);
  return t_caps && vec && w >= 7 && count % static_cast<size_t>(w) == 0 && (seg * es) % kVecBytes == 0 &&
         count * groups * es >= (4u << 20);
}
// All-gather: tiles per workgroup and workgroups per CU.
void ag_shape(int w, bool in_place, int* tpw, uint32_t* cap) {
  if (t_caps && (w >= 7 || (w == 6 && !in_place))) {
    *tpw = 2;
    *cap = 1;
    return;
  }
  *tpw = 1;
  *cap = ag_cap(w, in_place);
}
uint32_t rs_cap(int w) { return w <= 2 ? 8u : 5u; }  // W >= 10 runs in pairs (rs_pairs)
uint32_t ar_cap(int w) { return w <= 1 ? 8u : w == 2 ? 5u : 3u; }

// Per element type launchers (one translation unit each).
hipError_t launch_fold_by_type(int dtype, int op, int world, bool rs, bool vec, int tpw, const FoldArgs& a,
                               dim3 grid, uint32_t lds, hipStream_t s) {
  switch (dtype) {
    case RSX_FLOAT32:
      return launch_fold_f32(op, world, rs, vec, tpw, a, grid, lds, s);
    case RSX_BFLOAT16:
      return launch_fold_bf16(op, world, rs, vec, tpw, a, grid, lds, s);
    case RSX_INT32:
      return launch_fold_i32(op, world, rs, vec, tpw, a, grid, lds, s);
    case RSX_FLOAT64:
      return launch_fold_f64(op, world, rs, vec, tpw, a, grid, lds, s);
    case RSX_FLOAT16:
      return launch_fold_f16(op, world, rs, vec, tpw, a, grid, lds, s);
    case RSX_INT64:
      return launch_fold_i64(op, world, rs, vec, tpw, a, grid, lds, s);
    case RSX_UINT64:
      return launch_fold_u64(op, world, rs, vec, tpw, a, grid, lds, s);
    case RSX_INT8:
      return launch_fold_i8(op, world, rs, vec, tpw, a, grid, lds, s);
    case RSX_FLOAT32_HALF_WIRE:
      return launch_fold_f32h(op, world, rs, vec, tpw, a, grid, lds, s);
    default:
      return hipErrorInvalidValue;
  }
}

hipError_t launch_list_by_type(int dtype, int op, int world, const ListArgs& a, dim3 grid, uint32_t lds,
                               hipStream_t s) {
  switch (dtype) {
    case RSX_FLOAT32:
      return launch_list_f32(op, world, a, grid, lds, s);
    case RSX_BFLOAT16:
      return launch_list_bf16(op, world, a, grid, lds, s);
    case RSX_INT32:
      return launch_list_i32(op, world, a, grid, lds, s);
    case RSX_FLOAT64:
      return launch_list_f64(op, world, a, grid, lds, s);
    case RSX_FLOAT16:
      return launch_list_f16(op, world, a, grid, lds, s);
    case RSX_INT64:
      return launch_list_i64(op, world, a, grid, lds, s);
    case RSX_UINT64:
      return launch_list_u64(op, world, a, grid, lds, s);
    case RSX_INT8:
      return launch_list_i8(op, world, a, grid, lds, s);
    case RSX_FLOAT32_HALF_WIRE:
      return launch_list_f32h(op, world, a, grid, lds, s);
    default:
      return hipErrorInvalidValue;
  }
}

// a * b without wrapping; false on overflow.
bool mul_ok(size_t a, size_t b, size_t* out) {
  if (a != 0 && b > SIZE_MAX / a) return false;
  *out = a * b;
  return true;
}

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};
Range range_of(const void* p, size_t bytes) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return {lo, lo + bytes};
}
// A buffer whose end would wrap past the top of the address space.
bool wraps(Range r) { return r.hi < r.lo; }
bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi && a.lo < a.hi && b.lo < b.hi; }
bool same(Range a, Range b) { return a.lo == b.lo && a.hi == b.hi; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Buffers that are only read may coincide exactly; partial overlap is refused
// because no element index can then be tied to a single lane.
bool reads_consistent(const Range* r, int n) {
  for (int i = 0; i < n; ++i)
    for (int j = i + 1; j < n; ++j)
      if (overlap(r[i], r[j]) && !same(r[i], r[j])) return false;
  return true;
}
bool pairwise_disjoint(const Range* r, int n) {
  for (int i = 0; i < n; ++i)
    for (int j = i + 1; j < n; ++j)
      if (overlap(r[i], r[j])) return false;
  return true;
}

// Workgroups along one segment of `seg` elements.
uint64_t fold_tiles(uint64_t seg, int world, bool vec, int vl) {
  const uint64_t per = static_cast<uint64_t>(fold_units(world)) * kBlock;
  const uint64_t units = vec ? seg / vl : seg;
  return std::max<uint64_t>(1, (units + per - 1) / per);
}

rsx_status_t launch_fold_any(int dtype, int op, int world, bool rs, bool vec, FoldArgs a,
                             uint64_t tiles_per_seg, uint32_t nseg, hipStream_t s) {
  const uint64_t total = tiles_per_seg * nseg;
  if (total > 0x7ffffff0ull) return RSX_ERR_UNSUPPORTED;
  a.tiles_per_seg = static_cast<uint32_t>(tiles_per_seg);
  a.tiles_total = static_cast<uint32_t>(total);
  split_magic(a.tiles_per_seg, &a.tps_magic, &a.tps_shift);
  // The dwordx4 all-reduce at W >= 5 runs two tiles per workgroup, one
  // workgroup per CU (ar_pairs), the dwordx4 reduce-scatter at W >= 10 two
  // per workgroup, two workgroups per CU (rs_pairs); everything else one
  // tile per workgroup.
  const bool pairs = vec && (rs ? rs_pairs(world) : ar_pairs(world));
  const int tpw = pairs ? 2 : 1;
  const dim3 grid(static_cast<uint32_t>(xcd_grid((total + tpw - 1) / tpw)));
  const uint32_t lds = !vec ? 0u : pairs ? lds_for_cap(rs ? 2u : 1u) : lds_for_cap(rs ? rs_cap(world) : ar_cap(world));
  return hip_status(launch_fold_by_type(dtype, op, world, rs, vec, tpw, a, grid, lds, s));
}

// All-gather launch over validated buffers: piece k = src[k] goes to
// dst[r] + k * n elements for every r.  A piece already in place (src[k] ==
// dst[k] + k * n) is read but not written back.  With groups > 1 the same
// is done for each of `groups` consecutive blocks of W * n elements.
rsx_status_t launch_gather_any(const void* const* src, void* const* dst, int nranks, size_t n,
                               size_t es, hipStream_t stream, uint64_t groups = 1) {
  const size_t piece_bytes = n * es;
  // whole dwords: the dwordx4 kernels (dword-aligned loads where the pieces
  // are not whole vectors, aligned stores)
  bool vec = (piece_bytes % 4) == 0;
  const bool whole = (piece_bytes % kVecBytes) == 0;
  bool in_place = true;
  for (int r = 0; r < nranks; ++r) {
    vec = vec && aligned16(src[r]) && aligned16(dst[r]);
    in_place = in_place && src[r] == static_cast<const char*>(dst[r]) + static_cast<size_t>(r) * piece_bytes;
  }
  GatherArgs a;
  memset(&a, 0, sizeof(a));
  for (int r = 0; r < nranks; ++r) {
    a.src[r] = src[r];
    a.dst[r] = dst[r];
  }
  a.n = n;
  a.world = nranks;
  const uint64_t units = vec ? piece_bytes / kVecBytes : n;
  const uint64_t per = static_cast<uint64_t>(kCopyUnits) * kBlock;
  const uint64_t tiles = std::max<uint64_t>(1, (units + per - 1) / per);
  const uint64_t total = tiles * static_cast<uint64_t>(nranks) * groups;
  if (total > 0x7ffffff0ull) return RSX_ERR_UNSUPPORTED;
  a.tiles_per_piece = static_cast<uint32_t>(tiles);
  a.tiles_total = static_cast<uint32_t>(total);
  split_magic(a.tiles_per_piece, &a.tps_magic, &a.tps_shift);
  int tpw = 1;
  uint32_t cap = 8;  // the element-wise kernel runs uncapped
  if (vec) ag_shape(nranks, in_place, &tpw, &cap);
  return hip_status(launch_gather(static_cast<int>(es), !vec ? 0 : whole ? 1 : 2, tpw, a,
                                  dim3(static_cast<uint32_t>(xcd_grid((total + tpw - 1) / tpw))),
                                  lds_for_cap(cap), stream));
}

// Shared validation of the pointer arrays and enums of the collectives.
rsx_status_t check_common(const void* const* sendbufs, void* const* recvbufs, int nranks,
                          int dtype) {
  if (sendbufs == nullptr || recvbufs == nullptr) return RSX_ERR_INVALID_ARGUMENT;
  if (nranks < 1 || nranks > RSX_MAX_RANKS) return RSX_ERR_INVALID_ARGUMENT;
  if (esize_of(dtype) == 0) return RSX_ERR_INVALID_TYPE;
  return RSX_SUCCESS;
}

// Every element access of the kernels is naturally aligned: a buffer must
// start at a multiple of its element size (es is a power of two).
bool elem_aligned(const void* p, size_t es) { return (reinterpret_cast<uintptr_t>(p) & (es - 1)) == 0; }

rsx_status_t check_device_ptrs(const void* const* sendbufs, void* const* recvbufs, int nranks,
                               size_t es) {
  for (int r = 0; r < nranks; ++r) {
    if (sendbufs[r] == nullptr || recvbufs[r] == nullptr) return RSX_ERR_INVALID_ARGUMENT;
    if (!elem_aligned(sendbufs[r], es) || !elem_aligned(recvbufs[r], es)) return RSX_ERR_INVALID_ARGUMENT;
  }
  return RSX_SUCCESS;
}

// Pack (tensors -> fused) or unpack (fused -> tensors) at running offsets.
rsx_status_t fuse_copy(const void* const* tens, const size_t* counts, int ntensors,
                       const void* fused, bool pack, int dtype, hipStream_t stream) {
  if (counts == nullptr || ntensors < 0) return RSX_ERR_INVALID_ARGUMENT;
  const size_t es = esize_of(dtype);
  if (es == 0) return RSX_ERR_INVALID_TYPE;
  size_t total = 0;
  for (int i = 0; i < ntensors; ++i) {
    size_t b;
    if (!mul_ok(counts[i], es, &b) || total + b < total) return RSX_ERR_UNSUPPORTED;
    total += b;
  }
  if (total == 0) return RSX_SUCCESS;
  if (tens == nullptr || fused == nullptr || !elem_aligned(fused, es)) return RSX_ERR_INVALID_ARGUMENT;
  for (int i = 0; i < ntensors; ++i)
    if (counts[i] != 0 && (tens[i] == nullptr || !elem_aligned(tens[i], es))) return RSX_ERR_INVALID_ARGUMENT;
  const Range fr = range_of(fused, total);
  if (wraps(fr)) return RSX_ERR_INVALID_ARGUMENT;
  for (int i = 0; i < ntensors; ++i) {
    if (counts[i] == 0) continue;
    const Range ti = range_of(tens[i], counts[i] * es);
    if (wraps(ti)) return RSX_ERR_INVALID_ARGUMENT;
    if (overlap(fr, ti)) return RSX_ERR_ALIASING;
    if (!pack) {  // unpack writes the tensors: they must not overlap each other
      for (int j = i + 1; j < ntensors; ++j)
        if (counts[j] != 0 && overlap(ti, range_of(tens[j], counts[j] * es))) return RSX_ERR_ALIASING;
    }
  }

  if (total > kOffMask) return RSX_ERR_UNSUPPORTED;

  // Batches of up to RSX_FUSE_BATCH copies and kMaxCopyTiles tiles per
  // launch; a tensor beyond 16 GiB is copied as several pieces.
  constexpr uint64_t kPieceBytes = 1ull << 34;
  MultiCopyArgs a;
  memset(&a, 0, sizeof(a));
  a.fused = static_cast<char*>(const_cast<void*>(fused));
  a.unpack = pack ? 0u : 1u;
  uint64_t tiles = 0;
  size_t off = 0;
  auto flush = [&]() -> rsx_status_t {
    if (a.n == 0) return RSX_SUCCESS;
    a.d[a.n].tensor = nullptr;
    a.d[a.n].off_tile = off | (tiles << kOffBits);  // sentinel: end offset, tile total
    const rsx_status_t st = hip_status(launch_multicopy(static_cast<int>(es), a, 0u, stream));
    a.n = 0;
    tiles = 0;
    return st;
  };
  for (int i = 0; i < ntensors; ++i) {
    const size_t bytes = counts[i] * es;
    for (size_t done = 0; done < bytes;) {
      const size_t piece = std::min<size_t>(bytes - done, kPieceBytes);
      char* tp = static_cast<char*>(const_cast<void*>(tens[i])) + done;
      const void* dst = pack ? static_cast<const void*>(a.fused + off) : static_cast<const void*>(tp);
      const uint64_t pt = copy_tiles(dst, piece);
      if (a.n == RSX_FUSE_BATCH || tiles + pt > kMaxCopyTiles) {
        const rsx_status_t st = flush();
        if (st != RSX_SUCCESS) return st;
      }
      a.d[a.n].tensor = tp;
      a.d[a.n].off_tile = off | (tiles << kOffBits);
      a.n += 1;
      tiles += pt;
      off += piece;
      done += piece;
    }
  }
  return flush();
}

// Overlap rules of the tensor-list all-reduce, in O(n log n) for n buffers.
// Sources may coincide exactly but not overlap partially; destinations are
// pairwise disjoint; a destination may coincide with sources only when all of
// them belong to the same tensor index (each element is then read and
// written by the same lane).
struct Span {
  uintptr_t lo, hi;
  int tensor;
};
bool list_aliasing_ok(std::vector<Span>& sends, std::vector<Span>& recvs) {
  auto by_lo = [](const Span& a, const Span& b) { return a.lo < b.lo || (a.lo == b.lo && a.hi < b.hi); };
  std::sort(sends.begin(), sends.end(), by_lo);
  std::sort(recvs.begin(), recvs.end(), by_lo);
  // Unique source spans (sorted, pairwise disjoint after this check), each
  // with its tensor index or -1 when spans of several tensors coincide.
  std::vector<Span> uniq;
  for (const Span& x : sends) {
    if (!uniq.empty() && uniq.back().lo == x.lo && uniq.back().hi == x.hi) {
      if (uniq.back().tensor != x.tensor) uniq.back().tensor = -1;
      continue;
    }
    if (!uniq.empty() && x.lo < uniq.back().hi) return false;  // partial overlap of sources
    uniq.push_back(x);
  }
  for (size_t i = 1; i < recvs.size(); ++i)
    if (recvs[i].lo < recvs[i - 1].hi) return false;  // destinations overlap
  for (const Span& r : recvs) {
    // first unique source ending after r.lo
    size_t a = std::partition_point(uniq.begin(), uniq.end(),
                                    [&](const Span& u) { return u.hi <= r.lo; }) - uniq.begin();
    for (size_t j = a; j < uniq.size() && uniq[j].lo < r.hi; ++j) {
      const Span& u = uniq[j];
      if (u.lo != r.lo || u.hi != r.hi || u.tensor != r.tensor) return false;
    }
  }
  return true;
}

bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// Workspace of the sparsified all-reduce: per-tile counts and offsets,
// radix histograms, selection state, and one slot of kSpTile entries per
// tile.  Each region starts on a 256-byte boundary.
constexpr size_t kWsAlign = 256;
size_t ws_align(size_t v) { return (v + kWsAlign - 1) / kWsAlign * kWsAlign; }
struct SparseLayout {
  size_t tile_slot, tile_cnt, tile_eqc, tile_off, tile_eqb, hist, state, gap_idx, gap_val, total;
  uint32_t tiles;
};
bool sparse_layout(int w, size_t count, int mode, bool accum, SparseLayout* l) {
  if (w < 1 || w > RSX_MAX_RANKS) return false;
  if (mode != RSX_SPARSE_THRESHOLD && mode != RSX_SPARSE_TOPK) return false;
  if (count > UINT32_MAX) return false;
  const size_t ws = static_cast<size_t>(w);
  l->tiles = static_cast<uint32_t>((count + kSpTile - 1) / kSpTile);
  const size_t tile_bytes = ws_align(ws * (l->tiles + 1) * 4);
  const size_t slot_bytes = ws_align(ws * l->tiles * kSpTile * 4);
  size_t off = 0;
  l->tile_slot = off;
  off += tile_bytes;
  l->tile_cnt = off;
  off += tile_bytes;
  l->tile_eqc = off;
  off += tile_bytes;
  l->tile_off = off;
  off += tile_bytes;
  l->tile_eqb = off;
  off += tile_bytes;
  l->gap_idx = off;
  off += slot_bytes;
  l->gap_val = off;
  off += slot_bytes;
  l->hist = off;
  off += ws_align(kHistCount * ws * kSpBins * 4);
  l->state = off;
  off += ws_align(ws * kSpState * 4);
  (void)accum;  // the slots hold everything either mode keeps
  l->total = off;
  return true;
}

// Validation of a sparsified all-reduce, shared by both entry points; no HIP
// call.  own_scratch: the library's scratch array takes the place of the
// caller's workspace (no caller buffer can overlap it; its size is checked
// by the entry point).
rsx_status_t sparse_check(const float* const* grads, float* const* accums, float* const* outs,
                          int nranks, size_t count, rsx_sparse_mode_t mode, size_t k,
                          uint32_t* const* msg_idx, float* const* msg_val, size_t msg_capacity,
                          uint32_t* nnz, const void* workspace, size_t workspace_bytes,
                          bool own_scratch, SparseLayout* l) {
  if (grads == nullptr || outs == nullptr || msg_idx == nullptr || msg_val == nullptr)
    return RSX_ERR_INVALID_ARGUMENT;
  if (nranks < 1 || nranks > RSX_MAX_RANKS) return RSX_ERR_INVALID_ARGUMENT;
  if (mode != RSX_SPARSE_THRESHOLD && mode != RSX_SPARSE_TOPK) return RSX_ERR_INVALID_ARGUMENT;
  if (count > UINT32_MAX) return RSX_ERR_UNSUPPORTED;
  if (mode == RSX_SPARSE_TOPK && k > count) return RSX_ERR_INVALID_ARGUMENT;
  if (nnz == nullptr || !aligned4(nnz)) return RSX_ERR_INVALID_ARGUMENT;
  const Range nr = range_of(nnz, static_cast<size_t>(nranks) * 4);
  if (wraps(nr)) return RSX_ERR_INVALID_ARGUMENT;
  if (count == 0) return RSX_SUCCESS;

  const bool has_acc = accums != nullptr;
  const size_t sent_max = mode == RSX_SPARSE_THRESHOLD ? count : k;
  if (msg_capacity < sent_max) return RSX_ERR_INVALID_ARGUMENT;
  sparse_layout(nranks, count, mode, has_acc, l);
  if (!own_scratch && (workspace == nullptr || (reinterpret_cast<uintptr_t>(workspace) & (kWsAlign - 1)) != 0 ||
                       workspace_bytes < l->total))
    return RSX_ERR_INVALID_ARGUMENT;
  const size_t bytes = count * 4;
  for (int r = 0; r < nranks; ++r) {
    if (grads[r] == nullptr || outs[r] == nullptr || msg_idx[r] == nullptr || msg_val[r] == nullptr ||
        (has_acc && accums[r] == nullptr))
      return RSX_ERR_INVALID_ARGUMENT;
    if (!aligned16(grads[r]) || !aligned16(outs[r]) || (has_acc && !aligned16(accums[r])) ||
        !aligned4(msg_idx[r]) || !aligned4(msg_val[r]))
      return RSX_ERR_INVALID_ARGUMENT;
  }
  // Everything written must be pairwise disjoint and apart from the
  // gradients, except the outputs: they are written after every read of the
  // gradients, so they may overlap them (in place: outs[r] == grads[r]).
  std::vector<Range> writes, outs_r;
  Range grads_r[RSX_MAX_RANKS];
  for (int r = 0; r < nranks; ++r) {
    grads_r[r] = range_of(grads[r], bytes);
    outs_r.push_back(range_of(outs[r], bytes));
    writes.push_back(outs_r.back());
    if (has_acc) writes.push_back(range_of(accums[r], bytes));
    writes.push_back(range_of(msg_idx[r], sent_max * 4));
    writes.push_back(range_of(msg_val[r], sent_max * 4));
    if (wraps(grads_r[r])) return RSX_ERR_INVALID_ARGUMENT;
  }
  writes.push_back(nr);
  if (!own_scratch) writes.push_back(range_of(workspace, l->total));
  for (const Range& w : writes)
    if (wraps(w)) return RSX_ERR_INVALID_ARGUMENT;
  if (!pairwise_disjoint(writes.data(), static_cast<int>(writes.size()))) return RSX_ERR_ALIASING;
  for (const Range& w : writes) {
    bool is_out = false;
    for (const Range& o : outs_r) is_out = is_out || same(o, w);
    if (is_out) continue;
    for (int r = 0; r < nranks; ++r)
      if (overlap(w, grads_r[r])) return RSX_ERR_ALIASING;
  }
  return RSX_SUCCESS;
}

// Kernel arguments of a checked sparsified all-reduce over the workspace `ws`
// (laid out by `l`), and the launches.
rsx_status_t sparse_launch(const float* const* grads, float* const* accums, float* const* outs,
                           int nranks, size_t count, rsx_sparse_mode_t mode, float threshold,
                           size_t k, uint32_t* const* msg_idx, float* const* msg_val,
                           size_t msg_capacity, uint32_t* nnz, void* ws_base,
                           const SparseLayout& l, hipStream_t stream) {
  (void)msg_capacity;
  const bool has_acc = accums != nullptr;
  const size_t sent_max = mode == RSX_SPARSE_THRESHOLD ? count : k;
  SparseArgs a;
  memset(&a, 0, sizeof(a));
  char* ws = static_cast<char*>(ws_base);
  for (int r = 0; r < nranks; ++r) {
    a.grad[r] = grads[r];
    a.accum[r] = has_acc ? accums[r] : nullptr;
    a.out[r] = outs[r];
    a.msg_idx[r] = msg_idx[r];
    a.msg_val[r] = msg_val[r];
  }
  a.nnz = nnz;
  a.tile_slot = reinterpret_cast<uint32_t*>(ws + l.tile_slot);
  a.tile_cnt = reinterpret_cast<uint32_t*>(ws + l.tile_cnt);
  a.tile_eqc = reinterpret_cast<uint32_t*>(ws + l.tile_eqc);
  a.tile_off = reinterpret_cast<uint32_t*>(ws + l.tile_off);
  a.tile_eqb = reinterpret_cast<uint32_t*>(ws + l.tile_eqb);
  a.gap_idx = reinterpret_cast<uint32_t*>(ws + l.gap_idx);
  a.gap_val = reinterpret_cast<float*>(ws + l.gap_val);
  a.hist = reinterpret_cast<uint32_t*>(ws + l.hist);
  a.state = reinterpret_cast<uint32_t*>(ws + l.state);
  a.count = count;
  a.tiles = l.tiles;
  a.world = static_cast<uint32_t>(nranks);
  a.k = mode == RSX_SPARSE_TOPK ? static_cast<uint32_t>(k) : 0u;
  a.cap = static_cast<uint32_t>(sent_max);
  a.threshold = threshold;
  return hip_status(launch_sparse(a, mode, has_acc, stream));
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

rsx_status_t scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (dev < 0 || dev >= kMaxDevices) return RSX_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e);
    if (p == nullptr) return RSX_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return RSX_SUCCESS;
}

// An all-reduce of `groups` buckets of `count` elements each fits the
// launch grid in every form (one pass, naive, or reduce-scatter +
// all-gather: at most count/W + 1 whole-vector or element tiles per
// segment, W segments per bucket).
bool all_reduce_grid_ok(int nranks, size_t count, uint64_t groups = 1) {
  const uint64_t seg = (count + nranks - 1) / nranks;
  const uint64_t per = fold_tiles(seg, nranks, false, 1) * static_cast<uint64_t>(nranks);
  if (per > 0x7ffffff0ull / groups) return false;
  return per * groups <= 0x7ffffff0ull && fold_tiles(count * groups, nranks, false, 1) <= 0x7ffffff0ull;
}

// Checks of an all-reduce (no HIP call).  *nothing: valid, with no work.
rsx_status_t all_reduce_check(const void* const* sendbufs, void* const* recvbufs, int nranks,
                              size_t count, rsx_dtype_t dtype, rsx_op_t op, rsx_algo_t algo,
                              bool* nothing) {
  *nothing = false;
  rsx_status_t st = check_common(sendbufs, recvbufs, nranks, dtype);
  if (st != RSX_SUCCESS) return st;
  if (!valid_op(op)) return RSX_ERR_INVALID_OP;
  if (algo != RSX_ALGO_RING && algo != RSX_ALGO_NAIVE && algo != RSX_ALGO_AUTO &&
      algo != RSX_ALGO_RING_FUSED && algo != RSX_ALGO_RING_SPLIT)
    return RSX_ERR_INVALID_ARGUMENT;
  if (count == 0) {
    *nothing = true;
    return RSX_SUCCESS;
  }
  if ((st = check_device_ptrs(sendbufs, recvbufs, nranks, esize_of(dtype))) != RSX_SUCCESS) return st;
  const size_t es = esize_of(dtype);
  size_t bytes;
  if (!mul_ok(count, es, &bytes)) return RSX_ERR_UNSUPPORTED;
  if (algo == RSX_ALGO_RING_SPLIT && count % static_cast<size_t>(nranks) != 0)
    return RSX_ERR_UNSUPPORTED;
  Range in[RSX_MAX_RANKS], out[RSX_MAX_RANKS];
  bool in_place_all = true;
  for (int r = 0; r < nranks; ++r) {
    in[r] = range_of(sendbufs[r], bytes);
    out[r] = range_of(recvbufs[r], bytes);
    if (wraps(in[r]) || wraps(out[r])) return RSX_ERR_INVALID_ARGUMENT;
  }
  if (!reads_consistent(in, nranks) || !pairwise_disjoint(out, nranks)) return RSX_ERR_ALIASING;
  for (int r = 0; r < nranks; ++r) {
    in_place_all = in_place_all && same(out[r], in[r]);
    for (int j = 0; j < nranks; ++j)
      if (overlap(out[r], in[j]) && !same(out[r], in[j])) return RSX_ERR_ALIASING;
  }
  // One rank in place: nothing to do, except that a half wire still rounds.
  *nothing = nranks == 1 && in_place_all && dtype != RSX_FLOAT32_HALF_WIRE;
  if (!*nothing && !all_reduce_grid_ok(nranks, count)) return RSX_ERR_UNSUPPORTED;
  return RSX_SUCCESS;
}

// Launches of a checked all-reduce of `count` elements per rank, or of
// `groups` consecutive buckets of `count` elements each, every bucket
// all-reduced as one call on it would (W must divide count when groups >
// 1, so that the buckets' ring segments tile the whole range).
rsx_status_t all_reduce_launch(const void* const* sendbufs, void* const* recvbufs, int nranks,
                               size_t count, rsx_dtype_t dtype, rsx_op_t op, rsx_algo_t algo,
                               hipStream_t stream, uint64_t groups = 1) {
  const size_t es = esize_of(dtype);
  const size_t bytes = count * es;  // one bucket: the naive choice is per bucket
  rsx_status_t st = RSX_SUCCESS;
  const bool naive = algo == RSX_ALGO_NAIVE || (algo == RSX_ALGO_AUTO && bytes <= RSX_NAIVE_MAX_BYTES);
  bool vec = true;
  for (int r = 0; r < nranks; ++r) vec = vec && aligned16(sendbufs[r]) && aligned16(recvbufs[r]);
  const bool split = algo == RSX_ALGO_RING_SPLIT ||
                     (!naive && algo != RSX_ALGO_RING_FUSED && two_passes_pay(nranks, count, groups, es, vec));

  // Two passes ("Distributed primitives": Ring AllReduce = ReduceScatter +
  // AllGather): the reduce-scatter stores segment k into recvbufs[k] at its
  // own offset, and the all-gather copies it from there to the other ranks.
  // Each lane of the reduce-scatter reads its element of every input before
  // it stores, and touches no other segment, so every alias the one-pass
  // form accepts is still safe; the all-gather runs after the last read of
  // the inputs, in stream order.  RSX_ALGO_RING takes this form where it
  // measured faster (two_passes_pay), RSX_ALGO_RING_SPLIT always.
  if (split) {
    const size_t seg = count / static_cast<size_t>(nranks);
    const bool rs_vec = vec && (seg * es) % 4 == 0;
    FoldArgs a;
    memset(&a, 0, sizeof(a));
    const void* pieces[RSX_MAX_RANKS];
    for (int r = 0; r < nranks; ++r) {
      a.src[r] = sendbufs[r];
      a.dst[r] = static_cast<char*>(recvbufs[r]) + static_cast<size_t>(r) * seg * es;
      pieces[r] = a.dst[r];
    }
    a.count = count * groups;
    a.seg = seg;
    a.rot = 1;
    const int vl = static_cast<int>(kVecBytes / es);
    // The all-gather's grid has no more tiles than the reduce-scatter's (the
    // same segments, in 16-byte units whenever the reduce-scatter's are), so
    // its size check cannot fail after the reduce-scatter has launched.
    st = launch_fold_any(dtype, op, nranks, true, rs_vec, a, fold_tiles(seg, nranks, rs_vec, vl),
                         static_cast<uint32_t>(nranks * groups), stream);
    if (st != RSX_SUCCESS) return st;
    return launch_gather_any(pieces, recvbufs, nranks, seg, es, stream, groups);
  }

  FoldArgs a;
  memset(&a, 0, sizeof(a));
  for (int r = 0; r < nranks; ++r) {
    a.src[r] = sendbufs[r];
    a.dst[r] = recvbufs[r];
  }
  a.count = count * groups;
  // Rank order is the same for every bucket: one segment over all of them.
  const uint64_t seg = naive ? count * groups : (count + nranks - 1) / nranks;
  a.seg = seg;
  a.rot = naive ? 0 : 1;
  const uint32_t nseg = naive ? 1 : static_cast<uint32_t>(nranks * groups);
  const int vl = static_cast<int>(kVecBytes / es);
  return launch_fold_any(dtype, op, nranks, false, vec, a, fold_tiles(seg, nranks, vec, vl), nseg,
                         stream);
}

// Checks of a bucketed all-reduce (no HIP call): one all-reduce over the
// whole buffers, the bucket size, W dividing every bucket in the two-pass
// form, and every bucket's launch grid (the largest bucket's).
rsx_status_t bucketed_check(const void* const* sendbufs, void* const* recvbufs, int nranks, size_t count,
                            size_t bucket_elems, rsx_dtype_t dtype, rsx_op_t op, rsx_algo_t algo,
                            bool* nothing) {
  if (bucket_elems == 0) return RSX_ERR_INVALID_ARGUMENT;
  rsx_status_t st = all_reduce_check(sendbufs, recvbufs, nranks, count, dtype, op, algo, nothing);
  if (st != RSX_SUCCESS || *nothing) return st;
  const size_t w = static_cast<size_t>(nranks);
  const size_t full = std::min(bucket_elems, count), last = count % bucket_elems;
  if (algo == RSX_ALGO_RING_SPLIT && (full % w != 0 || last % w != 0)) return RSX_ERR_UNSUPPORTED;
  if (!all_reduce_grid_ok(nranks, full)) return RSX_ERR_UNSUPPORTED;
  return RSX_SUCCESS;
}

}  // namespace
}  // namespace rsx

using namespace rsx;

extern "C" {

rsx_status_t rsx_reduce_scatter(const void* const* sendbufs, void* const* recvbufs, int nranks,
                                size_t recvcount, rsx_dtype_t dtype, rsx_op_t op,
                                hipStream_t stream) {
  rsx_status_t st = check_common(sendbufs, recvbufs, nranks, dtype);
  if (st != RSX_SUCCESS) return st;
  if (!valid_op(op)) return RSX_ERR_INVALID_OP;
  if (recvcount == 0) return RSX_SUCCESS;
  if ((st = check_device_ptrs(sendbufs, recvbufs, nranks, esize_of(dtype))) != RSX_SUCCESS) return st;
  const size_t es = esize_of(dtype);
  size_t n, seg_bytes, in_bytes;
  if (!mul_ok(recvcount, static_cast<size_t>(nranks), &n) || !mul_ok(recvcount, es, &seg_bytes) ||
      !mul_ok(n, es, &in_bytes))
    return RSX_ERR_UNSUPPORTED;

  Range in[RSX_MAX_RANKS], out[RSX_MAX_RANKS];
  bool in_place_all = true;
  for (int r = 0; r < nranks; ++r) {
    in[r] = range_of(sendbufs[r], in_bytes);
    out[r] = range_of(recvbufs[r], seg_bytes);
    if (wraps(in[r]) || wraps(out[r])) return RSX_ERR_INVALID_ARGUMENT;
  }
  if (!reads_consistent(in, nranks) || !pairwise_disjoint(out, nranks)) return RSX_ERR_ALIASING;
  for (int k = 0; k < nranks; ++k) {
    const bool in_place = out[k].lo == in[k].lo + k * seg_bytes;
    in_place_all = in_place_all && in_place;
    if (in_place) continue;
    for (int r = 0; r < nranks; ++r)
      if (overlap(out[k], in[r])) return RSX_ERR_ALIASING;
  }
  // One rank in place: nothing to do, except that a half wire still rounds.
  if (nranks == 1 && in_place_all && dtype != RSX_FLOAT32_HALF_WIRE) return RSX_SUCCESS;

  bool vec = (seg_bytes % 4) == 0;  // dword-aligned block starts; the fold kernel takes any tail
  for (int r = 0; r < nranks; ++r) vec = vec && aligned16(sendbufs[r]) && aligned16(recvbufs[r]);

  FoldArgs a;
  memset(&a, 0, sizeof(a));
  for (int r = 0; r < nranks; ++r) {
    a.src[r] = sendbufs[r];
    a.dst[r] = recvbufs[r];
  }
  a.count = n;
  a.seg = recvcount;
  a.rot = 1;
  const int vl = static_cast<int>(kVecBytes / es);
  return launch_fold_any(dtype, op, nranks, true, vec, a, fold_tiles(recvcount, nranks, vec, vl),
                         static_cast<uint32_t>(nranks), stream);
}

rsx_status_t rsx_all_gather(const void* const* sendbufs, void* const* recvbufs, int nranks,
                            size_t sendcount, rsx_dtype_t dtype, hipStream_t stream) {
  rsx_status_t st = check_common(sendbufs, recvbufs, nranks, dtype);
  if (st != RSX_SUCCESS) return st;
  // A gather reduces nothing: the half wire format applies to reductions only.
  if (dtype == RSX_FLOAT32_HALF_WIRE) return RSX_ERR_INVALID_TYPE;
  if (sendcount == 0) return RSX_SUCCESS;
  if ((st = check_device_ptrs(sendbufs, recvbufs, nranks, esize_of(dtype))) != RSX_SUCCESS) return st;
  const size_t es = esize_of(dtype);
  size_t piece_bytes, out_bytes;
  if (!mul_ok(sendcount, es, &piece_bytes) ||
      !mul_ok(piece_bytes, static_cast<size_t>(nranks), &out_bytes))
    return RSX_ERR_UNSUPPORTED;
  Range in[RSX_MAX_RANKS], out[RSX_MAX_RANKS];
  for (int r = 0; r < nranks; ++r) {
    in[r] = range_of(sendbufs[r], piece_bytes);
    out[r] = range_of(recvbufs[r], out_bytes);
    if (wraps(in[r]) || wraps(out[r])) return RSX_ERR_INVALID_ARGUMENT;
  }
  if (!pairwise_disjoint(out, nranks)) return RSX_ERR_ALIASING;
  bool in_place_all = true;
  for (int k = 0; k < nranks; ++k) {
    const bool in_place = in[k].lo == out[k].lo + k * piece_bytes;
    in_place_all = in_place_all && in_place;
    if (in_place) continue;
    for (int r = 0; r < nranks; ++r)
      if (overlap(in[k], out[r])) return RSX_ERR_ALIASING;
  }
  if (nranks == 1 && in_place_all) return RSX_SUCCESS;

  return launch_gather_any(sendbufs, recvbufs, nranks, sendcount, es, stream);
}

rsx_status_t rsx_all_reduce(const void* const* sendbufs, void* const* recvbufs, int nranks,
                            size_t count, rsx_dtype_t dtype, rsx_op_t op, rsx_algo_t algo,
                            hipStream_t stream) {
  bool nothing = false;
  const rsx_status_t st = all_reduce_check(sendbufs, recvbufs, nranks, count, dtype, op, algo, &nothing);
  if (st != RSX_SUCCESS || nothing) return st;
  return all_reduce_launch(sendbufs, recvbufs, nranks, count, dtype, op, algo, stream);
}

size_t rsx_bucket_count(size_t count, size_t bucket_elems) {
  return bucket_elems == 0 ? 0 : count / bucket_elems + (count % bucket_elems != 0 ? 1 : 0);
}

rsx_status_t rsx_all_reduce_bucket(const void* const* sendbufs, void* const* recvbufs, int nranks,
                                   size_t count, size_t bucket_elems, size_t bucket, rsx_dtype_t dtype,
                                   rsx_op_t op, rsx_algo_t algo, hipStream_t stream) {
  bool nothing = false;
  rsx_status_t st = bucketed_check(sendbufs, recvbufs, nranks, count, bucket_elems, dtype, op, algo, &nothing);
  if (st != RSX_SUCCESS) return st;
  if (count > 0 && bucket >= rsx_bucket_count(count, bucket_elems)) return RSX_ERR_INVALID_ARGUMENT;
  if (nothing) return RSX_SUCCESS;
  const size_t es = esize_of(dtype);
  const size_t b0 = bucket * bucket_elems, n = std::min(bucket_elems, count - b0);
  const void* src[RSX_MAX_RANKS];
  void* dst[RSX_MAX_RANKS];
  for (int r = 0; r < nranks; ++r) {
    src[r] = static_cast<const char*>(sendbufs[r]) + b0 * es;
    dst[r] = static_cast<char*>(recvbufs[r]) + b0 * es;
  }
  return all_reduce_launch(src, dst, nranks, n, dtype, op, algo, stream);
}

rsx_status_t rsx_all_reduce_bucketed(const void* const* sendbufs, void* const* recvbufs, int nranks,
                                     size_t count, size_t bucket_elems, rsx_dtype_t dtype, rsx_op_t op,
                                     rsx_algo_t algo, hipStream_t stream) {
  bool nothing = false;
  rsx_status_t st = bucketed_check(sendbufs, recvbufs, nranks, count, bucket_elems, dtype, op, algo, &nothing);
  if (st != RSX_SUCCESS || nothing) return st;
  const size_t w = static_cast<size_t>(nranks);
  const size_t es = esize_of(dtype);
  const void* src[RSX_MAX_RANKS];
  void* dst[RSX_MAX_RANKS];
  size_t b0 = 0;
  // Equal buckets whose ring segments line up (W divides the bucket) are
  // reduced by one launch per pass; each bucket keeps its own ring segments
  // and fold order, so the result is the same as one call per bucket.
  const size_t nfull = count / bucket_elems;
  if (nfull > 1 && bucket_elems % w == 0 && all_reduce_grid_ok(nranks, bucket_elems, nfull)) {
    if ((st = all_reduce_launch(sendbufs, recvbufs, nranks, bucket_elems, dtype, op, algo, stream, nfull)) !=
        RSX_SUCCESS)
      return st;
    b0 = nfull * bucket_elems;
  }
  while (b0 < count) {
    const size_t n = std::min(bucket_elems, count - b0);
    for (int r = 0; r < nranks; ++r) {
      src[r] = static_cast<const char*>(sendbufs[r]) + b0 * es;
      dst[r] = static_cast<char*>(recvbufs[r]) + b0 * es;
    }
    if ((st = all_reduce_launch(src, dst, nranks, n, dtype, op, algo, stream)) != RSX_SUCCESS) return st;
    b0 += n;
  }
  return RSX_SUCCESS;
}

rsx_status_t rsx_fuse_pack(const void* const* tensors, const size_t* counts, int ntensors,
                           void* fused, rsx_dtype_t dtype, hipStream_t stream) {
  return fuse_copy(tensors, counts, ntensors, fused, true, dtype, stream);
}

rsx_status_t rsx_fuse_unpack(const void* fused, void* const* tensors, const size_t* counts,
                             int ntensors, rsx_dtype_t dtype, hipStream_t stream) {
  return fuse_copy(tensors, counts, ntensors, fused, false, dtype, stream);
}

rsx_status_t rsx_fused_all_reduce(const void* const* sendtensors, void* const* recvtensors,
                                  const size_t* counts, int ntensors, int nranks,
                                  rsx_dtype_t dtype, rsx_op_t op, rsx_algo_t algo,
                                  hipStream_t stream) {
  if (nranks < 1 || nranks > RSX_MAX_RANKS || ntensors < 0) return RSX_ERR_INVALID_ARGUMENT;
  const size_t es = esize_of(dtype);
  if (es == 0) return RSX_ERR_INVALID_TYPE;
  if (!valid_op(op)) return RSX_ERR_INVALID_OP;
  if (algo != RSX_ALGO_RING && algo != RSX_ALGO_NAIVE && algo != RSX_ALGO_AUTO &&
      algo != RSX_ALGO_RING_FUSED && algo != RSX_ALGO_RING_SPLIT)
    return RSX_ERR_INVALID_ARGUMENT;
  if (algo == RSX_ALGO_RING_SPLIT) return RSX_ERR_UNSUPPORTED;
  if (ntensors > 0 && counts == nullptr) return RSX_ERR_INVALID_ARGUMENT;
  size_t total = 0;
  for (int i = 0; i < ntensors; ++i) {
    size_t b;
    if (!mul_ok(counts[i], es, &b) || total + counts[i] < total) return RSX_ERR_UNSUPPORTED;
    total += counts[i];
  }
  size_t total_bytes;
  if (!mul_ok(total, es, &total_bytes)) return RSX_ERR_UNSUPPORTED;
  if (total == 0) return RSX_SUCCESS;
  if (sendtensors == nullptr || recvtensors == nullptr) return RSX_ERR_INVALID_ARGUMENT;

  const int w = nranks;
  std::vector<Span> sends, recvs;
  bool in_place_all = true;
  for (int r = 0; r < w; ++r) {
    for (int i = 0; i < ntensors; ++i) {
      if (counts[i] == 0) continue;
      const void* sp = sendtensors[static_cast<size_t>(r) * ntensors + i];
      const void* rp = recvtensors[static_cast<size_t>(r) * ntensors + i];
      if (sp == nullptr || rp == nullptr) return RSX_ERR_INVALID_ARGUMENT;
      if (!elem_aligned(sp, es) || !elem_aligned(rp, es)) return RSX_ERR_INVALID_ARGUMENT;
      const Range sr = range_of(sp, counts[i] * es), rr = range_of(rp, counts[i] * es);
      if (wraps(sr) || wraps(rr)) return RSX_ERR_INVALID_ARGUMENT;
      sends.push_back({sr.lo, sr.hi, i});
      recvs.push_back({rr.lo, rr.hi, i});
      in_place_all = in_place_all && sp == rp;
    }
  }
  if (!list_aliasing_ok(sends, recvs)) return RSX_ERR_ALIASING;
  if (w == 1 && in_place_all && dtype != RSX_FLOAT32_HALF_WIRE) return RSX_SUCCESS;

  const bool naive = algo == RSX_ALGO_NAIVE || (algo == RSX_ALGO_AUTO && total_bytes <= RSX_NAIVE_MAX_BYTES);
  const uint64_t seg = naive ? total : (total + w - 1) / w;
  const uint64_t per = static_cast<uint64_t>(fold_units(w)) * kBlock;
  const int vl = static_cast<int>(kVecBytes / es);

  // In place, a tensor needs W pointer slots instead of 2W.
  const int slots = in_place_all ? w : 2 * w;
  ListArgs a;
  uint64_t tiles = 0;
  int ntens = 0;        // tensors in the current launch
  bool all_vec = true;  // every piece of the current launch takes the dwordx4 path
  auto reset = [&]() {
    memset(&a, 0, sizeof(a));
    a.rot = naive ? 0 : 1;
    a.in_place = in_place_all ? 1 : 0;
    tiles = 0;
    ntens = 0;
    all_vec = true;
  };
  auto flush = [&]() -> rsx_status_t {
    if (a.npieces == 0) return RSX_SUCCESS;
    a.tile_start[a.npieces] = static_cast<uint32_t>(tiles);
    const dim3 grid(static_cast<uint32_t>(xcd_grid(tiles)));
    const uint32_t lds = all_vec ? lds_for_cap(list_cap(w)) : 0u;
    const rsx_status_t st = hip_status(launch_list_by_type(dtype, op, w, a, grid, lds, stream));
    reset();
    return st;
  };
  reset();
  uint64_t off = 0;  // fused offset of tensor i
  for (int i = 0; i < ntensors; ++i) {
    const uint64_t c = counts[i];
    if (c == 0) continue;
    const uint32_t k0 = naive ? 0 : static_cast<uint32_t>(off / seg);
    const uint32_t k1 = naive ? 0 : static_cast<uint32_t>((off + c - 1) / seg);
    const uint32_t npc = k1 - k0 + 1;
    if ((ntens + 1) * slots > kListPtrs || a.npieces + npc > static_cast<uint32_t>(kListPieces)) {
      const rsx_status_t st = flush();
      if (st != RSX_SUCCESS) return st;
    }
    bool vec = true;
    for (int r = 0; r < w; ++r) {
      void* sp = const_cast<void*>(sendtensors[static_cast<size_t>(r) * ntensors + i]);
      void* rp = recvtensors[static_cast<size_t>(r) * ntensors + i];
      a.ptr[ntens * slots + r] = sp;
      if (!in_place_all) a.ptr[ntens * slots + w + r] = rp;
      vec = vec && aligned16(sp) && aligned16(rp);
    }
    all_vec = all_vec && vec;
    for (uint32_t k = k0; k <= k1; ++k) {
      ListPiece& pc = a.piece[a.npieces];
      const uint64_t slo = naive ? 0 : static_cast<uint64_t>(k) * seg;
      const uint64_t shi = naive ? total : std::min<uint64_t>(slo + seg, total);
      pc.lo = std::max(off, slo) - off;
      pc.hi = std::min(off + c, shi) - off;
      pc.tensor = static_cast<uint32_t>(ntens);
      pc.seg = static_cast<uint16_t>(k);
      pc.vec = vec ? 1 : 0;
      const uint64_t len = pc.hi - pc.lo;
      const uint64_t units = vec ? len / vl : len;
      const uint64_t nt = std::max<uint64_t>(1, (units + per - 1) / per);
      a.tile_start[a.npieces] = static_cast<uint32_t>(tiles);
      tiles += nt;
      if (tiles > 0x7ffffff0ull) return RSX_ERR_UNSUPPORTED;
      a.npieces += 1;
    }
    ntens += 1;
    off += c;
  }
  return flush();
}

int rsx_fusion_plan(const size_t* counts, const rsx_dtype_t* dtypes, int ntensors,
                    size_t threshold_bytes, int* group_end) {
  if (ntensors < 0) return -1;
  if (ntensors == 0) return 0;
  if (counts == nullptr || dtypes == nullptr || group_end == nullptr) return -1;
  for (int i = 0; i < ntensors; ++i)
    if (esize_of(dtypes[i]) == 0) return -1;
  // Bytes of tensor i, saturating (a tensor that large is a group of its own).
  auto bytes_of = [&](int i) {
    size_t b;
    return mul_ok(counts[i], esize_of(dtypes[i]), &b) ? b : SIZE_MAX;
  };
  int ngroups = 0;
  int i = 0;
  while (i < ntensors) {
    size_t total = bytes_of(i);
    int j = i + 1;
    while (j < ntensors && dtypes[j] == dtypes[i]) {
      const size_t b = bytes_of(j);
      if (b > threshold_bytes || total > threshold_bytes - b) break;
      total += b;
      ++j;
    }
    group_end[ngroups++] = j;
    i = j;
  }
  return ngroups;
}

size_t rsx_sparse_topk_count(size_t count, float fraction) {
  const float p = fraction * static_cast<float>(count);  // fp32 product, as on the page
  if (!(p > 0.0f)) return 0;
  const float c = ceilf(p);
  if (c >= 18446744073709551616.0f) return SIZE_MAX;
  return static_cast<size_t>(c);
}

size_t rsx_sparse_workspace_size(int nranks, size_t count, rsx_sparse_mode_t mode, int has_accum) {
  SparseLayout l;
  return sparse_layout(nranks, count, mode, has_accum != 0, &l) ? l.total : 0;
}

rsx_status_t rsx_sparse_all_reduce(const float* const* grads, float* const* accums,
                                   float* const* outs, int nranks, size_t count,
                                   rsx_sparse_mode_t mode, float threshold, size_t k,
                                   uint32_t* const* msg_idx, float* const* msg_val,
                                   size_t msg_capacity, uint32_t* nnz, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream) {
  SparseLayout l;
  const rsx_status_t st = sparse_check(grads, accums, outs, nranks, count, mode, k, msg_idx, msg_val,
                                       msg_capacity, nnz, workspace, workspace_bytes, false, &l);
  if (st != RSX_SUCCESS) return st;
  if (count == 0) return hip_status(launch_sparse_zero_nnz(nnz, nranks, stream));
  return sparse_launch(grads, accums, outs, nranks, count, mode, threshold, k, msg_idx, msg_val,
                       msg_capacity, nnz, workspace, l, stream);
}

rsx_status_t rsx_sparse_all_reduce_noalloc(const float* const* grads, float* const* accums,
                                           float* const* outs, int nranks, size_t count,
                                           rsx_sparse_mode_t mode, float threshold, size_t k,
                                           uint32_t* const* msg_idx, float* const* msg_val,
                                           size_t msg_capacity, uint32_t* nnz, hipStream_t stream) {
  SparseLayout l;
  rsx_status_t st = sparse_check(grads, accums, outs, nranks, count, mode, k, msg_idx, msg_val,
                                 msg_capacity, nnz, nullptr, 0, true, &l);
  if (st != RSX_SUCCESS) return st;
  if (count == 0) return hip_status(launch_sparse_zero_nnz(nnz, nranks, stream));
  if (l.total > RSX_SPARSE_SCRATCH_BYTES) return RSX_ERR_UNSUPPORTED;
  void* ws = nullptr;
  if ((st = scratch_of_current_device(&ws)) != RSX_SUCCESS) return st;
  return sparse_launch(grads, accums, outs, nranks, count, mode, threshold, k, msg_idx, msg_val,
                       msg_capacity, nnz, ws, l, stream);
}

size_t rsx_segment_begin(size_t count, int nranks, int k) {
  if (nranks < 1 || k < 0) return 0;
  const size_t seg = count / nranks + (count % nranks != 0);
  const size_t kk = static_cast<size_t>(k);
  if (seg != 0 && kk > count / seg) return count;
  return std::min(kk * seg, count);
}

size_t rsx_dtype_size(rsx_dtype_t dtype) { return esize_of(dtype); }

const char* rsx_status_string(rsx_status_t status) {
  switch (status) {
    case RSX_SUCCESS:
      return "success";
    case RSX_ERR_INVALID_ARGUMENT:
      return "invalid argument";
    case RSX_ERR_INVALID_TYPE:
      return "invalid data type";
    case RSX_ERR_INVALID_OP:
      return "invalid reduction operation";
    case RSX_ERR_UNSUPPORTED:
      return "unsupported size";
    case RSX_ERR_ALIASING:
      return "buffers overlap in an unsupported way";
    case RSX_ERR_HIP:
      return g_hip_error;
    default:
      return "unknown status";
  }
}

int rsx_version(void) { return RSX_VERSION; }

int rsx_set_occupancy_caps(int enable) {
  const int prev = t_caps ? 1 : 0;
  t_caps = enable != 0;
  return prev;
}

}  // extern "C"
