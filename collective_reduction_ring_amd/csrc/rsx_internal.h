// Internal launch interface between the C-ABI layer (rsx_abi.hip) and the
// kernel translation units.  Not installed; users include include/rsx.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rsx.h"

namespace rsx {

constexpr int kBlock = 256;        // threads per workgroup: 4 wave64s
constexpr int kVecBytes = 16;      // one dwordx4 per lane per source

// Fold kernel arguments, passed by value in the kernarg segment so every
// per-rank pointer is an SGPR load.
//
// The fold domain of one launch is `count` elements per rank, cut into
// `nseg` segments of `seg` elements: segment k = [min(k*seg,count),
// min((k+1)*seg,count)).  Segment k folds rank (k+rot)%W first, then the ranks
// after it in ring order, so rot=1 is the ring (the block a ring position
// starts at step 0 is the one owned by the position before it) and
// rot=0 with one segment is rank order.  A launch may cover several equal
// buckets of W segments each (nseg = buckets * W, each bucket its own ring).
// The reduce-scatter form stores element i of segment k at
// dst[k%W][i - (k%W)*seg]: each rank's own block with W segments, and with
// several buckets and dst[r] at block r of the first bucket, every block at
// its own offset in its rank's buffer.
//
// Workgroups: `tiles_per_seg` tiles per segment, `tiles_total` = nseg *
// tiles_per_seg in all, launched as a 1-D grid rounded up to a multiple of
// the XCD count (see xcd_tile).  Tile t lies in segment
// (t * tps_magic) >> tps_shift = t / tiles_per_seg (see split_magic).
struct FoldArgs {
  uint64_t count;
  uint64_t seg;
  uint32_t rot;
  uint32_t tiles_per_seg;
  uint32_t tiles_total;
  uint32_t tps_magic;
  uint32_t tps_shift;
  uint32_t pad_;
  const void* src[RSX_MAX_RANKS];
  void* dst[RSX_MAX_RANKS];
};

// Division of t < 2^31 by a fixed d in [1, 2^31) as a multiply and a shift:
// with l = ceil(log2 d) and m = ceil(2^(31+l) / d) < 2^32, the error term of
// t*m / 2^(31+l) against t/d is below t/2^(31+l) < 2^-l <= 1/d, too small to
// reach the next integer, so floor(t*m / 2^(31+l)) = floor(t/d).
inline void split_magic(uint32_t d, uint32_t* magic, uint32_t* shift) {
  uint32_t l = 0;
  while ((1ull << l) < d) ++l;
  *magic = static_cast<uint32_t>(((1ull << (31 + l)) + d - 1) / d);
  *shift = 31 + l;
}

// All-gather: dst[r][k*n + i] = src[k][i].  Tiles as in FoldArgs: piece k
// owns tiles [k*tiles_per_piece, (k+1)*tiles_per_piece).  A launch may cover
// several groups of W pieces laid out back to back (the in-place all-gathers
// of several equal buckets): piece k >= W is read from src[k mod W] +
// (k - k mod W)*n elements and written at k*n, so tiles_total / tiles_per_piece
// counts the pieces.
struct GatherArgs {
  const void* src[RSX_MAX_RANKS];
  void* dst[RSX_MAX_RANKS];
  uint64_t n;
  int world;
  uint32_t tiles_per_piece;
  uint32_t tiles_total;
  uint32_t tps_magic;
  uint32_t tps_shift;
};

// Pack / unpack batch: copies between tensors and running offsets of one
// fusion buffer.  Descriptor i holds tensor i's pointer and one word with
// the byte offset of its data in the fusion buffer (low 40 bits) and its
// first tile (high 24 bits); its length is the next descriptor's offset
// minus its own, so entry n is a sentinel holding the end offset and the
// tile total.  16 bytes per copy keep RSX_FUSE_BATCH copies in the 4 KiB of
// kernel arguments.  Tiles are whole 16-byte destination vectors, kBlock per
// tile; a tensor larger than a launch's tile budget is split into several
// descriptors by the host.
struct CopyDesc {
  void* tensor;
  uint64_t off_tile;
};
constexpr int kOffBits = 40;
constexpr uint64_t kOffMask = (1ull << kOffBits) - 1;
constexpr uint64_t kMaxCopyTiles = (1ull << (64 - kOffBits)) - 1;  // per launch
struct MultiCopyArgs {
  char* fused;
  uint32_t n;       // copies in this batch
  uint32_t unpack;  // 0: tensor -> fused; 1: fused -> tensor
  CopyDesc d[RSX_FUSE_BATCH + 1];
};
// Kernel arguments are limited to 4 KiB.
static_assert(sizeof(MultiCopyArgs) <= 4096, "pack/unpack batch must fit the kernel arguments");

// MI355X: 256 CUs in 8 XCDs, each XCD with its own L2.  Workgroups of one
// launch are handed to the XCDs round-robin by workgroup id.
constexpr uint32_t kXcds = 8;

// dwordx4 per lane per source in the fold kernels.  One, for every W: a lane
// already has W loads in flight, and on MI355X more resident waves with one
// vector each beat fewer waves with several (measured for W = 2, 4, 8, 16,
// reduce-scatter and all-reduce alike).
constexpr int fold_units(int /*world*/) { return 1; }

// Grid size for `tiles` tiles: a multiple of the XCD count.
inline uint64_t xcd_grid(uint64_t tiles) { return (tiles + kXcds - 1) / kXcds * kXcds; }

// Copy kernels: 16-byte units per thread per tile.  One, as in the fold
// kernels: a plain copy of 2 GiB runs at 6.5 TB/s with one vector per lane
// against 5.9 TB/s with four (both non-temporal).
constexpr int kCopyUnits = 1;

// Bytes before the first 16-byte-aligned destination byte, at most `bytes`.
inline uint64_t copy_head(const void* dst, uint64_t bytes) {
  const uint64_t h = (16 - (reinterpret_cast<uintptr_t>(dst) & 15u)) & 15u;
  return h < bytes ? h : bytes;
}
// Tiles of a copy: whole aligned destination vectors, kCopyUnits per lane.
inline uint64_t copy_tiles(const void* dst, uint64_t bytes) {
  const uint64_t vecs = (bytes - copy_head(dst, bytes)) / 16;
  const uint64_t per = static_cast<uint64_t>(kCopyUnits) * kBlock;
  return vecs == 0 ? 1 : (vecs + per - 1) / per;
}

// Tensor-list all-reduce: the result of packing every rank's tensor list
// back to back, all-reducing the W fused buffers and unpacking, computed on
// the tensors themselves.  Each launch carries up to kListPieces pieces; a
// piece is the part of one tensor that lies in one segment of the fused
// layout, so its fold order is uniform.
constexpr int kListPtrs = 288;   // pointer slots per launch, 2*W per tensor (W in place)
constexpr int kListPieces = 63;  // pieces per launch (the two limits fill the 4 KiB of kernel arguments)
struct ListPiece {
  uint64_t lo, hi;   // tensor-local element range
  uint32_t tensor;   // the tensor's pointers start at slot tensor * 2W (tensor * W in place)
  uint16_t seg;      // segment of the fused layout (fold starts at rank seg + rot)
  uint16_t vec;      // 1: all 2W buffers of the tensor are 16-byte aligned
};
struct ListArgs {
  uint32_t npieces;
  uint32_t rot;
  uint32_t in_place;  // 1: every destination is its own source; W slots per tensor
  uint32_t tile_start[kListPieces + 1];  // piece i owns tiles [tile_start[i], tile_start[i+1])
  ListPiece piece[kListPieces];
  // tensor t: sources of ranks 0..W-1 at slots [t*2W, t*2W + W), destinations
  // at [t*2W + W, t*2W + 2W); in place, sources only, at [t*W, t*W + W).
  void* ptr[kListPtrs];
};
static_assert(sizeof(ListArgs) <= 4096, "a tensor-list launch must fit the kernel arguments");

// Launchers, one per dtype translation unit.  `rs` selects the reduce-scatter
// store (block k to dst[k]) over the all-reduce store (every element to every
// dst[r]); `vec` selects the dwordx4 kernel.  Return the launch status.
hipError_t launch_fold_f32(int op, int world, bool rs, bool vec, int tpw, const FoldArgs& a, dim3 grid, uint32_t lds,
                           hipStream_t s);
hipError_t launch_fold_bf16(int op, int world, bool rs, bool vec, int tpw, const FoldArgs& a, dim3 grid, uint32_t lds,
                           hipStream_t s);
hipError_t launch_fold_i32(int op, int world, bool rs, bool vec, int tpw, const FoldArgs& a, dim3 grid, uint32_t lds,
                           hipStream_t s);
hipError_t launch_fold_f64(int op, int world, bool rs, bool vec, int tpw, const FoldArgs& a, dim3 grid, uint32_t lds,
                           hipStream_t s);
hipError_t launch_fold_f16(int op, int world, bool rs, bool vec, int tpw, const FoldArgs& a, dim3 grid, uint32_t lds,
                           hipStream_t s);
hipError_t launch_fold_i64(int op, int world, bool rs, bool vec, int tpw, const FoldArgs& a, dim3 grid, uint32_t lds,
                           hipStream_t s);
hipError_t launch_fold_u64(int op, int world, bool rs, bool vec, int tpw, const FoldArgs& a, dim3 grid, uint32_t lds,
                           hipStream_t s);
hipError_t launch_fold_i8(int op, int world, bool rs, bool vec, int tpw, const FoldArgs& a, dim3 grid, uint32_t lds,
                           hipStream_t s);
hipError_t launch_fold_f32h(int op, int world, bool rs, bool vec, int tpw, const FoldArgs& a, dim3 grid, uint32_t lds,
                            hipStream_t s);
hipError_t launch_list_f32(int op, int world, const ListArgs& a, dim3 grid, uint32_t lds, hipStream_t s);
hipError_t launch_list_bf16(int op, int world, const ListArgs& a, dim3 grid, uint32_t lds, hipStream_t s);
hipError_t launch_list_i32(int op, int world, const ListArgs& a, dim3 grid, uint32_t lds, hipStream_t s);
hipError_t launch_list_f64(int op, int world, const ListArgs& a, dim3 grid, uint32_t lds, hipStream_t s);
hipError_t launch_list_f16(int op, int world, const ListArgs& a, dim3 grid, uint32_t lds, hipStream_t s);
hipError_t launch_list_i64(int op, int world, const ListArgs& a, dim3 grid, uint32_t lds, hipStream_t s);
hipError_t launch_list_u64(int op, int world, const ListArgs& a, dim3 grid, uint32_t lds, hipStream_t s);
hipError_t launch_list_i8(int op, int world, const ListArgs& a, dim3 grid, uint32_t lds, hipStream_t s);
hipError_t launch_list_f32h(int op, int world, const ListArgs& a, dim3 grid, uint32_t lds, hipStream_t s);

// kind 0: element-wise, 1: whole 16-byte vectors, 2: pieces of whole dwords.
hipError_t launch_gather(int esize, int kind, int tpw, const GatherArgs& a, dim3 grid, uint32_t lds,
                         hipStream_t s);
hipError_t launch_multicopy(int esize, const MultiCopyArgs& a, uint32_t lds, hipStream_t s);

}  // namespace rsx
