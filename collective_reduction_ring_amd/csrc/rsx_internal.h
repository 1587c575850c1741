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
// rot=0 with one segment is rank order.
//
// Workgroups: `tiles_per_seg` tiles per segment, `tiles_total` = nseg *
// tiles_per_seg in all, launched as a 1-D grid rounded up to a multiple of
// the XCD count (see xcd_tile).
struct FoldArgs {
  const void* src[RSX_MAX_RANKS];
  void* dst[RSX_MAX_RANKS];
  uint64_t count;
  uint64_t seg;
  uint32_t rot;
  uint32_t tiles_per_seg;
  uint32_t tiles_total;
};

// All-gather: dst[r][k*n + i] = src[k][i].
struct GatherArgs {
  const void* src[RSX_MAX_RANKS];
  void* dst[RSX_MAX_RANKS];
  uint64_t n;
  int world;
};

// One copy of a pack/unpack batch.  `path` is chosen on the host from the
// relative alignment of src and dst: 0 = dwordx4 body with element-size head
// and tail, 1 = dword body, 2 = element-size (2-byte) copies.
struct CopyDesc {
  const void* src;
  void* dst;
  uint64_t bytes;
  uint32_t path;
  uint32_t tiles;
};

struct MultiCopyArgs {
  CopyDesc d[RSX_FUSE_BATCH];
  uint32_t tile_start[RSX_FUSE_BATCH + 1];
  int n;
};

// MI355X: 256 CUs in 8 XCDs, each XCD with its own L2.  Workgroups of one
// launch are handed to the XCDs round-robin by workgroup id.
constexpr uint32_t kXcds = 8;

// dwordx4 per lane per source in the fold kernels, by rank count: with W
// sources a lane already has W loads in flight; fewer sources get more units.
constexpr int fold_units(int world) { return world <= 2 ? 4 : world <= 4 ? 2 : 1; }

// Grid size for `tiles` tiles: a multiple of the XCD count.
inline uint64_t xcd_grid(uint64_t tiles) { return (tiles + kXcds - 1) / kXcds * kXcds; }

// Copy kernels: 16-byte units per thread per tile.
constexpr int kCopyUnits = 4;

// Launchers, one per dtype translation unit.  `rs` selects the reduce-scatter
// store (block k to dst[k]) over the all-reduce store (every element to every
// dst[r]); `vec` selects the dwordx4 kernel.  Return the launch status.
hipError_t launch_fold_f32(int op, int world, bool rs, bool vec, const FoldArgs& a,
                           dim3 grid, hipStream_t s);
hipError_t launch_fold_bf16(int op, int world, bool rs, bool vec, const FoldArgs& a,
                            dim3 grid, hipStream_t s);
hipError_t launch_fold_i32(int op, int world, bool rs, bool vec, const FoldArgs& a,
                           dim3 grid, hipStream_t s);

hipError_t launch_gather(int esize, bool vec, const GatherArgs& a, dim3 grid, hipStream_t s);
hipError_t launch_multicopy(int esize, const MultiCopyArgs& a, uint32_t blocks, hipStream_t s);

}  // namespace rsx
