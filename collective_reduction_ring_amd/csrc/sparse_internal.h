// Internal launch interface of the sparsified all-reduce, between the C-ABI
// layer (rsx_abi.hip) and sparse_kernels.hip.  Not installed.
#pragma once

#include "rsx_internal.h"

namespace rsx {

// ------------------------------------------------ sparsified all-reduce
//
// Apache SINGA communicator.cc, valSparsAllReduce / topKSparsAllReduce: each
// rank sparsifies its gradient (plus an optional error-feedback
// accumulation) into an (index, value) message, and every rank adds all
// messages, rank 0 first, into a zeroed buffer.  Every kernel below covers
// the W ranks of one call in one launch.  Ranks are cut into tiles of
// kSpTile elements; the compaction writes a tile's selected entries in index
// order into a slot of its own, so the combine finds the entries of an output
// tile in every rank's slot, without a search, and places them in the
// message at offsets scanned in between.
constexpr uint32_t kSpTile = 4096;      // elements per tile: 1024 lanes x 1 dwordx4
constexpr uint32_t kSpUnits = 1;        // dwordx4 per lane per tile
constexpr uint32_t kSpTileBlock = kSpTile / (4 * kSpUnits);  // lanes of the per-tile kernels
constexpr uint32_t kSpBins = 2048;      // radix-select histogram bins (11-bit digits)
constexpr uint32_t kSpScanBlock = 1024; // threads of the per-rank offset scan

// Per-rank selection state, kSpState words per rank.  The radix search
// records its cut after each pass in a field of its own, so that the pass
// that computes it never overwrites what its other workgroups read.
enum : uint32_t {
  kStCut = 0,       // top-K: the K-th largest key (after the last pass)
  kStNeed = 1,      // top-K: entries still to take at the cut
  kStBound = 2,     // top-K: every key at or above it is gathered into the slots
  kStCand = 3,      // top-K: candidates the first gather found (fewer than K: the exact fallback runs)
  kStGuess = 4,     // top-K: keys at or above it get the sent-entry residual at the gather
  kStCut0 = 5,      // top-K: the cut's prefix after the first digit
  kStNeed0 = 6,     //        and the entries still to take below it
  kStCut1 = 7,      // top-K: the same after the second digit
  kStNeed1 = 8,
  kSpState = 16
};
// Histograms, kSpBins words per rank each: the three slot passes' and the
// fallback's (kHistFallback), [kHistCount][W][kSpBins].
constexpr uint32_t kHistFallback = 3;
constexpr uint32_t kHistCount = 4;

struct SparseArgs {
  const float* grad[RSX_MAX_RANKS];
  float* accum[RSX_MAX_RANKS];       // error-feedback buffers (read, then the residual)
  float* out[RSX_MAX_RANKS];
  uint32_t* msg_idx[RSX_MAX_RANKS];
  float* msg_val[RSX_MAX_RANKS];
  uint32_t* nnz;                     // [W] message lengths
  uint32_t* tile_slot;               // [W][tiles + 1] per tile: entries in its slot
  uint32_t* tile_cnt;                // [W][tiles + 1] per tile: entries sent for sure
  uint32_t* tile_eqc;                // [W][tiles + 1] per tile: ties with the cut (top-K)
  uint32_t* tile_off;                // [W][tiles + 1] per tile: offset in the message
  uint32_t* tile_eqb;                // [W][tiles + 1] per tile: ties in earlier tiles
  uint32_t* gap_idx;                 // [W][tiles][kSpTile] one slot of entries per tile:
  float* gap_val;                    //   (tile-local index, g value)
  uint32_t* hist;                    // [kHistCount][W][kSpBins]
  uint32_t* state;                   // [W][kSpState]: kSt* fields
  uint64_t count;                    // elements per rank
  uint32_t tiles;                    // tiles per rank
  uint32_t world;
  uint32_t k;                        // top-K: entries per rank
  uint32_t cap;                      // message entries that may be written: count or k
  float threshold;                   // threshold mode: |x| >= threshold is sent
  uint32_t hist_groups;              // histogram workgroups per rank
  uint32_t hist_chunk;               // tiles per histogram workgroup
};

// Enqueue the whole sparsified all-reduce.  `mode` is rsx_sparse_mode_t.
hipError_t launch_sparse(const SparseArgs& a, int mode, bool has_accum, hipStream_t s);
// nnz[r] = 0 for r < world (a call with count 0).
hipError_t launch_sparse_zero_nnz(uint32_t* nnz, int world, hipStream_t s);

}  // namespace rsx
