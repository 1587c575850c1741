// Memory-access helpers for gfx950 streaming kernels.
//
// Buffer resource descriptors give every workgroup a byte range checked by
// the hardware: a dwordx4 lane whose offset lies outside the range loads
// zeros and its store is dropped, so the ragged last tile of a segment needs
// no per-lane predicate.  Loads carry the non-temporal hint (the data is
// read exactly once, so it should not displace anything in L2 or the MALL).
// Stores take one of two hints, by how much a kernel writes: a small output
// (a reduce-scatter writes 1/W of what it reads) is written with the sc1
// scope bit, through the XCD-private L2 into the memory-side cache, while a
// large one (an all-reduce writes as much as it reads, far more than the
// 256 MB MALL) streams past the caches with the non-temporal hint.  Measured
// on MI355X, each choice is the faster one for its kernel.  The hints change
// speed only, never results.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rsx_internal.h"

namespace rsx {

// `aux` cache-policy operand of the buffer intrinsics on gfx950:
// bit 0 = sc0, bit 1 = nt, bit 4 = sc1.
constexpr int kLoadStream = 2;      // nt
constexpr int kStoreThrough = 16;   // sc1
constexpr int kStoreStream = 2;     // nt
// Descriptor word 3 of a raw (stride 0, untyped) buffer: 32-bit data format.
constexpr int kRawBufferWord3 = 0x00020000;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Tile run by workgroup `b` of an `nblocks` grid (a multiple of kXcds):
// workgroup b lands on XCD b % 8, and the workgroups of one XCD take one
// contiguous range of tiles, so each XCD streams through its own contiguous
// region of every buffer (fewer pages per XCD translation cache, whole DRAM
// rows per XCD).
__device__ __forceinline__ uint32_t xcd_tile(uint32_t b, uint32_t nblocks) {
  const uint32_t per = nblocks / kXcds;
  return (b % kXcds) * per + b / kXcds;
}

// Tile of this wave's half of the workgroup when a workgroup of TPW * 256
// lanes runs TPW consecutive tiles of 256 lanes (workgroup b takes tiles
// TPW * xcd_tile(b) ..., so each XCD's region stays contiguous).  The half
// index is the same for all 64 lanes of a wave; readfirstlane makes that
// explicit, so the tile and everything derived from it stay scalar.
template <int TPW>
__device__ __forceinline__ uint32_t workgroup_tile() {
  const uint32_t base = xcd_tile(blockIdx.x, gridDim.x) * TPW;
  if constexpr (TPW == 1) {
    return base;
  } else {
    return base + static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x / 256u)));
  }
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes),
                                           kRawBufferWord3);
}

__device__ __forceinline__ uint4 load_stream(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kLoadStream);
  return make_uint4(v.x, v.y, v.z, v.w);
}

template <int AUX>
__device__ __forceinline__ void store_b128(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                           const uint4& v) {
  const u32x4 w = {v.x, v.y, v.z, v.w};
  __builtin_amdgcn_raw_buffer_store_b128(w, r, voff, soff, AUX);
}

}  // namespace rsx
