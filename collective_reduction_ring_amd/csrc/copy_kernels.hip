// Copy kernels: the all-gather fan-out and the tensor-fusion pack/unpack.
//
// All-gather ("Distributed primitives": every node ends with every node's
// piece) reads piece k once and stores it into all W receive buffers, so its
// HBM traffic is W*n reads' worth of input plus W*W*n of output, the least the
// definition allows.
//
// Pack/unpack (Apache SINGA communicator.cc fusedSynch; Horovod
// operations.cc PerformOperation) copy many tensors to or from running
// offsets of one fusion buffer.  One launch carries up to RSX_FUSE_BATCH
// (src, dst, bytes) descriptors in its kernel arguments; workgroup b finds its
// descriptor from the prefix sums of per-descriptor tile counts.  Offsets in
// the fusion buffer are back to back, so a descriptor's src and dst need not
// share 16-byte alignment: the host picks the widest unit both allow.
#include "rsx_internal.h"

namespace rsx {

template <int ES>
struct Unit;
template <>
struct Unit<2> {
  using T = uint16_t;
};
template <>
struct Unit<4> {
  using T = uint32_t;
};

// ------------------------------------------------------------ all-gather

template <int ES, bool VEC>
__global__ __launch_bounds__(kBlock) void gather_kernel(const GatherArgs a) {
  using T = typename std::conditional<VEC, uint4, typename Unit<ES>::T>::type;
  constexpr int U = kCopyUnits;
  const uint32_t k = blockIdx.y;
  const uint64_t nbytes = a.n * ES;
  const uint64_t nu = nbytes / sizeof(T);
  const uint64_t t0 = static_cast<uint64_t>(blockIdx.x) * (U * kBlock);
  if (t0 >= nu) return;
  const bool full = t0 + U * kBlock <= nu;
  const uint32_t tid = threadIdx.x;
  const T* src = static_cast<const T*>(a.src[k]) + t0 + tid;
  T v[U];
#pragma unroll
  for (int u = 0; u < U; ++u)
    if (full || t0 + u * kBlock + tid < nu) v[u] = src[u * kBlock];
  for (int r = 0; r < a.world; ++r) {
    char* base = static_cast<char*>(a.dst[r]) + k * nbytes;
    if (base == static_cast<const char*>(a.src[k])) continue;  // in-place piece
    T* dst = reinterpret_cast<T*>(base) + t0 + tid;
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (full || t0 + u * kBlock + tid < nu) dst[u * kBlock] = v[u];
  }
}

hipError_t launch_gather(int esize, bool vec, const GatherArgs& a, dim3 grid, hipStream_t s) {
  void* args[] = {const_cast<GatherArgs*>(&a)};
  const void* fn;
  if (esize == 2) {
    fn = vec ? reinterpret_cast<const void*>(&gather_kernel<2, true>)
             : reinterpret_cast<const void*>(&gather_kernel<2, false>);
  } else if (esize == 4) {
    fn = vec ? reinterpret_cast<const void*>(&gather_kernel<4, true>)
             : reinterpret_cast<const void*>(&gather_kernel<4, false>);
  } else {
    return hipErrorInvalidValue;
  }
  return hipLaunchKernel(fn, grid, dim3(kBlock), args, 0, s);
}

// -------------------------------------------------------- pack / unpack

// Copy `n` units of type T from s to d, tile `t` of U*256 units.
template <class T>
__device__ __forceinline__ void copy_tile(const T* s, T* d, uint64_t n, uint32_t t) {
  constexpr int U = kCopyUnits;
  const uint64_t t0 = static_cast<uint64_t>(t) * (U * kBlock);
  if (t0 >= n) return;
  const bool full = t0 + U * kBlock <= n;
  const uint32_t tid = threadIdx.x;
  T v[U];
#pragma unroll
  for (int u = 0; u < U; ++u)
    if (full || t0 + u * kBlock + tid < n) v[u] = s[t0 + u * kBlock + tid];
#pragma unroll
  for (int u = 0; u < U; ++u)
    if (full || t0 + u * kBlock + tid < n) d[t0 + u * kBlock + tid] = v[u];
}

// Copy a body of `W`-byte units aligned on both sides, with an element-size
// head and tail; tile 0 of the descriptor also copies the head and tail.
template <int ES, class W>
__device__ __forceinline__ void copy_aligned(const char* s, char* d, uint64_t bytes, uint32_t t) {
  using E = typename Unit<ES>::T;
  constexpr uint64_t WB = sizeof(W);
  const uint64_t head = min((WB - (reinterpret_cast<uintptr_t>(s) & (WB - 1))) & (WB - 1), bytes);
  const uint64_t body = (bytes - head) / WB;
  const uint64_t tail = bytes - head - body * WB;
  copy_tile<W>(reinterpret_cast<const W*>(s + head), reinterpret_cast<W*>(d + head), body, t);
  if (t == 0) {
    const uint32_t nh = static_cast<uint32_t>(head / ES);
    const uint32_t nt = static_cast<uint32_t>(tail / ES);
    const uint32_t tid = threadIdx.x;
    if (tid < nh) {
      reinterpret_cast<E*>(d)[tid] = reinterpret_cast<const E*>(s)[tid];
    } else if (tid < nh + nt) {
      const uint64_t off = head + body * WB;
      reinterpret_cast<E*>(d + off)[tid - nh] = reinterpret_cast<const E*>(s + off)[tid - nh];
    }
  }
}

template <int ES>
__global__ __launch_bounds__(kBlock) void multicopy_kernel(const MultiCopyArgs a) {
  // Descriptor of this workgroup: the last i with tile_start[i] <= blockIdx.x.
  const uint32_t b = blockIdx.x;
  int lo = 0, hi = a.n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) / 2;
    if (a.tile_start[mid] <= b) lo = mid; else hi = mid - 1;
  }
  const CopyDesc& d = a.d[lo];
  const uint32_t t = b - a.tile_start[lo];
  const char* s = static_cast<const char*>(d.src);
  char* o = static_cast<char*>(d.dst);
  if (d.path == 0) {
    copy_aligned<ES, uint4>(s, o, d.bytes, t);
  } else if (d.path == 1) {
    copy_aligned<ES, uint32_t>(s, o, d.bytes, t);
  } else {
    using E = typename Unit<ES>::T;
    copy_tile<E>(reinterpret_cast<const E*>(s), reinterpret_cast<E*>(o), d.bytes / ES, t);
  }
}

hipError_t launch_multicopy(int esize, const MultiCopyArgs& a, uint32_t blocks, hipStream_t s) {
  void* args[] = {const_cast<MultiCopyArgs*>(&a)};
  const void* fn;
  if (esize == 2) {
    fn = reinterpret_cast<const void*>(&multicopy_kernel<2>);
  } else if (esize == 4) {
    fn = reinterpret_cast<const void*>(&multicopy_kernel<4>);
  } else {
    return hipErrorInvalidValue;
  }
  return hipLaunchKernel(fn, dim3(blocks), dim3(kBlock), args, 0, s);
}

}  // namespace rsx
