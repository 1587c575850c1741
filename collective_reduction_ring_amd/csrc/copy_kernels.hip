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
// copies in its kernel arguments (16 bytes each); a workgroup finds its copy
// from the tile starts packed into the descriptors.  Offsets in the fusion
// buffer are back to back, so source and destination of one copy are often
// not 16-byte aligned relative to each other.  Every lane stores one aligned
// dwordx4.  When the matching source address is a multiple of 4 bytes (every
// fp32 / int32 / fp64 / int64 copy) the lane loads those 16 bytes with one
// dword-aligned dwordx4 load, which the buffer unit serves in every
// alignment mode; otherwise (2- and 1-byte elements at odd offsets) it
// assembles them from the two aligned source vectors they straddle
// (v_alignbyte).  Measured on the 200-tensor fusion workload (W = 4, four
// packs, one launch each): 164 us with the two-load assembly for every
// misaligned copy, 152 us with the dword-aligned load; the same copies with
// every destination padded to 16 bytes take 145 us.  Exchanging the
// straddled chunk through LDS instead was slower (175 us), and so was a wave
// shuffle.  Stores are non-temporal (plain stores cost 10%).
#include "mem.h"
#include "rsx_internal.h"

namespace rsx {

template <int ES>
struct Unit;
template <>
struct Unit<1> {
  using T = uint8_t;
};
template <>
struct Unit<2> {
  using T = uint16_t;
};
template <>
struct Unit<4> {
  using T = uint32_t;
};
template <>
struct Unit<8> {
  using T = uint64_t;
};

// ------------------------------------------------------------ all-gather

// TPW tiles per workgroup: with TPW = 2, a workgroup of 512 lanes copies two
// consecutive tiles, one per half (workgroup_tile).
template <int ES, bool VEC, int TPW>
__global__ __launch_bounds__(kBlock * TPW) void gather_kernel(const GatherArgs a) {
  using T = typename std::conditional<VEC, uint4, typename Unit<ES>::T>::type;
  constexpr int U = kCopyUnits;
  const uint32_t t = workgroup_tile<TPW>();
  if (t >= a.tiles_total) return;
  const uint32_t k = static_cast<uint32_t>((static_cast<uint64_t>(t) * a.tps_magic) >> a.tps_shift);
  const uint32_t tile = t - k * a.tiles_per_piece;
  const uint64_t nbytes = a.n * ES;
  const uint64_t nu = nbytes / sizeof(T);
  const uint64_t t0 = static_cast<uint64_t>(tile) * (U * kBlock);
  if (t0 >= nu) return;
  const uint32_t tid = TPW == 1 ? threadIdx.x : threadIdx.x % kBlock;
  // Piece k is block k mod W of group k div W (GatherArgs).
  const uint32_t world = static_cast<uint32_t>(a.world);
  const uint32_t kr = k < world ? k : k % world;
  const char* srcb = static_cast<const char*>(a.src[kr]) + static_cast<uint64_t>(k - kr) * nbytes;
  if constexpr (VEC) {
    // Whole 16-byte vectors; the descriptor range drops lanes past the piece.
    const uint32_t bytes = static_cast<uint32_t>(min<uint64_t>(U * kBlock, nu - t0)) * kVecBytes;
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(srcb + t0 * kVecBytes, bytes);
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = load_stream(rs, tid * kVecBytes, u * kBlock * kVecBytes);
    for (int r = 0; r < a.world; ++r) {
      char* base = static_cast<char*>(a.dst[r]) + k * nbytes;
      if (base == srcb) continue;  // in-place piece
      const __amdgpu_buffer_rsrc_t rd = make_rsrc(base + t0 * kVecBytes, bytes);
#pragma unroll
      for (int u = 0; u < U; ++u) store_b128<kStoreStream>(rd, tid * kVecBytes, u * kBlock * kVecBytes, v[u]);
    }
  } else {
    const bool full = t0 + U * kBlock <= nu;
    const T* src = reinterpret_cast<const T*>(srcb) + t0 + tid;
    T v[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (full || t0 + u * kBlock + tid < nu) v[u] = src[u * kBlock];
    for (int r = 0; r < a.world; ++r) {
      char* base = static_cast<char*>(a.dst[r]) + k * nbytes;
      if (base == srcb) continue;  // in-place piece
      T* dst = reinterpret_cast<T*>(base) + t0 + tid;
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (full || t0 + u * kBlock + tid < nu) dst[u * kBlock] = v[u];
    }
  }
}

// The all-gather of pieces of whole dwords that are not whole 16-byte
// vectors (16-byte-aligned buffers): piece k starts k * n elements into every
// destination, at an offset that is a multiple of 4 but not always of 16.
// The bytes before the piece's first 16-byte-aligned destination byte, and
// those after its last whole vector, are copied element by element by tile 0;
// the vectors between are read with dword-aligned dwordx4 loads (multi-dword
// buffer loads need only dword alignment) and stored aligned.  The
// descriptor range drops lanes past the last vector.
template <int ES, int TPW>
__global__ __launch_bounds__(kBlock * TPW) void gather_dword_kernel(const GatherArgs a) {
  using E = typename Unit<ES>::T;
  constexpr int U = kCopyUnits;
  const uint32_t t = workgroup_tile<TPW>();
  if (t >= a.tiles_total) return;
  const uint32_t k = static_cast<uint32_t>((static_cast<uint64_t>(t) * a.tps_magic) >> a.tps_shift);
  const uint32_t tile = t - k * a.tiles_per_piece;
  const uint64_t nbytes = a.n * ES;
  const uint64_t doff = static_cast<uint64_t>(k) * nbytes;  // the piece's offset in every destination
  const uint64_t h = min<uint64_t>((16u - (doff & 15u)) & 15u, nbytes);
  const uint64_t nu = (nbytes - h) / kVecBytes;
  const uint64_t t0 = static_cast<uint64_t>(tile) * (U * kBlock);
  const uint32_t tid = TPW == 1 ? threadIdx.x : threadIdx.x % kBlock;
  const uint32_t world = static_cast<uint32_t>(a.world);
  const uint32_t kr = k < world ? k : k % world;
  const char* srcb = static_cast<const char*>(a.src[kr]) + static_cast<uint64_t>(k - kr) * nbytes;
  if (t0 < nu) {
    const uint32_t bytes = static_cast<uint32_t>(min<uint64_t>(U * kBlock, nu - t0)) * kVecBytes;
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(srcb + h + t0 * kVecBytes, bytes);
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = load_stream(rs, tid * kVecBytes, u * kBlock * kVecBytes);
    for (int r = 0; r < a.world; ++r) {
      char* base = static_cast<char*>(a.dst[r]) + doff;
      if (base == srcb) continue;  // in-place piece
      const __amdgpu_buffer_rsrc_t rd = make_rsrc(base + h + t0 * kVecBytes, bytes);
#pragma unroll
      for (int u = 0; u < U; ++u) store_b128<kStoreStream>(rd, tid * kVecBytes, u * kBlock * kVecBytes, v[u]);
    }
  }
  if (tile == 0) {
    const uint32_t nh = static_cast<uint32_t>(h / ES);
    const uint64_t tail = h + nu * kVecBytes;
    const uint32_t nt = static_cast<uint32_t>((nbytes - tail) / ES);
    if (tid < nh + nt) {
      const uint64_t e = tid < nh ? tid : tail / ES + (tid - nh);
      const E v = reinterpret_cast<const E*>(srcb)[e];
      for (int r = 0; r < a.world; ++r) {
        char* base = static_cast<char*>(a.dst[r]) + doff;
        if (base == srcb) continue;
        reinterpret_cast<E*>(base)[e] = v;
      }
    }
  }
}

// kind 0: element-wise; 1: whole 16-byte vectors; 2: pieces of whole
// dwords (gather_dword_kernel).  Two tiles per workgroup exist for kinds 1
// and 2.
hipError_t launch_gather(int esize, int kind, int tpw, const GatherArgs& a, dim3 grid, uint32_t lds,
                         hipStream_t s) {
  void* args[] = {const_cast<GatherArgs*>(&a)};
  if (kind < 0 || kind > 2 || (tpw != 1 && !(tpw == 2 && kind != 0))) return hipErrorInvalidValue;
  const void* fn;
  switch (esize) {
#define RSX_ES(n)                                                                                   \
  case n:                                                                                           \
    fn = kind == 0   ? reinterpret_cast<const void*>(&gather_kernel<n, false, 1>)                   \
         : kind == 1 ? (tpw == 2 ? reinterpret_cast<const void*>(&gather_kernel<n, true, 2>)        \
                                 : reinterpret_cast<const void*>(&gather_kernel<n, true, 1>))       \
                     : (tpw == 2 ? reinterpret_cast<const void*>(&gather_dword_kernel<n, 2>)        \
                                 : reinterpret_cast<const void*>(&gather_dword_kernel<n, 1>));      \
    break;
    RSX_ES(1) RSX_ES(2) RSX_ES(4) RSX_ES(8)
#undef RSX_ES
    default:
      return hipErrorInvalidValue;
  }
  return hipLaunchKernel(fn, grid, dim3(kBlock * tpw), args, lds, s);
}

// -------------------------------------------------------- pack / unpack

// Bytes [delta, delta + 16) of the 32-byte concatenation lo:hi, delta in
// [1, 15] (Q = delta / 4 whole words, then r bytes).
template <int Q>
__device__ __forceinline__ uint4 funnel_q(const uint32_t (&w)[8], uint32_t r) {
  return make_uint4(__builtin_amdgcn_alignbyte(w[Q + 1], w[Q], r),
                    __builtin_amdgcn_alignbyte(w[Q + 2], w[Q + 1], r),
                    __builtin_amdgcn_alignbyte(w[Q + 3], w[Q + 2], r),
                    __builtin_amdgcn_alignbyte(w[Q + 4], w[Q + 3], r));
}

__device__ __forceinline__ uint4 funnel(const uint4& lo, const uint4& hi, uint32_t delta) {
  const uint32_t w[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
  const uint32_t r = delta & 3u;
  switch (delta >> 2) {  // uniform per copy
    case 0:
      return funnel_q<0>(w, r);
    case 1:
      return funnel_q<1>(w, r);
    case 2:
      return funnel_q<2>(w, r);
    default:
      return funnel_q<3>(w, r);
  }
}

template <int ES>
__global__ __launch_bounds__(kBlock) void multicopy_kernel(const MultiCopyArgs a) {
  using E = typename Unit<ES>::T;
  constexpr int U = kCopyUnits;
  const uint32_t t = xcd_tile(blockIdx.x, gridDim.x);
  const uint32_t nd = a.n;
  if (t >= static_cast<uint32_t>(a.d[nd].off_tile >> kOffBits)) return;
  // Copy of this tile: the last i with tile_start(i) <= t.
  uint32_t lo = 0, hi = nd - 1;
  while (lo < hi) {
    const uint32_t mid = (lo + hi + 1) / 2;
    if (static_cast<uint32_t>(a.d[mid].off_tile >> kOffBits) <= t) lo = mid; else hi = mid - 1;
  }
  const uint64_t w0 = a.d[lo].off_tile;
  const uint64_t off = w0 & kOffMask;
  const uint64_t n = (a.d[lo + 1].off_tile & kOffMask) - off;
  char* const fz = a.fused + off;
  char* const tensor = static_cast<char*>(a.d[lo].tensor);
  const char* s = a.unpack ? fz : tensor;
  char* o = a.unpack ? tensor : fz;
  const uint32_t tile = t - static_cast<uint32_t>(w0 >> kOffBits);
  const uint32_t tid = threadIdx.x;

  // [0, h): head bytes up to the first aligned destination byte;
  // [h, h + 16 m): m aligned destination vectors; then a tail below 16 bytes.
  const uint64_t h = min<uint64_t>((16u - (reinterpret_cast<uintptr_t>(o) & 15u)) & 15u, n);
  const uint64_t m = (n - h) / 16;
  const uint64_t j0 = static_cast<uint64_t>(tile) * (U * kBlock);
  if (j0 < m) {
    const uint32_t nvt = static_cast<uint32_t>(min<uint64_t>(U * kBlock, m - j0));
    const char* s1 = s + h + 16 * j0;
    char* o1 = o + h + 16 * j0;
    const uint32_t delta = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(s1) & 15u);
    const __amdgpu_buffer_rsrc_t rd = make_rsrc(o1, nvt * 16);
    uint4 v[U];
    if ((delta & 3u) == 0) {
      // 16-byte or dword-aligned source: one load per vector.
      const __amdgpu_buffer_rsrc_t rs = make_rsrc(s1, nvt * 16);
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = load_stream(rs, tid * 16, u * kBlock * 16);
    } else {
      // The aligned 16-byte source chunks overlapping this tile's bytes:
      // nvt + 1 of them, starting delta bytes before s1.  They lie in the
      // pages of the source bytes, and the descriptor range ends with them.
      const __amdgpu_buffer_rsrc_t rs = make_rsrc(s1 - delta, (nvt + 1) * 16);
      uint4 x0[U], x1[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        x0[u] = load_stream(rs, tid * 16, u * kBlock * 16);
        x1[u] = load_stream(rs, tid * 16 + 16, u * kBlock * 16);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = funnel(x0[u], x1[u], delta);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) store_b128<kStoreStream>(rd, tid * 16, u * kBlock * 16, v[u]);
  }
  if (tile == 0) {
    // Head and tail elements (every pointer is element-aligned, so h and the
    // tail are whole elements).
    const uint32_t nh = static_cast<uint32_t>(h / ES);
    const uint32_t nt = static_cast<uint32_t>((n - h - 16 * m) / ES);
    if (tid < nh) {
      reinterpret_cast<E*>(o)[tid] = reinterpret_cast<const E*>(s)[tid];
    } else if (tid < nh + nt) {
      const uint64_t toff = h + 16 * m;
      reinterpret_cast<E*>(o + toff)[tid - nh] = reinterpret_cast<const E*>(s + toff)[tid - nh];
    }
  }
}

hipError_t launch_multicopy(int esize, const MultiCopyArgs& a, uint32_t lds, hipStream_t s) {
  void* args[] = {const_cast<MultiCopyArgs*>(&a)};
  const void* fn;
  switch (esize) {
    case 1:
      fn = reinterpret_cast<const void*>(&multicopy_kernel<1>);
      break;
    case 2:
      fn = reinterpret_cast<const void*>(&multicopy_kernel<2>);
      break;
    case 4:
      fn = reinterpret_cast<const void*>(&multicopy_kernel<4>);
      break;
    case 8:
      fn = reinterpret_cast<const void*>(&multicopy_kernel<8>);
      break;
    default:
      return hipErrorInvalidValue;
  }
  const uint64_t tiles = a.d[a.n].off_tile >> kOffBits;
  return hipLaunchKernel(fn, dim3(static_cast<uint32_t>(xcd_grid(tiles))), dim3(kBlock), args, lds, s);
}

}  // namespace rsx
