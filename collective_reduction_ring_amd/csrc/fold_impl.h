// Ring-order fold kernels: reduce-scatter, all-reduce (reduce-scatter and
// all-gather in one pass) and the naive all-reduce, for one element type.
//
// What is computed (NCCL 1.x src/reduce_scatter.cu, the ring kernel and
// GetBlock; "Distributed primitives", Ring AllReduce): block k of the result
// is the fold of every rank's block k, starting from the rank after k and
// going round the ring to rank k.  On W GPUs that fold is spread over W steps,
// each GPU adding its own input to the partial it received and passing it on.
// Here the W ranks are W buffers of one GPU, so a lane loads element i of
// block k from all W buffers and folds them in registers in the same order:
// the partial never leaves the register file, the flags and the staging
// buffers of the multi-GPU kernel have nothing left to guard, and HBM sees
// each input once and each output once.
//
// Layout of one launch: a 1-D grid of tiles of U * 256 dwordx4 (or
// elements, for the unaligned kernel), segment-major, mapped XCD-contiguous
// (xcd_tile).  A workgroup works inside one segment k, so the ring rotation
// and the W source pointers are scalar.  A lane issues all W*U loads before
// the first combine.
#pragma once

#include <type_traits>

#include "mem.h"
#include "rsx_internal.h"

namespace rsx {

// ------------------------------------------------------------ element types

struct F32T {
  using S = float;   // storage
  using A = float;   // accumulation
  static constexpr int kVL = 4;  // elements per dwordx4
};
struct I32T {
  using S = int32_t;
  using A = int32_t;
  static constexpr int kVL = 4;
};
struct BF16T {
  using S = uint16_t;
  using A = float;
  static constexpr int kVL = 8;
};
struct F64T {
  using S = double;
  using A = double;
  static constexpr int kVL = 2;
};
struct F16T {
  using S = uint16_t;  // IEEE half bit patterns
  using A = _Float16;  // the ring partial stays half (the page's T-typed ring buffers)
  static constexpr int kVL = 8;
};
struct I64T {
  using S = int64_t;
  using A = int64_t;
  static constexpr int kVL = 2;
};
struct U64T {
  using S = uint64_t;
  using A = uint64_t;
  static constexpr int kVL = 2;
};
struct I8T {
  using S = int8_t;
  using A = int8_t;
  static constexpr int kVL = 16;
};
// fp32 data with IEEE half as the wire format (Apache SINGA communicator.cc,
// synchHalf / fusedSynchHalf: float2half, a half all-reduce, half2float).
struct F32HT {
  using S = float;
  using A = _Float16;
  static constexpr int kVL = 4;
};

// bf16 -> fp32 is exact: the bf16 bits are the top half of the fp32 bits.
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// fp32 -> bf16, round to nearest, ties to even; a NaN becomes the quiet NaN
// with the sign kept.  Overflow goes to +-inf, as the rounding rule gives.
// Written as a select, not an early return, so it compiles to a compare and
// a v_cndmask instead of a branch per element.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t rounded = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
  const uint32_t quiet_nan = ((u >> 16) & 0x8000u) | 0x7fc0u;
  return (u & 0x7fffffffu) > 0x7f800000u ? quiet_nan : rounded;
}

template <class D>
struct Elem;

template <>
struct Elem<F32T> {
  __device__ static float widen(float x) { return x; }
  __device__ static float narrow(float a) { return a; }
  __device__ static void unpack(const uint4& v, float (&a)[4]) {
    a[0] = __uint_as_float(v.x);
    a[1] = __uint_as_float(v.y);
    a[2] = __uint_as_float(v.z);
    a[3] = __uint_as_float(v.w);
  }
  __device__ static uint4 pack(const float (&a)[4]) {
    return make_uint4(__float_as_uint(a[0]), __float_as_uint(a[1]), __float_as_uint(a[2]),
                      __float_as_uint(a[3]));
  }
};

template <>
struct Elem<I32T> {
  __device__ static int32_t widen(int32_t x) { return x; }
  __device__ static int32_t narrow(int32_t a) { return a; }
  __device__ static void unpack(const uint4& v, int32_t (&a)[4]) {
    a[0] = static_cast<int32_t>(v.x);
    a[1] = static_cast<int32_t>(v.y);
    a[2] = static_cast<int32_t>(v.z);
    a[3] = static_cast<int32_t>(v.w);
  }
  __device__ static uint4 pack(const int32_t (&a)[4]) {
    return make_uint4(static_cast<uint32_t>(a[0]), static_cast<uint32_t>(a[1]),
                      static_cast<uint32_t>(a[2]), static_cast<uint32_t>(a[3]));
  }
};

template <>
struct Elem<BF16T> {
  __device__ static float widen(uint16_t h) { return bf16_bits_to_f32(h); }
  __device__ static uint16_t narrow(float a) { return static_cast<uint16_t>(f32_to_bf16_bits(a)); }
  __device__ static void unpack_word(uint32_t w, float& lo, float& hi) {
    lo = __uint_as_float(w << 16);
    hi = __uint_as_float(w & 0xffff0000u);
  }
  __device__ static void unpack(const uint4& v, float (&a)[8]) {
    unpack_word(v.x, a[0], a[1]);
    unpack_word(v.y, a[2], a[3]);
    unpack_word(v.z, a[4], a[5]);
    unpack_word(v.w, a[6], a[7]);
  }
  __device__ static uint32_t pack_word(float lo, float hi) {
    return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
  }
  __device__ static uint4 pack(const float (&a)[8]) {
    return make_uint4(pack_word(a[0], a[1]), pack_word(a[2], a[3]), pack_word(a[4], a[5]),
                      pack_word(a[6], a[7]));
  }
};

// 64-bit elements: two per dwordx4, low word first.
template <class T>
struct Elem64 {
  __device__ static T widen(T x) { return x; }
  __device__ static T narrow(T a) { return a; }
  __device__ static void unpack(const uint4& v, T (&a)[2]) {
    a[0] = __builtin_bit_cast(T, (static_cast<uint64_t>(v.y) << 32) | v.x);
    a[1] = __builtin_bit_cast(T, (static_cast<uint64_t>(v.w) << 32) | v.z);
  }
  __device__ static uint4 pack(const T (&a)[2]) {
    const uint64_t lo = __builtin_bit_cast(uint64_t, a[0]), hi = __builtin_bit_cast(uint64_t, a[1]);
    return make_uint4(static_cast<uint32_t>(lo), static_cast<uint32_t>(lo >> 32),
                      static_cast<uint32_t>(hi), static_cast<uint32_t>(hi >> 32));
  }
};
template <>
struct Elem<F64T> : Elem64<double> {};
template <>
struct Elem<I64T> : Elem64<int64_t> {};
template <>
struct Elem<U64T> : Elem64<uint64_t> {};

// IEEE half, folded in half: every combine is one native half operation
// (v_add_f16 / v_mul_f16, IEEE and correctly rounded, denormals kept), so the
// partial is a half after every ring step, as it is in the NCCL ring, whose
// buffers between steps hold the element type (ReduceScatterKernelArgs<T>,
// ThisBuffer / NextBuffer).
template <>
struct Elem<F16T> {
  __device__ static _Float16 widen(uint16_t h) { return __builtin_bit_cast(_Float16, h); }
  __device__ static uint16_t narrow(_Float16 a) { return __builtin_bit_cast(uint16_t, a); }
  __device__ static void unpack(const uint4& v, _Float16 (&a)[8]) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[2 * i] = widen(static_cast<uint16_t>(w[i]));
      a[2 * i + 1] = widen(static_cast<uint16_t>(w[i] >> 16));
    }
  }
  __device__ static uint4 pack(const _Float16 (&a)[8]) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = narrow(a[2 * i]) | (static_cast<uint32_t>(narrow(a[2 * i + 1])) << 16);
    return make_uint4(w[0], w[1], w[2], w[3]);
  }
};

// fp32 through half: every input is rounded to half (round to nearest even)
// as the sender's float2half does, the halves are folded in half as the fp16
// type is, and the half result is widened exactly for the fp32 output, as
// half2float does.
template <>
struct Elem<F32HT> {
  __device__ static _Float16 widen(float x) { return static_cast<_Float16>(x); }
  __device__ static float narrow(_Float16 a) { return static_cast<float>(a); }
  __device__ static void unpack(const uint4& v, _Float16 (&a)[4]) {
    a[0] = widen(__uint_as_float(v.x));
    a[1] = widen(__uint_as_float(v.y));
    a[2] = widen(__uint_as_float(v.z));
    a[3] = widen(__uint_as_float(v.w));
  }
  __device__ static uint4 pack(const _Float16 (&a)[4]) {
    return make_uint4(__float_as_uint(narrow(a[0])), __float_as_uint(narrow(a[1])),
                      __float_as_uint(narrow(a[2])), __float_as_uint(narrow(a[3])));
  }
};

// int8: sixteen per dwordx4, byte i of word i / 4 at bit 8 * (i % 4).
template <>
struct Elem<I8T> {
  __device__ static int8_t widen(int8_t x) { return x; }
  __device__ static int8_t narrow(int8_t a) { return a; }
  __device__ static void unpack(const uint4& v, int8_t (&a)[16]) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 16; ++i) a[i] = static_cast<int8_t>(w[i / 4] >> (8 * (i % 4)));
  }
  __device__ static uint4 pack(const int8_t (&a)[16]) {
    uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 16; ++i) w[i / 4] |= static_cast<uint32_t>(static_cast<uint8_t>(a[i])) << (8 * (i % 4));
    return make_uint4(w[0], w[1], w[2], w[3]);
  }
};

// ------------------------------------------------------------------- ops

// Sums and products: IEEE in the float types; integers wrap, computed in the
// unsigned type of the same width (whose low bits are the two's-complement
// result, without signed-overflow undefined behaviour).
template <class T>
struct Unsigned;
template <>
struct Unsigned<int8_t> {
  using T = uint8_t;
};
template <>
struct Unsigned<int32_t> {
  using T = uint32_t;
};
template <>
struct Unsigned<int64_t> {
  using T = uint64_t;
};
template <>
struct Unsigned<uint64_t> {
  using T = uint64_t;
};

template <class A>
inline constexpr bool kIsFloat = std::is_floating_point<A>::value || std::is_same<A, _Float16>::value;

template <class A>
__device__ __forceinline__ A add_op(A a, A b) {
  if constexpr (kIsFloat<A>) {
    return a + b;
  } else {
    using U = typename Unsigned<A>::T;
    return static_cast<A>(static_cast<U>(static_cast<U>(a) + static_cast<U>(b)));
  }
}

template <class A>
__device__ __forceinline__ A mul_op(A a, A b) {
  if constexpr (kIsFloat<A>) {
    return a * b;
  } else {
    using U = typename Unsigned<A>::T;
    return static_cast<A>(static_cast<U>(static_cast<U>(a) * static_cast<U>(b)));
  }
}

// One ring step: the partial folded so far, combined with the next rank's value.
// max/min keep the partial unless the new value compares strictly greater /
// smaller (a compare and a select, never a hardware max/min instruction, so
// +-0 ties and NaNs follow the fold order).
template <int OP, class A>
__device__ __forceinline__ A combine(A acc, A x) {
  if constexpr (OP == RSX_MAX) {
    return (x > acc) ? x : acc;
  } else if constexpr (OP == RSX_MIN) {
    return (x < acc) ? x : acc;
  } else if constexpr (OP == RSX_PROD) {
    return mul_op(acc, x);
  } else {
    return add_op(acc, x);
  }
}

// avg: one division by W in the accumulation type (IEEE for floats; C
// integer division: toward zero for signed types, floor for uint64).  A half
// fold is divided in fp32 (correctly rounded here) and converted: fp32 holds
// 24 >= 2 * 11 + 2 significand bits, so the quotient rounded to fp32 and
// then to half equals the correctly rounded half quotient.  The empty asm
// keeps the quotient a plain fp32 value before the conversion.
template <int OP, int W, class A>
__device__ __forceinline__ A finish(A acc) {
  if constexpr (OP == RSX_AVG && std::is_same<A, _Float16>::value) {
    float q = static_cast<float>(acc) / static_cast<float>(W);
    asm volatile("" : "+v"(q));
    return static_cast<_Float16>(q);
  } else if constexpr (OP == RSX_AVG) {
    return static_cast<A>(acc / static_cast<A>(W));
  } else {
    return acc;
  }
}

// ------------------------------------------------------------ tile body

// Fold one element: the W values in fold order, then finish and narrow.
template <class D, int OP, int W>
__device__ __forceinline__ typename D::S fold_values(const typename D::S (&x)[W]) {
  typename D::A acc = Elem<D>::widen(x[0]);
#pragma unroll
  for (int j = 1; j < W; ++j) acc = combine<OP>(acc, Elem<D>::widen(x[j]));
  return Elem<D>::narrow(finish<OP, W>(acc));
}

// Fold one dwordx4 of each of the W sources (in fold order), lane-wise.
template <class D, int OP, int W>
__device__ __forceinline__ uint4 fold_vectors(const uint4 (&v)[W]) {
  using A = typename D::A;
  constexpr int VL = D::kVL;
  A acc[VL];
  Elem<D>::unpack(v[0], acc);
#pragma unroll
  for (int j = 1; j < W; ++j) {
    A x[VL];
    Elem<D>::unpack(v[j], x);
#pragma unroll
    for (int l = 0; l < VL; ++l) acc[l] = combine<OP>(acc[l], x[l]);
  }
#pragma unroll
  for (int l = 0; l < VL; ++l) acc[l] = finish<OP, W>(acc[l]);
  return Elem<D>::pack(acc);
}

// Tile `tile` of the element range [b, e) of W sources given in fold order.
// Element idx goes to dst[d][idx - shift] for each of the ND destinations
// (one reduce-scatter block, or every all-reduce rank).
//
// VEC: all source and destination bases are 16-byte aligned, so element
// offsets divisible by VL are too; the tile is U*256 whole vectors of the
// range and tile 0 also folds the unaligned head and tail elements.  WHOLE
// (the reduce-scatter): the vectors start at b itself, whose destination
// (dst + b - shift) is 16-byte aligned and whose sources are at least
// 4-byte aligned (multi-dword buffer loads need only dword alignment), and
// tile 0 folds the last (e - b) mod VL elements.  Otherwise the tile is
// U*256 elements, one per lane per unit, still coalesced.
template <class D, int OP, int W, int ND, int STORE_AUX, bool VEC, bool WHOLE>
__device__ __forceinline__ void fold_tile(const typename D::S* const (&src)[W],
                                          typename D::S* const (&dst)[ND], uint64_t shift,
                                          uint64_t b, uint64_t e, uint32_t tile, uint32_t tid) {
  using S = typename D::S;
  constexpr int U = fold_units(W);
  constexpr int VL = D::kVL;

  auto fold_element = [&](uint64_t idx) {
    S x[W];
#pragma unroll
    for (int j = 0; j < W; ++j) x[j] = src[j][idx];
    const S out = fold_values<D, OP, W>(x);
#pragma unroll
    for (int d = 0; d < ND; ++d) dst[d][idx - shift] = out;
  };

  if constexpr (VEC) {
    const uint64_t hb = WHOLE ? b : min((b + VL - 1) / VL * VL, e);
    const uint64_t be = WHOLE ? b + (e - b) / VL * VL : max(hb, e / VL * VL);
    const uint64_t nv = (be - hb) / VL;
    const uint64_t v0 = static_cast<uint64_t>(tile) * (U * kBlock);
    // A whole segment's tiles all hold vectors: the grid has ceil(nv / tile)
    // tiles per segment.
    if (WHOLE || v0 < nv) {
      // This tile's vectors, [v0, v0 + nvt), as a byte range per buffer;
      // lanes past the range read zeros and their stores are dropped.
      const uint32_t nvt = static_cast<uint32_t>(min<uint64_t>(U * kBlock, nv - v0));
      const uint32_t bytes = nvt * kVecBytes;
      const uint64_t e0 = hb + v0 * VL;
      const uint32_t voff = tid * kVecBytes;
      uint4 v[U][W];
#pragma unroll
      for (int j = 0; j < W; ++j) {
        const __amdgpu_buffer_rsrc_t r = make_rsrc(src[j] + e0, bytes);
#pragma unroll
        for (int u = 0; u < U; ++u) v[u][j] = load_stream(r, voff, u * kBlock * kVecBytes);
      }
      uint4 o[U];
#pragma unroll
      for (int u = 0; u < U; ++u) o[u] = fold_vectors<D, OP, W>(v[u]);
#pragma unroll
      for (int d = 0; d < ND; ++d) {
        const __amdgpu_buffer_rsrc_t r = make_rsrc(dst[d] + (e0 - shift), bytes);
#pragma unroll
        for (int u = 0; u < U; ++u) store_b128<STORE_AUX>(r, voff, u * kBlock * kVecBytes, o[u]);
      }
    }
    if (WHOLE && tile == 0) {
      if (tid < e - be) fold_element(be + tid);
    } else if (!WHOLE && tile == 0) {
      const uint32_t nh = static_cast<uint32_t>(hb - b);
      const uint32_t nt = static_cast<uint32_t>(e - be);
      if (tid < nh) {
        fold_element(b + tid);
      } else if (tid < nh + nt) {
        fold_element(be + (tid - nh));
      }
    }
  } else {
    const uint64_t t0 = b + static_cast<uint64_t>(tile) * (U * kBlock);
    if (t0 >= e) return;
    const bool full = t0 + U * kBlock <= e;
    S x[U][W];
#pragma unroll
    for (int j = 0; j < W; ++j)
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (full || t0 + u * kBlock + tid < e) x[u][j] = src[j][t0 + u * kBlock + tid];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint64_t idx = t0 + u * kBlock + tid;
      if (!full && idx >= e) continue;
      const S out = fold_values<D, OP, W>(x[u]);
#pragma unroll
      for (int d = 0; d < ND; ++d) dst[d][idx - shift] = out;
    }
  }
}

// ------------------------------------------------------------------ kernels

// Reduce-scatter (RS) or all-reduce over W rank buffers (FoldArgs).  TPW
// tiles per workgroup: with TPW = 2, a workgroup of 512 lanes runs two
// consecutive tiles of 256 lanes, one per half (see pair_tiles).
template <class D, int OP, int W, bool RS, bool VEC, int TPW>
__global__ __launch_bounds__(kBlock * TPW) void fold_kernel(const FoldArgs a) {
  using S = typename D::S;

  // Every scalar argument in one round of kernarg loads.  A workgroup runs a
  // single tile, so each dependent round before its first HBM load costs a
  // few percent of the kernel; the empty asm keeps the compiler from sinking
  // these loads below the exit test, one round at a time.  A reduce-scatter
  // always folds in ring order (rotation 1).
  const uint32_t tiles_total = a.tiles_total, magic = a.tps_magic, shift = a.tps_shift;
  const uint32_t tps = a.tiles_per_seg;
  const uint32_t rot = RS ? 1u : a.rot;
  const uint64_t seg = a.seg, count = a.count;
  const uint32_t t = workgroup_tile<TPW>();
  const uint32_t tid = TPW == 1 ? threadIdx.x : threadIdx.x % kBlock;
  asm volatile("" ::"s"(magic), "s"(shift), "s"(tps), "s"(rot), "s"(seg), "s"(count), "s"(t));
  if (t >= tiles_total) return;
  const uint32_t k = static_cast<uint32_t>((static_cast<uint64_t>(t) * magic) >> shift);
  const uint32_t tile = t - k * tps;
  // Reduce-scatter segments are whole (count = W * seg, seg % VL == 0 for
  // the dwordx4 kernel); all-reduce ones are clipped to count.
  const uint64_t b = RS ? static_cast<uint64_t>(k) * seg : min(static_cast<uint64_t>(k) * seg, count);
  const uint64_t e = RS ? b + seg : min(b + seg, count);

  // Ring rotation: source j of segment k is rank (k + rot + j) mod W.  Each
  // pointer is fetched on its own, just before its load is issued, so the
  // first HBM load leaves as early as it can (measured faster than fetching
  // the whole pointer table first and issuing the W loads back to back).
  const uint32_t first = (k + rot) % W;
  const S* src[W];
#pragma unroll
  for (int j = 0; j < W; ++j) src[j] = static_cast<const S*>(a.src[(first + j) % W]);

  if constexpr (RS) {
    // Segment k goes to rank k mod W, at its offset within its group of W
    // segments (one group per bucket when a launch covers several).
    const uint32_t kr = k % W;
    S* const dst[1] = {static_cast<S*>(a.dst[kr])};
    fold_tile<D, OP, W, 1, kStoreThrough, VEC, true>(src, dst, static_cast<uint64_t>(kr) * seg, b, e, tile,
                                                      tid);
  } else {
    S* dst[W];
#pragma unroll
    for (int d = 0; d < W; ++d) dst[d] = static_cast<S*>(a.dst[d]);
    fold_tile<D, OP, W, W, kStoreStream, VEC, false>(src, dst, 0, b, e, tile, tid);
  }
}

// Tensor-list all-reduce (ListArgs): one piece of one tensor per workgroup.
template <class D, int OP, int W>
__global__ __launch_bounds__(kBlock) void list_fold_kernel(const ListArgs a) {
  using S = typename D::S;
  const uint32_t n = a.npieces;
  const uint32_t t = xcd_tile(blockIdx.x, gridDim.x);  // one tile per workgroup
  if (t >= a.tile_start[n]) return;
  // Piece of this tile: the last i with tile_start[i] <= t.
  uint32_t lo = 0, hi = n - 1;
  while (lo < hi) {
    const uint32_t mid = (lo + hi + 1) / 2;
    if (a.tile_start[mid] <= t) lo = mid; else hi = mid - 1;
  }
  const ListPiece& pc = a.piece[lo];
  const uint32_t tile = t - a.tile_start[lo];
  const bool in_place = a.in_place != 0;
  const uint32_t base = pc.tensor * (in_place ? W : 2 * W);
  const uint32_t dbase = in_place ? base : base + W;
  const uint32_t first = (pc.seg + a.rot) % W;
  const S* src[W];
  S* dst[W];
#pragma unroll
  for (int j = 0; j < W; ++j) {
    uint32_t r = first + j;
    if (r >= static_cast<uint32_t>(W)) r -= W;
    src[j] = static_cast<const S*>(a.ptr[base + r]);
    dst[j] = static_cast<S*>(a.ptr[dbase + j]);
  }
  if (pc.vec) {
    fold_tile<D, OP, W, W, kStoreStream, true, false>(src, dst, 0, pc.lo, pc.hi, tile, threadIdx.x);
  } else {
    fold_tile<D, OP, W, W, kStoreStream, false, false>(src, dst, 0, pc.lo, pc.hi, tile, threadIdx.x);
  }
}

// --------------------------------------------------------------- dispatch

// Two tiles per workgroup exist for the dwordx4 all-reduce only (the launch
// chooses them; see rsx_abi.hip).
template <class D, int OP, int W>
hipError_t launch_world(bool rs, bool vec, int tpw, const FoldArgs& a, dim3 grid, uint32_t lds,
                        hipStream_t s) {
  void* args[] = {const_cast<FoldArgs*>(&a)};
  const void* fn;
  if (!rs && vec && tpw == 2) {
    fn = reinterpret_cast<const void*>(&fold_kernel<D, OP, W, false, true, 2>);
  } else if (rs && vec && tpw == 2) {
    // paired reduce-scatter tiles exist from W = 10 (rs_pairs)
    if constexpr (W >= 10) fn = reinterpret_cast<const void*>(&fold_kernel<D, OP, W, true, true, 2>);
    else return hipErrorInvalidValue;
  } else if (tpw != 1) {
    return hipErrorInvalidValue;
  } else if (rs) {
    fn = vec ? reinterpret_cast<const void*>(&fold_kernel<D, OP, W, true, true, 1>)
             : reinterpret_cast<const void*>(&fold_kernel<D, OP, W, true, false, 1>);
  } else {
    fn = vec ? reinterpret_cast<const void*>(&fold_kernel<D, OP, W, false, true, 1>)
             : reinterpret_cast<const void*>(&fold_kernel<D, OP, W, false, false, 1>);
  }
  return hipLaunchKernel(fn, grid, dim3(kBlock * tpw), args, lds, s);
}

template <class D, int OP>
hipError_t launch_op(int world, bool rs, bool vec, int tpw, const FoldArgs& a, dim3 grid, uint32_t lds,
                     hipStream_t s) {
  switch (world) {
#define RSX_W(n) \
  case n:        \
    return launch_world<D, OP, n>(rs, vec, tpw, a, grid, lds, s);
    RSX_W(1) RSX_W(2) RSX_W(3) RSX_W(4) RSX_W(5) RSX_W(6) RSX_W(7) RSX_W(8)
    RSX_W(9) RSX_W(10) RSX_W(11) RSX_W(12) RSX_W(13) RSX_W(14) RSX_W(15) RSX_W(16)
#undef RSX_W
    default:
      return hipErrorInvalidValue;
  }
}

template <class D, int OP>
hipError_t launch_list_op(int world, const ListArgs& a, dim3 grid, uint32_t lds, hipStream_t s) {
  void* args[] = {const_cast<ListArgs*>(&a)};
  const void* fn;
  switch (world) {
#define RSX_W(n)                                                            \
  case n:                                                                   \
    fn = reinterpret_cast<const void*>(&list_fold_kernel<D, OP, n>);        \
    break;
    RSX_W(1) RSX_W(2) RSX_W(3) RSX_W(4) RSX_W(5) RSX_W(6) RSX_W(7) RSX_W(8)
    RSX_W(9) RSX_W(10) RSX_W(11) RSX_W(12) RSX_W(13) RSX_W(14) RSX_W(15) RSX_W(16)
#undef RSX_W
    default:
      return hipErrorInvalidValue;
  }
  return hipLaunchKernel(fn, grid, dim3(kBlock), args, lds, s);
}

template <class D>
hipError_t launch_list(int op, int world, const ListArgs& a, dim3 grid, uint32_t lds, hipStream_t s) {
  switch (op) {
    case RSX_SUM:
      return launch_list_op<D, RSX_SUM>(world, a, grid, lds, s);
    case RSX_MAX:
      return launch_list_op<D, RSX_MAX>(world, a, grid, lds, s);
    case RSX_MIN:
      return launch_list_op<D, RSX_MIN>(world, a, grid, lds, s);
    case RSX_AVG:
      return launch_list_op<D, RSX_AVG>(world, a, grid, lds, s);
    case RSX_PROD:
      return launch_list_op<D, RSX_PROD>(world, a, grid, lds, s);
    default:
      return hipErrorInvalidValue;
  }
}

template <class D>
hipError_t launch_fold(int op, int world, bool rs, bool vec, int tpw, const FoldArgs& a, dim3 grid,
                       uint32_t lds, hipStream_t s) {
  switch (op) {
    case RSX_SUM:
      return launch_op<D, RSX_SUM>(world, rs, vec, tpw, a, grid, lds, s);
    case RSX_MAX:
      return launch_op<D, RSX_MAX>(world, rs, vec, tpw, a, grid, lds, s);
    case RSX_MIN:
      return launch_op<D, RSX_MIN>(world, rs, vec, tpw, a, grid, lds, s);
    case RSX_AVG:
      return launch_op<D, RSX_AVG>(world, rs, vec, tpw, a, grid, lds, s);
    case RSX_PROD:
      return launch_op<D, RSX_PROD>(world, rs, vec, tpw, a, grid, lds, s);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace rsx
