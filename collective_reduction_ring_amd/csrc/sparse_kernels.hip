// Sparsified all-reduce with error feedback, for W ranks on one GPU.
//
// What is computed (Apache SINGA src/io/communicator.cc, valSparsAllReduce
// and topKSparsAllReduce): each rank adds its accumulation buffer to its
// gradient (when it has one), keeps either the entries whose magnitude
// reaches a threshold (zeros never count) or the K largest values, sends the
// kept (index, value) pairs, and stores what it did not send back into the
// accumulation buffer.  The messages of all ranks are all-gathered, and every
// rank adds rank 0's message, then rank 1's, ..., into a zeroed buffer.
//
// On one GPU the W messages are W arrays in HBM, so the all-gather is the
// combine kernel reading them.  The page sorts all values to find the top K;
// only the set matters to the result (message entries of one rank have
// distinct indices, so their order does not change any sum), so the K-th
// largest value is found by a radix select instead:
//
//   init      zero the histograms; the selection state of every rank
//   hist/pick three passes (11, 11 and 10 bits of an order-preserving key):
//             a histogram of the next digit among the keys that match the
//             digits chosen so far, then the digit at which the K-th largest
//             key lies (top-K only)
//   compact   per tile: the candidate entries (to send: threshold; above
//             or equal to the cut: top-K) in index order into the tile's own
//             slot of the workspace, their counts, and the residual
//   scan      per rank: each tile's offset in the message, its length
//   combine   per output tile: zero an LDS tile; for each rank in order,
//             place the tile's sent entries in the message and add them into
//             the tile; store the tile to all W outputs
//
// Ties at the cut are taken in index order, as a stable sort from large to
// small values would take them.  Writing each tile's entries into a slot of
// its own lets the compaction run before the offsets are known, so every
// element is read once after the selection passes.  No kernel waits on
// another workgroup.
#include "mem.h"
#include "rsx_internal.h"

namespace rsx {
namespace {

constexpr uint32_t kSpLaneElems = kSpUnits * 4;  // 16 elements per lane per tile
static_assert(kSpLaneElems * kBlock == kSpTile, "tile = 256 lanes x 16 elements");

// Order-preserving key of an fp32 value for the top-K cut: a larger value has
// a larger key; -0 and +0 share one key; every NaN has key 0, below -inf.
__device__ __forceinline__ uint32_t order_key(float x) {
  uint32_t b = __float_as_uint(x);
  if (b == 0x80000000u) b = 0;
  const uint32_t k = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return (x != x) ? 0u : k;
}

// Inclusive sum over the 64 lanes of a wave.
__device__ __forceinline__ uint32_t wave_incl(uint32_t v) {
  const uint32_t lane = threadIdx.x & 63u;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t o = __shfl_up(v, d, 64);
    if (lane >= static_cast<uint32_t>(d)) v += o;
  }
  return v;
}

// Exclusive prefix sum over a workgroup of NW waves; `total` receives the
// sum of all.  `scratch` is NW words of LDS, free again on return.
template <int NW>
__device__ __forceinline__ uint32_t block_excl(uint32_t v, uint32_t* scratch, uint32_t& total) {
  const uint32_t inc = wave_incl(v);
  const uint32_t w = threadIdx.x >> 6;
  if ((threadIdx.x & 63u) == 63u) scratch[w] = inc;
  __syncthreads();
  uint32_t before = 0, sum = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const uint32_t s = scratch[i];
    before += (static_cast<uint32_t>(i) < w) ? s : 0u;
    sum += s;
  }
  __syncthreads();
  total = sum;
  return before + inc - v;
}

// The 16 values of this lane in tile `base` of a rank: x[u][j] is element
// u*1024 + 4*lane + j of the tile.  With ACC, x = g + acc (one fp32 add, the
// page's error feedback); lanes past the rank's end read zeros.
template <bool ACC>
__device__ __forceinline__ void load_tile(const float* g, const float* acc, uint64_t base, uint32_t n,
                                          float (&x)[kSpUnits][4]) {
  const uint32_t tid = threadIdx.x;
  const __amdgpu_buffer_rsrc_t rg = make_rsrc(g + base, n * 4);
  uint4 vg[kSpUnits];
#pragma unroll
  for (int u = 0; u < static_cast<int>(kSpUnits); ++u) vg[u] = load_stream(rg, tid * 16, u * kBlock * 16);
  if constexpr (ACC) {
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(acc + base, n * 4);
    uint4 va[kSpUnits];
#pragma unroll
    for (int u = 0; u < static_cast<int>(kSpUnits); ++u) va[u] = load_stream(ra, tid * 16, u * kBlock * 16);
#pragma unroll
    for (int u = 0; u < static_cast<int>(kSpUnits); ++u) {
      x[u][0] = __uint_as_float(vg[u].x) + __uint_as_float(va[u].x);
      x[u][1] = __uint_as_float(vg[u].y) + __uint_as_float(va[u].y);
      x[u][2] = __uint_as_float(vg[u].z) + __uint_as_float(va[u].z);
      x[u][3] = __uint_as_float(vg[u].w) + __uint_as_float(va[u].w);
    }
  } else {
#pragma unroll
    for (int u = 0; u < static_cast<int>(kSpUnits); ++u) {
      x[u][0] = __uint_as_float(vg[u].x);
      x[u][1] = __uint_as_float(vg[u].y);
      x[u][2] = __uint_as_float(vg[u].z);
      x[u][3] = __uint_as_float(vg[u].w);
    }
  }
}

__device__ __forceinline__ void store_tile(float* dst, uint64_t base, uint32_t n,
                                           const float (&x)[kSpUnits][4]) {
  const __amdgpu_buffer_rsrc_t rd = make_rsrc(dst + base, n * 4);
#pragma unroll
  for (int u = 0; u < static_cast<int>(kSpUnits); ++u)
    store_b128<kStoreStream>(rd, threadIdx.x * 16, u * kBlock * 16,
                             make_uint4(__float_as_uint(x[u][0]), __float_as_uint(x[u][1]),
                                        __float_as_uint(x[u][2]), __float_as_uint(x[u][3])));
}

// Element u*1024 + 4*lane + j of a tile lies inside the rank when below n.
__device__ __forceinline__ bool in_tile(int u, int j, uint32_t n) {
  return static_cast<uint32_t>(u) * kBlock * 4 + threadIdx.x * 4 + static_cast<uint32_t>(j) < n;
}

// Radix digits of the top-K cut, most significant first.
template <int PASS>
struct Digit {
  static constexpr uint32_t kShift = PASS == 0 ? 21 : (PASS == 1 ? 10 : 0);
  static constexpr uint32_t kBins = PASS == 2 ? 1024 : 2048;
  static constexpr uint32_t kHigh = PASS == 0 ? 0u : (PASS == 1 ? 0xFFE00000u : 0xFFFFFC00u);
};

// ----------------------------------------------------------------- kernels

// Zero every rank's histogram; selection state = (cut key 0, K ties to
// find).  K = 0 selects nothing: the cut key is above every key.
__global__ __launch_bounds__(kBlock) void sp_init_kernel(const SparseArgs a) {
  const uint32_t r = blockIdx.x;
  for (uint32_t i = threadIdx.x; i < kSpBins; i += kBlock) a.hist[r * kSpBins + i] = 0;
  if (threadIdx.x == 0) {
    uint32_t* st = a.state + 4 * r;
    st[0] = a.k == 0 ? 0xFFFFFFFFu : 0u;
    st[1] = a.k;
    st[2] = 0;
    st[3] = 0;
  }
}

// Histogram of digit PASS among the keys whose higher digits equal the cut
// chosen so far.  hist_groups workgroups per rank, each over hist_chunk
// consecutive tiles.  Pass 0 with an accumulation also stores g + acc, the
// values every later pass selects on.
template <int PASS, bool ACC>
__global__ __launch_bounds__(kBlock) void sp_hist_kernel(const SparseArgs a) {
  using Dg = Digit<PASS>;
  __shared__ uint32_t h[kSpBins];
  const uint32_t r = blockIdx.x / a.hist_groups;
  const uint32_t grp = blockIdx.x - r * a.hist_groups;
  for (uint32_t i = threadIdx.x; i < kSpBins; i += kBlock) h[i] = 0;
  __syncthreads();
  const uint32_t prefix = PASS == 0 ? 0u : a.state[4 * r];
  const uint32_t t0 = grp * a.hist_chunk;
  const uint32_t t1 = min(a.tiles, t0 + a.hist_chunk);
  for (uint32_t t = t0; t < t1; ++t) {
    const uint64_t base = static_cast<uint64_t>(t) * kSpTile;
    const uint32_t n = static_cast<uint32_t>(min<uint64_t>(kSpTile, a.count - base));
    float x[kSpUnits][4];
    if constexpr (PASS == 0 && ACC) {
      load_tile<true>(a.grad[r], a.accum[r], base, n, x);
      store_tile(a.key_store[r], base, n, x);
    } else {
      load_tile<false>(a.key[r], nullptr, base, n, x);
    }
#pragma unroll
    for (int u = 0; u < static_cast<int>(kSpUnits); ++u)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t k = order_key(x[u][j]);
        if (in_tile(u, j, n) && (k & Dg::kHigh) == prefix)
          atomicAdd(&h[(k >> Dg::kShift) & (Dg::kBins - 1)], 1u);
      }
  }
  __syncthreads();
  uint32_t* gh = a.hist + r * kSpBins;
  for (uint32_t i = threadIdx.x; i < Dg::kBins; i += kBlock)
    if (h[i] != 0) atomicAdd(&gh[i], h[i]);
}

// The digit at which the K-th largest key lies: walking the bins from the
// top, the first bin at which the running count reaches the number still to
// find.  The keys of the bins above it are all selected; the search goes on
// inside that bin.  One workgroup per rank; clears the histogram afterwards.
template <int PASS>
__global__ __launch_bounds__(kBlock) void sp_pick_kernel(const SparseArgs a) {
  using Dg = Digit<PASS>;
  constexpr uint32_t kPer = Dg::kBins / kBlock;
  __shared__ uint32_t scratch[kBlock / 64];
  const uint32_t r = blockIdx.x;
  uint32_t* gh = a.hist + r * kSpBins;
  uint32_t* st = a.state + 4 * r;
  const uint32_t prefix = st[0];
  const uint32_t need = st[1];
  // thread i holds bins top, top-1, ..., top-kPer+1 (thread 0 the highest)
  const uint32_t top = Dg::kBins - 1 - threadIdx.x * kPer;
  uint32_t c[kPer];
  uint32_t sum = 0;
#pragma unroll
  for (uint32_t i = 0; i < kPer; ++i) {
    c[i] = gh[top - i];
    sum += c[i];
  }
  uint32_t total;
  const uint32_t above = block_excl<kBlock / 64>(sum, scratch, total);
  if (above < need && need <= above + sum) {
    uint32_t run = above;
    for (uint32_t i = 0; i < kPer; ++i) {
      if (run + c[i] >= need) {
        st[0] = prefix | ((top - i) << Dg::kShift);
        st[1] = need - run;
        break;
      }
      run += c[i];
    }
  }
#pragma unroll
  for (uint32_t i = 0; i < kPer; ++i) gh[top - i] = 0;
}

// Rank and tile of workgroup b in a (rank, tile) grid; false past the end.
__device__ __forceinline__ bool rank_tile(const SparseArgs& a, uint32_t& r, uint32_t& t) {
  const uint32_t lin = xcd_tile(blockIdx.x, gridDim.x);
  if (lin >= a.world * a.tiles) return false;
  r = lin / a.tiles;
  t = lin - r * a.tiles;
  return true;
}

// Selection flags of one element: bit 0 = sent for sure (threshold mode:
// |x| >= threshold and x != 0; top-K: key above the cut), bit 16 = key equal
// to the cut (top-K; sent while ties are left, in index order).
template <int MODE>
__device__ __forceinline__ uint32_t flags(float x, bool valid, float thr, uint32_t cut) {
  if (!valid) return 0;
  if constexpr (MODE == RSX_SPARSE_THRESHOLD) {
    return (fabsf(x) >= thr && x != 0.0f) ? 1u : 0u;
  } else {
    const uint32_t k = order_key(x);
    return (k > cut ? 1u : 0u) | (k == cut ? 0x10000u : 0u);
  }
}

template <int MODE, bool ACC>
__device__ __forceinline__ void load_selected_on(const SparseArgs& a, uint32_t r, uint64_t base, uint32_t n,
                                                 float (&x)[kSpUnits][4]) {
  if constexpr (MODE == RSX_SPARSE_TOPK)
    load_tile<false>(a.key[r], nullptr, base, n, x);  // grad, or the stored grad + acc
  else
    load_tile<ACC>(a.grad[r], ACC ? a.accum[r] : nullptr, base, n, x);
}

// Per tile: the candidate entries (sent for sure, or tied with the cut) in
// index order, into the tile's own slot of kSpTile entries in the workspace,
// their two counts, and, with an accumulation, the residual.  A tie's
// residual is written as if it were not sent; the combine rewrites the ties
// that are taken.  Residuals follow the page's arithmetic: the threshold
// mode subtracts the thresholded array (which keeps a +-0 reaching the
// threshold), the top-K mode subtracts the sent values added to zeros (so a
// sent -0 leaves -0); a sent inf leaves NaN in both.
template <int MODE, bool ACC>
__global__ __launch_bounds__(kBlock) void sp_compact_kernel(const SparseArgs a) {
  __shared__ uint32_t scratch[kBlock / 64];
  uint32_t r, t;
  if (!rank_tile(a, r, t)) return;
  const uint64_t base = static_cast<uint64_t>(t) * kSpTile;
  const uint32_t n = static_cast<uint32_t>(min<uint64_t>(kSpTile, a.count - base));
  float x[kSpUnits][4];
  load_selected_on<MODE, ACC>(a, r, base, n, x);
  const uint32_t cut = MODE == RSX_SPARSE_TOPK ? a.state[4 * r] : 0u;
  const uint64_t slot = (static_cast<uint64_t>(r) * a.tiles + t) * kSpTile;
  uint32_t* gi = a.gap_idx + slot;
  float* gv = a.gap_val + slot;
  float res[kSpUnits][4];
  uint32_t run = 0;  // packed counts of the earlier units of the tile
#pragma unroll
  for (int u = 0; u < static_cast<int>(kSpUnits); ++u) {
    uint32_t f[4];
    uint32_t c = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f[j] = flags<MODE>(x[u][j], in_tile(u, j, n), a.threshold, cut);
      c += f[j];
    }
    uint32_t tot;
    uint32_t pre = block_excl<kBlock / 64>(c, scratch, tot) + run;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t local = static_cast<uint32_t>(u) * kBlock * 4 + threadIdx.x * 4 + j;
      if (f[j] != 0) {
        const uint32_t at = (pre & 0xFFFFu) + (pre >> 16);  // entries before it in the tile
        gi[at] = local;
        gv[at] = x[u][j];
      }
      if constexpr (ACC) {
        const float v = x[u][j];
        if constexpr (MODE == RSX_SPARSE_THRESHOLD)
          res[u][j] = fabsf(v) >= a.threshold ? v - v : v - 0.0f;
        else
          res[u][j] = (f[j] & 1u) ? v - (0.0f + v) : v - 0.0f;
      }
      pre += f[j];
    }
    run += tot;
  }
  if constexpr (ACC) store_tile(a.accum[r], base, n, res);
  if (threadIdx.x == 0) {
    const uint32_t i = r * (a.tiles + 1) + t;
    a.tile_cnt[i] = run & 0xFFFFu;
    a.tile_eqc[i] = run >> 16;
  }
}

// Per rank: exclusive prefixes of the tile counts.  A tile's message offset
// is the entries sent for sure before it plus the ties before it, up to the
// number of ties to take; tile_eqb holds the ties before it.  The last slot
// and nnz[r] get the message length.
template <int MODE>
__global__ __launch_bounds__(kSpScanBlock) void sp_scan_kernel(const SparseArgs a) {
  constexpr uint32_t kPer = 4;
  constexpr int kWaves = kSpScanBlock / 64;
  __shared__ uint32_t scratch[kWaves];
  const uint32_t r = blockIdx.x;
  const uint32_t n = a.tiles;
  const uint32_t* cnt = a.tile_cnt + r * (n + 1);
  const uint32_t* eqc = a.tile_eqc + r * (n + 1);
  uint32_t* off = a.tile_off + r * (n + 1);
  uint32_t* eqb = a.tile_eqb + r * (n + 1);
  const uint32_t need = MODE == RSX_SPARSE_TOPK ? a.state[4 * r + 1] : 0u;
  uint32_t carry_s = 0, carry_e = 0;
  for (uint32_t c0 = 0; c0 < n; c0 += kSpScanBlock * kPer) {
    uint32_t s[kPer], e[kPer];
    uint32_t ss = 0, se = 0;
#pragma unroll
    for (uint32_t i = 0; i < kPer; ++i) {
      const uint32_t idx = c0 + threadIdx.x * kPer + i;
      s[i] = idx < n ? cnt[idx] : 0u;
      e[i] = (MODE == RSX_SPARSE_TOPK && idx < n) ? eqc[idx] : 0u;
      ss += s[i];
      se += e[i];
    }
    uint32_t ts, te = 0;
    uint32_t bs = block_excl<kWaves>(ss, scratch, ts) + carry_s;
    uint32_t be = 0;
    if constexpr (MODE == RSX_SPARSE_TOPK) be = block_excl<kWaves>(se, scratch, te) + carry_e;
#pragma unroll
    for (uint32_t i = 0; i < kPer; ++i) {
      const uint32_t idx = c0 + threadIdx.x * kPer + i;
      if (idx < n) {
        off[idx] = bs + min(be, need);
        eqb[idx] = be;
      }
      bs += s[i];
      be += e[i];
    }
    carry_s += ts;
    carry_e += te;
  }
  if (threadIdx.x == 0) {
    const uint32_t len = carry_s + min(carry_e, need);
    off[n] = len;
    eqb[n] = carry_e;
    a.nnz[r] = len;
  }
}

// Per output tile: a zeroed LDS tile; for each rank in order, the entries of
// the tile's slot that are sent (all of them, except ties beyond the number
// to take, taken in index order) are added into it, written to their place
// in the rank's message, and, for a taken tie, its residual is rewritten as
// sent; then the tile is stored to every rank's output.  One barrier per rank
// keeps the adds in rank order; entries of one rank have distinct indices.
template <int MODE, bool ACC>
__global__ __launch_bounds__(kBlock) void sp_combine_kernel(const SparseArgs a) {
  __shared__ float4 acc4[kSpTile / 4];
  __shared__ uint32_t scratch[kBlock / 64];
  float* acc = reinterpret_cast<float*>(acc4);
  const uint32_t t = xcd_tile(blockIdx.x, gridDim.x);
  if (t >= a.tiles) return;
  const uint64_t base = static_cast<uint64_t>(t) * kSpTile;
  const uint32_t n = static_cast<uint32_t>(min<uint64_t>(kSpTile, a.count - base));
#pragma unroll
  for (int u = 0; u < static_cast<int>(kSpUnits); ++u) acc4[u * kBlock + threadIdx.x] = make_float4(0.f, 0.f, 0.f, 0.f);
  __syncthreads();
  for (uint32_t r = 0; r < a.world; ++r) {
    const uint32_t i = r * (a.tiles + 1) + t;
    const uint32_t c = min(a.tile_cnt[i] + a.tile_eqc[i], n);
    const uint32_t off = a.tile_off[i];
    uint32_t cut = 0, ties = 0;
    if constexpr (MODE == RSX_SPARSE_TOPK) {
      cut = a.state[4 * r];
      const uint32_t need = a.state[4 * r + 1];
      const uint32_t before = a.tile_eqb[i];
      ties = need > before ? need - before : 0u;
    }
    const uint64_t slot = (static_cast<uint64_t>(r) * a.tiles + t) * kSpTile;
    const uint32_t* gi = a.gap_idx + slot;
    const float* gv = a.gap_val + slot;
    uint32_t* mi = a.msg_idx[r];
    float* mv = a.msg_val[r];
    uint32_t run = 0;
    for (uint32_t c0 = 0; c0 < c; c0 += kBlock) {
      const uint32_t e = c0 + threadIdx.x;
      const bool valid = e < c;
      const uint32_t local = valid ? min(gi[e], kSpTile - 1) : 0u;
      const float v = valid ? gv[e] : 0.0f;
      uint32_t f = 0;
      if (valid) {
        if constexpr (MODE == RSX_SPARSE_TOPK)
          f = order_key(v) == cut ? 0x10000u : 1u;
        else
          f = 1u;
      }
      uint32_t tot;
      const uint32_t pre = block_excl<kBlock / 64>(f, scratch, tot) + run;
      const uint32_t sure_before = pre & 0xFFFFu, ties_before = pre >> 16;
      const bool sent = (f & 1u) || ((f >> 16) && ties_before < ties);
      const uint32_t pos = off + sure_before + min(ties_before, ties);
      if (sent && pos < a.cap) {  // always below: the counts bound every position
        mi[pos] = static_cast<uint32_t>(base) + local;
        mv[pos] = v;
        acc[local] = acc[local] + v;
        if constexpr (MODE == RSX_SPARSE_TOPK && ACC)
          if (f >> 16) a.accum[r][base + local] = v - (0.0f + v);
      }
      run += tot;
    }
    __syncthreads();
  }
  float x[kSpUnits][4];
#pragma unroll
  for (int u = 0; u < static_cast<int>(kSpUnits); ++u) {
    const float4 v = acc4[u * kBlock + threadIdx.x];
    x[u][0] = v.x;
    x[u][1] = v.y;
    x[u][2] = v.z;
    x[u][3] = v.w;
  }
  for (uint32_t r = 0; r < a.world; ++r) store_tile(a.out[r], base, n, x);
}

__global__ void sp_zero_nnz_kernel(uint32_t* nnz, int world) {
  if (static_cast<int>(threadIdx.x) < world) nnz[threadIdx.x] = 0;
}

template <int MODE, bool ACC>
hipError_t launch_mode(const SparseArgs& a, hipStream_t s) {
  void* args[] = {const_cast<SparseArgs*>(&a)};
  auto go = [&](const void* fn, uint64_t grid, uint32_t block) {
    return hipLaunchKernel(fn, dim3(static_cast<uint32_t>(grid)), dim3(block), args, 0, s);
  };
  hipError_t e = go(reinterpret_cast<const void*>(&sp_init_kernel), a.world, kBlock);
  const uint64_t hg = static_cast<uint64_t>(a.world) * a.hist_groups;
  // Pass 0 also stores grad + accum for the later kernels, so it runs even
  // when K = 0 leaves nothing to select.
  if (MODE == RSX_SPARSE_TOPK && (a.k > 0 || ACC) && e == hipSuccess)
    e = go(reinterpret_cast<const void*>(&sp_hist_kernel<0, ACC>), hg, kBlock);
  if (MODE == RSX_SPARSE_TOPK && a.k > 0 && e == hipSuccess) {
    if (e == hipSuccess) e = go(reinterpret_cast<const void*>(&sp_pick_kernel<0>), a.world, kBlock);
    if (e == hipSuccess) e = go(reinterpret_cast<const void*>(&sp_hist_kernel<1, ACC>), hg, kBlock);
    if (e == hipSuccess) e = go(reinterpret_cast<const void*>(&sp_pick_kernel<1>), a.world, kBlock);
    if (e == hipSuccess) e = go(reinterpret_cast<const void*>(&sp_hist_kernel<2, ACC>), hg, kBlock);
    if (e == hipSuccess) e = go(reinterpret_cast<const void*>(&sp_pick_kernel<2>), a.world, kBlock);
  }
  const uint64_t rt = xcd_grid(static_cast<uint64_t>(a.world) * a.tiles);
  if (e == hipSuccess) e = go(reinterpret_cast<const void*>(&sp_compact_kernel<MODE, ACC>), rt, kBlock);
  if (e == hipSuccess) e = go(reinterpret_cast<const void*>(&sp_scan_kernel<MODE>), a.world, kSpScanBlock);
  if (e == hipSuccess) e = go(reinterpret_cast<const void*>(&sp_combine_kernel<MODE, ACC>), xcd_grid(a.tiles), kBlock);
  return e;
}

}  // namespace

hipError_t launch_sparse(const SparseArgs& a, int mode, bool has_accum, hipStream_t s) {
  if (mode == RSX_SPARSE_THRESHOLD)
    return has_accum ? launch_mode<RSX_SPARSE_THRESHOLD, true>(a, s) : launch_mode<RSX_SPARSE_THRESHOLD, false>(a, s);
  if (mode == RSX_SPARSE_TOPK)
    return has_accum ? launch_mode<RSX_SPARSE_TOPK, true>(a, s) : launch_mode<RSX_SPARSE_TOPK, false>(a, s);
  return hipErrorInvalidValue;
}

hipError_t launch_sparse_zero_nnz(uint32_t* nnz, int world, hipStream_t s) {
  void* args[] = {&nnz, &world};
  return hipLaunchKernel(reinterpret_cast<const void*>(&sp_zero_nnz_kernel), dim3(1), dim3(64), args, 0, s);
}

}  // namespace rsx
