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
// largest value is found by a radix select on an order-preserving key
// (digits of 11, 11 and 10 bits) instead.  Ranks are cut into tiles of 4096
// elements, and each tile owns a slot of 4096 entries in the workspace.
//
//   threshold:  compact  (every element) entries to send, in index order,
//                        into the tile's slot; the residual
//   top-K:      sample   per rank: a lower bound for the K-th largest key
//                        from a sample of 65536 keys (runs of 16 spread
//                        over the rank)
//               gather   (every element) every key at or above the bound
//                        into the tile's slot, in index order; into the
//                        accumulation buffer g = grad + acc, or from a
//                        guessed cut up the residual of a sent entry
//               fallback per rank, only when the gather found fewer than K
//                        keys: a top-digit histogram over every element,
//                        and the gather again from its exact bound
//               hist0-2  (slots) top-, middle- and low-digit histograms;
//                        each pass first finds the previous digit of the
//                        K-th key in the finished histogram before it
//               count    (slots) the last digit, then per tile the
//                        candidates above / equal to the cut
//   both:       scan     per rank: each tile's offset in the message (one
//                        workgroup per 4096 tiles)
//               combine  per output tile: for each rank in order, its sent
//                        entries into the message and into an LDS tile (top-K
//                        corrects the residuals the guess got wrong); the
//                        tile to all W outputs
//
// Ties at the cut are taken in index order, as a stable sort from large to
// small values would take them.  A slot per tile lets a tile write its
// entries before any offset is known; after the selection only slots are
// read.  The sample only decides how many candidates are gathered; the
// result never depends on it.  No kernel waits on another workgroup.
#include <algorithm>

#include "mem.h"
#include "rsx_internal.h"
#include "sparse_internal.h"

namespace rsx {
namespace {

constexpr uint32_t kSpLaneElems = kSpUnits * 4;  // elements per lane per tile
constexpr uint32_t kSpWalkGroups = 2048;          // workgroups of the tile-walking kernels
constexpr uint32_t kSampleMax = 65536;            // top-K: keys sampled per rank for the gather bound
constexpr int kSampleBlock = 1024;                // lanes of the sampling workgroup
constexpr uint32_t kScanChunk = 4 * kSpScanBlock;  // tiles per workgroup of the offset scan
constexpr uint32_t kCombBlock = 256;               // lanes of the combine (see the kernel)
static_assert(kSpLaneElems * kSpTileBlock == kSpTile, "a tile is one element group per lane");
static_assert(kSampleMax % (16 * kSampleBlock) == 0, "whole sample batches");

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

// This lane's values in tile `base` of a rank (kSpTileBlock lanes): x[u][j]
// is element 4 (u kSpTileBlock + lane) + j of the tile.  One 16-byte vector
// per lane and stream: on this GPU that streams faster than several per lane
// (two reads and an in-place write of 2 GiB: 6.5 against 6.0 TB/s).  With
// ACC, x = g + acc (one fp32 add, the page's error feedback); lanes past the
// rank's end read zeros.
template <bool ACC>
__device__ __forceinline__ void load_tile(const float* g, const float* acc, uint64_t base, uint32_t n,
                                          float (&x)[kSpUnits][4]) {
  const uint32_t tid = threadIdx.x;
  const __amdgpu_buffer_rsrc_t rg = make_rsrc(g + base, n * 4);
  uint4 vg[kSpUnits];
#pragma unroll
  for (int u = 0; u < static_cast<int>(kSpUnits); ++u) vg[u] = load_stream(rg, tid * 16, u * kSpTileBlock * 16);
  if constexpr (ACC) {
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(acc + base, n * 4);
    uint4 va[kSpUnits];
#pragma unroll
    for (int u = 0; u < static_cast<int>(kSpUnits); ++u) va[u] = load_stream(ra, tid * 16, u * kSpTileBlock * 16);
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

// Dense tile stores are non-temporal.  In these kernels, which also read,
// plain stores lose (compaction 1068 -> 1198 us, and the combine that
// follows slows too) and sc1 stores lose a little (1068 -> 1084 us).
__device__ __forceinline__ void store_tile(float* dst, uint64_t base, uint32_t n,
                                           const float (&x)[kSpUnits][4]) {
  const __amdgpu_buffer_rsrc_t rd = make_rsrc(dst + base, n * 4);
#pragma unroll
  for (int u = 0; u < static_cast<int>(kSpUnits); ++u)
    store_b128<kStoreStream>(rd, threadIdx.x * 16, u * kSpTileBlock * 16,
                             make_uint4(__float_as_uint(x[u][0]), __float_as_uint(x[u][1]),
                                        __float_as_uint(x[u][2]), __float_as_uint(x[u][3])));
}

// Elements of tile t of a rank (kSpTile except in the last tile).
__device__ __forceinline__ uint32_t tile_len(const SparseArgs& a, uint32_t t) {
  return static_cast<uint32_t>(min<uint64_t>(kSpTile, a.count - static_cast<uint64_t>(t) * kSpTile));
}

// Element 4 (u kSpTileBlock + lane) + j of a tile lies inside the rank when
// below n.
__device__ __forceinline__ bool in_tile(int u, int j, uint32_t n) {
  return (static_cast<uint32_t>(u) * kSpTileBlock + threadIdx.x) * 4 + static_cast<uint32_t>(j) < n;
}

// Radix digits of the top-K cut, most significant first.
template <int PASS>
struct Digit {
  static constexpr uint32_t kShift = PASS == 0 ? 21 : (PASS == 1 ? 10 : 0);
  static constexpr uint32_t kBins = PASS == 2 ? 1024 : 2048;
  static constexpr uint32_t kHigh = PASS == 0 ? 0u : (PASS == 1 ? 0xFFE00000u : 0xFFFFFC00u);
};

// ----------------------------------------------------------------- kernels

// Histogram `pass` of rank r: the slot passes' (0, 1, 2) and the fallback's.
__device__ __forceinline__ uint32_t* hist_of(const SparseArgs& a, uint32_t pass, uint32_t r) {
  return a.hist + (static_cast<uint64_t>(pass) * a.world + r) * kSpBins;
}

// Top-K: a rank whose first gather holds fewer than K candidates (its sampled
// bound missed) takes the exact fallback.
__device__ __forceinline__ bool needs_fallback(const SparseArgs& a, uint32_t r) {
  return a.state[kSpState * r + kStCand] < a.k;
}

// Per rank: zero the histograms and the per-tile counts, and set the
// selection state: cut key 0 with K still to find, no candidate yet.  K = 0
// selects nothing: the cut key, the gather bound and the guess are then
// above every key.  NT lanes of a workgroup of the rank.  SAMPLED: the
// sampling kernel calls it and then sets the gather bound and the guess
// itself, so those two fields are left alone here (one writer each).
template <uint32_t NT, bool SAMPLED = false>
__device__ __forceinline__ void init_rank(const SparseArgs& a, uint32_t r) {
  for (uint32_t p = 0; p < kHistCount; ++p) {
    uint32_t* h = hist_of(a, p, r);
    for (uint32_t i = threadIdx.x; i < kSpBins; i += NT) h[i] = 0;
  }
  const uint32_t nt = a.tiles + 1;
  for (uint32_t i = threadIdx.x; i < nt; i += NT) {
    a.tile_slot[r * nt + i] = 0;
    a.tile_cnt[r * nt + i] = 0;
    a.tile_eqc[r * nt + i] = 0;
  }
  if (threadIdx.x == 0) {
    uint32_t* st = a.state + kSpState * r;
    const uint32_t none = a.k == 0 ? 0xFFFFFFFFu : 0u;  // K = 0: above every key
    st[kStCut] = none;
    st[kStNeed] = a.k;
    st[kStCand] = 0;
    if constexpr (!SAMPLED) {
      st[kStBound] = none;
      st[kStGuess] = none;
    }
  }
}

// One workgroup per rank (top-K with K > 0: the sampling kernel does it).
__global__ __launch_bounds__(kBlock) void sp_init_kernel(const SparseArgs a) { init_rank<kBlock>(a, blockIdx.x); }

// Workgroup-local histogram -> the rank's histogram in HBM (NT lanes).
template <uint32_t BINS, uint32_t NT = kBlock>
__device__ __forceinline__ void merge_hist(const uint32_t* h, uint32_t* gh) {
  __syncthreads();
  for (uint32_t i = threadIdx.x; i < BINS; i += NT)
    if (h[i] != 0) atomicAdd(&gh[i], h[i]);
}

template <uint32_t NT = kBlock>
__device__ __forceinline__ void zero_hist(uint32_t* h) {
  for (uint32_t i = threadIdx.x; i < kSpBins; i += NT) h[i] = 0;
  __syncthreads();
}

// One step of the radix select: the bin of a BINS-bin histogram (of the keys
// matching the cut's higher digits) in which the need-th largest key lies,
// walking the bins from the top: the first bin at which the running count
// reaches `need` (1 <= need <= the histogram's total).  Every one of the NT
// lanes gets the bin and the count of keys in the bins above it.  `scratch`
// is NT / 64 words of LDS, `sh` two.
template <uint32_t BINS, uint32_t NT>
__device__ __forceinline__ void find_digit(const uint32_t* gh, uint32_t need, uint32_t* scratch, uint32_t* sh,
                                           uint32_t& bin, uint32_t& above_bin) {
  constexpr uint32_t kPer = BINS / NT;
  static_assert(kPer * NT == BINS, "whole bins per lane");
  // thread i holds bins top, top-1, ..., top-kPer+1 (thread 0 the highest)
  const uint32_t top = BINS - 1 - threadIdx.x * kPer;
  uint32_t c[kPer];
  uint32_t sum = 0;
#pragma unroll
  for (uint32_t i = 0; i < kPer; ++i) {
    c[i] = gh[top - i];
    sum += c[i];
  }
  if (threadIdx.x == 0) {
    sh[0] = 0;
    sh[1] = 0;
  }
  uint32_t total;
  const uint32_t above = block_excl<NT / 64>(sum, scratch, total);  // barriers order sh's reset first
  if (above < need && need <= above + sum) {
    uint32_t run = above;
    for (uint32_t i = 0; i < kPer; ++i) {
      if (run + c[i] >= need) {
        sh[0] = top - i;
        sh[1] = run;
        break;
      }
      run += c[i];
    }
  }
  __syncthreads();
  bin = sh[0];
  above_bin = sh[1];
}

// The cut after radix pass P: the cut so far and the entries still to take
// (before pass 0: no digit fixed, K), extended by the digit of pass P in
// which the needed key lies, from pass P's complete histogram.  Every
// workgroup of the kernel after pass P computes it for itself; the rank's
// first workgroup records it (fields kStCut0 / kStCut1 / kStCut and their
// counts) for the kernels after that one.
template <int P>
__device__ __forceinline__ uint32_t pick_cut(const SparseArgs& a, uint32_t r, uint32_t grp, uint32_t* scratch,
                                             uint32_t* sh) {
  using Dg = Digit<P>;
  uint32_t* st = a.state + kSpState * r;
  const uint32_t prefix = P == 0 ? 0u : st[P == 1 ? kStCut0 : kStCut1];
  const uint32_t need = P == 0 ? a.k : st[P == 1 ? kStNeed0 : kStNeed1];
  uint32_t bin, above;
  find_digit<Dg::kBins, kBlock>(hist_of(a, P, r), need, scratch, sh, bin, above);
  const uint32_t cut = prefix | (bin << Dg::kShift);
  if (grp == 0 && threadIdx.x == 0) {
    st[P == 0 ? kStCut0 : (P == 1 ? kStCut1 : kStCut)] = cut;
    st[P == 0 ? kStNeed0 : (P == 1 ? kStNeed1 : kStNeed)] = need - above;
  }
  return cut;
}

// Top-K fallback, over every element of a rank whose sampled bound missed:
// histogram of the top digit of g.  With an accumulation the first gather
// left, at each of its candidates, the residual of a sent entry in the
// accumulation buffer, and g in the tile's slot: those g are counted from
// the slot and put back, so that the buffer holds g everywhere again for
// the fallback's gather.  Ranks that need no fallback leave at once.
template <bool ACC>
__global__ __launch_bounds__(kSpTileBlock) void sp_hist0_fb_kernel(const SparseArgs a) {
  using Dg = Digit<0>;
  __shared__ uint32_t h[kSpBins];
  __shared__ uint32_t cand[kSpTile / 32];  // the tile's first-gather candidates
  const uint32_t r = blockIdx.x / a.hist_groups;
  if (!needs_fallback(a, r)) return;
  const uint32_t grp = blockIdx.x - r * a.hist_groups;
  zero_hist<kSpTileBlock>(h);
  const float* key = ACC ? a.accum[r] : a.grad[r];
  const uint32_t t0 = grp * a.hist_chunk;
  const uint32_t t1 = min(a.tiles, t0 + a.hist_chunk);
  for (uint32_t t = t0; t < t1; ++t) {
    const uint32_t n = tile_len(a, t);
    const uint64_t base = static_cast<uint64_t>(t) * kSpTile;
    if constexpr (ACC) {
      for (uint32_t i = threadIdx.x; i < kSpTile / 32; i += kSpTileBlock) cand[i] = 0;
      __syncthreads();
      const uint32_t c = min(a.tile_slot[r * (a.tiles + 1) + t], n);
      const uint64_t slot = (static_cast<uint64_t>(r) * a.tiles + t) * kSpTile;
      for (uint32_t e = threadIdx.x; e < c; e += kSpTileBlock) {
        const uint32_t local = min(a.gap_idx[slot + e], n - 1);
        const float v = a.gap_val[slot + e];
        atomicOr(&cand[local >> 5], 1u << (local & 31u));
        atomicAdd(&h[order_key(v) >> Dg::kShift], 1u);
        a.accum[r][base + local] = v;
      }
      __syncthreads();
    }
    float x[kSpUnits][4];
    load_tile<false>(key, nullptr, base, n, x);
#pragma unroll
    for (int u = 0; u < static_cast<int>(kSpUnits); ++u)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t local = (static_cast<uint32_t>(u) * kSpTileBlock + threadIdx.x) * 4 + j;
        const bool counted = ACC && ((cand[local >> 5] >> (local & 31u)) & 1u);
        if (in_tile(u, j, n) && !counted) atomicAdd(&h[order_key(x[u][j]) >> Dg::kShift], 1u);
      }
    if constexpr (ACC) __syncthreads();  // the bitmap is reused by the next tile
  }
  merge_hist<Dg::kBins, kSpTileBlock>(h, hist_of(a, kHistFallback, r));
}

// Top-K sample of a rank of n keys: m = min(n, kSampleMax) keys, in runs
// of 16 consecutive elements (one 64-byte line) spread evenly over the rank,
// and the rank j (from the top) of the sample key taken as the gather
// bound: ceil(K m / n) + 4 sqrt(ceil(K m / n)) + 4.  That key is expected to
// have about j n / m keys at or above it, comfortably more than K.  j > m
// means the bound is 0: everything is gathered.
struct SamplePlan {
  uint32_t m, kk, j;    // sample size, K scaled to it, the bound's rank
  uint64_t run_stride;  // elements from one sampled run of 16 to the next
  __device__ explicit SamplePlan(const SparseArgs& a) {
    const uint64_t n = a.count;
    m = static_cast<uint32_t>(min<uint64_t>(n, kSampleMax));
    run_stride = 16 * max<uint64_t>(1, n / kSampleMax);
    kk = static_cast<uint32_t>((static_cast<uint64_t>(a.k) * m + n - 1) / n);
    uint64_t root = 0;
    while ((root + 1) * (root + 1) <= kk) ++root;  // isqrt, kk <= kSampleMax
    j = static_cast<uint32_t>(kk + 4 * root + 4);
  }
  // Element of sample key s < m: run s / 16, position s % 16 in it.  With
  // n <= kSampleMax the sample is every element.
  __device__ uint64_t index(uint32_t s) const { return (s >> 4) * run_stride + (s & 15u); }
};

// Top-K, one workgroup of kSampleBlock lanes per rank, from one histogram
// of the 14-bit key prefixes (about 2% of the value) of the sampled keys of
// g = grad + acc:
// - the gather bound, the lower edge of the j-th largest sampled key's
//   prefix.  Everything at or above it is gathered; if that is fewer than K
//   keys the sample misled, and the exact fallback takes over;
// - the guess, the same for the ceil(K m / n)-th largest sampled key: an
//   estimate of the cut.  At keys from the guess up, the gather stores the
//   residual of a sent entry, below it g; the combine corrects the
//   candidates on the wrong side, which are few when the guess is good.
// The result never depends on the sample.
template <bool ACC>
__global__ __launch_bounds__(kSampleBlock) void sp_sample_kernel(const SparseArgs a) {
  constexpr int kWaves = kSampleBlock / 64;
  constexpr uint32_t kPer = kSampleMax / kSampleBlock;
  constexpr uint32_t kBatch = 16;
  constexpr uint32_t kBins = 16384, kShift = 18;
  constexpr uint32_t kLaneBins = kBins / kSampleBlock;
  __shared__ uint32_t h[kBins];
  __shared__ uint32_t scratch[kWaves];
  const uint32_t r = blockIdx.x;
  // The rank's initial state first (all but the bound and the guess, which
  // are set below whatever the sample holds).
  init_rank<kSampleBlock, true>(a, r);
  __syncthreads();
  const SamplePlan p(a);
  if (p.j > p.m) {  // everything is gathered, and guessed sent
    if (threadIdx.x == 0) {
      a.state[kSpState * r + kStBound] = 0;
      a.state[kSpState * r + kStGuess] = 0;
    }
    return;
  }
  const float* g = a.grad[r];
  const float* acc = ACC ? a.accum[r] : nullptr;
  for (uint32_t i = threadIdx.x; i < kBins; i += kSampleBlock) h[i] = 0;
  __syncthreads();
#pragma unroll 1
  for (uint32_t q0 = 0; q0 < kPer; q0 += kBatch) {
    // consecutive lanes take consecutive sample keys: 16 lanes per run
    float gv[kBatch], av[kBatch];
#pragma unroll
    for (uint32_t q = 0; q < kBatch; ++q) {
      const uint64_t idx = p.index(min(threadIdx.x + (q0 + q) * kSampleBlock, p.m - 1));
      gv[q] = g[idx];
      if constexpr (ACC) av[q] = acc[idx];
    }
#pragma unroll
    for (uint32_t q = 0; q < kBatch; ++q)
      if (threadIdx.x + (q0 + q) * kSampleBlock < p.m)
        atomicAdd(&h[order_key(ACC ? gv[q] + av[q] : gv[q]) >> kShift], 1u);
  }
  __syncthreads();
  // thread i holds bins top, top-1, ..., top-kLaneBins+1 (thread 0 the highest)
  const uint32_t top = kBins - 1 - threadIdx.x * kLaneBins;
  uint32_t c[kLaneBins];
  uint32_t sum = 0;
#pragma unroll
  for (uint32_t i = 0; i < kLaneBins; ++i) {
    c[i] = h[top - i];
    sum += c[i];
  }
  uint32_t total;
  const uint32_t above = block_excl<kWaves>(sum, scratch, total);
  // the bin of the rank-th largest sampled key, in the one lane that holds it
  // (1 <= rank <= m = total)
  auto bin_of = [&](uint32_t rank) {
    uint32_t run = above, bin = top;
#pragma unroll
    for (uint32_t i = 0; i < kLaneBins; ++i) {
      if (run < rank) bin = top - i;
      run += c[i];
    }
    return bin << kShift;
  };
  if (above < p.j && p.j <= above + sum) a.state[kSpState * r + kStBound] = bin_of(p.j);
  if (above < p.kk && p.kk <= above + sum) a.state[kSpState * r + kStGuess] = bin_of(p.kk);
}

static_assert(kSpUnits == 1, "compact_to_slot takes one element group per lane");

// Lanes below this one whose bit is set in a wave-wide mask.
__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u));
}

// The flagged entries of this tile (f[0][j] set: element 4 lane + j, value
// x[0][j]) into its slot, in index order; returns their count.  Lane
// positions come from one ballot per element group and a sum over the
// waves; the entries are staged in LDS and then written as whole 16-byte
// vectors from the slot's start.  Written straight from each lane (two
// scattered 4-byte stores per entry), the slot stores cost the compaction
// 7% (1,064 against 991 us without them, W = 8 x 64 Mi fp32).  Entries
// past the count in the last vector are junk inside the slot, which no
// reader looks at.  Two barriers; the first orders every read of the
// previous call's staging before this call's writes, so the function may run
// once per tile in a loop.
__device__ __forceinline__ uint32_t compact_to_slot(const SparseArgs& a, uint64_t slot,
                                                    const uint32_t (&f)[kSpUnits][4],
                                                    const float (&x)[kSpUnits][4], uint32_t* scratch) {
  constexpr uint32_t kWaves = kSpTileBlock / 64;
  __shared__ __align__(16) uint32_t st_idx[kSpTile];
  __shared__ __align__(16) float st_val[kSpTile];
  uint32_t at = 0, wave_total = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint64_t m = __ballot(f[0][j] != 0u);
    at += lanes_below(m);
    wave_total += static_cast<uint32_t>(__popcll(m));
  }
  const uint32_t w = threadIdx.x >> 6;
  if ((threadIdx.x & 63u) == 0) scratch[w] = wave_total;
  __syncthreads();
  uint32_t tot = 0;
#pragma unroll
  for (uint32_t i = 0; i < kWaves; ++i) {
    const uint32_t c = scratch[i];
    at += i < w ? c : 0u;
    tot += c;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (f[0][j]) {
      st_idx[at] = threadIdx.x * 4 + j;
      st_val[at] = x[0][j];
    }
    at += f[0][j];
  }
  __syncthreads();
  if (threadIdx.x * 4 < tot) {
    const uint32_t e = threadIdx.x * 4;
    *reinterpret_cast<uint4*>(a.gap_idx + slot + e) = *reinterpret_cast<const uint4*>(st_idx + e);
    *reinterpret_cast<float4*>(a.gap_val + slot + e) = *reinterpret_cast<const float4*>(st_val + e);
  }
  return tot;
}

// Rank and tile of workgroup b in a (rank, tile) grid; false past the end.
__device__ __forceinline__ bool rank_tile(const SparseArgs& a, uint32_t& r, uint32_t& t) {
  const uint32_t lin = xcd_tile(blockIdx.x, gridDim.x);
  if (lin >= a.world * a.tiles) return false;
  r = lin / a.tiles;
  t = lin - r * a.tiles;
  return true;
}

// Every key of tile t of rank r at or above `lo` into the tile's slot, in
// index order.  COUNT: also add the tile's count to the rank's candidates
// (the first gather; the fallback's test reads the sum).
template <bool COUNT>
__device__ __forceinline__ void gather_tile(const SparseArgs& a, uint32_t r, uint32_t t, uint32_t lo,
                                            const float (&x)[kSpUnits][4], uint32_t n, uint32_t* scratch) {
  uint32_t f[kSpUnits][4];
#pragma unroll
  for (int u = 0; u < static_cast<int>(kSpUnits); ++u)
#pragma unroll
    for (int j = 0; j < 4; ++j) f[u][j] = (in_tile(u, j, n) && order_key(x[u][j]) >= lo) ? 1u : 0u;
  const uint64_t slot = (static_cast<uint64_t>(r) * a.tiles + t) * kSpTile;
  const uint32_t cnt = compact_to_slot(a, slot, f, x, scratch);
  if (threadIdx.x == 0) {
    a.tile_slot[r * (a.tiles + 1) + t] = cnt;
    if (COUNT && cnt != 0) atomicAdd(&a.state[kSpState * r + kStCand], cnt);
  }
}

// What the accumulation buffer holds after a gather: at keys from the guess
// up (all of them candidates) the residual of a sent entry, g - (0 + g),
// elsewhere g itself, the residual of an entry not sent.  The combine
// corrects the candidates that the guess put on the wrong side of the cut.
__device__ __forceinline__ void store_residual(float* acc, uint64_t base, uint32_t n, uint32_t guess,
                                               const float (&x)[kSpUnits][4]) {
  float y[kSpUnits][4];
#pragma unroll
  for (int u = 0; u < static_cast<int>(kSpUnits); ++u)
#pragma unroll
    for (int j = 0; j < 4; ++j) y[u][j] = order_key(x[u][j]) >= guess ? x[u][j] - (0.0f + x[u][j]) : x[u][j];
  store_tile(acc, base, n, y);
}

// Top-K gather, one workgroup per tile, against the sampled bound
// (kStBound).  It forms g = grad + acc, and with an accumulation stores the
// residual each entry has if the candidates are exactly the entries sent
// (g - 0 = g for the rest).  Later kernels read the slots only.
template <bool ACC>
__global__ __launch_bounds__(kSpTileBlock) void sp_gather_kernel(const SparseArgs a) {
  __shared__ uint32_t scratch[kSpTileBlock / 64];
  uint32_t r, t;
  if (!rank_tile(a, r, t)) return;
  const uint32_t lo = a.state[kSpState * r + kStBound];
  const uint64_t base = static_cast<uint64_t>(t) * kSpTile;
  const uint32_t n = tile_len(a, t);
  float x[kSpUnits][4];
  load_tile<ACC>(a.grad[r], ACC ? a.accum[r] : nullptr, base, n, x);
  if constexpr (ACC) store_residual(a.accum[r], base, n, a.state[kSpState * r + kStGuess], x);
  gather_tile<true>(a, r, t, lo, x, n, scratch);
}

// The fallback's gather, for a rank whose sampled bound missed (its groups
// walk the rank's tiles; other ranks leave at once), from g: the gradient,
// or the accumulation buffer as the fallback's histogram restored it, which
// then gets the guessed residuals as the first gather would store them.
// Its bound is the lower edge of the K-th largest key's top-digit bin in the
// fallback's histogram, which every workgroup finds for itself; the guess is
// raised to it if below, so that every key given the sent residual is
// gathered (the rank's first workgroup records both).
template <bool ACC>
__global__ __launch_bounds__(kSpTileBlock) void sp_gather_fb_kernel(const SparseArgs a) {
  __shared__ uint32_t scratch[kSpTileBlock / 64];
  __shared__ uint32_t sh[2];
  const uint32_t r = blockIdx.x / a.hist_groups;
  if (!needs_fallback(a, r)) return;
  const uint32_t grp = blockIdx.x - r * a.hist_groups;
  uint32_t bin, above;
  find_digit<Digit<0>::kBins, kSpTileBlock>(hist_of(a, kHistFallback, r), a.k, scratch, sh, bin, above);
  const uint32_t lo = bin << Digit<0>::kShift;
  // the recorded guess is either the sample's or already raised to lo: the same max
  const uint32_t guess = max(a.state[kSpState * r + kStGuess], lo);
  if (grp == 0 && threadIdx.x == 0) {
    a.state[kSpState * r + kStBound] = lo;
    a.state[kSpState * r + kStGuess] = guess;
  }
  const float* key = ACC ? a.accum[r] : a.grad[r];
  const uint32_t t1 = min(a.tiles, (grp + 1) * a.hist_chunk);
  for (uint32_t t = grp * a.hist_chunk; t < t1; ++t) {
    const uint32_t n = tile_len(a, t);
    float x[kSpUnits][4];
    load_tile<false>(key, nullptr, static_cast<uint64_t>(t) * kSpTile, n, x);
    if constexpr (ACC) store_residual(a.accum[r], static_cast<uint64_t>(t) * kSpTile, n, guess, x);
    gather_tile<false>(a, r, t, lo, x, n, scratch);
  }
}

// Sum over the 64 lanes of a wave, in every lane.
__device__ __forceinline__ uint32_t wave_sum(uint32_t v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
  return v;
}

// Walks the slots of tiles [t0, t1) of rank r: each wave of the workgroup
// takes every (kBlock / 64)-th tile, its lanes the tile's entries.  The
// lanes first load the entry counts of the wave's next 64 tiles at once,
// then the first 64 entries of 4 tiles at a time (measured against 16), so
// that few loads wait on each other.  fn(tile, value, valid, last) runs for
// every entry of a tile (valid), in tile order, and with last set on the
// tile's final call, once per 64 entries (a tile with no entry gets one call
// with none valid).
template <class F>
__device__ __forceinline__ void walk_slots(const SparseArgs& a, uint32_t r, uint32_t t0, uint32_t t1, F&& fn) {
  constexpr uint32_t kWaves = kBlock / 64;
  constexpr uint32_t kAhead = 4;
  const uint32_t wave = threadIdx.x >> 6, lane = threadIdx.x & 63u;
  const uint32_t* cnt = a.tile_slot + r * (a.tiles + 1);
  const float* slots = a.gap_val + static_cast<uint64_t>(r) * a.tiles * kSpTile;
  for (uint32_t tb = t0 + wave; tb < t1; tb += 64 * kWaves) {
    const uint32_t mine = tb + lane * kWaves;
    const uint32_t c_l = mine < t1 ? min(cnt[mine], kSpTile) : 0u;
    const uint32_t nt = min(64u, (t1 - tb + kWaves - 1) / kWaves);
    for (uint32_t i = 0; i < nt; i += kAhead) {
      uint32_t c[kAhead];
      float v[kAhead];
#pragma unroll
      for (uint32_t k = 0; k < kAhead; ++k) {
        const uint32_t t = tb + (i + k) * kWaves;
        c[k] = i + k < nt ? __shfl(c_l, i + k, 64) : 0u;
        v[k] = lane < c[k] ? slots[static_cast<uint64_t>(t) * kSpTile + lane] : 0.0f;
      }
#pragma unroll
      for (uint32_t k = 0; k < kAhead; ++k) {
        if (i + k >= nt) break;
        const uint32_t t = tb + (i + k) * kWaves;
        fn(t, v[k], lane < c[k], c[k] <= 64);
        // a tile with more than 64 entries: 4 chunks of 64 loaded at a time
        for (uint32_t e0 = 64; e0 < c[k]; e0 += 4 * 64) {
          float w4[4];
#pragma unroll
          for (uint32_t q = 0; q < 4; ++q) {
            const uint32_t e = e0 + q * 64 + lane;
            w4[q] = e < c[k] ? slots[static_cast<uint64_t>(t) * kSpTile + e] : 0.0f;
          }
#pragma unroll
          for (uint32_t q = 0; q < 4; ++q)
            if (e0 + q * 64 < c[k]) fn(t, w4[q], e0 + q * 64 + lane < c[k], e0 + (q + 1) * 64 >= c[k]);
        }
      }
    }
  }
}

// Top-K, over the slots: histogram of digit PASS among the keys matching
// the cut's higher digits.  Passes 1 and 2 first take the previous pass's
// digit (pick_cut).
template <int PASS>
__global__ __launch_bounds__(kBlock) void sp_hist_slots_kernel(const SparseArgs a) {
  using Dg = Digit<PASS>;
  __shared__ uint32_t h[kSpBins];
  __shared__ uint32_t scratch[kBlock / 64];
  __shared__ uint32_t sh[2];
  const uint32_t r = blockIdx.x / a.hist_groups;
  const uint32_t grp = blockIdx.x - r * a.hist_groups;
  uint32_t prefix = 0;
  if constexpr (PASS > 0) prefix = pick_cut<PASS - 1>(a, r, grp, scratch, sh);
  zero_hist(h);
  const uint32_t t0 = grp * a.hist_chunk;
  walk_slots(a, r, t0, min(a.tiles, t0 + a.hist_chunk), [&](uint32_t, float v, bool valid, bool) {
    const uint32_t k = order_key(v);
    if (valid && (k & Dg::kHigh) == prefix) atomicAdd(&h[(k >> Dg::kShift) & (Dg::kBins - 1)], 1u);
  });
  merge_hist<Dg::kBins>(h, hist_of(a, PASS, r));
}

// Flags of a top-K candidate against the cut: 1 = above it (sent), 0x10000 =
// equal to it (sent while ties are left, in index order), 0 = below.
__device__ __forceinline__ uint32_t cut_flags(float v, uint32_t cut) {
  const uint32_t k = order_key(v);
  return k > cut ? 1u : (k == cut ? 0x10000u : 0u);
}

// Top-K, over the slots: per tile, the candidates above the cut and those
// equal to it, after taking the last digit of the cut (pick_cut).
__global__ __launch_bounds__(kBlock) void sp_slot_count_kernel(const SparseArgs a) {
  __shared__ uint32_t scratch[kBlock / 64];
  __shared__ uint32_t sh[2];
  const uint32_t r = blockIdx.x / a.hist_groups;
  const uint32_t grp = blockIdx.x - r * a.hist_groups;
  const uint32_t cut = pick_cut<2>(a, r, grp, scratch, sh);
  const uint32_t t0 = grp * a.hist_chunk;
  uint32_t f = 0;  // this lane's flags in the current tile
  walk_slots(a, r, t0, min(a.tiles, t0 + a.hist_chunk), [&](uint32_t t, float v, bool valid, bool last) {
    if (valid) f += cut_flags(v, cut);
    if (last) {
      const uint32_t tot = wave_sum(f);
      f = 0;
      if ((threadIdx.x & 63u) == 0) {
        const uint32_t i = r * (a.tiles + 1) + t;
        a.tile_cnt[i] = tot & 0xFFFFu;
        a.tile_eqc[i] = tot >> 16;
      }
    }
  });
}

// Threshold mode, over every element: per tile, the entries to send
// (|g| >= threshold, g != 0) in index order into the tile's slot, their
// count, and with an accumulation the final residual: g minus the
// thresholded array, which keeps a +-0 reaching the threshold (a sent inf
// leaves NaN).
template <bool ACC>
__global__ __launch_bounds__(kSpTileBlock) void sp_compact_kernel(const SparseArgs a) {
  __shared__ uint32_t scratch[kSpTileBlock / 64];
  uint32_t r, t;
  if (!rank_tile(a, r, t)) return;
  const uint64_t base = static_cast<uint64_t>(t) * kSpTile;
  const uint32_t n = static_cast<uint32_t>(min<uint64_t>(kSpTile, a.count - base));
  float x[kSpUnits][4];
  load_tile<ACC>(a.grad[r], ACC ? a.accum[r] : nullptr, base, n, x);
  const uint64_t slot = (static_cast<uint64_t>(r) * a.tiles + t) * kSpTile;
  uint32_t f[kSpUnits][4];
  float res[kSpUnits][4];
#pragma unroll
  for (int u = 0; u < static_cast<int>(kSpUnits); ++u)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float v = x[u][j];
      f[u][j] = (in_tile(u, j, n) && fabsf(v) >= a.threshold && v != 0.0f) ? 1u : 0u;
      if constexpr (ACC) res[u][j] = fabsf(v) >= a.threshold ? v - v : v - 0.0f;
    }
  if constexpr (ACC) store_tile(a.accum[r], base, n, res);
  const uint32_t cnt = compact_to_slot(a, slot, f, x, scratch);
  if (threadIdx.x == 0) {
    const uint32_t i = r * (a.tiles + 1) + t;
    a.tile_slot[i] = cnt;
    a.tile_cnt[i] = cnt;
  }
}

// Exclusive prefixes of a rank's tile counts, one workgroup per chunk of
// kScanChunk tiles.  A workgroup first sums the counts of every tile before
// its chunk itself (coalesced reads, many in flight), so no workgroup waits
// for another.  A tile's message offset is the entries sent for sure before
// it plus the ties before it, up to the number of ties to take; tile_eqb
// holds the ties before it.  The last chunk's workgroup also writes the
// message length into the last slot and nnz[r].
template <int MODE>
__global__ __launch_bounds__(kSpScanBlock) void sp_scan_kernel(const SparseArgs a) {
  constexpr bool TOPK = MODE == RSX_SPARSE_TOPK;
  constexpr uint32_t kPer = kScanChunk / kSpScanBlock;
  constexpr int kWaves = kSpScanBlock / 64;
  __shared__ uint32_t scratch[kWaves];
  const uint32_t n = a.tiles;
  const uint32_t groups = (n + kScanChunk - 1) / kScanChunk;
  const uint32_t r = blockIdx.x / groups;
  const uint32_t c0 = (blockIdx.x - r * groups) * kScanChunk;
  const uint32_t* cnt = a.tile_cnt + r * (n + 1);
  const uint32_t* eqc = a.tile_eqc + r * (n + 1);
  uint32_t* off = a.tile_off + r * (n + 1);
  uint32_t* eqb = a.tile_eqb + r * (n + 1);
  const uint32_t need = TOPK ? a.state[kSpState * r + kStNeed] : 0u;
  // this chunk's counts: 4 consecutive tiles per lane
  uint32_t s[kPer], e[kPer];
  uint32_t ss = 0, se = 0;
#pragma unroll
  for (uint32_t i = 0; i < kPer; ++i) {
    const uint32_t idx = c0 + threadIdx.x * kPer + i;
    s[i] = idx < n ? cnt[idx] : 0u;
    e[i] = (TOPK && idx < n) ? eqc[idx] : 0u;
    ss += s[i];
    se += e[i];
  }
  // every tile before the chunk
  uint32_t ps = 0, pe = 0;
#pragma unroll 8
  for (uint32_t i = threadIdx.x; i < c0; i += kSpScanBlock) {
    ps += cnt[i];
    if constexpr (TOPK) pe += eqc[i];
  }
  uint32_t carry_s, carry_e = 0, ts, te = 0;
  block_excl<kWaves>(ps, scratch, carry_s);
  if constexpr (TOPK) block_excl<kWaves>(pe, scratch, carry_e);
  uint32_t bs = block_excl<kWaves>(ss, scratch, ts) + carry_s;
  uint32_t be = 0;
  if constexpr (TOPK) be = block_excl<kWaves>(se, scratch, te) + carry_e;
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
  if (c0 + kScanChunk >= n && threadIdx.x == 0) {
    const uint32_t len = carry_s + ts + min(carry_e + te, need);
    off[n] = len;
    eqb[n] = carry_e + te;
    a.nnz[r] = len;
  }
}

// Per output tile: a zeroed LDS tile; for each rank in order, the entries of
// the tile's slot that are sent (threshold: all of them; top-K: those above
// the cut, and ties in index order while ties are left) are written to
// their place in the rank's message and added into the tile, and with an
// accumulation the residual of a top-K candidate that the gather guessed
// wrong is corrected; then the tile is stored to every rank's output.  One
// barrier per rank keeps the adds in rank order; entries of one rank have
// distinct indices.  Every rank's counts are read at once, and the next
// rank's first entries are loaded while this rank's are placed.  256 lanes,
// 4 vectors each: a tile holds few entries per rank, and more lanes spend the
// time in their per-rank scans and barriers (threshold combine 434 -> 481 us
// with 512 lanes, 662 us with 1024).
template <int MODE, bool ACC>
__global__ __launch_bounds__(kCombBlock) void sp_combine_kernel(const SparseArgs a) {
  constexpr uint32_t kVecs = kSpTile / 4 / kCombBlock;  // 16-byte vectors per lane of the output tile
  __shared__ float4 acc4[kSpTile / 4];
  __shared__ uint32_t meta[RSX_MAX_RANKS][5];  // entries, message offset, cut, ties to take, guess
  __shared__ uint32_t scratch[kCombBlock / 64];
  float* acc = reinterpret_cast<float*>(acc4);
  const uint32_t t = xcd_tile(blockIdx.x, gridDim.x);
  if (t >= a.tiles) return;
  const uint64_t base = static_cast<uint64_t>(t) * kSpTile;
  const uint32_t n = tile_len(a, t);
  const uint32_t world = a.world;
  const uint32_t tid = threadIdx.x;
#pragma unroll
  for (uint32_t u = 0; u < kVecs; ++u) acc4[u * kCombBlock + tid] = make_float4(0.f, 0.f, 0.f, 0.f);
  if (tid < world) {
    const uint32_t i = tid * (a.tiles + 1) + t;
    meta[tid][0] = min(a.tile_slot[i], n);
    meta[tid][1] = a.tile_off[i];
    if constexpr (MODE == RSX_SPARSE_TOPK) {
      const uint32_t need = a.state[kSpState * tid + kStNeed];
      const uint32_t before = a.tile_eqb[i];
      meta[tid][2] = a.state[kSpState * tid + kStCut];
      meta[tid][3] = need > before ? need - before : 0u;
      meta[tid][4] = a.state[kSpState * tid + kStGuess];
    } else {
      meta[tid][2] = 0;
      meta[tid][3] = 0;
      meta[tid][4] = 0;
    }
  }
  __syncthreads();

  // Entry c0 + tid of rank r's slot (index clamped into the tile).
  auto fetch = [&](uint32_t r, uint32_t c0, uint32_t& local, float& v) {
    const uint32_t e = c0 + tid;
    local = 0;
    v = 0.0f;
    if (e < meta[r][0]) {
      const uint64_t slot = (static_cast<uint64_t>(r) * a.tiles + t) * kSpTile;
      local = min(a.gap_idx[slot + e], kSpTile - 1);
      v = a.gap_val[slot + e];
    }
  };
  uint32_t nlocal;
  float nv;
  fetch(0, 0, nlocal, nv);
  for (uint32_t r = 0; r < world; ++r) {
    const uint32_t c = meta[r][0], off = meta[r][1], cut = meta[r][2], ties = meta[r][3], guess = meta[r][4];
    uint32_t local = nlocal;
    float v = nv;
    if (r + 1 < world) fetch(r + 1, 0, nlocal, nv);
    uint32_t* mi = a.msg_idx[r];
    float* mv = a.msg_val[r];
    uint32_t run = 0;  // packed counts of the chunks before this one
    for (uint32_t c0 = 0; c0 < c; c0 += kCombBlock) {
      // a slot with more than kCombBlock entries: its next chunk loads while
      // this one is placed
      uint32_t local_next = 0;
      float v_next = 0.0f;
      if (c0 + kCombBlock < c) fetch(r, c0 + kCombBlock, local_next, v_next);
      uint32_t f = 0;
      if (c0 + tid < c) {
        if constexpr (MODE == RSX_SPARSE_TOPK)
          f = cut_flags(v, cut);
        else
          f = 1u;
      }
      uint32_t p, tot;
      if constexpr (MODE == RSX_SPARSE_TOPK) {
        p = block_excl<kCombBlock / 64>(f, scratch, tot) + run;
      } else {  // every slot entry is sent: its place is its index
        p = run + tid;
        tot = min(c - c0, kCombBlock);
      }
      run += tot;
      const uint32_t sure_before = p & 0xFFFFu, ties_before = p >> 16;
      const bool sent = (f & 1u) || ((f >> 16) && ties_before < ties);
      const uint32_t pos = off + sure_before + min(ties_before, ties);
      if (sent && pos < a.cap) {  // always below: the counts bound every position
        mi[pos] = static_cast<uint32_t>(base) + local;
        mv[pos] = v;
        acc[local] = acc[local] + v;
      }
      // the candidates the gather's guess put on the wrong side of the cut
      if constexpr (MODE == RSX_SPARSE_TOPK && ACC) {
        if (c0 + tid < c) {
          const bool guessed_sent = order_key(v) >= guess;
          if (sent && !guessed_sent) a.accum[r][base + local] = v - (0.0f + v);
          if (!sent && guessed_sent) a.accum[r][base + local] = v;
        }
      }
      local = local_next;
      v = v_next;
    }
    __syncthreads();
  }
  uint4 q[kVecs];
#pragma unroll
  for (uint32_t u = 0; u < kVecs; ++u) {
    const float4 v = acc4[u * kCombBlock + tid];
    q[u] = make_uint4(__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z), __float_as_uint(v.w));
  }
  for (uint32_t r = 0; r < world; ++r) {
    const __amdgpu_buffer_rsrc_t rd = make_rsrc(a.out[r] + base, n * 4);
#pragma unroll
    for (uint32_t u = 0; u < kVecs; ++u) store_b128<kStoreStream>(rd, tid * 16, u * kCombBlock * 16, q[u]);
  }
}

__global__ void sp_zero_nnz_kernel(uint32_t* nnz, int world) {
  if (static_cast<int>(threadIdx.x) < world) nnz[threadIdx.x] = 0;
}

template <int MODE, bool ACC>
hipError_t launch_mode(SparseArgs a, hipStream_t s) {
  // Kernels that walk tiles: about 2048 workgroups in all (8 per CU), each
  // over whole tiles of one rank.  Measured faster than a grid that fits
  // the device in one resident round.
  const uint32_t groups = std::max<uint32_t>(1, std::min<uint32_t>(kSpWalkGroups / a.world, a.tiles));
  a.hist_chunk = (a.tiles + groups - 1) / groups;
  a.hist_groups = (a.tiles + a.hist_chunk - 1) / a.hist_chunk;
  void* args[] = {&a};
  auto go = [&](const void* fn, uint64_t grid, uint32_t block) {
    return hipLaunchKernel(fn, dim3(static_cast<uint32_t>(grid)), dim3(block), args, 0, s);
  };
  const uint64_t hg = static_cast<uint64_t>(a.world) * a.hist_groups;
  const uint64_t rt = xcd_grid(static_cast<uint64_t>(a.world) * a.tiles);
  hipError_t e = hipSuccess;
  if (MODE != RSX_SPARSE_TOPK || a.k == 0) e = go(reinterpret_cast<const void*>(&sp_init_kernel), a.world, kBlock);
  if constexpr (MODE == RSX_SPARSE_TOPK) {
    auto fn = [](auto k) { return reinterpret_cast<const void*>(k); };
    // the sample kernel also initialises each rank (init_rank)
    if (a.k > 0 && e == hipSuccess) e = go(fn(&sp_sample_kernel<ACC>), a.world, kSampleBlock);
    // The first gather also leaves g in the accumulation buffer, so it runs
    // even when K = 0 has nothing to select.
    if ((a.k > 0 || ACC) && e == hipSuccess) e = go(fn(&sp_gather_kernel<ACC>), rt, kSpTileBlock);
    if (a.k > 0) {
      if (e == hipSuccess) e = go(fn(&sp_hist0_fb_kernel<ACC>), hg, kSpTileBlock);
      if (e == hipSuccess) e = go(fn(&sp_gather_fb_kernel<ACC>), hg, kSpTileBlock);
      if (e == hipSuccess) e = go(fn(&sp_hist_slots_kernel<0>), hg, kBlock);
      if (e == hipSuccess) e = go(fn(&sp_hist_slots_kernel<1>), hg, kBlock);
      if (e == hipSuccess) e = go(fn(&sp_hist_slots_kernel<2>), hg, kBlock);
      if (e == hipSuccess) e = go(fn(&sp_slot_count_kernel), hg, kBlock);
    }
  } else {
    if (e == hipSuccess) e = go(reinterpret_cast<const void*>(&sp_compact_kernel<ACC>), rt, kSpTileBlock);
  }
  const uint64_t scan_groups = (a.tiles + kScanChunk - 1) / kScanChunk;
  if (e == hipSuccess)
    e = go(reinterpret_cast<const void*>(&sp_scan_kernel<MODE>), a.world * scan_groups, kSpScanBlock);
  if (e == hipSuccess)
    e = go(reinterpret_cast<const void*>(&sp_combine_kernel<MODE, ACC>), xcd_grid(a.tiles), kCombBlock);
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
