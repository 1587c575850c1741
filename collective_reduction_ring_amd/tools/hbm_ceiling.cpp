// HBM bandwidth ceilings of the GPU this runs on: streaming read, copy and
// write, 16-byte lanes, XCD-contiguous tiles, buffer descriptors and the
// same cache hints as the library's kernels.  These bound what a
// reduce-scatter (mostly reads) and an all-reduce (as many writes as reads)
// can reach; reading 8 buffers into a sum written to a ninth, or to all 8
// (in place) or to 8 other buffers, are the reduce-scatter's and the
// all-reduce's own patterns at W = 8 without the ring order; reading 16
// buffers into a sum written to a seventeenth is the reduce-scatter's at
// W = 16 (buffers 128 MiB apart, as 16 ranks of 128 MiB are).  Two more
// patterns bound the sparsified all-reduce: reading two
// buffers and writing the second in place (its compaction and gather), and
// writing each tile to 8 buffers (its combine).  Every pattern runs with
// 256, 512 and 1024 lanes of one vector each, with 256 lanes of four, and
// with 256 lanes of one at 6, 5, 4, 3 and 2 workgroups per CU (LDS reserved
// to cap them, as the library's launches do); the best is the ceiling.  Prints one JSON line: per pattern the best rate
// and the configuration that reached it, and the rate with 256 lanes of one
// vector.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <vector>

#define CHECK(x)                                                                        \
  do {                                                                                  \
    hipError_t e_ = (x);                                                                \
    if (e_ != hipSuccess) {                                                             \
      fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__);    \
      exit(1);                                                                          \
    }                                                                                   \
  } while (0)

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ unsigned xcd_tile(unsigned b, unsigned n) { return (b % 8) * (n / 8) + b / 8; }
template <unsigned BYTES>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, BYTES, 0x00020000);
}

// MODE 0: read only; 1: copy; 2: write only; 3: dst += src (two reads, one
// write in place); 4: write each tile to 8 buffers (dst cut in 8, the grid
// covering one eighth); 5: the sum of a tile of NB buffers (src cut in NB,
// the grid covering one NB-th) written to dst; 6: the same sum (NB = 8)
// written back to all 8 (in place); 7: to 8 other buffers.  B lanes of U
// vectors per tile; the grid is a multiple of 8.
template <int MODE, int LOAD_AUX, int STORE_AUX, int B, int U, int NB = 8>
__global__ __launch_bounds__(B) void stream_kernel(const char* src, char* dst, float* sink) {
  constexpr int kUnits = U, kBlock = B;
  constexpr unsigned kTileBytes = B * U * 16;
  const size_t off = size_t(xcd_tile(blockIdx.x, gridDim.x)) * kTileBytes;
  const unsigned voff = threadIdx.x * 16u;
  u32x4 v[kUnits];
  if (MODE == 0 || MODE == 1 || MODE == 3) {
    const __amdgpu_buffer_rsrc_t r = rsrc<kTileBytes>(src + off);
#pragma unroll
    for (int u = 0; u < kUnits; ++u) v[u] = __builtin_amdgcn_raw_buffer_load_b128(r, voff, u * kBlock * 16, LOAD_AUX);
  } else {
#pragma unroll
    for (int u = 0; u < kUnits; ++u) v[u] = u32x4{threadIdx.x, 1u, 2u, 3u};
  }
  if (MODE == 3) {
    const __amdgpu_buffer_rsrc_t r = rsrc<kTileBytes>(dst + off);
#pragma unroll
    for (int u = 0; u < kUnits; ++u) v[u] += __builtin_amdgcn_raw_buffer_load_b128(r, voff, u * kBlock * 16, LOAD_AUX);
  }
  if (MODE == 5 || MODE == 6 || MODE == 7) {
    const size_t part = size_t(gridDim.x) * kTileBytes;
    u32x4 w[NB][kUnits];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const __amdgpu_buffer_rsrc_t r = rsrc<kTileBytes>(src + b * part + off);
#pragma unroll
      for (int u = 0; u < kUnits; ++u) w[b][u] = __builtin_amdgcn_raw_buffer_load_b128(r, voff, u * kBlock * 16, LOAD_AUX);
    }
#pragma unroll
    for (int u = 0; u < kUnits; ++u) {
      v[u] = w[0][u];
#pragma unroll
      for (int b = 1; b < NB; ++b) v[u] += w[b][u];
    }
    if (MODE == 5) {
      const __amdgpu_buffer_rsrc_t d = rsrc<kTileBytes>(dst + off);
#pragma unroll
      for (int u = 0; u < kUnits; ++u) __builtin_amdgcn_raw_buffer_store_b128(v[u], d, voff, u * kBlock * 16, STORE_AUX);
    } else {
#pragma unroll
      for (int b = 0; b < 8; ++b) {
        // MODE 6 writes back over the 8 sources; MODE 7 to 8 separate buffers
        char* const base = MODE == 6 ? const_cast<char*>(src) : dst;
        const __amdgpu_buffer_rsrc_t d = rsrc<kTileBytes>(base + b * part + off);
#pragma unroll
        for (int u = 0; u < kUnits; ++u) __builtin_amdgcn_raw_buffer_store_b128(v[u], d, voff, u * kBlock * 16, STORE_AUX);
      }
    }
    return;
  }
  if (MODE == 4) {
    const size_t part = size_t(gridDim.x) * kTileBytes;
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const __amdgpu_buffer_rsrc_t w = rsrc<kTileBytes>(dst + b * part + off);
#pragma unroll
      for (int u = 0; u < kUnits; ++u)
        __builtin_amdgcn_raw_buffer_store_b128(v[u], w, voff, u * kBlock * 16, STORE_AUX);
    }
    return;
  }
  if (MODE == 0) {
    unsigned acc = 0;
#pragma unroll
    for (int u = 0; u < kUnits; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    if (acc == 0x9e3779b9u) sink[blockIdx.x] = float(acc);  // keeps the loads (sink has one slot per tile)
  } else {
    const __amdgpu_buffer_rsrc_t w = rsrc<kTileBytes>(dst + off);
#pragma unroll
    for (int u = 0; u < kUnits; ++u) __builtin_amdgcn_raw_buffer_store_b128(v[u], w, voff, u * kBlock * 16, STORE_AUX);
  }
}

// Source words from a multiplicative hash of their index: data like a real
// gradient's (the memory system moves all-zero lines measurably faster, so a
// zeroed buffer would overstate every ceiling).
__global__ void fill_kernel(unsigned* p, size_t n) {
  for (size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += size_t(gridDim.x) * blockDim.x) {
    const unsigned x = unsigned(i) * 0x9e3779b1u;
    p[i] = x ^ (x >> 15) ^ unsigned(i >> 32);
  }
}

template <class F>
float median_ms(F launch) {
  hipEvent_t a, b;
  CHECK(hipEventCreate(&a));
  CHECK(hipEventCreate(&b));
  for (int i = 0; i < 3; ++i) launch();
  CHECK(hipDeviceSynchronize());
  std::vector<float> t;
  for (int i = 0; i < 30; ++i) {
    CHECK(hipEventRecord(a));
    launch();
    CHECK(hipEventRecord(b));
    CHECK(hipEventSynchronize(b));
    float ms;
    CHECK(hipEventElapsedTime(&ms, a, b));
    t.push_back(ms);
  }
  CHECK(hipEventDestroy(a));
  CHECK(hipEventDestroy(b));
  std::sort(t.begin(), t.end());
  return t[t.size() / 2];
}

struct Best {
  double gbs = 0, first = 0;
  const char* cfg = "";
};

// Rate of one pattern in each lane configuration; the best and the first
// (256 lanes of one vector).
template <int MODE, int LA, int SA, int NB = 8>
Best measure(const char* src, char* dst, float* sink, size_t bytes, double moved) {
  Best best;
  auto one = [&](auto kernel, unsigned tile_bytes, unsigned block, const char* cfg, unsigned wg_per_cu = 8) {
    const unsigned tiles = unsigned(bytes / tile_bytes) / (MODE >= 4 ? NB : 1);  // a multiple of 8
    const unsigned lds = wg_per_cu >= 8 ? 0u : (160u * 1024u / wg_per_cu) & ~1023u;
    const float ms = median_ms([&] { hipLaunchKernelGGL(kernel, dim3(tiles), dim3(block), lds, 0, src, dst, sink); });
    CHECK(hipGetLastError());
    const double g = moved / (ms * 1e-3) / 1e9;
    fprintf(stderr, "pattern %d/%d/%d/%d  %-16s %8.1f GB/s\n", MODE, LA, SA, NB, cfg, g);
    if (best.first == 0) best.first = g;
    if (g > best.gbs) {
      best.gbs = g;
      best.cfg = cfg;
    }
  };
  one(stream_kernel<MODE, LA, SA, 256, 1, NB>, 256 * 16, 256, "256x1");
  one(stream_kernel<MODE, LA, SA, 512, 1, NB>, 512 * 16, 512, "512x1");
  one(stream_kernel<MODE, LA, SA, 1024, 1, NB>, 1024 * 16, 1024, "1024x1");
  if (NB <= 8) one(stream_kernel<MODE, LA, SA, 256, 4, NB>, 256 * 64, 256, "256x4");
  one(stream_kernel<MODE, LA, SA, 256, 1, NB>, 256 * 16, 256, "256x1, 6 WG/CU", 6);
  one(stream_kernel<MODE, LA, SA, 256, 1, NB>, 256 * 16, 256, "256x1, 5 WG/CU", 5);
  one(stream_kernel<MODE, LA, SA, 256, 1, NB>, 256 * 16, 256, "256x1, 4 WG/CU", 4);
  one(stream_kernel<MODE, LA, SA, 256, 1, NB>, 256 * 16, 256, "256x1, 3 WG/CU", 3);
  one(stream_kernel<MODE, LA, SA, 256, 1, NB>, 256 * 16, 256, "256x1, 2 WG/CU", 2);
  return best;
}

}  // namespace

int main() {
  const size_t bytes = size_t(2) << 30;  // 2 GiB per buffer
  char *src, *dst;
  float* sink;
  CHECK(hipMalloc(&src, bytes));
  CHECK(hipMalloc(&dst, bytes));
  CHECK(hipMalloc(&sink, bytes / (256 * 16) * sizeof(float)));  // one slot per tile of the smallest tiles
  // The same read on a zeroed buffer, for comparison only.
  CHECK(hipMemset(src, 0, bytes));
  CHECK(hipDeviceSynchronize());
  const Best r_nt_zero = measure<0, 2, 0>(src, dst, sink, bytes, double(bytes));
  hipLaunchKernelGGL(fill_kernel, dim3(4096), dim3(256), 0, 0, reinterpret_cast<unsigned*>(src), bytes / 4);
  CHECK(hipGetLastError());
  CHECK(hipDeviceSynchronize());
  const Best r_plain = measure<0, 0, 0>(src, dst, sink, bytes, double(bytes));
  const Best r_nt = measure<0, 2, 0>(src, dst, sink, bytes, double(bytes));
  const Best c_plain = measure<1, 0, 0>(src, dst, sink, bytes, 2.0 * bytes);
  const Best c_nt = measure<1, 2, 2>(src, dst, sink, bytes, 2.0 * bytes);
  const Best w_plain = measure<2, 0, 0>(src, dst, sink, bytes, double(bytes));
  const Best w_nt = measure<2, 0, 2>(src, dst, sink, bytes, double(bytes));
  // dst += src needs dst to hold data too
  CHECK(hipMemcpy(dst, src, bytes, hipMemcpyDeviceToDevice));
  const Best rw_nt = measure<3, 2, 2>(src, dst, sink, bytes, 3.0 * bytes);
  const Best w8_plain = measure<4, 0, 0>(src, dst, sink, bytes, double(bytes));
  const Best w8_nt = measure<4, 0, 2>(src, dst, sink, bytes, double(bytes));
  const Best r8w1 = measure<5, 2, 16>(src, dst, sink, bytes, bytes + bytes / 8.0);
  const Best r16w1 = measure<5, 2, 16, 16>(src, dst, sink, bytes, bytes + bytes / 16.0);
  const Best r8w8o = measure<7, 2, 2>(src, dst, sink, bytes, 2.0 * bytes);
  const Best r8w8 = measure<6, 2, 2>(src, dst, sink, bytes, 2.0 * bytes);  // last: it rewrites src
  printf("{\"ceilings\": \"HBM streaming, 2 GiB buffers; per pattern the best of 256x1, 512x1, 1024x1, "
         "256x4 (lanes x 16-byte vectors per lane) and 256x1 at 6..2 workgroups per CU, and the rate at "
         "256x1 uncapped\", \"unit\": \"GB/s\"");
  auto put = [](const char* name, const Best& b) {
    printf(", \"%s\": {\"best\": %.1f, \"at\": \"%s\", \"256x1\": %.1f}", name, b.gbs, b.cfg, b.first);
  };
  put("read", r_plain);
  put("read_nt", r_nt);
  put("copy", c_plain);
  put("copy_nt", c_nt);
  put("write", w_plain);
  put("write_nt", w_nt);
  put("read2_write1_in_place_nt", rw_nt);
  put("write_8_buffers", w8_plain);
  put("write_8_buffers_nt", w8_nt);
  put("read_8_sum_write_1", r8w1);
  put("read_16_sum_write_1", r16w1);
  put("read_8_sum_write_8_in_place", r8w8);
  put("read_8_sum_write_8_other_buffers", r8w8o);
  put("read_nt_zeroed_buffer", r_nt_zero);
  printf("}\n");
  CHECK(hipFree(src));
  CHECK(hipFree(dst));
  CHECK(hipFree(sink));
  return 0;
}
