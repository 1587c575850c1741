// HBM bandwidth ceilings of the GPU this runs on: streaming read, copy and
// write, 16-byte lanes, XCD-contiguous tiles, buffer descriptors and the
// same cache hints as the library's kernels.  These bound what a
// reduce-scatter (mostly reads) and an all-reduce (as many writes as reads)
// can reach.  Two more patterns bound the sparsified all-reduce: reading two
// buffers and writing the second in place (its compaction and gather), and
// writing each tile to 8 buffers (its combine).  Prints one JSON line.
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

constexpr int kBlock = 256;
constexpr int kUnits = 4;                        // dwordx4 per lane per tile
constexpr unsigned kTileBytes = kBlock * kUnits * 16;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ unsigned xcd_tile(unsigned b, unsigned n) { return (b % 8) * (n / 8) + b / 8; }
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, kTileBytes, 0x00020000);
}

// MODE 0: read only; 1: copy; 2: write only; 3: dst += src (two reads, one
// write in place); 4: write each tile to 8 buffers (dst cut in 8, the grid
// covering one eighth).  The grid is a multiple of 8.
template <int MODE, int LOAD_AUX, int STORE_AUX>
__global__ __launch_bounds__(kBlock) void stream_kernel(const char* src, char* dst, float* sink) {
  const size_t off = size_t(xcd_tile(blockIdx.x, gridDim.x)) * kTileBytes;
  const unsigned voff = threadIdx.x * 16u;
  u32x4 v[kUnits];
  if (MODE == 0 || MODE == 1 || MODE == 3) {
    const __amdgpu_buffer_rsrc_t r = rsrc(src + off);
#pragma unroll
    for (int u = 0; u < kUnits; ++u) v[u] = __builtin_amdgcn_raw_buffer_load_b128(r, voff, u * kBlock * 16, LOAD_AUX);
  } else {
#pragma unroll
    for (int u = 0; u < kUnits; ++u) v[u] = u32x4{threadIdx.x, 1u, 2u, 3u};
  }
  if (MODE == 3) {
    const __amdgpu_buffer_rsrc_t r = rsrc(dst + off);
#pragma unroll
    for (int u = 0; u < kUnits; ++u) v[u] += __builtin_amdgcn_raw_buffer_load_b128(r, voff, u * kBlock * 16, LOAD_AUX);
  }
  if (MODE == 4) {
    const size_t part = size_t(gridDim.x) * kTileBytes;
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const __amdgpu_buffer_rsrc_t w = rsrc(dst + b * part + off);
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
    const __amdgpu_buffer_rsrc_t w = rsrc(dst + off);
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

}  // namespace

int main() {
  const size_t bytes = size_t(2) << 30;           // 2 GiB per buffer
  const unsigned tiles = unsigned(bytes / kTileBytes);  // 131072, a multiple of 8
  char *src, *dst;
  float* sink;
  CHECK(hipMalloc(&src, bytes));
  CHECK(hipMalloc(&dst, bytes));
  CHECK(hipMalloc(&sink, tiles * sizeof(float)));
  const dim3 grid(tiles), block(kBlock);
  auto gbs = [&](double moved, float ms) { return moved / (ms * 1e-3) / 1e9; };
  // The same read on a zeroed buffer, for comparison only.
  CHECK(hipMemset(src, 0, bytes));
  CHECK(hipDeviceSynchronize());
  const float r_nt_zero = median_ms([&] { hipLaunchKernelGGL((stream_kernel<0, 2, 0>), grid, block, 0, 0, src, dst, sink); });
  hipLaunchKernelGGL(fill_kernel, dim3(4096), dim3(256), 0, 0, reinterpret_cast<unsigned*>(src), bytes / 4);
  CHECK(hipGetLastError());
  CHECK(hipDeviceSynchronize());
  const float r_plain = median_ms([&] { hipLaunchKernelGGL((stream_kernel<0, 0, 0>), grid, block, 0, 0, src, dst, sink); });
  const float r_nt = median_ms([&] { hipLaunchKernelGGL((stream_kernel<0, 2, 0>), grid, block, 0, 0, src, dst, sink); });
  const float c_plain = median_ms([&] { hipLaunchKernelGGL((stream_kernel<1, 0, 0>), grid, block, 0, 0, src, dst, sink); });
  const float c_nt = median_ms([&] { hipLaunchKernelGGL((stream_kernel<1, 2, 2>), grid, block, 0, 0, src, dst, sink); });
  const float w_plain = median_ms([&] { hipLaunchKernelGGL((stream_kernel<2, 0, 0>), grid, block, 0, 0, src, dst, sink); });
  const float w_nt = median_ms([&] { hipLaunchKernelGGL((stream_kernel<2, 0, 2>), grid, block, 0, 0, src, dst, sink); });
  // dst += src needs dst to hold data too
  CHECK(hipMemcpy(dst, src, bytes, hipMemcpyDeviceToDevice));
  const float rw_nt = median_ms([&] { hipLaunchKernelGGL((stream_kernel<3, 2, 2>), grid, block, 0, 0, src, dst, sink); });
  const dim3 grid8(tiles / 8);  // a multiple of 8: each workgroup writes its tile to all 8 parts
  const float w8_plain = median_ms([&] { hipLaunchKernelGGL((stream_kernel<4, 0, 0>), grid8, block, 0, 0, src, dst, sink); });
  const float w8_nt = median_ms([&] { hipLaunchKernelGGL((stream_kernel<4, 0, 2>), grid8, block, 0, 0, src, dst, sink); });
  CHECK(hipGetLastError());
  printf("{\"ceilings\": \"HBM streaming, 2 GiB buffers\", \"unit\": \"GB/s\", "
         "\"read\": %.1f, \"read_nt\": %.1f, \"copy\": %.1f, \"copy_nt\": %.1f, "
         "\"write\": %.1f, \"write_nt\": %.1f, \"read2_write1_in_place_nt\": %.1f, "
         "\"write_8_buffers\": %.1f, \"write_8_buffers_nt\": %.1f, \"read_nt_zeroed_buffer\": %.1f}\n",
         gbs(bytes, r_plain), gbs(bytes, r_nt), gbs(2.0 * bytes, c_plain), gbs(2.0 * bytes, c_nt),
         gbs(bytes, w_plain), gbs(bytes, w_nt), gbs(3.0 * bytes, rw_nt), gbs(bytes, w8_plain), gbs(bytes, w8_nt),
         gbs(bytes, r_nt_zero));
  CHECK(hipFree(src));
  CHECK(hipFree(dst));
  CHECK(hipFree(sink));
  return 0;
}
