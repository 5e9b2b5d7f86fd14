// A plain streaming read of a device buffer, for measuring the HBM read bandwidth the decode and
// compaction kernels are compared against: every thread reads 16-byte pieces in a grid-stride
// loop, eight in flight, and folds them into one word per workgroup (so that no load is dead).
#include "../common.h"
#include "../launch.h"

namespace sals {
namespace {

constexpr int kThreads = 256;
constexpr int kU = 8;

__global__ __launch_bounds__(kThreads) void hbm_read_kernel(const u32x4* __restrict__ src, size_t n,
                                                            uint32_t* __restrict__ sink) {
  __shared__ uint32_t red[kThreads / 64];
  const size_t stride = (size_t)gridDim.x * kThreads;
  uint32_t acc = 0;
  for (size_t base = (size_t)blockIdx.x * kThreads + threadIdx.x; base < n; base += stride * kU) {
    u32x4 v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const size_t i = base + (size_t)u * stride;
      v[u] = i < n ? src[i] : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

}  // namespace

hipError_t launch_hbm_read(const void* src, size_t bytes, uint32_t* sink, int blocks, hipStream_t st) {
  hbm_read_kernel<<<blocks, kThreads, 0, st>>>((const u32x4*)src, bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace sals
