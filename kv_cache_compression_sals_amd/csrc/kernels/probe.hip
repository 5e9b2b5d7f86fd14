// Probes of the machine's own peaks, which the kernels' fractions are also stated against:
//   hbm_read_kernel: a plain streaming read of a device buffer: every thread reads 16-byte pieces
//     in a grid-stride loop, eight in flight, and folds them into one word per workgroup (so that
//     no load is dead);
//   mfma_peak_kernel: bf16 32x32x16 MFMAs from registers only, four independent accumulators per
//     wave, folded into one word per workgroup. Measured on MI355X: 2.34-2.40 PFLOP/s with 2 to 8
//     accumulators; the 16x16x32 instruction needs 16 independent accumulators per wave to come
//     near that (2.27 PFLOP/s; 1.2-1.5 with 4 or 8).
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

constexpr int kAcc = 4;  // independent accumulators per wave
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

__global__ __launch_bounds__(kThreads) void mfma_peak_kernel(int iters, uint32_t* __restrict__ sink) {
  // operands from the thread index (not compile-time constants, so nothing folds away)
  const uint32_t seed = threadIdx.x * 2654435761u + blockIdx.x;
  bf16x8_t a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(float)((seed >> i) & 7u) * (__bf16)0.125f;
    b[i] = (__bf16)(float)((seed >> (i + 3)) & 7u) * (__bf16)0.0625f;
  }
  f32x16 acc[kAcc];
#pragma unroll
  for (int j = 0; j < kAcc; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[j][e] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < kAcc; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
  }
  float x = 0.f;
#pragma unroll
  for (int j = 0; j < kAcc; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) x += acc[j][e];
  uint32_t w = __float_as_uint(x);
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) w ^= (uint32_t)__shfl_xor((int)w, o);
  __shared__ uint32_t red[kThreads / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = w;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

}  // namespace

hipError_t launch_mfma_peak(int blocks, int iters, uint32_t* sink, hipStream_t st) {
  mfma_peak_kernel<<<blocks, kThreads, 0, st>>>(iters, sink);
  return hipGetLastError();
}

hipError_t launch_hbm_read(const void* src, size_t bytes, uint32_t* sink, int blocks, hipStream_t st) {
  hbm_read_kernel<<<blocks, kThreads, 0, st>>>((const u32x4*)src, bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace sals
