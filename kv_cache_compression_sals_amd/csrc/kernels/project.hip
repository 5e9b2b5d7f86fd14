// Latent projection of new cache rows (SALS 技术框架 stage 1; 关键设计 item 1 for P):
//   L[b][t0 + t][j] = sum_i X[b][t][i] * P[i][j]
// A dense contraction, so it runs on MFMA: each workgroup owns 64 tokens x 64 latent columns,
// each wave 16 tokens x 64 columns. The k dimension (D) is walked in chunks of 64. The X rows are
// read straight from HBM as the A operand (each lane a contiguous 16-element run per chunk); the
// P chunk is staged in LDS transposed (column-major) so that B fragments are contiguous 16-byte
// reads. Products accumulate in fp32 and are rounded once to the storage type.
#include "../common.h"
#include "../launch.h"

namespace sals {
namespace {

constexpr int kThreads = 256;
constexpr int KC = 64;       // k chunk
constexpr int KPAD = 8;      // LDS padding (elements) per transposed row
constexpr int NT = 64;       // latent columns per workgroup
constexpr int MT = 64;       // tokens per workgroup

template <class T>
__device__ __forceinline__ void store_out(typename T::elem* p, float v);
template <>
__device__ __forceinline__ void store_out<F32>(float* p, float v) { *p = v; }
template <>
__device__ __forceinline__ void store_out<BF16>(uint16_t* p, float v) {
  *p = (uint16_t)f32_to_bf16_bits(v);
}

// grid (ceil(T/64), ceil(r/64), B)
template <class T>
__global__ __launch_bounds__(kThreads) void project_kernel(const typename T::elem* __restrict__ X,
                                                           const typename T::elem* __restrict__ P,
                                                           typename T::elem* __restrict__ L, int T_,
                                                           int D, int r, int ctx_cap, int t0) {
  using elem = typename T::elem;
  constexpr int EPC = 16 / (int)sizeof(elem);  // elements per 16-byte chunk
  constexpr int RUN = KC / 4;                  // contiguous k elements per lane per chunk
  constexpr int NCH = RUN / EPC;               // 16-byte chunks per lane per chunk
  constexpr int STEPS = KC / T::KSTEP;         // MFMA steps per chunk
  constexpr int PST = KC + KPAD;
  __shared__ __attribute__((aligned(16))) elem PT[NT * PST];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n16 = lane & 15, q4 = lane >> 4;
  const int b = blockIdx.z;
  const int col0 = blockIdx.y * NT;
  const int tok = min(blockIdx.x * MT + wave * 16 + n16, T_ - 1);
  const elem* xrow = X + ((size_t)b * T_ + tok) * D + q4 * RUN;

  f32x4 acc[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int k0 = 0; k0 < D; k0 += KC) {
    __syncthreads();
    // P[k0 .. k0+KC)[col0 .. col0+NT) -> PT[col][k]
    for (int e = tid; e < KC * (NT / EPC); e += kThreads) {
      const int kk = e / (NT / EPC), cc = (e % (NT / EPC)) * EPC;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (col0 + cc < r) v = *(const u32x4*)(P + (size_t)(k0 + kk) * r + col0 + cc);
      const elem* ve = (const elem*)&v;
#pragma unroll
      for (int j = 0; j < EPC; ++j) PT[(cc + j) * PST + kk] = ve[j];
    }
    u32x4 ach[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) ach[c] = *(const u32x4*)(xrow + k0 + c * EPC);
    __syncthreads();
#pragma unroll
    for (int kb = 0; kb < STEPS; ++kb) {
      const typename T::frag a = frag_at<T>(ach, kb);
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const elem* bp = PT + (nb * 16 + n16) * PST + q4 * RUN + kb * T::KPL;
        typename T::frag bf;
        if constexpr (T::HILO)
          bf = *(const bf16x8_t*)bp;
        else
          bf = *bp;
        acc[nb] = T::mma(a, bf, acc[nb]);
      }
    }
  }
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    const int col = col0 + nb * 16 + n16;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = blockIdx.x * MT + wave * 16 + q4 * 4 + i;
      if (t < T_ && col < r) store_out<T>(L + ((size_t)b * ctx_cap + t0 + t) * r + col, acc[nb][i]);
    }
  }
}

}  // namespace

hipError_t launch_project(int dtype, const void* X, const void* P, void* L, int B, int T, int D,
                          int r, int ctx_cap, int t0, hipStream_t st) {
  dim3 grid(ceil_div(T, MT), ceil_div(r, NT), B);
  if (dtype == 0)
    project_kernel<F32><<<grid, kThreads, 0, st>>>((const float*)X, (const float*)P, (float*)L, T,
                                                   D, r, ctx_cap, t0);
  else
    project_kernel<BF16><<<grid, kThreads, 0, st>>>((const uint16_t*)X, (const uint16_t*)P,
                                                    (uint16_t*)L, T, D, r, ctx_cap, t0);
  return hipGetLastError();
}

}  // namespace sals
