// Latent query (SALS 技术框架 stage 2, first half): the RoPE-free decode query of every
// selection group, mapped into the latent space,
//   q~[b][s][j] = sum_{h : group(kv(h)) = s} sum_c q[b][h][c] * P_k[kv(h)*d + c][j].
// Reordered as a sum over the rows of P_k: row i (KV head g = i / d, c = i % d) is weighted by
// qsum[b][i] = sum over the query heads of g of q[b][h][c]. P_k is read once per launch; the
// rows are split across workgroups and the partial sums reduced by a second small kernel
// (skipped when one split covers a whole group).
#include "../common.h"
#include "../launch.h"

namespace sals {
namespace {

constexpr int kBC = 8;        // sequences per pass
constexpr int kThreads = 256; // 8 column groups x 32 row phases

template <class T>
__device__ __forceinline__ void load8(const typename T::elem* p, float* v);

template <>
__device__ __forceinline__ void load8<BF16>(const uint16_t* p, float* v) {
  u32x4 c = *(const u32x4*)p;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    v[2 * j] = __uint_as_float(c[j] << 16);
    v[2 * j + 1] = __uint_as_float(c[j] & 0xffff0000u);
  }
}

template <>
__device__ __forceinline__ void load8<F32>(const float* p, float* v) {
  u32x4 a = *(const u32x4*)p, b = *(const u32x4*)(p + 4);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    v[j] = __uint_as_float(a[j]);
    v[4 + j] = __uint_as_float(b[j]);
  }
}

// grid (ceil(r/64), D/rps); rows [rs*rps, (rs+1)*rps) of P_k, 64 columns.
template <class T>
__global__ __launch_bounds__(kThreads) void lq_partial_kernel(
    const typename T::elem* __restrict__ q, const typename T::elem* __restrict__ Pk,
    float* __restrict__ dst, int B, int H_q, int H_kv, int d, int r, int G, int rps,
    int direct) {
  __shared__ float qsum[kBC][512];
  __shared__ float red[4][kBC][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int cg = tid & 7, rp = tid >> 3;
  const int rs = blockIdx.y;
  const int row0 = rs * rps;
  const int col0 = blockIdx.x * 64 + cg * 8;
  const bool col_ok = col0 < r;
  const int nqh = H_q / H_kv;
  const int D = H_kv * d;
  const int grp = row0 / (D / G);

  for (int b0 = 0; b0 < B; b0 += kBC) {
    const int nb = min(kBC, B - b0);
    __syncthreads();
    // qsum[bb][i] = sum over the query heads of KV head g of q[b][h][c]: one load per head,
    // batched so that many are in flight
    for (int h = 0; h < nqh; ++h) {
      batched_copy<8>(
          nb * rps, tid, kThreads,
          [&](int e) {
            const int bb = e / rps, row = row0 + e % rps;
            return T::to_f32(q[((size_t)(b0 + bb) * H_q + (size_t)(row / d) * nqh + h) * d + row % d]);
          },
          [&](int e, float v) { qsum[e / rps][e % rps] = (h == 0 ? 0.f : qsum[e / rps][e % rps]) + v; });
    }
    __syncthreads();
    float acc[kBC][8];
#pragma unroll
    for (int bb = 0; bb < kBC; ++bb)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[bb][j] = 0.f;
    if (col_ok) {
#pragma unroll 8
      for (int i = rp; i < rps; i += 32) {
        float p[8];
        load8<T>(Pk + (size_t)(row0 + i) * r + col0, p);
#pragma unroll
        for (int bb = 0; bb < kBC; ++bb) {
          const float wgt = qsum[bb][i];
#pragma unroll
          for (int j = 0; j < 8; ++j) acc[bb][j] = fmaf(wgt, p[j], acc[bb][j]);
        }
      }
    }
    // reduce the 8 row phases of a wave (lane bits 3..5), then the 4 waves
#pragma unroll
    for (int bb = 0; bb < kBC; ++bb)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float v = acc[bb][j];
        v += __shfl_xor(v, 8);
        v += __shfl_xor(v, 16);
        v += __shfl_xor(v, 32);
        acc[bb][j] = v;
      }
    if (lane < 8) {
#pragma unroll
      for (int bb = 0; bb < kBC; ++bb)
#pragma unroll
        for (int j = 0; j < 8; ++j) red[wave][bb][lane * 8 + j] = acc[bb][j];
    }
    __syncthreads();
    for (int e = tid; e < nb * 64; e += kThreads) {
      const int bb = e / 64, cc = e % 64;
      const int col = blockIdx.x * 64 + cc;
      if (col < r) {
        const float v = red[0][bb][cc] + red[1][bb][cc] + red[2][bb][cc] + red[3][bb][cc];
        if (direct)
          dst[((size_t)(b0 + bb) * G + grp) * r + col] = v;
        else
          dst[((size_t)rs * B + b0 + bb) * r + col] = v;
      }
    }
  }
}

// qt[b][s][j] = sum over the row splits of group s of qpart[rs][b][j].
__global__ void lq_reduce_kernel(const float* __restrict__ qpart, float* __restrict__ qt, int B,
                                 int G, int r, int splits_per_group) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= B * G * r) return;
  const int j = e % r, s = (e / r) % G, b = e / (r * G);
  float v = 0.f;
#pragma unroll 8
  for (int i = 0; i < splits_per_group; ++i)
    v += qpart[((size_t)(s * splits_per_group + i) * B + b) * r + j];
  qt[e] = v;
}

}  // namespace

hipError_t launch_latent_query(int dtype, const void* q, const void* Pk, float* qpart, float* qt,
                               int B, int H_q, int H_kv, int d, int r, int G, int rps,
                               hipStream_t st) {
  const int D = H_kv * d;
  const int n_rs = D / rps;
  const int spg = (D / G) / rps;
  const bool direct = spg == 1;
  dim3 grid(ceil_div(r, 64), n_rs);
  float* dst = direct ? qt : qpart;
  if (dtype == 0)
    lq_partial_kernel<F32><<<grid, kThreads, 0, st>>>((const float*)q, (const float*)Pk, dst, B,
                                                      H_q, H_kv, d, r, G, rps, direct);
  else
    lq_partial_kernel<BF16><<<grid, kThreads, 0, st>>>((const uint16_t*)q, (const uint16_t*)Pk,
                                                       dst, B, H_q, H_kv, d, r, G, rps, direct);
  if (!direct) {
    const int n = B * G * r;
    lq_reduce_kernel<<<ceil_div(n, 256), 256, 0, st>>>(qpart, qt, B, G, r, spg);
  }
  return hipGetLastError();
}

}  // namespace sals
