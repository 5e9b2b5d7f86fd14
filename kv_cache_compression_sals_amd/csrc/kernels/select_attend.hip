// Dispatch of the gather + rebuild + RoPE + attention kernel over the instantiated shapes, and
// the LSE merge of split partials.
#include "../common.h"
#include "../launch.h"
#include "select_attend.inc"
#include "select_attend_variants.h"

namespace sals {

int select_attend_max_split(int dtype, int d, int r, int nqh) {
  if (dtype == 1 && d == 128) return sa::bf16_d128_max_split(r, nqh);
  if (dtype == 1 && d == 64) return sa::bf16_d64_max_split(r, nqh);
  if (dtype == 0 && d == 128) return sa::f32_d128_max_split(r, nqh);
  if (dtype == 0 && d == 64) return sa::f32_d64_max_split(r, nqh);
  return 0;
}

hipError_t launch_select_attend(int dtype, const void* q, const void* Lk, const void* Lv,
                                const void* Pk, const void* Pv, const int32_t* sel, const int32_t* cnt,
                                float* out, float* part, float* pbuf, float* pstat, int B, int H_q,
                                int H_kv, int d, int r, int G, int ctx_cap, int ctx, int n_sel,
                                int split_len, int n_splits, float rope_base, hipStream_t st,
                                hipEvent_t t_start, hipEvent_t t_stop) {
  const sa::SAArgs a{q,     Lk,   Lv, Pk,      Pv,  sel,   cnt,   out,       part,     pbuf,     pstat,
                     B,     H_q,  H_kv, G,     ctx_cap, ctx, n_sel, split_len, n_splits, rope_base,
                     t_start, t_stop};
  bool ok = false;
  if (dtype == 1 && d == 128) ok = sa::bf16_d128_launch(r, a, st);
  else if (dtype == 1 && d == 64) ok = sa::bf16_d64_launch(r, a, st);
  else if (dtype == 0 && d == 128) ok = sa::f32_d128_launch(r, a, st);
  else if (dtype == 0 && d == 64) ok = sa::f32_d64_launch(r, a, st);
  return ok ? hipGetLastError() : hipErrorInvalidValue;
}

// LSE merge: out[bh] = sum_s o_s e^{m_s - M} / sum_s l_s e^{m_s - M}, M = max_s m_s.
// The split maxima are read in parallel, then the splits are merged in chunks of kChunk: each
// chunk's weights e^{m_s - M} are staged in LDS and every thread sums its columns over the chunk
// with independent loads.
constexpr int kChunk = 1024;
__global__ __launch_bounds__(128) void combine_kernel(const float* __restrict__ part,
                                                      float* __restrict__ out, int d,
                                                      int n_splits) {
  __shared__ float wgt[kChunk];
  __shared__ float red[2];
  const float* p = part + (size_t)blockIdx.x * n_splits * (d + 2);
  const int tid = threadIdx.x;
  float M = -INFINITY;
  for (int s = tid; s < n_splits; s += 128) M = fmaxf(M, p[(size_t)s * (d + 2)]);
  M = wave_max(M);
  if ((tid & 63) == 0) red[tid >> 6] = M;
  __syncthreads();
  M = fmaxf(red[0], red[1]);
  __syncthreads();
  float lsum = 0.f;
  float o[2] = {0.f, 0.f};  // columns tid and tid + 128 (d <= 256)
  for (int c0 = 0; c0 < n_splits; c0 += kChunk) {
    const int nc = min(kChunk, n_splits - c0);
    batched_copy<8>(nc, tid, 128, [&](int s) { return p[(size_t)(c0 + s) * (d + 2)]; },
                    [&](int s, float m) { wgt[s] = expf(m - M); });
    __syncthreads();
    for (int s = tid; s < nc; s += 128) lsum += wgt[s] * p[(size_t)(c0 + s) * (d + 2) + 1];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = tid + 128 * h;
      if (c < d) {
        const float* col = p + (size_t)c0 * (d + 2) + 2 + c;
        float acc = 0.f;
#pragma unroll 8
        for (int s = 0; s < nc; ++s) acc += col[(size_t)s * (d + 2)] * wgt[s];
        o[h] += acc;
      }
    }
    __syncthreads();
  }
  lsum = wave_sum(lsum);
  if ((tid & 63) == 0) red[tid >> 6] = lsum;
  __syncthreads();
  const float L = red[0] + red[1];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int c = tid + 128 * h;
    if (c < d) out[(size_t)blockIdx.x * d + c] = o[h] / L;
  }
}

hipError_t launch_combine(const float* part, float* out, int BH, int d, int n_splits,
                          hipStream_t st) {
  if (BH <= 0) return hipSuccess;
  combine_kernel<<<BH, 128, 0, st>>>(part, out, d, n_splits);
  return hipGetLastError();
}

}  // namespace sals
