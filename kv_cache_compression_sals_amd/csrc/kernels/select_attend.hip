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
                                const void* Pk, const void* Pv, const int32_t* sel, float* out,
                                float* part, int B, int H_q, int H_kv, int d, int r, int G,
                                int ctx_cap, int ctx, int n_sel, int split_len, int n_splits,
                                float rope_base, hipStream_t st) {
  const sa::SAArgs a{q, Lk, Lv, Pk, Pv, sel, out, part, B, H_q, H_kv, G, ctx_cap, ctx, n_sel,
                     split_len, n_splits, rope_base};
  bool ok = false;
  if (dtype == 1 && d == 128) ok = sa::bf16_d128_launch(r, a, st);
  else if (dtype == 1 && d == 64) ok = sa::bf16_d64_launch(r, a, st);
  else if (dtype == 0 && d == 128) ok = sa::f32_d128_launch(r, a, st);
  else if (dtype == 0 && d == 64) ok = sa::f32_d64_launch(r, a, st);
  return ok ? hipGetLastError() : hipErrorInvalidValue;
}

// LSE merge: out[bh] = sum_s o_s e^{m_s - M} / sum_s l_s e^{m_s - M}, M = max_s m_s.
__global__ void combine_kernel(const float* __restrict__ part, float* __restrict__ out, int d,
                               int n_splits) {
  const float* p = part + (size_t)blockIdx.x * n_splits * (d + 2);
  float M = -INFINITY;
  for (int s = 0; s < n_splits; ++s) M = fmaxf(M, p[(size_t)s * (d + 2)]);
  float L = 0.f;
  for (int s = 0; s < n_splits; ++s) L += p[(size_t)s * (d + 2) + 1] * expf(p[(size_t)s * (d + 2)] - M);
  for (int c = threadIdx.x; c < d; c += blockDim.x) {
    float o = 0.f;
    for (int s = 0; s < n_splits; ++s) o += p[(size_t)s * (d + 2) + 2 + c] * expf(p[(size_t)s * (d + 2)] - M);
    out[(size_t)blockIdx.x * d + c] = o / L;
  }
}

hipError_t launch_combine(const float* part, float* out, int BH, int d, int n_splits,
                          hipStream_t st) {
  if (BH <= 0) return hipSuccess;
  combine_kernel<<<BH, 128, 0, st>>>(part, out, d, n_splits);
  return hipGetLastError();
}

}  // namespace sals
