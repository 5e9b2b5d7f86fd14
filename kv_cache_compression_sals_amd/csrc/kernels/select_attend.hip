// Dispatch of the gather + rebuild + RoPE + attention kernel over the instantiated shapes, the
// LSE merge of split partials, and the merge + value product of its latent partials.
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

bool select_attend_rank_fits(int dtype, int d, int r, int nqh, int split_len, int nc, int kp) {
  return dtype == 1 && d == 128 && sa::bf16_d128_rank_fits(r, nqh, split_len, nc, kp);
}

hipError_t launch_select_attend(int dtype, const void* q, const void* Lk, const void* Lv,
                                const void* Pk, const void* Pv, const int32_t* sel, const int32_t* cnt,
                                float* out, float* part, float* pbuf, float* pstat, int B, int H_q,
                                int H_kv, int d, int r, int G, int ctx_cap, int ctx, int n_sel,
                                int split_len, int n_splits, float rope_base, hipStream_t st,
                                hipEvent_t t_start, hipEvent_t t_stop, const int32_t* cand, int ns, int m,
                                const float* S, int ldS, int Tc, int kp, int32_t* selw) {
  sa::RankArgs rk{};
  if (cand) {
    if (cnt || !selw || !S || ns < 1 || m < 1 || kp < 1 || n_sel != kp + (ctx - Tc) ||
        !select_attend_rank_fits(dtype, d, r, H_q / H_kv, split_len, ns * m, kp))
      return hipErrorInvalidValue;
    const size_t per = (size_t)B * G * ns * m;
    rk = sa::RankArgs{cand, (const uint32_t*)(cand + per), (const uint32_t*)(cand + 2 * per), S, selw,
                      ns, m, ldS, Tc, kp};
  }
  const sa::SAArgs a{q,     Lk,   Lv, Pk,      Pv,  sel,   cnt,   out,       part,     pbuf,     pstat,
                     B,     H_q,  H_kv, G,     ctx_cap, ctx, n_sel, split_len, n_splits, rope_base,
                     t_start, t_stop, rk};
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

// Split merge of the gather + attention kernel's latent partials, then the value product:
//   M = max_s m_s,  w_s = e^{m_s - M},  L = sum_s w_s l_s,  z = sum_s w_s z_s   (z in latent space)
//   out[b][h][c] = sum_k P_v[g*d + c][k] z[k] / L
// z is linear in the probabilities, so merging before the product gives the result of the
// per-split products at one product per head. Workgroup (b*H_q + h, row block): every workgroup
// merges all r columns (thread j owns columns j, j + 256, ..., splits in chunks of kSch with an
// online rescale) while its P_v rows, requested first, are in flight; NPH consecutive lanes share
// one row, each holding LPT 16-byte chunks of it, so that one load instruction covers whole
// 128-byte lines. The product runs in fp32.
constexpr int kSch = 16;
template <class T, int R>
__global__ __launch_bounds__(256) void latent_combine_kernel(const float* __restrict__ part,
                                                             const typename T::elem* __restrict__ Pv,
                                                             float* __restrict__ out, int H_q, int H_kv,
                                                             int d, int n_splits) {
  using E = typename T::elem;
  constexpr int EPL = 16 / (int)sizeof(E);
  constexpr int CPR = R / EPL;               // 16-byte chunks per P_v row
  constexpr int NPH = CPR < 8 ? CPR : 8;     // lanes per row
  constexpr int LPT = CPR / NPH;             // chunks per lane
  constexpr int RW = 256 / NPH;              // rows per workgroup
  constexpr int ZC = (R + 255) / 256;        // merged columns per thread
  static_assert(CPR % NPH == 0 && LPT <= 16, "row split");
  __shared__ float zs[R];
  const int bh = blockIdx.x, tid = threadIdx.x;
  const int h = bh % H_q, g = h / (H_q / H_kv);
  const int row = tid / NPH, ph = tid % NPH;
  const int c = blockIdx.y * RW + row;
  const E* prow = Pv + ((size_t)g * d + min(c, d - 1)) * R;
  u32x4 pa[LPT];
#pragma unroll
  for (int t = 0; t < LPT; ++t) pa[t] = *(const u32x4*)(prow + (ph + NPH * t) * EPL);

  const float* pp = part + (size_t)bh * n_splits * (R + 2);
  float M = -INFINITY, L = 0.f, z[ZC];
#pragma unroll
  for (int u = 0; u < ZC; ++u) z[u] = 0.f;
  for (int s0 = 0; s0 < n_splits; s0 += kSch) {
    const int ns = min(kSch, n_splits - s0);
    float mv[kSch], lv[kSch], zv[kSch][ZC];
#pragma unroll
    for (int s = 0; s < kSch; ++s) {
      const float* ps = pp + (size_t)(s0 + min(s, ns - 1)) * (R + 2);
      mv[s] = ps[0];
      lv[s] = ps[1];
#pragma unroll
      for (int u = 0; u < ZC; ++u) zv[s][u] = ps[2 + min(tid + 256 * u, R - 1)];
    }
    float Mc = M;
#pragma unroll
    for (int s = 0; s < kSch; ++s)
      if (s < ns) Mc = fmaxf(Mc, mv[s]);
    if (Mc == -INFINITY) continue;  // only empty splits so far
    const float f = expf(M - Mc);    // 0 while M is still -inf
    L *= f;
#pragma unroll
    for (int u = 0; u < ZC; ++u) z[u] *= f;
#pragma unroll
    for (int s = 0; s < kSch; ++s) {
      const float w = s < ns ? expf(mv[s] - Mc) : 0.f;  // an empty split (m = -inf) weighs 0
      L = fmaf(w, lv[s], L);
#pragma unroll
      for (int u = 0; u < ZC; ++u) z[u] = fmaf(w, zv[s][u], z[u]);
    }
    M = Mc;
  }
#pragma unroll
  for (int u = 0; u < ZC; ++u)
    if (tid + 256 * u < R) zs[tid + 256 * u] = z[u];
  __syncthreads();
  float acc = 0.f;
#pragma unroll
  for (int t = 0; t < LPT; ++t) {
    const int k0 = (ph + NPH * t) * EPL;
    float x[EPL];
    sa::unpack_chunk<T>(pa[t], x);
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc = fmaf(x[e], zs[k0 + e], acc);
  }
#pragma unroll
  for (int o = 1; o < NPH; o <<= 1) acc += __shfl_xor(acc, o);
  if (ph == 0 && c < d) out[(size_t)bh * d + c] = acc / L;
}

template <class T, int R>
void launch_latent_combine_t(const float* part, const void* Pv, float* out, int BH, int H_q, int H_kv,
                             int d, int n_splits, hipStream_t st) {
  constexpr int EPL = 16 / (int)sizeof(typename T::elem);
  constexpr int CPR = R / EPL;
  constexpr int RW = 256 / (CPR < 8 ? CPR : 8);
  const dim3 grid(BH, (d + RW - 1) / RW);
  latent_combine_kernel<T, R><<<grid, 256, 0, st>>>(part, (const typename T::elem*)Pv, out, H_q, H_kv, d,
                                                    n_splits);
}

hipError_t launch_latent_combine(int dtype, const float* part, const void* Pv, float* out, int B, int H_q,
                                 int H_kv, int d, int r, int n_splits, hipStream_t st) {
  const int BH = B * H_q;
  if (BH <= 0) return hipSuccess;
#define SALS_CASE(RR)                                                                    \
  case RR:                                                                               \
    if (dtype == 1)                                                                      \
      launch_latent_combine_t<BF16, RR>(part, Pv, out, BH, H_q, H_kv, d, n_splits, st);  \
    else                                                                                 \
      launch_latent_combine_t<F32, RR>(part, Pv, out, BH, H_q, H_kv, d, n_splits, st);   \
    break;
  switch (r) {
    SALS_CASE(32) SALS_CASE(64) SALS_CASE(128) SALS_CASE(256) SALS_CASE(384) SALS_CASE(512)
    default:
      return hipErrorInvalidValue;
  }
#undef SALS_CASE
  return hipGetLastError();
}

}  // namespace sals
