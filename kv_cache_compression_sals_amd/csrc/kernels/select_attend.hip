// Gather + rebuild + RoPE + attention over the selected tokens (SALS 技术框架 stages 3-4,
// 关键创新 3; 问题定义 and abstract: RoPE is applied after the rebuild, at true positions).
//
// One workgroup per (sequence b, KV head g, split of the selected set). The KV head's slice of
// P_k (d x r) sits in LDS; each wave takes 16 selected tokens at a time, gathers their latent
// rows straight from HBM as the MFMA A operand and multiplies by the slice (B operand from LDS),
// giving K_hat for 16 tokens x d columns in registers. RoPE is applied in place (the pair
// (c, c + d/2) lives in the same lane), the logits of the KV head's query heads are formed with
// a 16-lane reduction and kept in LDS. After an exact softmax over the split, the slice of P_v
// replaces P_k and a second pass rebuilds V_hat the same way and accumulates p * V_hat. K_hat
// and V_hat never leave the chip. With one split the normalised output is written directly;
// otherwise (m, l, unnormalised o) partials are written for the LSE merge.
#include "../common.h"
#include "../launch.h"

namespace sals {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxQH = 8;
constexpr double kTwoPi = 6.283185307179586476925286766559;

template <class T, int R, int DH>
struct SACfg {
  using elem = typename T::elem;
  static constexpr int PAD = 16 / (int)sizeof(elem);
  static constexpr int PST = R + PAD;  // LDS row stride (elements) of the P slice
  static constexpr int P_BYTES = DH * PST * (int)sizeof(elem);
  static constexpr int QS_FLOATS = kMaxQH * DH;
  static constexpr int RED_FLOATS = 4 * DH + 64;
  static constexpr int FIXED = P_BYTES + (QS_FLOATS + RED_FLOATS) * 4;
  // two workgroups per CU when the fixed part leaves room for a short split, else one
  static constexpr int TOTAL = (FIXED + 4096 <= 81408) ? 81408 : 162816;
  static constexpr int TAIL = TOTAL - FIXED;  // logits/probabilities + positions
  static_assert(TAIL >= 4096, "P slice too large for LDS");
};

template <class T>
__device__ __forceinline__ typename T::frag lds_frag(const typename T::elem* p);
template <>
__device__ __forceinline__ float lds_frag<F32>(const float* p) { return *p; }
template <>
__device__ __forceinline__ bf16x8_t lds_frag<BF16>(const uint16_t* p) {
  return *(const bf16x8_t*)p;
}

template <class T, int R, int DH>
__device__ __forceinline__ void load_p_slice(const typename T::elem* __restrict__ src,
                                             typename T::elem* dst, int tid) {
  using C = SACfg<T, R, DH>;
  constexpr int EPC = 16 / (int)sizeof(typename T::elem);
  constexpr int CPR = R / EPC;  // 16-byte chunks per row
  for (int e = tid; e < DH * CPR; e += kThreads) {
    const int row = e / CPR, c = e % CPR;
    *(u32x4*)(dst + row * C::PST + c * EPC) = *(const u32x4*)(src + (size_t)row * R + c * EPC);
  }
}

// acc[nb][i] = sum_k L[token q4*4+i][k] * P[nb*16 + n16][k]  (the 16-token tile x DH columns)
template <class T, int R, int DH>
__device__ __forceinline__ void rebuild_tile(const u32x4* ach, const typename T::elem* Pbuf,
                                             int n16, int q4, f32x4* acc) {
  using C = SACfg<T, R, DH>;
  using SG = Seg<T, R>;
  constexpr int NB = DH / 16;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kb = 0; kb < SG::KS; ++kb) {
    const typename T::frag a = frag_at<T>(ach, kb);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const typename T::frag bf =
          lds_frag<T>(Pbuf + (nb * 16 + n16) * C::PST + q4 * SG::SEG + kb * T::KPL);
      acc[nb] = T::mma(a, bf, acc[nb]);
    }
  }
}

template <class T, int R>
__device__ __forceinline__ void load_latent_row(const typename T::elem* __restrict__ L, size_t row,
                                                int q4, u32x4* ch) {
  using SG = Seg<T, R>;
  const u32x4* p = (const u32x4*)(L + row * R + q4 * SG::SEG);
#pragma unroll
  for (int c = 0; c < SG::NCH; ++c) ch[c] = p[c];
}

// sin/cos of 2*pi * (pos * frev) with the product reduced to [-1/2, 1/2] revolutions in fp64.
__device__ __forceinline__ void rope_sincos(int pos, double frev, float* s, float* c) {
  double rv = (double)pos * frev;
  rv -= rint(rv);
  sincospif(2.0f * (float)rv, s, c);
}

template <class T, int R, int DH>
__global__ __launch_bounds__(kThreads) void select_attend_kernel(
    const typename T::elem* __restrict__ q, const typename T::elem* __restrict__ Lk,
    const typename T::elem* __restrict__ Lv, const typename T::elem* __restrict__ Pk,
    const typename T::elem* __restrict__ Pv, const int32_t* __restrict__ sel,
    float* __restrict__ out, float* __restrict__ part, int H_q, int H_kv, int G, int ctx_cap,
    int ctx, int n_sel, int split_len, int n_splits, float rope_base) {
  using C = SACfg<T, R, DH>;
  using SG = Seg<T, R>;
  using elem = typename T::elem;
  constexpr int NB = DH / 16, HB = NB / 2;
  __shared__ __attribute__((aligned(16))) unsigned char smem[C::TOTAL];
  elem* Pbuf = (elem*)smem;
  float* qs = (float*)(smem + C::P_BYTES);
  float* red = qs + C::QS_FLOATS;
  float* lg = red + C::RED_FLOATS;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n16 = lane & 15, q4 = lane >> 4;
  const int sp = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int nqh = H_q / H_kv;
  const int s = (g * G) / H_kv;
  const int j0 = sp * split_len;
  const int n_tok = min(split_len, n_sel - j0);
  const int n_tiles = (n_tok + 15) / 16;
  int* pos = (int*)(lg + nqh * split_len);

  const int32_t* selrow = sel + ((size_t)b * G + s) * n_sel + j0;
  for (int j = tid; j < n_tok; j += kThreads) pos[j] = selrow[j];
  load_p_slice<T, R, DH>(Pk + (size_t)g * DH * R, Pbuf, tid);
  const float qscale = 1.0f / sqrtf((float)DH);
  for (int e = tid; e < nqh * (DH / 2); e += kThreads) {
    const int hh = e / (DH / 2), i = e % (DH / 2);
    const elem* qp = q + ((size_t)b * H_q + (size_t)g * nqh + hh) * DH;
    const float x1 = T::to_f32(qp[i]), x2 = T::to_f32(qp[i + DH / 2]);
    const double frev = pow((double)rope_base, -2.0 * i / DH) / kTwoPi;
    float sn, cs;
    rope_sincos(ctx - 1, frev, &sn, &cs);
    qs[hh * DH + i] = (x1 * cs - x2 * sn) * qscale;
    qs[hh * DH + i + DH / 2] = (x2 * cs + x1 * sn) * qscale;
  }
  double frev[HB];
#pragma unroll
  for (int nb = 0; nb < HB; ++nb)
    frev[nb] = pow((double)rope_base, -2.0 * (nb * 16 + n16) / DH) / kTwoPi;
  const size_t brow = (size_t)b * ctx_cap;
  __syncthreads();

  // ---- pass 1: rebuild K_hat, rotate, logits ----
  for (int tile = wave; tile < n_tiles; tile += 4) {
    u32x4 ach[SG::NCH];
    load_latent_row<T, R>(Lk, brow + pos[min(tile * 16 + n16, n_tok - 1)], q4, ach);
    f32x4 acc[NB];
    rebuild_tile<T, R, DH>(ach, Pbuf, n16, q4, acc);
    int p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = pos[min(tile * 16 + q4 * 4 + i, n_tok - 1)];
#pragma unroll
    for (int nb = 0; nb < HB; ++nb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float sn, cs;
        rope_sincos(p[i], frev[nb], &sn, &cs);
        const float x1 = acc[nb][i], x2 = acc[nb + HB][i];
        acc[nb][i] = x1 * cs - x2 * sn;
        acc[nb + HB][i] = x2 * cs + x1 * sn;
      }
    }
#pragma unroll
    for (int hh = 0; hh < kMaxQH; ++hh) {
      if (hh < nqh) {
        float pr[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const float qv = qs[hh * DH + nb * 16 + n16];
#pragma unroll
          for (int i = 0; i < 4; ++i) pr[i] = fmaf(qv, acc[nb][i], pr[i]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float v = pr[i];
          v += __shfl_xor(v, 1);
          v += __shfl_xor(v, 2);
          v += __shfl_xor(v, 4);
          v += __shfl_xor(v, 8);
          pr[i] = v;
        }
        if (n16 == 0) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int sl = tile * 16 + q4 * 4 + i;
            if (sl < n_tok) lg[hh * split_len + sl] = pr[i];
          }
        }
      }
    }
  }
  __syncthreads();

  // ---- exact softmax over the split, per query head ----
  float mh[kMaxQH], lh[kMaxQH];
#pragma unroll
  for (int hh = 0; hh < kMaxQH; ++hh) {
    mh[hh] = 0.f;
    lh[hh] = 1.f;
    if (hh < nqh) {
      float* row = lg + hh * split_len;
      float m = -INFINITY;
      for (int j = tid; j < n_tok; j += kThreads) m = fmaxf(m, row[j]);
      m = wave_max(m);
      if (lane == 0) red[wave] = m;
      __syncthreads();
      m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
      __syncthreads();
      float l = 0.f;
      for (int j = tid; j < n_tok; j += kThreads) {
        const float e = expf(row[j] - m);
        row[j] = e;
        l += e;
      }
      l = wave_sum(l);
      if (lane == 0) red[wave] = l;
      __syncthreads();
      l = (red[0] + red[1]) + (red[2] + red[3]);
      __syncthreads();
      mh[hh] = m;
      lh[hh] = l;
    }
  }

  // ---- pass 2: rebuild V_hat, accumulate p * V_hat ----
  load_p_slice<T, R, DH>(Pv + (size_t)g * DH * R, Pbuf, tid);
  __syncthreads();
  float oacc[kMaxQH][NB];
#pragma unroll
  for (int hh = 0; hh < kMaxQH; ++hh)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) oacc[hh][nb] = 0.f;
  for (int tile = wave; tile < n_tiles; tile += 4) {
    u32x4 ach[SG::NCH];
    load_latent_row<T, R>(Lv, brow + pos[min(tile * 16 + n16, n_tok - 1)], q4, ach);
    f32x4 acc[NB];
    rebuild_tile<T, R, DH>(ach, Pbuf, n16, q4, acc);
#pragma unroll
    for (int hh = 0; hh < kMaxQH; ++hh) {
      if (hh < nqh) {
        float pw[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int sl = tile * 16 + q4 * 4 + i;
          pw[i] = sl < n_tok ? lg[hh * split_len + sl] : 0.f;
        }
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int i = 0; i < 4; ++i) oacc[hh][nb] = fmaf(pw[i], acc[nb][i], oacc[hh][nb]);
      }
    }
  }
#pragma unroll
  for (int hh = 0; hh < kMaxQH; ++hh)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      float v = oacc[hh][nb];
      v += __shfl_xor(v, 16);
      v += __shfl_xor(v, 32);
      oacc[hh][nb] = v;
    }
#pragma unroll
  for (int hh = 0; hh < kMaxQH; ++hh) {
    if (hh < nqh) {
      __syncthreads();
      if (lane < 16) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) red[wave * DH + nb * 16 + lane] = oacc[hh][nb];
      }
      __syncthreads();
      const int h = g * nqh + hh;
      for (int c = tid; c < DH; c += kThreads) {
        const float o = (red[c] + red[DH + c]) + (red[2 * DH + c] + red[3 * DH + c]);
        if (n_splits == 1) {
          out[((size_t)b * H_q + h) * DH + c] = o / lh[hh];
        } else {
          float* pp = part + (((size_t)b * H_q + h) * n_splits + sp) * (DH + 2);
          pp[2 + c] = o;
          if (c == 0) {
            pp[0] = mh[hh];
            pp[1] = lh[hh];
          }
        }
      }
    }
  }
}

template <class T, int R, int DH>
void launch_t(const void* q, const void* Lk, const void* Lv, const void* Pk, const void* Pv,
              const int32_t* sel, float* out, float* part, int B, int H_q, int H_kv, int G,
              int ctx_cap, int ctx, int n_sel, int split_len, int n_splits, float base,
              hipStream_t st) {
  using E = typename T::elem;
  dim3 grid(n_splits, H_kv, B);
  select_attend_kernel<T, R, DH><<<grid, kThreads, 0, st>>>(
      (const E*)q, (const E*)Lk, (const E*)Lv, (const E*)Pk, (const E*)Pv, sel, out, part, H_q,
      H_kv, G, ctx_cap, ctx, n_sel, split_len, n_splits, base);
}

template <class T, int R, int DH>
int max_split_t(int nqh) {
  using C = SACfg<T, R, DH>;
  return (C::TAIL / (4 * (nqh + 1))) / 16 * 16;
}

}  // namespace

// Instantiated shapes: (dtype, r, d) with d * r * elemsize <= 128 KiB.
#define SALS_SA_CASES(X)                                                                     \
  X(BF16, 32, 64) X(BF16, 64, 64) X(BF16, 128, 64) X(BF16, 192, 64) X(BF16, 256, 64)       \
  X(BF16, 320, 64) X(BF16, 384, 64) X(BF16, 448, 64) X(BF16, 512, 64) X(BF16, 32, 128)     \
  X(BF16, 64, 128) X(BF16, 128, 128) X(BF16, 192, 128) X(BF16, 256, 128) X(BF16, 320, 128) \
  X(BF16, 384, 128) X(BF16, 448, 128) X(BF16, 512, 128) X(F32, 32, 64) X(F32, 64, 64)      \
  X(F32, 128, 64) X(F32, 192, 64) X(F32, 256, 64) X(F32, 320, 64) X(F32, 384, 64)          \
  X(F32, 448, 64) X(F32, 512, 64) X(F32, 32, 128) X(F32, 64, 128) X(F32, 128, 128)         \
  X(F32, 192, 128) X(F32, 256, 128)

int select_attend_max_split(int dtype, int d, int r, int nqh) {
#define SALS_SA_MAX(TT, RR, DD) \
  if ((dtype == 0) == (sizeof(TT::elem) == 4) && r == RR && d == DD) return max_split_t<TT, RR, DD>(nqh);
  SALS_SA_CASES(SALS_SA_MAX)
#undef SALS_SA_MAX
  return 0;
}

hipError_t launch_select_attend(int dtype, const void* q, const void* Lk, const void* Lv,
                                const void* Pk, const void* Pv, const int32_t* sel, float* out,
                                float* part, int B, int H_q, int H_kv, int d, int r, int G,
                                int ctx_cap, int ctx, int n_sel, int split_len, int n_splits,
                                float rope_base, hipStream_t st) {
#define SALS_SA_LAUNCH(TT, RR, DD)                                                              \
  if ((dtype == 0) == (sizeof(TT::elem) == 4) && r == RR && d == DD) {                         \
    launch_t<TT, RR, DD>(q, Lk, Lv, Pk, Pv, sel, out, part, B, H_q, H_kv, G, ctx_cap, ctx, n_sel, \
                         split_len, n_splits, rope_base, st);                                   \
    return hipGetLastError();                                                                   \
  }
  SALS_SA_CASES(SALS_SA_LAUNCH)
#undef SALS_SA_LAUNCH
  return hipErrorInvalidValue;
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
