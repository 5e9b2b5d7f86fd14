// Frequency-domain outlier importance of a KV cache (FlashCache page, summary and abstract: the
// energy of the KV matrices along the token axis sits at low frequencies; a low-pass filter
// extracts that principal component; the KV pairs that deviate most from it are kept), with no
// attention score involved.
//
// Per (sequence b, KV head g), with X = K[b, g, :ctx] or V[b, g, :ctx] ([ctx, d], bf16) and the
// orthonormal DCT-II basis C[t, f] = a_f cos(pi (2t + 1) f / (2 ctx)) of its first F columns:
//   coef = C^T X            (F x d)                     pass 1, a reduction over the tokens
//   I[t] = ||K[t] - (C coef_K)[t]||^2 + ||V[t] - (C coef_V)[t]||^2   pass 2, per token
// Both contractions run on bf16 MFMAs. The cache is exact in bf16; the basis values (fp32) and
// the coefficients (fp32) enter as high + low bf16 parts, so every product carries about 2^-16
// relative error and every sum is fp32. A basis value takes its angle in revolutions,
// (2t + 1) f / (4 ctx) reduced to [-1/2, 1/2) in fp64, and the hardware cosine of it.
//
// Pass 1: one workgroup per (b, g, K or V, chunk of 4096 tokens), in sub-tiles of 128 tokens.
// The MFMA contracts over tokens, which is the slow axis of the cache, so each sub-tile is
// transposed through LDS: a thread loads two consecutive token rows and writes, per channel, one
// 32-bit word holding both tokens (a wave writes 64 consecutive words per channel: no bank
// conflicts); a B fragment (8 tokens of one channel) is then one 16-byte read. The basis of the
// sub-tile is computed once per workgroup into LDS in the A-fragment layout. The chunk's partial
// coefficients go to the workspace.
// A small kernel then adds each pair's chunk partials in chunk order and writes the coefficients,
// split into bf16 parts, in the A-fragment layout of pass 2.
// Pass 2: one workgroup per (b, g, chunk of 2048 tokens), with its pair's fragments in LDS. The
// product is taken transposed, X_lp^T = coef^T C^T, with the A rows permuted so
// that a lane ends up holding 32 (d = 128) contiguous channels of its token: the deviation is then
// formed against 64 contiguous bytes of the cached row, and the four lane groups are added in a
// fixed order.
#include "../common.h"
#include "../launch.h"

namespace sals {
namespace {

constexpr int kTch1 = 4096;  // tokens per pass-1 workgroup
constexpr int kSub = 128;    // tokens per pass-1 sub-tile
constexpr int kRW = kSub / 2 + 4;  // LDS words per channel row of a transposed sub-tile (padded)
constexpr int kTch2 = 2048;  // tokens per pass-2 workgroup

// a_f cos(pi (2t + 1) f / (2 T)) in fp32, zero past the kept frequencies. The angle in revolutions
// is (2t + 1) f / (4 T): the product is an exact fp64 integer (below 2^34), times an fp64 1 / (4 T),
// minus its floor, so the fraction carries ~1e-14 absolute error before the rounding to fp32.
__device__ __forceinline__ float dct_value(int t, int f, double inv4T, int n_freq, float a0, float a1) {
  if (f >= n_freq) return 0.f;
  const double x = (2.0 * (double)t + 1.0) * (double)f * inv4T;
  float rev = (float)(x - floor(x));  // [0, 1) revolutions
  rev = rev >= 0.5f ? rev - 1.0f : rev;
  return (f == 0 ? a0 : a1) * __builtin_amdgcn_cosf(rev);
}

// 8 fp32 values -> high and low bf16 parts (nearest even), packed as two MFMA fragments.
__device__ __forceinline__ void split8(const float (&v)[8], u32x4& hi, u32x4& lo) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t h0 = f32_to_bf16_bits(v[2 * i]), h1 = f32_to_bf16_bits(v[2 * i + 1]);
    const uint32_t l0 = f32_to_bf16_bits(v[2 * i] - bf16_bits_to_f32(h0));
    const uint32_t l1 = f32_to_bf16_bits(v[2 * i + 1] - bf16_bits_to_f32(h1));
    hi[i] = h0 | (h1 << 16);
    lo[i] = l0 | (l1 << 16);
  }
}

__device__ __forceinline__ f32x4 mma(const u32x4& a, const u32x4& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}

// ---- pass 1: partial coefficients ----------------------------------------------------------
// grid: B * H_kv * 2 * nch workgroups; part[((pair * 2 + x) * nch + ch) * FP * D + f * D + c].
template <int D, int FP>
__global__ __launch_bounds__(256) void outlier_coef_kernel(const uint16_t* __restrict__ K,
                                                           const uint16_t* __restrict__ V,
                                                           float* __restrict__ part, int ctx_cap, int ctx,
                                                           int n_freq, int nch) {
  constexpr int FT = FP / 16;          // frequency tiles
  constexpr int CT = D / 16 / 4;       // channel tiles per wave
  constexpr int CPT = D / 4;           // channels per thread in the transposed write
  constexpr int LPR = CPT * 2 / 16;    // 16-byte loads per row per thread
  constexpr int NB = FT * 4 * 64;      // basis fragments per sub-tile (each hi + lo)
  __shared__ __attribute__((aligned(16))) uint32_t xt[D * kRW];
  __shared__ __attribute__((aligned(16))) u32x4 bas[2][NB];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n16 = lane & 15, q4 = lane >> 4;
  const int wg = blockIdx.x;
  const int ch = wg % nch, x = (wg / nch) & 1, pair = wg / (2 * nch);
  const uint16_t* X = (x ? V : K) + (size_t)pair * ctx_cap * D;
  const int t_begin = ch * kTch1, t_end = min(ctx, t_begin + kTch1);
  const float a0 = sqrtf(1.0f / (float)ctx), a1 = sqrtf(2.0f / (float)ctx);
  const double inv4T = 1.0 / (4.0 * (double)ctx);

  // this thread's rows of a sub-tile: tokens 2p, 2p + 1; channels cq * CPT .. + CPT
  const int p = tid & 63, cq = tid >> 6;
  u32x4 rows[2][LPR];
  auto load_rows = [&](int s0) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int t = s0 + 2 * p + r;
      const bool ok = t < t_end;
      const uint16_t* src = X + (size_t)(ok ? t : t_begin) * D + cq * CPT;
#pragma unroll
      for (int u = 0; u < LPR; ++u) {
        const u32x4 v = *(const u32x4*)(src + 8 * u);
        rows[r][u] = ok ? v : u32x4{0u, 0u, 0u, 0u};
      }
    }
  };

  f32x4 acc[FT][CT];
#pragma unroll
  for (int ft = 0; ft < FT; ++ft)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) acc[ft][ct] = f32x4{0.f, 0.f, 0.f, 0.f};

  load_rows(t_begin);
  for (int s0 = t_begin; s0 < t_end; s0 += kSub) {
    // transposed write: word (channel c, token pair p) = X[2p][c] | X[2p + 1][c] << 16
#pragma unroll
    for (int u = 0; u < LPR; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t w0 = rows[0][u][e], w1 = rows[1][u][e];
        const int c = cq * CPT + 8 * u + 2 * e;
        xt[c * kRW + p] = (w0 & 0xffffu) | (w1 << 16);
        xt[(c + 1) * kRW + p] = (w0 >> 16) | (w1 & 0xffff0000u);
      }
    // basis of the sub-tile in the A layout: fragment (ft, ks, l) holds C[s0 + 32 ks + 8 (l / 16) + i]
    // [16 ft + l % 16], i < 8, as high and low parts
    for (int e = tid; e < NB; e += 256) {
      const int l = e & 63, ks = (e >> 6) & 3, ft = e >> 8;
      float v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int t = s0 + 32 * ks + 8 * (l >> 4) + i;
        v[i] = t < t_end ? dct_value(t, 16 * ft + (l & 15), inv4T, n_freq, a0, a1) : 0.f;
      }
      split8(v, bas[0][e], bas[1][e]);
    }
    __syncthreads();
    if (s0 + kSub < t_end) load_rows(s0 + kSub);  // in flight during the products
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      u32x4 bf[CT];
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const int c = (wave * CT + ct) * 16 + n16;
        bf[ct] = *(const u32x4*)&xt[c * kRW + ks * 16 + 4 * q4];
      }
#pragma unroll
      for (int ft = 0; ft < FT; ++ft) {
        const u32x4 ah = bas[0][(ft * 4 + ks) * 64 + lane], al = bas[1][(ft * 4 + ks) * 64 + lane];
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          acc[ft][ct] = mma(ah, bf[ct], acc[ft][ct]);
          acc[ft][ct] = mma(al, bf[ct], acc[ft][ct]);
        }
      }
    }
    __syncthreads();
  }
  float* dst = part + ((size_t)(pair * 2 + x) * nch + ch) * FP * D;
#pragma unroll
  for (int ft = 0; ft < FT; ++ft)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[(16 * ft + 4 * q4 + i) * D + (wave * CT + ct) * 16 + n16] = acc[ft][ct][i];
}

// ---- coefficients: chunk partials added in chunk order, as pass-2 A fragments ----------------
// Fragment (x, channel tile j, k-step kf, lane l) of a pair holds coef_x[32 kf + 8 (l / 16) + i]
// [perm(j, l % 16)], i < 8, with perm(j, m) = (D / 4)(m / 4) + 4 j + m % 4, as high and low
// bf16 parts: afrag[(pair * NA + e) * 2 + {0, 1}], NA = 2 * (D / 16) * (FP / 32) * 64.
template <int D, int FP>
__global__ __launch_bounds__(256) void outlier_reduce_kernel(const float* __restrict__ part,
                                                             u32x4* __restrict__ afrag, int BH, int nch) {
  constexpr int CTL = D / 16, KF = FP / 32, CPL = D / 4;
  constexpr int NA = 2 * CTL * KF * 64;
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= BH * NA) return;
  const int pair = idx / NA, e = idx % NA;
  const int l = e & 63, kf = (e >> 6) % KF, j = (e >> 6) / KF % CTL, x = (e >> 6) / (KF * CTL);
  const int m = l & 15;
  const int c = CPL * (m >> 2) + 4 * j + (m & 3);
  const float* src = part + (size_t)(pair * 2 + x) * nch * FP * D + c;
  float v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int f = 32 * kf + 8 * (l >> 4) + i;
    float sum = 0.f;
    for (int ch = 0; ch < nch; ++ch) sum += src[((size_t)ch * FP + f) * D];
    v[i] = sum;
  }
  split8(v, afrag[(size_t)idx * 2], afrag[(size_t)idx * 2 + 1]);
}

// ---- pass 2: deviation energy per token ----------------------------------------------------
// grid: B * H_kv * ceil(ctx / kTch2) workgroups.
template <int D, int FP>
__global__ __launch_bounds__(256) void outlier_dev_kernel(const uint16_t* __restrict__ K,
                                                          const uint16_t* __restrict__ V,
                                                          const u32x4* __restrict__ afrag, float* __restrict__ I,
                                                          int ctx_cap, int ctx, int n_freq, int nch2) {
  constexpr int CTL = D / 16;   // channel tiles
  constexpr int KF = FP / 32;   // k-steps over the frequencies
  constexpr int CPL = D / 4;    // channels per lane after the product
  constexpr int NA = 2 * CTL * KF * 64;  // A fragments (K and V), each hi + lo
  __shared__ __attribute__((aligned(16))) u32x4 afr[2 * NA];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n16 = lane & 15, q4 = lane >> 4;
  const int wg = blockIdx.x;
  const int c2 = wg % nch2, pair = wg / nch2;
  const float a0 = sqrtf(1.0f / (float)ctx), a1 = sqrtf(2.0f / (float)ctx);
  const double inv4T = 1.0 / (4.0 * (double)ctx);
  batched_copy<8>(2 * NA, tid, 256, [&](int i) { return afrag[(size_t)pair * 2 * NA + i]; },
                  [&](int i, const u32x4& v) { afr[i] = v; });
  __syncthreads();

  const int t_begin = c2 * kTch2, t_end = min(ctx, t_begin + kTch2);
  for (int t0 = t_begin + 16 * wave; t0 < t_end; t0 += 64) {
    const int t = t0 + n16;
    const bool ok = t < t_end;
    // the lane's row pieces of K and V: channels CPL q4 .. + CPL
    u32x4 xr[2][CPL / 8];
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const uint16_t* src = (x ? V : K) + ((size_t)pair * ctx_cap + (ok ? t : t_begin)) * D + CPL * q4;
#pragma unroll
      for (int u = 0; u < CPL / 8; ++u) xr[x][u] = *(const u32x4*)(src + 8 * u);
    }
    // basis fragments: C[t][32 kf + 8 q4 + i]
    u32x4 bh[KF], bl[KF];
#pragma unroll
    for (int kf = 0; kf < KF; ++kf) {
      float v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = ok ? dct_value(t, 32 * kf + 8 * q4 + i, inv4T, n_freq, a0, a1) : 0.f;
      split8(v, bh[kf], bl[kf]);
    }
    float dev = 0.f;
#pragma unroll
    for (int x = 0; x < 2; ++x) {
#pragma unroll
      for (int j = 0; j < CTL; ++j) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kf = 0; kf < KF; ++kf) {
          const int e = ((x * CTL + j) * KF + kf) * 64 + lane;
          const u32x4 ah = afr[2 * e], al = afr[2 * e + 1];
          acc = mma(ah, bh[kf], acc);
          acc = mma(ah, bl[kf], acc);
          acc = mma(al, bh[kf], acc);
        }
        // acc[i] = low-pass value of channel CPL q4 + 4 j + i of token t
        const u32x4 w = xr[x][j >> 1];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t word = w[2 * (j & 1) + (i >> 1)];
          const float xv = __uint_as_float((i & 1) ? (word & 0xffff0000u) : (word << 16));
          const float r = xv - acc[i];
          dev = fmaf(r, r, dev);
        }
      }
    }
    // the four lane groups of a token, in a fixed order: (q0 + q1) + (q2 + q3)
    dev += __shfl_xor(dev, 16);
    dev += __shfl_xor(dev, 32);
    if (ok && q4 == 0) I[(size_t)pair * ctx + t] = dev;
  }
}

constexpr size_t align256(size_t x) { return (x + 255) / 256 * 256; }

size_t part_bytes(int BH, int d, int ctx, int fp) { return align256((size_t)BH * 2 * ceil_div(ctx, kTch1) * fp * d * 4); }
size_t afrag_bytes(int BH, int d, int fp) { return (size_t)BH * 2 * (2 * (d / 16) * (fp / 32) * 64) * 16; }

template <int D, int FP>
void launch_t(const void* K, const void* V, void* ws, float* I, int BH, int ctx_cap, int ctx, int n_freq,
              hipStream_t st) {
  constexpr int NA = 2 * (D / 16) * (FP / 32) * 64;
  const int nch = ceil_div(ctx, kTch1), nch2 = ceil_div(ctx, kTch2);
  const auto* k = (const uint16_t*)K;
  const auto* v = (const uint16_t*)V;
  float* part = (float*)ws;
  u32x4* afrag = (u32x4*)((char*)ws + part_bytes(BH, D, ctx, FP));
  outlier_coef_kernel<D, FP><<<BH * 2 * nch, 256, 0, st>>>(k, v, part, ctx_cap, ctx, n_freq, nch);
  outlier_reduce_kernel<D, FP><<<ceil_div(BH * NA, 256), 256, 0, st>>>(part, afrag, BH, nch);
  outlier_dev_kernel<D, FP><<<BH * nch2, 256, 0, st>>>(k, v, afrag, I, ctx_cap, ctx, n_freq, nch2);
}

}  // namespace

int outlier_freq_pad(int n_freq) { return n_freq <= 32 ? 32 : 64; }

size_t outlier_workspace_bytes(int BH, int d, int ctx, int n_freq) {
  const int fp = outlier_freq_pad(n_freq);
  return part_bytes(BH, d, ctx, fp) + afrag_bytes(BH, d, fp);
}

hipError_t launch_outlier_importance(const void* K, const void* V, void* ws, float* I, int BH, int d,
                                     int ctx_cap, int ctx, int n_freq, hipStream_t st) {
  const int fp = outlier_freq_pad(n_freq);
  if (d == 128 && fp == 32) launch_t<128, 32>(K, V, ws, I, BH, ctx_cap, ctx, n_freq, st);
  else if (d == 128) launch_t<128, 64>(K, V, ws, I, BH, ctx_cap, ctx, n_freq, st);
  else if (d == 64 && fp == 32) launch_t<64, 32>(K, V, ws, I, BH, ctx_cap, ctx, n_freq, st);
  else if (d == 64) launch_t<64, 64>(K, V, ws, I, BH, ctx_cap, ctx, n_freq, st);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace sals
