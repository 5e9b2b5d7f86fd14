// Importance-based mixed-precision KV cache and attention over it (ZipVL abstract: high-bit
// quantization for the caches of important tokens, low-bit quantization for the rest, to ease
// the memory bottleneck of decoding).
//
// Per (sequence, KV head): the n_hi most important positions (their sorted list pos_hi comes from
// the top-k kernel) are stored at 8 bits, every other position at 4 bits, both sets in ascending
// position order. Each token row is quantized per group of 32 channels, asymmetric and uniform:
//   span = mx - mn, inv = levels / span, scale = span / levels  (fp32, each rounded to nearest)
//   code = clamp(floor((x - mn) * inv + 0.5), 0, levels),  levels = 2^bits - 1
// with code 0, scale 0 and zero point mn when span < 2^-96. The code is an integer decided in
// floating point, so these steps are taken exactly as written: fp contraction is off in this file
// and division is the correctly rounded one, so the codes are a fixed function of the inputs.
//
// mixed_quant_kernel: one thread per (token, group of 32 channels), for K and V. A thread finds
// its token's set and slot by a binary search in pos_hi (slot in the 8-bit set = its index there;
// slot in the 4-bit set = position - number of important positions below it, which also writes
// pos_lo), loads the group's
// 64 bytes, and writes 32 bytes (8-bit) or 16 bytes (4-bit, the even channel in the low nibble)
// of codes plus (scale, zero point).
// mixed_decode_kernel: flash-decode over both sets, one token row per four lanes (each lane a
// quarter of the channels), dequantizing on load as zero point + code * scale (one fp32 fma);
// online softmax per wave, the waves of a workgroup merged in LDS, split partials merged by the
// same LSE combine as the plain decode.
#include "../common.h"
#include "../launch.h"

#pragma clang fp contract(off)

namespace sals {
namespace {

constexpr int kGroup = 32;
constexpr float kTinySpan = 0x1p-96f;

// Quantizes 32 fp32 values in place into codes (as floats) and returns (scale, zero point).
template <int BITS>
__device__ __forceinline__ float2 quantize32(float (&x)[kGroup]) {
  constexpr float levels = (float)((1 << BITS) - 1);
  float mn = x[0], mx = x[0];
#pragma unroll
  for (int i = 1; i < kGroup; ++i) {
    mn = fminf(mn, x[i]);
    mx = fmaxf(mx, x[i]);
  }
  const float span = mx - mn;
  if (!(span >= kTinySpan)) {
#pragma unroll
    for (int i = 0; i < kGroup; ++i) x[i] = 0.f;
    return make_float2(0.f, mn);
  }
  const float inv = levels / span;
  const float scale = span / levels;
#pragma unroll
  for (int i = 0; i < kGroup; ++i) {
    const float u = (x[i] - mn) * inv;
    x[i] = fminf(fmaxf(floorf(u + 0.5f), 0.f), levels);
  }
  return make_float2(scale, mn);
}

// grid: BH * ceil(ctx / tokens per block); block 256 threads, D / 32 threads per token.
template <int D>
__global__ __launch_bounds__(256) void mixed_quant_kernel(const uint16_t* __restrict__ K,
                                                          const uint16_t* __restrict__ V,
                                                          const int32_t* __restrict__ pos_hi,
                                                          uint8_t* __restrict__ codes_hi,
                                                          float* __restrict__ params_hi,
                                                          uint8_t* __restrict__ codes_lo,
                                                          float* __restrict__ params_lo,
                                                          int32_t* __restrict__ pos_lo, int BH, int ctx_cap,
                                                          int ctx, int n_hi, int nblk) {
  constexpr int GPT = D / kGroup;  // groups (threads) per token
  constexpr int TPB = 256 / GPT;   // tokens per block
  const int pair = blockIdx.x / nblk, blk = blockIdx.x % nblk;
  const int t = blk * TPB + threadIdx.x / GPT, gi = threadIdx.x % GPT;
  if (t >= ctx) return;
  const int n_lo = ctx - n_hi;
  // rank = number of important positions below t; t is important if it sits at pos_hi[rank]
  const int32_t* ph = pos_hi + (size_t)pair * n_hi;
  int lo = 0, hi = n_hi;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (ph[mid] < t) lo = mid + 1;
    else hi = mid;
  }
  const bool important = lo < n_hi && ph[lo] == t;
  const int slot = important ? lo : t - lo;
  if (!important && gi == 0) pos_lo[(size_t)pair * n_lo + slot] = t;
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    const uint16_t* src = (x ? V : K) + ((size_t)pair * ctx_cap + t) * D + gi * kGroup;
    u32x4 raw[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) raw[u] = *(const u32x4*)(src + 8 * u);
    float v[kGroup];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[8 * u + 2 * e] = __uint_as_float(raw[u][e] << 16);
        v[8 * u + 2 * e + 1] = __uint_as_float(raw[u][e] & 0xffff0000u);
      }
    if (important) {
      const float2 sp = quantize32<8>(v);
      const size_t row = (size_t)x * BH * n_hi + (size_t)pair * n_hi + slot;
      u32x4 w[2];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int b0 = 16 * h + 4 * e;
          w[h][e] = (uint32_t)v[b0] | ((uint32_t)v[b0 + 1] << 8) | ((uint32_t)v[b0 + 2] << 16) |
                    ((uint32_t)v[b0 + 3] << 24);
        }
      u32x4* dst = (u32x4*)(codes_hi + row * D + gi * kGroup);
      dst[0] = w[0];
      dst[1] = w[1];
      *(float2*)(params_hi + (row * GPT + gi) * 2) = sp;
    } else {
      const float2 sp = quantize32<4>(v);
      const size_t row = (size_t)x * BH * n_lo + (size_t)pair * n_lo + slot;
      u32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        uint32_t word = 0;
#pragma unroll
        for (int k = 0; k < 8; ++k) word |= (uint32_t)v[8 * e + k] << (4 * k);
        w[e] = word;
      }
      *(u32x4*)(codes_lo + row * (D / 2) + gi * (kGroup / 2)) = w;
      *(float2*)(params_lo + (row * GPT + gi) * 2) = sp;
    }
  }
}

// ---- decode ----------------------------------------------------------------------------------

constexpr int kThreads = 256;

// grid: n_splits * (H_q / NG) * B (as the plain decode); tokens j < n_hi are slot j of the
// 8-bit set, the rest slot j - n_hi of the 4-bit set.
template <int D>
__global__ __launch_bounds__(kThreads) void mixed_decode_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ codes_hi, const float* __restrict__ params_hi,
    const uint8_t* __restrict__ codes_lo, const float* __restrict__ params_lo, float* __restrict__ out,
    float* __restrict__ part, int B, int H_q, int H_kv, int n_hi, int n_lo, int split_len, int n_splits) {
  constexpr int CW = D / 4;  // channels per lane (contiguous)
  constexpr int GPT = D / kGroup;
  __shared__ float qsh[4][D];
  __shared__ float red[4][D + 2];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nqh = H_q / H_kv;
  const int NG = dense_heads_per_group(nqh), NPH = 4 / NG, ngr = nqh / NG;
  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int gr = wg % ngr, sp = (wg / ngr) % n_splits, g = (wg / (ngr * n_splits)) % H_kv;
  const int b = wg / (ngr * n_splits * H_kv);
  const int myh = wave % NG, phase = wave / NG;
  const float qscale = 1.0f / sqrtf((float)D);
  for (int c = tid; c < NG * D; c += kThreads)
    qsh[c / D][c % D] = bf16_bits_to_f32(q[((size_t)b * H_q + g * nqh + gr * NG + c / D) * D + c % D]) * qscale;
  __syncthreads();
  const int lq = lane & 3;
  const int c0 = lq * CW;           // this lane's channels c0 .. c0 + CW
  const int gi = c0 / kGroup;       // their group
  float qv[CW];
#pragma unroll
  for (int j = 0; j < CW; ++j) qv[j] = qsh[myh][c0 + j];
  const int pair = b * H_kv + g;
  const size_t BHk = (size_t)B * H_kv;
  const int n = n_hi + n_lo;
  const int jbeg = sp * split_len, jend = min(n, jbeg + split_len);
  float m = -INFINITY, l = 0.f;
  float o[CW];
#pragma unroll
  for (int j = 0; j < CW; ++j) o[j] = 0.f;
  // dequantized channels of token j for tensor x (0 keys, 1 values)
  auto row = [&](int j, int x, float (&v)[CW]) {
    if (j < n_hi) {
      const size_t r = (size_t)x * BHk * n_hi + (size_t)pair * n_hi + j;
      const float2 sz = *(const float2*)(params_hi + (r * GPT + gi) * 2);
      const uint8_t* cp = codes_hi + r * D + c0;
#pragma unroll
      for (int u = 0; u < CW / 16; ++u) {
        const u32x4 w = *(const u32x4*)(cp + 16 * u);
#pragma unroll
        for (int k = 0; k < 16; ++k) v[16 * u + k] = fmaf((float)((w[k >> 2] >> (8 * (k & 3))) & 0xffu), sz.x, sz.y);
      }
    } else {
      const size_t r = (size_t)x * BHk * n_lo + (size_t)pair * n_lo + (j - n_hi);
      const float2 sz = *(const float2*)(params_lo + (r * GPT + gi) * 2);
      const uint8_t* cp = codes_lo + r * (D / 2) + c0 / 2;
      if constexpr (CW >= 32) {
#pragma unroll
        for (int u = 0; u < CW / 32; ++u) {
          const u32x4 w = *(const u32x4*)(cp + 16 * u);
#pragma unroll
          for (int k = 0; k < 32; ++k) v[32 * u + k] = fmaf((float)((w[k >> 3] >> (4 * (k & 7))) & 0xfu), sz.x, sz.y);
        }
      } else {
        const uint2 w = *(const uint2*)cp;
#pragma unroll
        for (int k = 0; k < CW; ++k) v[k] = fmaf((float)((((k >> 3) ? w.y : w.x) >> (4 * (k & 7))) & 0xfu), sz.x, sz.y);
      }
    }
  };
  const int tstep = 16 * NPH;
  for (int t0 = jbeg + phase * 16; t0 < jend; t0 += tstep) {
    const int j = t0 + (lane >> 2);
    const bool ok = j < jend;
    const int jj = ok ? j : jend - 1;
    float kv[CW];
    row(jj, 0, kv);
    float xs = 0.f;
#pragma unroll
    for (int c = 0; c < CW; ++c) xs = fmaf(qv[c], kv[c], xs);
    xs += __shfl_xor(xs, 1);
    xs += __shfl_xor(xs, 2);
    if (!ok) xs = -INFINITY;
    const float tm = wave_max(xs);
    const float mn = fmaxf(m, tm);
    const float corr = expf(m - mn);
    const float p = ok ? expf(xs - mn) : 0.f;
    float ps = p;
    ps += __shfl_xor(ps, 4);
    ps += __shfl_xor(ps, 8);
    ps += __shfl_xor(ps, 16);
    ps += __shfl_xor(ps, 32);
    l = l * corr + ps;
    m = mn;
    float vv[CW];
    row(jj, 1, vv);
#pragma unroll
    for (int c = 0; c < CW; ++c) o[c] = fmaf(p, vv[c], o[c] * corr);
  }
  // o over the 16 tokens of the wave (lanes with equal lane % 4)
#pragma unroll
  for (int c = 0; c < CW; ++c) {
    float v = o[c];
    v += __shfl_xor(v, 4);
    v += __shfl_xor(v, 8);
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    o[c] = v;
  }
  if (lane < 4) {
#pragma unroll
    for (int c = 0; c < CW; ++c) red[wave][c0 + c] = o[c];
  }
  if (lane == 0) {
    red[wave][D] = m;
    red[wave][D + 1] = l;
  }
  __syncthreads();
  for (int c2 = tid; c2 < NG * D; c2 += kThreads) {
    const int e = c2 / D, c = c2 % D;
    float M = -INFINITY;
    for (int ph = 0; ph < NPH; ++ph) M = fmaxf(M, red[ph * NG + e][D]);
    float L = 0.f, oc = 0.f;
    for (int ph = 0; ph < NPH; ++ph) {
      const int wv = ph * NG + e;
      const float wgt = red[wv][D] == -INFINITY ? 0.f : expf(red[wv][D] - M);
      L += red[wv][D + 1] * wgt;
      oc += red[wv][c] * wgt;
    }
    const int hq = g * nqh + gr * NG + e;
    if (n_splits == 1) {
      out[((size_t)b * H_q + hq) * D + c] = oc / L;
    } else {
      float* pp = part + (((size_t)b * H_q + hq) * n_splits + sp) * (D + 2);
      pp[2 + c] = oc;
      if (c == 0) {
        pp[0] = M;
        pp[1] = L;
      }
    }
  }
}

}  // namespace

hipError_t launch_mixed_quant(const void* K, const void* V, const int32_t* pos_hi, uint8_t* codes_hi,
                              float* params_hi, uint8_t* codes_lo, float* params_lo, int32_t* pos_lo, int BH, int d,
                              int ctx_cap, int ctx, int n_hi, hipStream_t st) {
  const int tpb = 256 / (d / kGroup);
  const int nblk = ceil_div(ctx, tpb);
  if ((long)BH * nblk > 0x7fffffffL) return hipErrorInvalidValue;
  const auto* k = (const uint16_t*)K;
  const auto* v = (const uint16_t*)V;
  if (d == 128)
    mixed_quant_kernel<128><<<BH * nblk, 256, 0, st>>>(k, v, pos_hi, codes_hi, params_hi, codes_lo, params_lo, pos_lo, BH,
                                                       ctx_cap, ctx, n_hi, nblk);
  else if (d == 64)
    mixed_quant_kernel<64><<<BH * nblk, 256, 0, st>>>(k, v, pos_hi, codes_hi, params_hi, codes_lo, params_lo, pos_lo, BH,
                                                      ctx_cap, ctx, n_hi, nblk);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_mixed_decode(const void* q, const uint8_t* codes_hi, const float* params_hi, const uint8_t* codes_lo,
                               const float* params_lo, float* out, float* part, int B, int H_q, int H_kv, int d,
                               int n_hi, int n_lo, int split_len, int n_splits, hipStream_t st) {
  dim3 grid(n_splits * (H_q / dense_heads_per_group(H_q / H_kv)) * B);
  const auto* qq = (const uint16_t*)q;
  if (d == 128)
    mixed_decode_kernel<128><<<grid, kThreads, 0, st>>>(qq, codes_hi, params_hi, codes_lo, params_lo, out, part, B,
                                                        H_q, H_kv, n_hi, n_lo, split_len, n_splits);
  else if (d == 64)
    mixed_decode_kernel<64><<<grid, kThreads, 0, st>>>(qq, codes_hi, params_hi, codes_lo, params_lo, out, part, B,
                                                       H_q, H_kv, n_hi, n_lo, split_len, n_splits);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace sals
