// Latent scoring (SALS 技术框架 stage 2, second half; 关键创新 1-2): the RoPE-free score of
// every cached token for every selection group,
//   S[b][s][t] = q~[b][s] . L_k[b][t],  t < Tc.
// This streams the whole latent key cache once and is HBM-bound. Each wave computes 16 tokens
// per step with one 16x16 MFMA chain over the rank: the 16 MFMA rows are the groups' fp32
// queries, split into bf16 high and low parts for a bf16 cache (8 groups per launch slice), so
// the bf16 MFMA reproduces an fp32 dot product to ~2^-16 relative; for an fp32 cache the rows
// are 16 groups and the fp32 MFMA is used. Every lane reads a contiguous R/4-element run of one
// token row (see Seg in common.h); the next tile is loaded while the current one is reduced.
#include "../common.h"
#include "../launch.h"

namespace sals {
namespace {

constexpr int kWavesPerBlock = 4;

template <class T, int R>
__device__ __forceinline__ void build_query_frags(const float* __restrict__ qt, int b, int G, int gb,
                                                  int lane, typename T::frag* a);

template <class T, int R>
__device__ __forceinline__ void build_query_frags(const float* __restrict__ qt, int b, int G, int gb,
                                                  int lane, typename T::frag* a) {
  using SG = Seg<T, R>;
  const int n16 = lane & 15, q4 = lane >> 4;
  if constexpr (T::HILO) {
    const int g = gb * 8 + (n16 & 7);
    const bool lo = n16 >= 8;
    const bool ok = g < G;
    const float* row = qt + ((size_t)b * G + (ok ? g : 0)) * R + q4 * SG::SEG;
#pragma unroll
    for (int kb = 0; kb < SG::KS; ++kb) {
      u32x4 w;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        uint32_t bits[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const float v = ok ? row[kb * 8 + jj * 2 + e] : 0.f;
          const uint32_t hi = f32_to_bf16_bits(v);
          bits[e] = lo ? f32_to_bf16_bits(v - bf16_bits_to_f32(hi)) : hi;
        }
        w[jj] = bits[0] | (bits[1] << 16);
      }
      a[kb] = __builtin_bit_cast(bf16x8_t, w);
    }
  } else {
    const int g = gb * 16 + n16;
    const bool ok = g < G;
    const float* row = qt + ((size_t)b * G + (ok ? g : 0)) * R + q4 * SG::SEG;
#pragma unroll
    for (int kb = 0; kb < SG::KS; ++kb) a[kb] = ok ? row[kb] : 0.f;
  }
}

template <class T, int R>
__device__ __forceinline__ void load_rows(const typename T::elem* __restrict__ Lk, size_t brow,
                                          int t, int q4, u32x4* ch) {
  using SG = Seg<T, R>;
  const u32x4* p = (const u32x4*)(Lk + (brow + (size_t)t) * R + q4 * SG::SEG);
#pragma unroll
  for (int c = 0; c < SG::NCH; ++c) ch[c] = p[c];
}

template <class T, int R>
__device__ __forceinline__ void score_tile(const typename T::frag* a, const u32x4* ch, float* __restrict__ S,
                                           int b, int G, int gb, int Tc, int t0, int lane) {
  using SG = Seg<T, R>;
  const int n16 = lane & 15, q4 = lane >> 4;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kb = 0; kb < SG::KS; ++kb) acc = T::mma(a[kb], frag_at<T>(ch, kb), acc);
  const int t = t0 + n16;
  if constexpr (T::HILO) {
    // rows 0..7 hold the high parts, rows 8..15 the low parts of the same 8 groups: lane l and
    // lane l + 32 hold the same (group, token) pair.
    f32x4 other;
#pragma unroll
    for (int i = 0; i < 4; ++i) other[i] = __shfl_xor(acc[i], 32);
    if (lane < 32 && t < Tc) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int g = gb * 8 + q4 * 4 + i;
        if (g < G) S[((size_t)b * G + g) * Tc + t] = acc[i] + other[i];
      }
    }
  } else {
    if (t < Tc) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int g = gb * 16 + q4 * 4 + i;
        if (g < G) S[((size_t)b * G + g) * Tc + t] = acc[i];
      }
    }
  }
}

// grid (ceil(tiles / (4 * tpw)), B, group slices); block 256.
template <class T, int R>
__global__ __launch_bounds__(256) void latent_score_kernel(const float* __restrict__ qt,
                                                           const typename T::elem* __restrict__ Lk,
                                                           float* __restrict__ S, int G, int Tc,
                                                           int ctx_cap, int tpw) {
  using SG = Seg<T, R>;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n16 = lane & 15, q4 = lane >> 4;
  const int b = blockIdx.y, gb = blockIdx.z;
  const int tile0 = (blockIdx.x * kWavesPerBlock + wave) * tpw;
  if (tile0 * 16 >= Tc) return;
  typename T::frag a[SG::KS];
  build_query_frags<T, R>(qt, b, G, gb, lane, a);
  const size_t brow = (size_t)b * ctx_cap;
  const int ntile = min(tpw, (Tc - tile0 * 16 + 15) / 16);
  u32x4 c0[SG::NCH], c1[SG::NCH];
  load_rows<T, R>(Lk, brow, min(tile0 * 16 + n16, Tc - 1), q4, c0);
  for (int it = 0; it < ntile; it += 2) {
    const int t0 = (tile0 + it) * 16;
    if (it + 1 < ntile) load_rows<T, R>(Lk, brow, min(t0 + 16 + n16, Tc - 1), q4, c1);
    score_tile<T, R>(a, c0, S, b, G, gb, Tc, t0, lane);
    if (it + 1 >= ntile) break;
    if (it + 2 < ntile) load_rows<T, R>(Lk, brow, min(t0 + 32 + n16, Tc - 1), q4, c0);
    score_tile<T, R>(a, c1, S, b, G, gb, Tc, t0 + 16, lane);
  }
}

template <class T, int R>
void launch_t(const float* qt, const void* Lk, float* S, int B, int G, int Tc, int ctx_cap,
              hipStream_t st) {
  constexpr int GPB = T::HILO ? 8 : 16;
  const int tiles = ceil_div(Tc, 16);
  const int n_gb = ceil_div(G, GPB);
  const long total = (long)tiles * B * n_gb;
  int tpw = (int)((total + 4095) / 4096);
  tpw = tpw < 1 ? 1 : (tpw > 64 ? 64 : tpw);
  dim3 grid(ceil_div(tiles, kWavesPerBlock * tpw), B, n_gb);
  latent_score_kernel<T, R><<<grid, 256, 0, st>>>(qt, (const typename T::elem*)Lk, S, G, Tc,
                                                  ctx_cap, tpw);
}

}  // namespace

hipError_t launch_latent_score(int dtype, const float* qt, const void* Lk, float* S, int B, int G,
                               int r, int Tc, int ctx_cap, hipStream_t st) {
  if (Tc <= 0) return hipSuccess;
#define SALS_SCORE_CASE(RR)                                              \
  case RR:                                                               \
    if (dtype == 0)                                                      \
      launch_t<F32, RR>(qt, Lk, S, B, G, Tc, ctx_cap, st);               \
    else                                                                 \
      launch_t<BF16, RR>(qt, Lk, S, B, G, Tc, ctx_cap, st);              \
    break;
  switch (r) {
    SALS_SCORE_CASE(32)
    SALS_SCORE_CASE(64)
    SALS_SCORE_CASE(128)
    SALS_SCORE_CASE(192)
    SALS_SCORE_CASE(256)
    SALS_SCORE_CASE(320)
    SALS_SCORE_CASE(384)
    SALS_SCORE_CASE(448)
    SALS_SCORE_CASE(512)
    default:
      return hipErrorInvalidValue;
  }
#undef SALS_SCORE_CASE
  return hipGetLastError();
}

}  // namespace sals
