// Latent scoring (SALS 技术框架 stage 2, second half; 关键创新 1-2): the RoPE-free score of
// every cached token for every selection group,
//   S[b][s][t] = q~[b][s] . L_k[b][t],  t < Tc (rows of ldS floats).
// This streams the whole latent key cache once and is HBM-bound. Each wave computes 16 tokens
// per step with one 16x16 MFMA chain over the rank: the 16 MFMA rows are the groups' fp32
// queries, split into bf16 high and low parts for a bf16 cache (8 groups per launch slice), so
// the bf16 MFMA reproduces an fp32 dot product to ~2^-16 relative; for an fp32 cache the rows
// are 16 groups and the fp32 MFMA is used. The latent-query kernel writes these rows already in
// operand form, so each wave loads its A fragments straight from L2. Latent rows are read in the natural k layout (each
// load instruction covers 64 contiguous bytes of 16 consecutive rows); a wave takes 2 or 4 tiles
// (fewer when the cache is short, so that every CU gets work), loading two tiles at a time.
#include "../common.h"
#include "../launch.h"

namespace sals {
namespace {

constexpr int kWaves = 4;
template <class T, int R>
__device__ __forceinline__ void load_tile(const typename T::elem* __restrict__ Lk, size_t brow, int t,
                                          int q4, u32x4 (&ch)[R / Win<T>::WLEN]) {
  using W = Win<T>;
  const typename T::elem* p = Lk + (brow + (size_t)t) * R + q4 * W::EPC;
#pragma unroll
  for (int w = 0; w < R / W::WLEN; ++w) ch[w] = *(const u32x4*)(p + w * W::WLEN);
}

template <class T, int R>
__device__ __forceinline__ void score_tile(const u32x4 (&a)[R / Win<T>::WLEN],
                                           const u32x4 (&ch)[R / Win<T>::WLEN],
                                           float* __restrict__ S, int b, int G, int gb, int Tc,
                                           int ldS, int t0, int lane) {
  using W = Win<T>;
  const int n16 = lane & 15, q4 = lane >> 4;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int w = 0; w < R / W::WLEN; ++w)
#pragma unroll
    for (int st = 0; st < W::KW; ++st) acc = T::mma(chunk_frag<T>(a[w], st), chunk_frag<T>(ch[w], st), acc);
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
        if (g < G) S[((size_t)b * G + g) * ldS + t] = acc[i] + other[i];
      }
    }
  } else {
    if (t < Tc) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int g = gb * 16 + q4 * 4 + i;
        if (g < G) S[((size_t)b * G + g) * ldS + t] = acc[i];
      }
    }
  }
}

// grid (ceil(tiles / (4 * TW)), B, group slices); block 256. Workgroup x covers tiles
// [x*4*TW, (x+1)*4*TW); wave w takes tiles x*4*TW + w + 4*i, i < TW, two at a time: the loads of
// both tiles of a pair are issued before either is reduced.
template <class T, int R, int TW>
__global__ __launch_bounds__(256) void latent_score_kernel(const typename T::elem* __restrict__ qa,
                                                           const typename T::elem* __restrict__ Lk,
                                                           float* __restrict__ S, int G, int Tc,
                                                           int ldS, int ctx_cap) {
  using W = Win<T>;
  constexpr int NW = R / W::WLEN;
  constexpr int GPB = T::HILO ? 8 : 16;
  static_assert(TW % 2 == 0, "tiles are taken in pairs");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n16 = lane & 15, q4 = lane >> 4;
  const int b = blockIdx.y, gb = blockIdx.z;
  const size_t brow = (size_t)b * ctx_cap;
  const int tile0 = blockIdx.x * (kWaves * TW) + wave;
  // the first pair's rows (HBM) are requested first, then the operand rows (L2)
  u32x4 c0[NW], c1[NW];
  load_tile<T, R>(Lk, brow, min(tile0 * 16 + n16, Tc - 1), q4, c0);
  load_tile<T, R>(Lk, brow, min((tile0 + 4) * 16 + n16, Tc - 1), q4, c1);
  // MFMA A operand: row n16 of this slice's 16 operand rows, natural k layout
  u32x4 a[NW];
  {
    const int nsl = (G + GPB - 1) / GPB;
    const typename T::elem* arow = qa + ((size_t)(b * nsl + gb) * 16 + n16) * R + q4 * W::EPC;
#pragma unroll
    for (int w = 0; w < NW; ++w) a[w] = *(const u32x4*)(arow + w * W::WLEN);
  }
#pragma unroll
  for (int i = 0; i < TW; i += 2) {
    const int ta = tile0 + 4 * i, tb = ta + 4;
    if (ta * 16 >= Tc) break;
    if (i > 0) {
      load_tile<T, R>(Lk, brow, min(ta * 16 + n16, Tc - 1), q4, c0);
      load_tile<T, R>(Lk, brow, min(tb * 16 + n16, Tc - 1), q4, c1);
      __builtin_amdgcn_sched_barrier(0);
    }
    score_tile<T, R>(a, c0, S, b, G, gb, Tc, ldS, ta * 16, lane);
    if (tb * 16 < Tc) score_tile<T, R>(a, c1, S, b, G, gb, Tc, ldS, tb * 16, lane);
  }
}

template <class T, int R>
void launch_t(const void* qa, const void* Lk, float* S, int ldS, int B, int G, int Tc, int ctx_cap,
              hipStream_t st) {
  using E = typename T::elem;
  constexpr int GPB = T::HILO ? 8 : 16;
  const int tiles = ceil_div(Tc, 16);
  const int slices = ceil_div(G, GPB);
  // two tiles per wave unless that already gives the chip several workgroups per CU
  const bool four = (long)ceil_div(tiles, kWaves * 4) * B * slices >= 1024;
  if (four) {
    dim3 grid(ceil_div(tiles, kWaves * 4), B, slices);
    latent_score_kernel<T, R, 4><<<grid, 256, 0, st>>>((const E*)qa, (const E*)Lk, S, G, Tc, ldS, ctx_cap);
  } else {
    dim3 grid(ceil_div(tiles, kWaves * 2), B, slices);
    latent_score_kernel<T, R, 2><<<grid, 256, 0, st>>>((const E*)qa, (const E*)Lk, S, G, Tc, ldS, ctx_cap);
  }
}

}  // namespace

hipError_t launch_latent_score(int dtype, const void* qa, const void* Lk, float* S, int ldS, int B,
                               int G, int r, int Tc, int ctx_cap, hipStream_t st) {
  if (Tc <= 0) return hipSuccess;
#define SALS_SCORE_CASE(RR)                                              \
  case RR:                                                               \
    if (dtype == 0)                                                      \
      launch_t<F32, RR>(qa, Lk, S, ldS, B, G, Tc, ctx_cap, st);          \
    else                                                                 \
      launch_t<BF16, RR>(qa, Lk, S, ldS, B, G, Tc, ctx_cap, st);         \
    break;
  switch (r) {
    SALS_SCORE_CASE(32)
    SALS_SCORE_CASE(64)
    SALS_SCORE_CASE(128)
    SALS_SCORE_CASE(256)
    SALS_SCORE_CASE(384)
    SALS_SCORE_CASE(512)
    default:
      return hipErrorInvalidValue;
  }
#undef SALS_SCORE_CASE
  return hipGetLastError();
}

}  // namespace sals
