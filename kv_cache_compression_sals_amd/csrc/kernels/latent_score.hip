// Latent scoring (SALS 技术框架 stage 2, second half; 关键创新 1-2): the RoPE-free score of
// every cached token for every selection group,
//   S[b][s][t] = q~[b][s] . L_k[b][t],  t < Tc (rows of ldS floats).
// This streams the whole latent key cache once and is HBM-bound. Each wave computes 16 tokens
// per step with one 16x16 MFMA chain over the rank: the 16 MFMA rows are the groups' fp32
// queries, split into bf16 high and low parts for a bf16 cache (8 groups per launch slice), so
// the bf16 MFMA reproduces an fp32 dot product to ~2^-16 relative; for an fp32 cache the rows
// are 16 groups and the fp32 MFMA is used. A workgroup first issues the loads of its first
// latent tiles, then adds the latent-query partial sums of its groups (part order), writes the
// operand rows to LDS and takes its A fragments from there. Latent rows are read in the
// natural k layout (each load instruction covers 64 contiguous bytes of 16 consecutive rows); a
// wave takes 2 or 4 tiles (fewer when the cache is short, so that every CU gets work), loading
// two tiles at a time.
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

// Operand row entries of group slot gs, columns 4 cq .. 4 cq + 3 (bf16: high parts in row gs,
// low parts in row 8 + gs).
template <class T>
__device__ __forceinline__ void store_operand_quad(typename T::elem* opnd, int ost, int gs, int cq,
                                                   const float4& v) {
  const float x[4] = {v.x, v.y, v.z, v.w};
  if constexpr (T::HILO) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t hi = f32_to_bf16_bits(x[i]);
      opnd[gs * ost + cq * 4 + i] = (typename T::elem)hi;
      opnd[(8 + gs) * ost + cq * 4 + i] = (typename T::elem)f32_to_bf16_bits(x[i] - bf16_bits_to_f32(hi));
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) opnd[gs * ost + cq * 4 + i] = x[i];
  }
}

// grid (ceil(tiles / (4 * TW)), B, group slices); block 256. Workgroup x covers tiles
// [x*4*TW, (x+1)*4*TW); wave w takes tiles x*4*TW + w + 4*i, i < TW, two at a time: the loads of
// both tiles of a pair are issued before either is reduced.
// PB: latent-query part loads in flight per thread (1 when every group has a single part).
template <class T, int R, int TW, int PB>
__global__ __launch_bounds__(256) void latent_score_kernel(const float* __restrict__ qpart, int npart,
                                                           const typename T::elem* __restrict__ Lk,
                                                           float* __restrict__ S, int B, int G, int Tc,
                                                           int ldS, int ctx_cap) {
  using W = Win<T>;
  using elem = typename T::elem;
  constexpr int NW = R / W::WLEN;
  constexpr int GPB = T::HILO ? 8 : 16;
  constexpr int OST = R + W::EPC;  // operand row stride in LDS (elements), padded by one chunk
  static_assert(TW % 2 == 0, "tiles are taken in pairs");
  __shared__ __attribute__((aligned(16))) elem opnd[16 * OST];
  __shared__ float4 rsum[256];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n16 = lane & 15, q4 = lane >> 4;
  const int b = blockIdx.y, gb = blockIdx.z;
  const size_t brow = (size_t)b * ctx_cap;
  const int tile0 = blockIdx.x * (kWaves * TW) + wave;
  u32x4 c0[NW], c1[NW];
  if constexpr (PB == 1) {
    // one part per group: the first pair's rows (HBM) are requested first, then the part (one
    // L2 load per quad)
    load_tile<T, R>(Lk, brow, min(tile0 * 16 + n16, Tc - 1), q4, c0);
    load_tile<T, R>(Lk, brow, min((tile0 + 4) * 16 + n16, Tc - 1), q4, c1);
    // operand rows: q~ of group slot gs in row gs (bf16: high part; row 8 + gs the low part).
    // Rows of slots past G are never written; the MFMA rows they feed are never stored. The parts
    // of a column quad are split into npg contiguous ranges (npg = 256 / quads when there are
    // fewer than 256 quads), each summed by one thread with all its loads in flight; the range
    // sums are then added in range order.
    {
      const int gv = min(GPB, G - gb * GPB);
      const int nq = gv * (R / 4);  // column quads of the slice
      const int npg = nq >= 256 ? 1 : min(256 / nq, npart);
      const int per = (npart + npg - 1) / npg;
      const size_t pstride = (size_t)B * G * R;
      for (int e = tid; e < nq * npg; e += 256) {
        const int quad = e % nq, pg = e / nq;
        const int gs = quad / (R / 4), cq = quad % (R / 4);
        const float* src = qpart + ((size_t)b * G + gb * GPB + gs) * R + cq * 4;
        const int pa = pg * per, pe = min(npart, pa + per);
        float4 sum = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int p0 = pa; p0 < pe; p0 += PB) {
          float4 v[PB];
#pragma unroll
          for (int u = 0; u < PB; ++u) v[u] = *(const float4*)(src + (size_t)min(p0 + u, pe - 1) * pstride);
#pragma unroll
          for (int u = 0; u < PB; ++u) {
            if (p0 + u < pe) {
              sum.x += v[u].x;
              sum.y += v[u].y;
              sum.z += v[u].z;
              sum.w += v[u].w;
            }
          }
        }
        if (npg == 1) {
          store_operand_quad<T>(opnd, OST, gs, cq, sum);
        } else {
          rsum[pg * nq + quad] = sum;
        }
      }
      if (npg > 1) {
        __syncthreads();
        for (int quad = tid; quad < nq; quad += 256) {
          float4 sum = rsum[quad];
          for (int pg = 1; pg < npg; ++pg) {
            const float4 v = rsum[pg * nq + quad];
            sum.x += v.x;
            sum.y += v.y;
            sum.z += v.z;
            sum.w += v.w;
          }
          store_operand_quad<T>(opnd, OST, quad / (R / 4), quad % (R / 4), sum);
        }
      }
    }
    __syncthreads();
  } else {
    // several parts per group: their sums are the longer dependent chain before the MFMAs
    // operand rows: q~ of group slot gs in row gs (bf16: high part; row 8 + gs the low part).
    // Rows of slots past G are never written; the MFMA rows they feed are never stored. The parts
    // of a column quad are split into npg contiguous ranges (npg = 256 / quads when there are
    // fewer than 256 quads), each summed by one thread with all its loads in flight; the range
    // sums are then added in range order.
    const int gv = min(GPB, G - gb * GPB);
    const int nq = gv * (R / 4);  // column quads of the slice
    const int npg = nq >= 256 ? 1 : min(256 / nq, npart);
    const int per = (npart + npg - 1) / npg;
    const size_t pstride = (size_t)B * G * R;
    auto part_src = [&](int e, int& gs, int& cq, int& pg, int& pa, int& pe) {
      const int quad = e % nq;
      pg = e / nq;
      gs = quad / (R / 4);
      cq = quad % (R / 4);
      pa = pg * per;
      pe = min(npart, pa + per);
      return qpart + ((size_t)b * G + gb * GPB + gs) * R + cq * 4;
    };
    auto add_parts = [&](const f32x4 (&v)[PB], int p0, int pe, float4& sum) {
#pragma unroll
      for (int u = 0; u < PB; ++u) {
        const bool in = p0 + u < pe;  // branch-free: clamped loads past the range add 0
        sum.x += in ? v[u][0] : 0.f;
        sum.y += in ? v[u][1] : 0.f;
        sum.z += in ? v[u][2] : 0.f;
        sum.w += in ? v[u][3] : 0.f;
      }
    };
    auto put = [&](int e, int gs, int cq, int pg, const float4& sum) {
      if (npg == 1) {
        store_operand_quad<T>(opnd, OST, gs, cq, sum);
      } else {
        rsum[pg * nq + e % nq] = sum;
      }
    };
    // Loads complete in issue order: this thread's first batch of part loads (L2) goes out first
    // as straight-line code, then the first pair's rows (HBM), so that the part sums wait for the
    // parts alone and the operand is built while the rows stream in. The first batch is summed and
    // stored unconditionally (a thread past the last quad repeats it and writes the same values),
    // so that the compiler keeps the loads in this order.
    {
      const int e = min(tid, nq * npg - 1);
      int gs, cq, pg, pa, pe;
      const float* src = part_src(e, gs, cq, pg, pa, pe);
      f32x4 v[PB];
#pragma unroll
      for (int u = 0; u < PB; ++u) v[u] = *(const f32x4*)(src + (size_t)min(pa + u, pe - 1) * pstride);
      // compiler-only fences (no instruction): memory accesses keep their order across them
      asm volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
      load_tile<T, R>(Lk, brow, min(tile0 * 16 + n16, Tc - 1), q4, c0);
      load_tile<T, R>(Lk, brow, min((tile0 + 4) * 16 + n16, Tc - 1), q4, c1);
      // the part registers pass through an empty asm here, so that no sum of them is placed above
      // the row loads (the wait for the parts then follows the row loads' issue)
#pragma unroll
      for (int u = 0; u < PB; ++u) asm volatile("" : "+v"(v[u]) :: "memory");
      __builtin_amdgcn_sched_barrier(0);
      float4 sum = make_float4(0.f, 0.f, 0.f, 0.f);
      add_parts(v, pa, pe, sum);
      for (int p0 = pa + PB; p0 < pe; p0 += PB) {
#pragma unroll
        for (int u = 0; u < PB; ++u) v[u] = *(const f32x4*)(src + (size_t)min(p0 + u, pe - 1) * pstride);
        add_parts(v, p0, pe, sum);
      }
      put(e, gs, cq, pg, sum);
    }
    for (int e = tid + 256; e < nq * npg; e += 256) {
      int gs, cq, pg, pa, pe;
      const float* src = part_src(e, gs, cq, pg, pa, pe);
      float4 sum = make_float4(0.f, 0.f, 0.f, 0.f);
      for (int p0 = pa; p0 < pe; p0 += PB) {
        f32x4 v[PB];
#pragma unroll
        for (int u = 0; u < PB; ++u) v[u] = *(const f32x4*)(src + (size_t)min(p0 + u, pe - 1) * pstride);
        add_parts(v, p0, pe, sum);
      }
      put(e, gs, cq, pg, sum);
    }
    if (npg > 1) {
      lds_barrier();  // range sums visible; the row loads stay in flight
      for (int quad = tid; quad < nq; quad += 256) {
        float4 sum = rsum[quad];
        for (int pg = 1; pg < npg; ++pg) {
          const float4 v = rsum[pg * nq + quad];
          sum.x += v.x;
          sum.y += v.y;
          sum.z += v.z;
          sum.w += v.w;
        }
        store_operand_quad<T>(opnd, OST, quad / (R / 4), quad % (R / 4), sum);
      }
    }
    // nothing that uses the rows moves above the operand
    __builtin_amdgcn_sched_barrier(0);
    lds_barrier();
  }
  // MFMA A operand: row n16 of the operand, natural k layout
  u32x4 a[NW];
#pragma unroll
  for (int w = 0; w < NW; ++w) a[w] = *(const u32x4*)(opnd + n16 * OST + w * W::WLEN + q4 * W::EPC);
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

template <class T, int R, int TW>
void launch_tw(dim3 grid, const float* qpart, int npart, const void* Lk, float* S, int ldS, int B,
               int G, int Tc, int ctx_cap, hipStream_t st) {
  using E = typename T::elem;
  // parts per thread (as the kernel splits them): all of a thread's part loads in one round trip
  constexpr int GPB = T::HILO ? 8 : 16;
  const int nq = (G < GPB ? G : GPB) * (R / 4);
  const int npg = nq >= 256 ? 1 : (256 / nq < npart ? 256 / nq : npart);
  const int per = (npart + npg - 1) / npg;
  if (npart == 1)
    latent_score_kernel<T, R, TW, 1><<<grid, 256, 0, st>>>(qpart, npart, (const E*)Lk, S, B, G, Tc, ldS, ctx_cap);
  else if (per <= 8)
    latent_score_kernel<T, R, TW, 8><<<grid, 256, 0, st>>>(qpart, npart, (const E*)Lk, S, B, G, Tc, ldS, ctx_cap);
  else
    latent_score_kernel<T, R, TW, 16><<<grid, 256, 0, st>>>(qpart, npart, (const E*)Lk, S, B, G, Tc, ldS, ctx_cap);
}

template <class T, int R>
void launch_t(const float* qpart, int npart, const void* Lk, float* S, int ldS, int B, int G, int Tc,
              int ctx_cap, hipStream_t st) {
  constexpr int GPB = T::HILO ? 8 : 16;
  const int tiles = ceil_div(Tc, 16);
  const int slices = ceil_div(G, GPB);
  // two tiles per wave unless that already gives the chip several workgroups per CU
  const bool four = (long)ceil_div(tiles, kWaves * 4) * B * slices >= 1024;
  if (four)
    launch_tw<T, R, 4>(dim3(ceil_div(tiles, kWaves * 4), B, slices), qpart, npart, Lk, S, ldS, B, G, Tc,
                       ctx_cap, st);
  else
    launch_tw<T, R, 2>(dim3(ceil_div(tiles, kWaves * 2), B, slices), qpart, npart, Lk, S, ldS, B, G, Tc,
                       ctx_cap, st);
}

}  // namespace

hipError_t launch_latent_score(int dtype, const float* qpart, int npart, const void* Lk, float* S,
                               int ldS, int B, int G, int r, int Tc, int ctx_cap, hipStream_t st) {
  if (Tc <= 0) return hipSuccess;
  if (npart < 1) return hipErrorInvalidValue;
#define SALS_SCORE_CASE(RR)                                                  \
  case RR:                                                                   \
    if (dtype == 0)                                                          \
      launch_t<F32, RR>(qpart, npart, Lk, S, ldS, B, G, Tc, ctx_cap, st);    \
    else                                                                     \
      launch_t<BF16, RR>(qpart, npart, Lk, S, ldS, B, G, Tc, ctx_cap, st);   \
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
