// Latent query (SALS 技术框架 stage 2, first half): the RoPE-free decode query of every
// selection group, mapped into the latent space,
//   q~[b][s][j] = sum_{h : group(kv(h)) = s} sum_c q[b][h][c] * P_k[kv(h)*d + c][j].
// Reordered as a sum over the rows of P_k: row i (KV head g = i / d, c = i % d) is weighted by
// qsum[b][i] = sum over the query heads of g of q[b][h][c]. P_k is read once per launch, spread
// over many workgroups: each takes RB rows inside one group and 64 latent columns. It issues
// all of its P_k loads first (a wave instruction reads 8 rows x 128 bytes, whole cache lines),
// forms qsum for its rows while they are in flight, and accumulates per thread over its rows.
// The 32 row phases of a workgroup are added by one DPP step and then through LDS, in a fixed
// order. The result is the partial sum over the block's rows, qpart[part][b][s][j]; with one
// block per group it is q~ itself, otherwise the scoring kernel adds the parts of a group in
// part order before use. Every sum has a fixed order, so the result is deterministic.
#include "../common.h"
#include "../launch.h"

namespace sals {
namespace {

constexpr int kBC = 8;         // sequences per pass
constexpr int kThreads = 256;  // 8 column groups x 32 row phases
constexpr int kQB = 8;         // query-head loads in flight per qsum chunk

template <class T>
__device__ __forceinline__ void unpack8(const u32x4 (&c)[16 / sizeof(typename T::elem) == 8 ? 1 : 2],
                                        float* v);

template <>
__device__ __forceinline__ void unpack8<BF16>(const u32x4 (&c)[1], float* v) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    v[2 * j] = __uint_as_float(c[0][j] << 16);
    v[2 * j + 1] = __uint_as_float(c[0][j] & 0xffff0000u);
  }
}

template <>
__device__ __forceinline__ void unpack8<F32>(const u32x4 (&c)[2], float* v) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    v[j] = __uint_as_float(c[0][j]);
    v[4 + j] = __uint_as_float(c[1][j]);
  }
}

// grid (ceil(r/64), D/RB): block y covers rows [y*RB, (y+1)*RB) of P_k (inside one group),
// block x latent columns [x*64, x*64 + 64). Thread (cg = tid & 7, rp = tid >> 3) owns columns
// x*64 + cg*8 .. +8 and rows rp + 32*i.
template <class T, int RB>
__global__ __launch_bounds__(kThreads) void latent_query_kernel(const typename T::elem* __restrict__ q,
                                                                const typename T::elem* __restrict__ Pk,
                                                                float* __restrict__ qpart, int B,
                                                                int H_q, int H_kv, int d, int r, int G) {
  using elem = typename T::elem;
  constexpr int EPC = 16 / (int)sizeof(elem);  // elements per 16-byte chunk
  constexpr int NC = 8 / EPC;                  // chunks per 8 columns
  constexpr int RPT = RB / 32;                 // rows per thread
  constexpr int QCH = RB / EPC;                // 16-byte query chunks per sequence
  static_assert(RB % 32 == 0 && RB <= 256, "row block");
  __shared__ float qsum[kBC][RB];
  __shared__ __attribute__((aligned(16))) float red[16][kBC][64];  // even row phases after DPP
  const int tid = threadIdx.x;
  const int cg = tid & 7, rp = tid >> 3;
  const int row0 = blockIdx.y * RB;
  const int c0 = blockIdx.x * 64;
  const int col = min(c0 + cg * 8, r - 8);  // columns past r are computed but never stored
  const int nqh = H_q / H_kv;
  const int group_rows = H_kv * d / G;
  const int s = row0 / group_rows, part = (row0 % group_rows) / RB;

  // qsum[bb][i] = sum_h q[b0 + bb][g * nqh + h][c] for row row0 + i = g * d + c; a chunk of
  // EPC rows never straddles a KV head (d is a multiple of EPC). Thread tid owns the chunks
  // e = tid + kThreads * n of each pass.
  auto qload = [&](int b0, int e, u32x4 (&v)[kQB], int h0) {
    const int nb = min(kBC, B - b0);
    const int ee = min(e, nb * QCH - 1);
    const int bb = ee / QCH, ch = ee % QCH;
    const int row = row0 + ch * EPC;
    const int g = row / d, c = row % d;
    const elem* qp = q + ((size_t)(b0 + bb) * H_q + (size_t)g * nqh) * d + c;
#pragma unroll
    for (int u = 0; u < kQB; ++u) v[u] = *(const u32x4*)(qp + (size_t)min(h0 + u, nqh - 1) * d);
  };
  auto qadd = [&](const u32x4 (&v)[kQB], int h0, float (&acc)[EPC]) {
    // branch-free: heads past nqh (clamped loads of the last head) add zero
#pragma unroll
    for (int u = 0; u < kQB; ++u) {
      const uint32_t keep = h0 + u < nqh ? 0xffffffffu : 0u;
      if constexpr (EPC == 8) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[2 * j] += __uint_as_float((v[u][j] << 16) & keep);
          acc[2 * j + 1] += __uint_as_float(v[u][j] & 0xffff0000u & keep);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] += __uint_as_float(v[u][j] & keep);
      }
    }
  };
  // stages qsum for chunks e0, e0 + kThreads, ... of the pass starting at sequence b0
  auto stage_q = [&](int b0, int e0) {
    const int nb = min(kBC, B - b0);
    for (int e = e0; e < nb * QCH; e += kThreads) {
      const int bb = e / QCH, ch = e % QCH;
      float acc[EPC];
#pragma unroll
      for (int x = 0; x < EPC; ++x) acc[x] = 0.f;
      for (int h0 = 0; h0 < nqh; h0 += kQB) {
        u32x4 v[kQB];
        qload(b0, e, v, h0);
        qadd(v, h0, acc);
      }
#pragma unroll
      for (int x = 0; x < EPC; ++x) qsum[bb][ch * EPC + x] = acc[x];
    }
  };
  // The first chunk of the first pass is straight-line code: its query loads go out first, then
  // the P_k rows (loads complete in issue order, so the query sums wait for the queries alone),
  // then its sums, written unconditionally (a thread past the last chunk repeats the last one
  // and writes the same values), so that the compiler keeps the loads in this order.
  u32x4 qv0[kQB];
  qload(0, tid, qv0, 0);
  __builtin_amdgcn_sched_barrier(0);
  u32x4 pc[RPT][NC];
#pragma unroll
  for (int i = 0; i < RPT; ++i)
#pragma unroll
    for (int m = 0; m < NC; ++m) pc[i][m] = *(const u32x4*)(Pk + (size_t)(row0 + rp + 32 * i) * r + col + m * EPC);
  __builtin_amdgcn_sched_barrier(0);
  {
    const int nb0 = min(kBC, B);
    const int ee = min(tid, nb0 * QCH - 1);
    float acc[EPC];
#pragma unroll
    for (int x = 0; x < EPC; ++x) acc[x] = 0.f;
    qadd(qv0, 0, acc);
    for (int h0 = kQB; h0 < nqh; h0 += kQB) {
      u32x4 v[kQB];
      qload(0, ee, v, h0);
      qadd(v, h0, acc);
    }
#pragma unroll
    for (int x = 0; x < EPC; ++x) qsum[ee / QCH][(ee % QCH) * EPC + x] = acc[x];
  }
  stage_q(0, tid + kThreads);
  // nothing that uses P_k (the compiler hoists their unpacking out of the pass loop) moves above
  // the query sums
  __builtin_amdgcn_sched_barrier(0);
  lds_barrier();  // qsum visible; the P_k loads stay in flight

  for (int b0 = 0; b0 < B; b0 += kBC) {
    const int nb = min(kBC, B - b0);
    if (b0 > 0) {
      __syncthreads();  // the previous pass is done with qsum and red
      stage_q(b0, tid);
      __syncthreads();
    }
    float acc[kBC][8];
#pragma unroll
    for (int bb = 0; bb < kBC; ++bb)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[bb][j] = 0.f;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int rr = rp + 32 * i;
      float p[8];
      unpack8<T>(pc[i], p);
#pragma unroll
      for (int bb = 0; bb < kBC; ++bb) {
        const float wgt = bb < nb ? qsum[bb][rr] : 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[bb][j] = fmaf(wgt, p[j], acc[bb][j]);
      }
    }
    // row phases rp and rp ^ 1 sit 8 lanes apart in one DPP row: one rotation by 8 adds them
#pragma unroll
    for (int bb = 0; bb < kBC; ++bb)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[bb][j] += dpp_f32<0x128>(acc[bb][j]);
    if ((rp & 1) == 0) {
#pragma unroll
      for (int bb = 0; bb < kBC; ++bb) {
        float4* dst = (float4*)&red[rp >> 1][bb][cg * 8];
        dst[0] = make_float4(acc[bb][0], acc[bb][1], acc[bb][2], acc[bb][3]);
        dst[1] = make_float4(acc[bb][4], acc[bb][5], acc[bb][6], acc[bb][7]);
      }
    }
    __syncthreads();
    // 16 column quads per sequence; the 16 pair sums are added in row-phase order
    if (tid < nb * 16) {
      const int bb = tid >> 4, cq = tid & 15;
      if (c0 + cq * 4 < r) {
        float4 v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) v[u] = *(const float4*)&red[u][bb][cq * 4];
        float4 sum = v[0];
#pragma unroll
        for (int u = 1; u < 16; ++u) {
          sum.x += v[u].x;
          sum.y += v[u].y;
          sum.z += v[u].z;
          sum.w += v[u].w;
        }
        *(float4*)(qpart + (((size_t)part * B + b0 + bb) * G + s) * r + c0 + cq * 4) = sum;
      }
    }
  }
}

template <class T>
void launch_t(const void* q, const void* Pk, float* qpart, int B, int H_q, int H_kv, int d, int r,
              int G, int rb, hipStream_t st) {
  using E = typename T::elem;
  const dim3 grid(ceil_div(r, 64), H_kv * d / rb);
  if (rb == 64)
    latent_query_kernel<T, 64><<<grid, kThreads, 0, st>>>((const E*)q, (const E*)Pk, qpart, B, H_q, H_kv, d, r, G);
  else if (rb == 128)
    latent_query_kernel<T, 128><<<grid, kThreads, 0, st>>>((const E*)q, (const E*)Pk, qpart, B, H_q, H_kv, d, r, G);
  else
    latent_query_kernel<T, 256><<<grid, kThreads, 0, st>>>((const E*)q, (const E*)Pk, qpart, B, H_q, H_kv, d, r, G);
}

}  // namespace

int latent_query_rows(int H_kv, int d, int r, int G) {
  const int group_heads = H_kv / G;
  // two KV heads per block when that still gives the chip enough workgroups: fewer parts for
  // the scoring kernel to add
  if (2 * d <= 256 && group_heads % 2 == 0 && (long)ceil_div(r, 64) * (H_kv / 2) >= kLqMinBlocks)
    return 2 * d;
  return d;
}

hipError_t launch_latent_query(int dtype, const void* q, const void* Pk, float* qpart, int B,
                               int H_q, int H_kv, int d, int r, int G, int rb, hipStream_t st) {
  if (rb != 64 && rb != 128 && rb != 256) return hipErrorInvalidValue;
  if (dtype == 0)
    launch_t<F32>(q, Pk, qpart, B, H_q, H_kv, d, r, G, rb, st);
  else
    launch_t<BF16>(q, Pk, qpart, B, H_q, H_kv, d, r, G, rb, st);
  return hipGetLastError();
}

}  // namespace sals
