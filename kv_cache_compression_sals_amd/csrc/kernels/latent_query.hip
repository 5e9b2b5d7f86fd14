// Latent query (SALS 技术框架 stage 2, first half): the RoPE-free decode query of every
// selection group, mapped into the latent space,
//   q~[b][s][j] = sum_{h : group(kv(h)) = s} sum_c q[b][h][c] * P_k[kv(h)*d + c][j].
// Reordered as a sum over the rows of P_k: row i (KV head g = i / d, c = i % d) is weighted by
// qsum[b][i] = sum over the query heads of g of q[b][h][c]. P_k is read once per launch, spread
// over many workgroups: each takes the d rows of one KV head and 64 columns, stages the query
// values of its rows with 16-byte loads, and issues all of its P_k loads before the first use.
// The partial sums of the row blocks of one group are added by a second small kernel in a fixed
// order (skipped when one block covers a whole group), so the result is deterministic.
#include "../common.h"
#include "../launch.h"

namespace sals {
namespace {

constexpr int kBC = 8;         // sequences per pass
constexpr int kThreads = 256;  // 8 column groups x 32 row phases
constexpr int kMaxRows = 128;  // rows per block (one KV head: rps = d)
constexpr int kMaxQH = 8;      // query heads per KV head
constexpr int kRowIt = kMaxRows / 32;

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

// Writes the final q~[b][s][j] into the scoring operand (see launch.h).
template <class T>
__device__ __forceinline__ void store_operand(void* qa, int b, int s, int j, float v, int G, int r) {
  if constexpr (T::HILO) {
    const int nsl = (G + 7) / 8;
    uint16_t* base = (uint16_t*)qa + ((size_t)(b * nsl + s / 8) * 16) * r + j;
    const uint32_t hi = f32_to_bf16_bits(v);
    base[(size_t)(s % 8) * r] = (uint16_t)hi;
    base[(size_t)(8 + s % 8) * r] = (uint16_t)f32_to_bf16_bits(v - bf16_bits_to_f32(hi));
  } else {
    const int nsl = (G + 15) / 16;
    ((float*)qa)[((size_t)(b * nsl + s / 16) * 16 + s % 16) * r + j] = v;
  }
}

// grid (ceil(r/64), D/rps); rows [rs*rps, (rs+1)*rps) of P_k, 64 columns; rps = d, so a block
// is exactly one KV head.
template <class T>
__global__ __launch_bounds__(kThreads) void lq_partial_kernel(
    const typename T::elem* __restrict__ q, const typename T::elem* __restrict__ Pk,
    float* __restrict__ dst, void* __restrict__ qa, int B, int H_q, int H_kv, int d, int r, int G,
    int rps, int direct) {
  using elem = typename T::elem;
  constexpr int EPC = 16 / (int)sizeof(elem);  // elements per 16-byte chunk
  constexpr int NC = 8 / EPC;                  // chunks per 8 columns
  __shared__ float qv[kMaxQH][kBC][kMaxRows];  // query values of this block's rows, per head
  __shared__ float qsum[kBC][kMaxRows];
  __shared__ float red[4][kBC][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int cg = tid & 7, rp = tid >> 3;
  const int rs = blockIdx.y;
  const int row0 = rs * rps;
  const int col0 = min(blockIdx.x * 64 + cg * 8, r - 8);  // columns past r are never written
  const int nqh = H_q / H_kv;
  const int D = H_kv * d;
  const int grp = row0 / (D / G);
  const int g = row0 / d, c0 = row0 % d;  // the block lies inside KV head g (rps <= d)

  // P_k rows of this thread, all in flight before the query staging completes
  u32x4 pc[kRowIt][NC];
#pragma unroll
  for (int it = 0; it < kRowIt; ++it) {
    const int i = min(rp + 32 * it, rps - 1);
#pragma unroll
    for (int m = 0; m < NC; ++m) pc[it][m] = *(const u32x4*)(Pk + (size_t)(row0 + i) * r + col0 + m * EPC);
  }

  for (int b0 = 0; b0 < B; b0 += kBC) {
    const int nb = min(kBC, B - b0);
    __syncthreads();
    // qv[h][bb][i] = q[b0 + bb][g * nqh + h][c0 + i], 16 bytes per load
    const int cpr = rps / EPC;  // chunks per (head, sequence)
    batched_copy<4>(
        nqh * nb * cpr, tid, kThreads,
        [&](int e) {
          const int h = e / (nb * cpr), bb = (e / cpr) % nb, ch = e % cpr;
          return *(const u32x4*)(q + ((size_t)(b0 + bb) * H_q + (size_t)g * nqh + h) * d + c0 + ch * EPC);
        },
        [&](int e, const u32x4& v) {
          const int h = e / (nb * cpr), bb = (e / cpr) % nb, ch = e % cpr;
          float* dstp = &qv[h][bb][ch * EPC];
          if constexpr (EPC == 8) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              dstp[2 * j] = __uint_as_float(v[j] << 16);
              dstp[2 * j + 1] = __uint_as_float(v[j] & 0xffff0000u);
            }
          } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) dstp[j] = __uint_as_float(v[j]);
          }
        });
    __syncthreads();
    for (int e = tid; e < nb * rps; e += kThreads) {
      const int bb = e / rps, i = e % rps;
      float s = 0.f;
      for (int h = 0; h < nqh; ++h) s += qv[h][bb][i];
      qsum[bb][i] = s;
    }
    __syncthreads();
    float acc[kBC][8];
#pragma unroll
    for (int bb = 0; bb < kBC; ++bb)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[bb][j] = 0.f;
#pragma unroll
    for (int it = 0; it < kRowIt; ++it) {
      const int i = rp + 32 * it;
      if (i < rps) {
        float p[8];
        unpack8<T>(pc[it], p);
#pragma unroll
        for (int bb = 0; bb < kBC; ++bb) {
          const float wgt = bb < nb ? qsum[bb][i] : 0.f;
#pragma unroll
          for (int j = 0; j < 8; ++j) acc[bb][j] = fmaf(wgt, p[j], acc[bb][j]);
        }
      }
    }
    // reduce the 8 row phases of a wave (lane bits 3..5), then the 4 waves
#pragma unroll
    for (int bb = 0; bb < kBC; ++bb)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float v = acc[bb][j];
        v += __shfl_xor(v, 8);
        v += __shfl_xor(v, 16);
        v += __shfl_xor(v, 32);
        acc[bb][j] = v;
      }
    if (lane < 8) {
#pragma unroll
      for (int bb = 0; bb < kBC; ++bb)
#pragma unroll
        for (int j = 0; j < 8; ++j) red[wave][bb][lane * 8 + j] = acc[bb][j];
    }
    __syncthreads();
    for (int e = tid; e < nb * 64; e += kThreads) {
      const int bb = e / 64, cc = e % 64;
      const int col = blockIdx.x * 64 + cc;
      // (col0 is clamped only for column groups lying wholly at or past r, skipped here)
      if (col < r) {
        const float v = red[0][bb][cc] + red[1][bb][cc] + red[2][bb][cc] + red[3][bb][cc];
        if (direct)
          store_operand<T>(qa, b0 + bb, grp, col, v, G, r);
        else
          dst[((size_t)rs * B + b0 + bb) * r + col] = v;
      }
    }
  }
}

// q~[b][s][j] = sum over the row blocks of group s of qpart[rs][b][j], in block order, stored
// into the scoring operand.
template <class T>
__global__ __launch_bounds__(256) void lq_reduce_kernel(const float* __restrict__ qpart,
                                                        void* __restrict__ qa, int B, int G, int r,
                                                        int splits_per_group) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= B * G * r) return;
  const int j = e % r, s = (e / r) % G, b = e / (r * G);
  const float* src = qpart + ((size_t)s * splits_per_group * B + b) * r + j;
  const size_t stride = (size_t)B * r;
  float v = 0.f;
  for (int i0 = 0; i0 < splits_per_group; i0 += 16) {
    float x[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) x[u] = src[(size_t)min(i0 + u, splits_per_group - 1) * stride];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < 16; ++u) v += i0 + u < splits_per_group ? x[u] : 0.f;
  }
  store_operand<T>(qa, b, s, j, v, G, r);
}

}  // namespace

hipError_t launch_latent_query(int dtype, const void* q, const void* Pk, float* qpart, void* qa,
                               int B, int H_q, int H_kv, int d, int r, int G, int rps,
                               hipStream_t st) {
  const int D = H_kv * d;
  const int n_rs = D / rps;
  const int spg = (D / G) / rps;
  const bool direct = spg == 1;
  dim3 grid(ceil_div(r, 64), n_rs);
  if (dtype == 0)
    lq_partial_kernel<F32><<<grid, kThreads, 0, st>>>((const float*)q, (const float*)Pk, qpart, qa, B,
                                                      H_q, H_kv, d, r, G, rps, direct);
  else
    lq_partial_kernel<BF16><<<grid, kThreads, 0, st>>>((const uint16_t*)q, (const uint16_t*)Pk, qpart,
                                                       qa, B, H_q, H_kv, d, r, G, rps, direct);
  if (!direct) {
    const int n = B * G * r;
    if (dtype == 0)
      lq_reduce_kernel<F32><<<ceil_div(n, 256), 256, 0, st>>>(qpart, qa, B, G, r, spg);
    else
      lq_reduce_kernel<BF16><<<ceil_div(n, 256), 256, 0, st>>>(qpart, qa, B, G, r, spg);
  }
  return hipGetLastError();
}

}  // namespace sals
