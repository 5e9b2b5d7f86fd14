// Exact per-row top-k with the recent window appended (SALS 关键设计 items 2 and 4; the top-k
// index set S_{psi,k} of the VL-Cache responses, reviewer XVzL weakness 2).
//
// One workgroup of 1024 threads per row. Scores become order-preserving uint32 keys (signed
// zeros equal). The k-th largest key tau is found by an MSB-first radix select:
//   1. a 2048-bin histogram of the top 11 key bits (sign, exponent, 2 mantissa bits) over the
//      whole row; scores spread over many such bins, so LDS atomics rarely collide;
//   2. the keys of the bin holding the k-th largest are gathered into an LDS candidate list and
//      the remaining 21 bits are resolved on that short list (11 + 10 bits);
//   3. if that bin is too full for the list (heavily tied or degenerate rows), the remaining
//      bits are resolved over the whole row instead (same digits, slower).
// An ordered compaction then writes the selected indices ascending: the output slot of index i
// is #(keys > tau before i) + min(#(keys == tau before i), take_eq), from one block-wide
// exclusive scan of packed (gt, eq) counts per chunk. Rows up to 32768 candidates are staged
// in LDS once; longer rows are re-read from global memory (L2) on every pass.
#include "../common.h"
#include "../launch.h"

namespace sals {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kLdsKeys = 32768;
constexpr int kCandMax = 4096;
constexpr int kBins = 2048;
constexpr int kIPT = 8;  // consecutive items per thread in the compaction

// Finds, in hist[0 .. nbins), the bin b holding the `remaining`-th largest item (bins ordered by
// value, highest bin = largest) and the number of items in bins above it. Uses all threads.
__device__ __forceinline__ void find_bin(const uint32_t* hist, int nbins, uint32_t remaining,
                                         uint32_t* scan, uint32_t* bcast) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // each thread owns bins [2*tid, 2*tid + 2) of a 2048-bin histogram (fewer bins: zeros)
  const int b0 = 2 * tid;
  const uint32_t c0 = b0 < nbins ? hist[b0] : 0u, c1 = b0 + 1 < nbins ? hist[b0 + 1] : 0u;
  const uint32_t tot = c0 + c1;
  // suffix sum over the bins: within the wave, then over the waves above this one
  uint32_t v = tot;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t t = __shfl_down(v, o);
    if (lane + o < 64) v += t;
  }
  // v = sum over lanes >= lane of this wave
  if (lane == 0) scan[wave] = v;
  __syncthreads();
  uint32_t above_waves = 0;
  for (int w = wave + 1; w < kWaves; ++w) above_waves += scan[w];
  const uint32_t suf = v + above_waves;  // items in this thread's bins and all higher bins
  const uint32_t above = suf - tot;
  if (above < remaining && remaining <= suf) {
    if (above + c1 >= remaining) {
      bcast[0] = (uint32_t)(b0 + 1);
      bcast[1] = above;
    } else {
      bcast[0] = (uint32_t)b0;
      bcast[1] = above + c1;
    }
  }
  __syncthreads();
}

template <bool IN_LDS>
__global__ __launch_bounds__(kThreads) void topk_window_kernel(const float* __restrict__ S,
                                                               int32_t* __restrict__ sel, int Tc,
                                                               int kp, int ctx, int n_sel) {
  __shared__ uint32_t keys[IN_LDS ? kLdsKeys : 1];
  __shared__ uint32_t hist[kBins];
  __shared__ int32_t cand[kCandMax];
  __shared__ uint32_t scan[kWaves];
  __shared__ uint32_t bcast[4];
  const int row = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* __restrict__ src = S + (size_t)row * Tc;
  int32_t* __restrict__ out = sel + (size_t)row * n_sel;

  for (int j = tid; j < ctx - Tc; j += kThreads) out[kp + j] = Tc + j;
  if (kp <= 0) return;
  if (kp >= Tc) {
    for (int j = tid; j < Tc; j += kThreads) out[j] = j;
    return;
  }
  if constexpr (IN_LDS) {
    batched_copy<8>(Tc, tid, kThreads, [&](int i) { return src[i]; },
                    [&](int i, float v) { keys[i] = float_key(v); });
  }
  auto key_at = [&](int i) -> uint32_t {
    if constexpr (IN_LDS) return keys[i];
    else return float_key(src[i]);
  };

  // ---- digit 1: key bits [31:21] over the whole row ----
  for (int i = tid; i < kBins; i += kThreads) hist[i] = 0;
  if (tid == 0) bcast[2] = 0;
  __syncthreads();
  batched_copy<8>(Tc, tid, kThreads, key_at, [&](int, uint32_t k) { atomicAdd(&hist[k >> 21], 1u); });
  __syncthreads();
  uint32_t remaining = (uint32_t)kp;
  find_bin(hist, kBins, remaining, scan, bcast);
  const uint32_t bin1 = bcast[0];
  remaining -= bcast[1];
  const uint32_t n_in_bin = hist[bin1];
  __syncthreads();

  uint32_t prefix = bin1 << 21;
  if (n_in_bin <= (uint32_t)kCandMax) {
    // ---- gather the bin's keys, resolve bits [20:10] and [9:0] on the short list ----
    batched_copy<8>(Tc, tid, kThreads, key_at, [&](int i, uint32_t k) {
      if ((k >> 21) == bin1) {
        const uint32_t slot = atomicAdd(&bcast[2], 1u);
        cand[slot] = i;
      }
    });
    __syncthreads();
    const int nc = (int)n_in_bin;
#pragma unroll 1
    for (int pass = 0; pass < 2; ++pass) {
      const int shift = pass == 0 ? 10 : 0;
      const uint32_t dmask = pass == 0 ? 0x7ffu : 0x3ffu;
      const uint32_t pmask = pass == 0 ? 0xffe00000u : 0xfffffc00u;
      for (int i = tid; i < kBins; i += kThreads) hist[i] = 0;
      __syncthreads();
      for (int j = tid; j < nc; j += kThreads) {
        const uint32_t k = key_at(cand[j]);
        if ((k & pmask) == prefix) atomicAdd(&hist[(k >> shift) & dmask], 1u);
      }
      __syncthreads();
      find_bin(hist, kBins, remaining, scan, bcast);
      prefix |= bcast[0] << shift;
      remaining -= bcast[1];
      __syncthreads();
    }
  } else {
    // ---- heavily tied row: resolve the remaining digits over the whole row ----
#pragma unroll 1
    for (int pass = 0; pass < 2; ++pass) {
      const int shift = pass == 0 ? 10 : 0;
      const uint32_t dmask = pass == 0 ? 0x7ffu : 0x3ffu;
      const uint32_t pmask = pass == 0 ? 0xffe00000u : 0xfffffc00u;
      for (int i = tid; i < kBins; i += kThreads) hist[i] = 0;
      __syncthreads();
      batched_copy<8>(Tc, tid, kThreads, key_at, [&](int, uint32_t k) {
        if ((k & pmask) == prefix) atomicAdd(&hist[(k >> shift) & dmask], 1u);
      });
      __syncthreads();
      find_bin(hist, kBins, remaining, scan, bcast);
      prefix |= bcast[0] << shift;
      remaining -= bcast[1];
      __syncthreads();
    }
  }
  const uint32_t tau = prefix;
  const uint32_t take_eq = remaining;  // >= 1

  uint32_t run_gt = 0, run_eq = 0;
  for (int base = 0; base < Tc; base += kThreads * kIPT) {
    const int i0 = base + tid * kIPT;
    uint32_t fgt = 0, feq = 0;
#pragma unroll
    for (int j = 0; j < kIPT; ++j) {
      const int i = i0 + j;
      if (i < Tc) {
        const uint32_t k = key_at(i);
        fgt |= (uint32_t)(k > tau) << j;
        feq |= (uint32_t)(k == tau) << j;
      }
    }
    const uint32_t packed = (uint32_t)__popc(fgt) | ((uint32_t)__popc(feq) << 16);
    const uint32_t incl = wave_incl_scan(packed, lane);
    if (lane == 63) scan[wave] = incl;
    __syncthreads();
    uint32_t wbase = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const uint32_t s = scan[w];
      wbase += (w < wave) ? s : 0u;
      total += s;
    }
    const uint32_t excl = wbase + incl - packed;
    uint32_t ngt = run_gt + (excl & 0xffffu), neq = run_eq + (excl >> 16);
#pragma unroll
    for (int j = 0; j < kIPT; ++j) {
      if ((fgt >> j) & 1u) {
        out[ngt + min(neq, take_eq)] = i0 + j;
        ++ngt;
      } else if ((feq >> j) & 1u) {
        if (neq < take_eq) out[ngt + neq] = i0 + j;
        ++neq;
      }
    }
    run_gt += total & 0xffffu;
    run_eq += total >> 16;
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_topk_window(const float* S, int32_t* sel, int rows, int Tc, int kp, int ctx,
                              int n_sel, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  if (Tc <= kLdsKeys)
    topk_window_kernel<true><<<rows, kThreads, 0, st>>>(S, sel, Tc, kp, ctx, n_sel);
  else
    topk_window_kernel<false><<<rows, kThreads, 0, st>>>(S, sel, Tc, kp, ctx, n_sel);
  return hipGetLastError();
}

}  // namespace sals
