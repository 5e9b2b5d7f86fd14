// Exact per-row top-k with the recent window appended (SALS 关键设计 items 2 and 4; the top-k
// index set S_{psi,k} of the VL-Cache responses, reviewer XVzL weakness 2).
//
// One workgroup of 1024 threads per row. Scores become order-preserving uint32 keys (signed
// zeros equal). An MSB-first radix select (four 8-bit digit passes, per-wave LDS histograms)
// finds the kp-th largest key tau and how many keys equal to tau are taken (the lowest-index
// ones). An ordered compaction then writes the selected indices ascending: the output slot of
// index i is #(keys > tau before i) + min(#(keys == tau before i), take_eq), from one block-wide
// exclusive scan of packed (gt, eq) counts per chunk. Rows up to 32768 candidates are staged
// in LDS once; longer rows are re-read from global memory (L2) on every pass.
#include "../common.h"
#include "../launch.h"

namespace sals {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kLdsKeys = 32768;
constexpr int kIPT = 8;  // consecutive items per thread in the compaction

template <bool IN_LDS>
__global__ __launch_bounds__(kThreads) void topk_window_kernel(const float* __restrict__ S,
                                                               int32_t* __restrict__ sel, int Tc,
                                                               int kp, int ctx, int n_sel) {
  __shared__ uint32_t keys[IN_LDS ? kLdsKeys : 1];
  __shared__ uint32_t hist[kWaves][256];
  __shared__ uint32_t bcast[2];
  __shared__ uint32_t wsum[kWaves];
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
    for (int i = tid; i < Tc; i += kThreads) keys[i] = float_key(src[i]);
  }
  auto key_at = [&](int i) -> uint32_t {
    if constexpr (IN_LDS) return keys[i];
    else return float_key(src[i]);
  };

  uint32_t prefix = 0, mask = 0;
  uint32_t remaining = (uint32_t)kp;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < kWaves * 256; i += kThreads) (&hist[0][0])[i] = 0;
    __syncthreads();
    for (int i = tid; i < Tc; i += kThreads) {
      const uint32_t k = key_at(i);
      if ((k & mask) == prefix) atomicAdd(&hist[wave][(k >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid < 256) {
      uint32_t s = 0;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) s += hist[w][tid];
      hist[0][tid] = s;
    }
    __syncthreads();
    if (wave == 0) {
      uint32_t c[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) c[j] = hist[0][4 * lane + j];
      const uint32_t tot = c[0] + c[1] + c[2] + c[3];
      uint32_t suf = tot;  // keys in this lane's bins and all higher bins
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t t = __shfl_down(suf, o);
        if (lane + o < 64) suf += t;
      }
      const uint32_t above = suf - tot;
      if (above < remaining && remaining <= suf) {
        uint32_t a = above;
        int bin = 4 * lane;
        for (int j = 3; j >= 0; --j) {
          if (a + c[j] >= remaining) {
            bin = 4 * lane + j;
            break;
          }
          a += c[j];
        }
        bcast[0] = (uint32_t)bin;
        bcast[1] = a;
      }
    }
    __syncthreads();
    prefix |= bcast[0] << shift;
    mask |= 0xffu << shift;
    remaining -= bcast[1];
    __syncthreads();
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
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    uint32_t wbase = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const uint32_t s = wsum[w];
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
