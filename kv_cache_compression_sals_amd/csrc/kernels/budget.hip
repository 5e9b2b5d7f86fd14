// Importance-mass budgets: per (sequence, KV head) row of a non-negative importance, the smallest
// number of tokens whose importance holds a fraction `mass` of the row's total (ZipVL abstract:
// the ratio of important tokens follows the layer's attention-score distribution instead of a
// fixed hyper-parameter), plus the row totals, the layer's ratio and the layer's summed
// importance (the energy a FlashCache-style per-layer budget is proportional to).
//
// One 1024-thread workgroup per row, the row staged in LDS (rows up to 32768 tokens; longer rows
// are read from memory in every pass). For non-negative floats the bit pattern orders like the
// value, so the search runs over 31-bit keys: the total and every partial mass are fp64 sums in a
// fixed order (per-thread runs, then the waves in order; the layer energy adds the fp32 row
// totals in fp64), and a binary search finds the largest
// key kappa with mass(key >= kappa) >= mass * total. The smallest value v at or above kappa is the
// boundary; n = #(> v) + the number of values equal to v needed to reach the target. Negative
// inputs count as zero.
#include "../common.h"
#include "../launch.h"

namespace sals {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kLds = 32768;

__device__ __forceinline__ uint32_t nonneg_bits(float v) { return v > 0.f ? __float_as_uint(v) : 0u; }

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) v += __shfl_xor(v, o);
  return v;
}

template <bool IN_LDS>
__global__ __launch_bounds__(kThreads) void mass_budget_kernel(const float* __restrict__ imp, int ctx, float mass,
                                                               int32_t* __restrict__ n_keep, float* __restrict__ total_out) {
  __shared__ uint32_t keys[IN_LDS ? kLds : 1];
  __shared__ double wred[kWaves];
  __shared__ uint32_t ured[kWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* row = imp + (size_t)blockIdx.x * ctx;
  auto key_at = [&](int i) -> uint32_t {
    if constexpr (IN_LDS) return keys[i];
    else return nonneg_bits(row[i]);
  };
  if constexpr (IN_LDS) {
    batched_copy<kLds / kThreads>(ctx, tid, kThreads, [&](int i) { return row[i]; },
                                  [&](int i, float v) { keys[i] = nonneg_bits(v); });
    __syncthreads();
  }
  // fixed-order block sums: per-thread runs, then the wave totals in wave order
  auto block_sum = [&](double v) -> double {
    v = wave_sum_f64(v);
    if (lane == 0) wred[wave] = v;
    __syncthreads();
    double s = 0.0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) s += wred[w];
    __syncthreads();
    return s;
  };
  auto block_count = [&](uint32_t v) -> uint32_t {
    v = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan(v, lane), 63);
    if (lane == 0) ured[wave] = v;
    __syncthreads();
    uint32_t s = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) s += ured[w];
    __syncthreads();
    return s;
  };
  auto mass_at_least = [&](uint32_t kappa) -> double {
    double m = 0.0;
    for (int i = tid; i < ctx; i += kThreads) {
      const uint32_t k = key_at(i);
      m += k >= kappa ? (double)__uint_as_float(k) : 0.0;
    }
    return block_sum(m);
  };
  const double total = mass_at_least(0u);
  const double target = (double)mass * total;
  int n = 1;
  if (target > 0.0) {
    uint32_t lo = 0u, hi = 0x7f7fffffu;  // mass(>= lo) >= target always holds
    while (lo < hi) {
      const uint32_t mid = lo + (hi - lo + 1u) / 2u;
      if (mass_at_least(mid) >= target) lo = mid;
      else hi = mid - 1u;
    }
    // boundary value: the smallest key at or above lo
    uint32_t vmin = 0xffffffffu;
    for (int i = tid; i < ctx; i += kThreads) {
      const uint32_t k = key_at(i);
      if (k >= lo) vmin = min(vmin, k);
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) vmin = min(vmin, (uint32_t)__shfl_xor((int)vmin, o));
    if (lane == 0) ured[wave] = vmin;
    __syncthreads();
    uint32_t vb = 0xffffffffu;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) vb = min(vb, ured[w]);
    __syncthreads();
    const double mass_gt = mass_at_least(vb + 1u);
    uint32_t cgt = 0, ceq = 0;
    for (int i = tid; i < ctx; i += kThreads) {
      const uint32_t k = key_at(i);
      cgt += k > vb ? 1u : 0u;
      ceq += k == vb ? 1u : 0u;
    }
    cgt = block_count(cgt);
    ceq = block_count(ceq);
    // values equal to the boundary needed on top of the larger ones
    const double v = (double)__uint_as_float(vb);  // > 0: all mass sits at positive keys
    double m = ceil((target - mass_gt) / v);
    m = fmin(fmax(m, 1.0), (double)ceq);
    n = (int)cgt + (int)m;
  }
  if (tid == 0) {
    n_keep[blockIdx.x] = n;
    total_out[blockIdx.x] = (float)total;
  }
}

// layer aggregates in a fixed order: ratio = sum(n_keep) / (rows * ctx), energy = sum(totals)
__global__ __launch_bounds__(256) void layer_budget_kernel(const int32_t* __restrict__ n_keep,
                                                           const float* __restrict__ row_total, int rows, int ctx,
                                                           float* __restrict__ ratio, float* __restrict__ energy) {
  __shared__ double sred[4][2];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  double sn = 0.0, se = 0.0;
  for (int i = tid; i < rows; i += 256) {
    sn += (double)n_keep[i];
    se += (double)row_total[i];
  }
  sn = wave_sum_f64(sn);
  se = wave_sum_f64(se);
  if (lane == 0) {
    sred[wave][0] = sn;
    sred[wave][1] = se;
  }
  __syncthreads();
  if (tid == 0) {
    const double n = (sred[0][0] + sred[1][0]) + (sred[2][0] + sred[3][0]);
    const double e = (sred[0][1] + sred[1][1]) + (sred[2][1] + sred[3][1]);
    if (ratio) *ratio = (float)(n / ((double)rows * ctx));
    if (energy) *energy = (float)e;
  }
}

}  // namespace

hipError_t launch_mass_budget(const float* imp, int rows, int ctx, float mass, int32_t* n_keep, float* total,
                              float* ratio, float* energy, hipStream_t st) {
  if (ctx <= kLds)
    mass_budget_kernel<true><<<rows, kThreads, 0, st>>>(imp, ctx, mass, n_keep, total);
  else
    mass_budget_kernel<false><<<rows, kThreads, 0, st>>>(imp, ctx, mass, n_keep, total);
  if (ratio || energy) layer_budget_kernel<<<1, 256, 0, st>>>(n_keep, total, rows, ctx, ratio, energy);
  return hipGetLastError();
}

}  // namespace sals
