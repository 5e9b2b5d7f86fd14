// Device-side helpers shared by the gfx950 kernels: element types, MFMA fragment access,
// key transforms and wave-level reductions. Wavefronts are 64 lanes wide.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sals {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// fp32 -> bf16 bits, round to nearest, ties to even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// Storage element types. HILO: the latent query is split into bf16 high + low parts so that a
// bf16 MFMA reproduces an fp32 dot product to ~2^-16 relative.
struct F32 {
  using elem = float;
  static constexpr int KSTEP = 4;  // k per 16x16 MFMA
  static constexpr int KPL = 1;    // k elements per lane per MFMA
  static constexpr bool HILO = false;
  using frag = float;
  __device__ static __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
  __device__ static __forceinline__ float to_f32(elem e) { return e; }
};

struct BF16 {
  using elem = uint16_t;
  static constexpr int KSTEP = 32;
  static constexpr int KPL = 8;
  static constexpr bool HILO = true;
  using frag = bf16x8_t;
  __device__ static __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static __forceinline__ float to_f32(elem e) { return bf16_bits_to_f32(e); }
};

// A lane's MFMA operand data for one 16-row tile is a contiguous run of SEG = R/4 elements of
// one row (the k dimension is permuted so that lane group q = lane/16 owns elements
// [q*R/4, (q+1)*R/4) and step kb uses elements kb*KPL .. kb*KPL+KPL-1 of that run; A and B use
// the same permutation, so the contraction is unchanged). The run is held as 16-byte chunks.
template <class T, int R>
struct Seg {
  static constexpr int SEG = R / 4;
  static constexpr int BYTES = SEG * (int)sizeof(typename T::elem);
  static constexpr int NCH = BYTES / 16;
  static constexpr int KS = R / T::KSTEP;  // MFMA steps over the full rank
  static_assert(BYTES % 16 == 0, "lane segment must be a whole number of 16-byte chunks");
};

template <class T>
__device__ __forceinline__ typename T::frag frag_at(const u32x4* ch, int kb);

template <>
__device__ __forceinline__ float frag_at<F32>(const u32x4* ch, int kb) {
  return __uint_as_float(ch[kb >> 2][kb & 3]);
}

template <>
__device__ __forceinline__ bf16x8_t frag_at<BF16>(const u32x4* ch, int kb) {
  return __builtin_bit_cast(bf16x8_t, ch[kb]);
}

// Natural k layout for 16x16 MFMA operands read in 16-byte chunks: the contraction is cut into
// windows of 4 chunks; lane group q = lane/16 holds chunk q of every window, so one load
// instruction of a wave covers 64 contiguous bytes of each of its 16 rows. A window spans KW
// MFMA steps (bf16: 1 step of k=32; fp32: 4 steps of k=4, one chunk element per step).
template <class T>
struct Win {
  static constexpr int EPC = 16 / (int)sizeof(typename T::elem);  // elements per chunk
  static constexpr int WLEN = 4 * EPC;                             // elements per window
  static constexpr int KW = WLEN / T::KSTEP;                       // MFMA steps per window
};

template <class T>
__device__ __forceinline__ typename T::frag chunk_frag(const u32x4& ch, int s);

template <>
__device__ __forceinline__ float chunk_frag<F32>(const u32x4& ch, int s) {
  return __uint_as_float(ch[s]);
}

template <>
__device__ __forceinline__ bf16x8_t chunk_frag<BF16>(const u32x4& ch, int) {
  return __builtin_bit_cast(bf16x8_t, ch);
}

// Order-preserving uint32 key of a float: larger float -> larger key; -0.0 and +0.0 map to the
// same key. Inputs are finite.
__device__ __forceinline__ uint32_t float_key(float x) {
  uint32_t u = __float_as_uint(x == 0.0f ? 0.0f : x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// DPP lane moves (no LDS traffic). CTRL: quad_perm 0xB1 swaps neighbouring lanes, 0x4E swaps
// lane pairs in a quad, 0x141 mirrors each half row, 0x140 mirrors each row of 16 lanes,
// 0x110 + n shifts a row right by n lanes (lanes shifted in from outside the row read 0).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float lane_f32(float v, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}

// Workgroup barrier for LDS traffic only: waits for this wave's LDS operations, not for its
// global loads (which stay in flight), then synchronises the waves. __syncthreads() also
// waits for every outstanding global load.
__device__ __forceinline__ void lds_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0); vmcnt and expcnt at their maxima
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// v[l] + v[l ^ 32] in every lane l, as (lower half + upper half) in both halves, by one
// cross-half lane swap (no LDS traffic).
__device__ __forceinline__ float xor32_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Transposing pair sums (no LDS traffic). xor32_pair_sum(a, b): lanes 0-31 hold a[l] + a[l ^ 32],
// lanes 32-63 hold b[l] + b[l ^ 32]. xor16_pair_sum(a, b): lane rows (16 lanes) 0 and 2 hold
// a[l] + a[l ^ 16], rows 1 and 3 hold b[l] + b[l ^ 16].
__device__ __forceinline__ float xor32_pair_sum(float a, float b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor16_pair_sum(float a, float b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Sum / max over the 16 lanes of a DPP row (lanes sharing lane/16), result in every lane of it.
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f32<0xB1>(v);
  v += dpp_f32<0x4E>(v);
  v += dpp_f32<0x141>(v);
  v += dpp_f32<0x140>(v);
  return v;
}
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_f32<0xB1>(v));
  v = fmaxf(v, dpp_f32<0x4E>(v));
  v = fmaxf(v, dpp_f32<0x141>(v));
  v = fmaxf(v, dpp_f32<0x140>(v));
  return v;
}

// Sum / max over the 64 lanes of a wave: row reductions, then the four row results (uniform).
__device__ __forceinline__ float wave_sum(float v) {
  v = row16_sum(v);
  return (lane_f32(v, 0) + lane_f32(v, 16)) + (lane_f32(v, 32) + lane_f32(v, 48));
}

__device__ __forceinline__ float wave_max(float v) {
  v = row16_max(v);
  return fmaxf(fmaxf(lane_f32(v, 0), lane_f32(v, 16)), fmaxf(lane_f32(v, 32), lane_f32(v, 48)));
}

// Inclusive prefix sum over the 64 lanes of a wave: a shift-and-add scan inside each row of 16
// lanes, then the totals of the rows below are added.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v, int lane) {
  v += dpp_u32<0x111>(v);
  v += dpp_u32<0x112>(v);
  v += dpp_u32<0x114>(v);
  v += dpp_u32<0x118>(v);
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 15);
  const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 31);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 47);
  v += (lane >= 16 ? r0 : 0u) + (lane >= 32 ? r1 : 0u) + (lane >= 48 ? r2 : 0u);
  return v;
}

__host__ __device__ constexpr int ceil_div(int a, int b) { return (a + b - 1) / b; }

// The dispatcher deals the workgroups of a launch to the 8 XCDs in turn (workgroup L runs on XCD
// L % 8), and every XCD has its own L2. xcd_remap turns the hardware index L into a logical
// index such that each XCD receives one contiguous range of logical indices: workgroups that are
// neighbours in logical order (and read the same rows) then share an L2. It is a bijection on
// [0, N) for any N, so correctness never depends on the hardware's actual placement.
constexpr int kXCDs = 8;
__device__ __forceinline__ int xcd_remap(int L, int N) {
  const int xcd = L % kXCDs, slot = L / kXCDs;
  const int q = N / kXCDs, rmd = N % kXCDs;
  return xcd < rmd ? xcd * (q + 1) + slot : rmd * (q + 1) + (xcd - rmd) * q + slot;
}

// Element-wise copy with up to U loads in flight per thread: all U loads of a batch are issued
// before any of them is consumed. A plain loop of (load, store) waits out the full memory
// latency once per element, which dominates short kernels.
template <int U, class LoadF, class StoreF>
__device__ __forceinline__ void batched_copy(int n, int tid, int nthreads, LoadF load, StoreF store) {
  for (int base = tid; base < n; base += U * nthreads) {
    decltype(load(0)) v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = base + u * nthreads;
      if (i < n) v[u] = load(i);
    }
    __builtin_amdgcn_sched_barrier(0);  // all loads of the batch before the first store
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = base + u * nthreads;
      if (i < n) store(i, v[u]);
    }
  }
}



}  // namespace sals
