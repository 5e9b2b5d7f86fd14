// Exact per-row top-k with the recent window appended (SALS 关键设计 items 2 and 4; the top-k
// index set S_{psi,k} of the VL-Cache responses, reviewer XVzL weakness 2).
//
// One workgroup of 1024 threads per row. Scores become order-preserving uint32 keys (signed
// zeros equal); the k-th largest key tau is found, and the selection is every key > tau plus
// the first take_eq keys == tau, in index order.
//
// Rows up to 32768 candidates (topk_rows) keep KPT = 4..32 keys per thread in registers, so that
// every pass over the keys is VALU work on registers and each phase ends in one barrier:
//   1. coalesced 16-byte loads (values kept in registers, keys staged in LDS in a padded layout)
//      and the row's key range;
//   2. a 2048-bin histogram of equal-width value bins over that range (a monotone map, so bins
//      are ordered like the keys) gives the bin b1 holding the k-th largest. Scores fill a few
//      float exponents, so bins of the key bits would crowd them into a handful of bins; value
//      bins spread them;
//   3. b1 usually holds a few keys: they are gathered and tau is the one whose counts of larger
//      and equal keys in b1 bracket the rank left over. A crowded b1 (heavy ties, or a range
//      stretched by outliers) falls back to three key-bit digits;
//   4. ordered compaction: thread t owns the KPT consecutive keys from t * KPT (read back from
//      LDS), its output slots follow from a block prefix sum of its counts, and the positions
//      are scattered to LDS and written out with coalesced stores.
// Longer rows are split into slices whose candidates are merged by the same routine
// (topk_slices), or, when that does not fit, go through topk_global: key-bit digits with the row
// read from global memory, listing every position in the threshold bin or above and filtering
// that list.
// With one row per CU a row is bound by that CU's load bandwidth, its VALU issue rate and barrier
// latency, not by HBM.
#include <string.h>

#include <type_traits>

#include "../common.h"
#include "../launch.h"

namespace sals {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kShortThreads = 256;              // workgroup of the short-row kernel
constexpr int kShortRow = 16 * kShortThreads;   // longest short row (16 keys per thread)
constexpr int kMaxSlices = 64;                  // slices of a long row
constexpr int kLdsKeys = 32768;
constexpr int kBins = 2048;
constexpr int kIPT = 16;     // keys per lane per chunk when a wave ranks a run (16 slices of 64)
constexpr int kSmall = 512;  // the largest threshold bin resolved by counting
constexpr int kList = 16384; // short-list capacity of topk_global (positions)

// Finds, in hist[0 .. kBins), the bin b holding the `remaining`-th largest item (bins ordered by
// value, highest bin = largest): bcast[0] = b, bcast[1] = items in bins above b, bcast[2] =
// items in b. Uses all NT threads (kBins / NT consecutive bins each); hist is no longer read once
// it returns.
template <int NT>
__device__ __forceinline__ void find_bin(const uint32_t* hist, uint32_t remaining, uint32_t* scan,
                                         uint32_t* bcast) {
  constexpr int NW = NT / 64, BPT = kBins / NT;
  static_assert(BPT * NT == kBins && NW % 4 == 0, "bins per thread");
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int b0 = BPT * tid;  // each thread owns bins [b0, b0 + BPT)
  uint32_t c[BPT];
  uint32_t tot = 0;
#pragma unroll
  for (int j = 0; j < BPT; ++j) {
    c[j] = hist[b0 + j];
    tot += c[j];
  }
  // suffix sum over the bins: within the wave (total minus the exclusive prefix), then the
  // waves above
  const uint32_t incl = wave_incl_scan(tot, lane);
  const uint32_t wtot = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
  const uint32_t v = wtot - incl + tot;
  if (lane == 0) scan[wave] = v;
  __syncthreads();
  // the totals of all waves in 16-byte reads, then the ones above this wave (no chain of
  // dependent LDS reads)
  uint32_t sv[NW];
#pragma unroll
  for (int q = 0; q < NW / 4; ++q) {
    const uint4 t = ((const uint4*)scan)[q];
    sv[4 * q] = t.x;
    sv[4 * q + 1] = t.y;
    sv[4 * q + 2] = t.z;
    sv[4 * q + 3] = t.w;
  }
  uint32_t above_waves = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) above_waves += w > wave ? sv[w] : 0u;
  const uint32_t suf = v + above_waves;  // items in this thread's bins and all higher bins
  const uint32_t above = suf - tot;
  if (above < remaining && remaining <= suf) {
    // this thread's bins from the highest down
    uint32_t acc = above;
    bool done = false;
#pragma unroll
    for (int j = BPT - 1; j >= 0; --j) {
      if (!done && acc + c[j] >= remaining) {
        bcast[0] = (uint32_t)(b0 + j);
        bcast[1] = acc;
        bcast[2] = c[j];
        done = true;
      }
      acc += c[j];
    }
  }
  __syncthreads();
}

// The float value of an order-preserving key (inverse of float_key).
__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// Exclusive prefix of a per-wave count over the NT / 64 waves of the workgroup, and the block total.
template <int NT>
__device__ __forceinline__ void block_prefix(uint32_t mine, uint32_t* scan, uint32_t& before, uint32_t& total) {
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (lane == 0) scan[wave] = mine;
  __syncthreads();
  before = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const uint32_t v = scan[w];
    before += (w < wave) ? v : 0u;
    total += v;
  }
  __syncthreads();
}

// The part of a selection that needs no ranking: the window out[kp + j] = wstart + j (j < wcount)
// and, in threshold mode (thr), the cap of kp by the number of keys >= tkey (counted over
// key(i), i < Tc), the padding out[kp + wcount .. pad_to) = -1 and *cnt_out = kp + wcount.
// Returns the number of keys left to select by rank, or 0 when the selection is complete
// (kp <= 0, or every key selected: out[j] = map(j)). The same value in every thread.
// For candidate keys the threshold count runs over the candidates: a row with fewer than kp
// passing keys has all of them among the candidates, otherwise at least kp pass there too, so
// min(kp, count) is the row's.
template <class KeyF, class MapF>
__device__ __forceinline__ int topk_prologue(KeyF key, MapF map, int Tc, int kp, int32_t* __restrict__ out,
                                             int wcount, int wstart, bool thr, uint32_t tkey,
                                             int32_t* __restrict__ cnt_out, int pad_to, uint32_t* scan) {
  const int tid = threadIdx.x, lane = tid & 63;
  if (thr) {
    if (kp > 0) {
      uint32_t mine = 0;
      for (int i = tid; i < Tc; i += kThreads) mine += key(i) >= tkey ? 1u : 0u;
      uint32_t before, total;
      block_prefix<kThreads>((uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan(mine, lane), 63), scan, before, total);
      kp = (int)min((uint32_t)kp, total);
    }
    for (int j = kp + wcount + tid; j < pad_to; j += kThreads) out[j] = -1;
    if (tid == 0 && cnt_out) *cnt_out = kp + wcount;
  }
  for (int j = tid; j < wcount; j += kThreads) out[kp + j] = wstart + j;
  if (kp <= 0) return 0;
  if (kp >= Tc) {
    for (int j = tid; j < Tc; j += kThreads) out[j] = map(j);
    return 0;
  }
  return kp;
}

// LDS word of key i in the staging layout: 4 pad words after every 32 keys, so that a thread
// reading its 32 consecutive keys as 16-byte pieces and a wave writing consecutive 16-byte pieces
// both spread over the banks.
__device__ __forceinline__ int padded(int i) { return i + ((i >> 5) << 2); }

// The selection of one workgroup over at most kThreads * KPT keys (thread t owns the KPT
// consecutive keys from t * KPT and holds them in registers): the kp largest of n keys, ties to
// the lowest position, written to out[0 .. kp) in ascending position order as map(position)
// (and, with okeys, for rows of scores only, their keys to okeys[0 .. kp)), followed by the
// window out[kp + j] = wstart + j, j < wcount. Keys are float_key(src[i]) with map(i) = obase + i, or (GATHER) the
// given keys ckeys[i] with map(i) = cand[i]. Threshold mode (thr): only keys >= tkey may be
// selected, so kp becomes min(kp, #keys >= tkey); out[kp + wcount .. pad_to) is filled with -1
// and *cnt_out receives kp + wcount. For GATHER the count runs over the candidates: a row with
// fewer than kp passing keys has all of them among the candidates, otherwise at least kp pass
// there too, so min(kp, count) is the row's. With tcheck (GATHER, tcheck[0 .. ntcheck) the
// threshold keys of the slices the candidates came from) the selection is exact only if its
// threshold key exceeds their maximum T; otherwise topk_rows writes no selection and returns false
// (the same in every thread). It returns true when the selection is written.
template <int NT, int KPT, bool GATHER>
__device__ __forceinline__ bool topk_rows(const float* __restrict__ src, const int32_t* __restrict__ cand,
                                          const uint32_t* __restrict__ ckeys, int n, int kp,
                                          int32_t* __restrict__ out, uint32_t* __restrict__ okeys,
                                          int obase, int wcount, int wstart, bool vec, bool thr,
                                          uint32_t tkey, int32_t* __restrict__ cnt_out, int pad_to,
                                          uint32_t* __restrict__ tau_out = nullptr,
                                          const uint32_t* __restrict__ tcheck = nullptr, int ntcheck = 0) {
  static_assert(KPT % 4 == 0 && KPT <= 32 && NT * KPT <= kLdsKeys, "keys per thread");
  constexpr int NW = NT / 64;
  constexpr int kStage = NT * KPT / 32 * 36;  // staging words for NT * KPT keys
  // staged keys (padded layout); after the ranking, the selection's positions in output order
  __shared__ __attribute__((aligned(16))) uint32_t stage[kStage];
  __shared__ __attribute__((aligned(16))) uint32_t hist[kBins];
  __shared__ __attribute__((aligned(16))) uint32_t scan[NW];
  __shared__ uint32_t bcast[4];
  __shared__ uint32_t mm[4 * NW];  // per-wave key minima, maxima, threshold counts, tcheck maxima
  __shared__ uint32_t nsmall, tsel[2];  // small-bin gather count; (tau, take_eq)
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int Tc = n;
  for (int i = tid; i < kBins; i += NT) hist[i] = 0;
  if (tid == 0) nsmall = 0;

  // ---- 1. coalesced loads: this thread's 16-byte pieces u = tid + NT * q hold positions
  //      4u .. 4u + 3. They are kept in registers (values for the histogram) and staged in LDS as
  //      keys; the row's range (and, in threshold mode, the count of keys >= tkey) follows ----
  using Reg = std::conditional_t<GATHER, uint32_t, float>;  // candidate keys, or scores
  Reg pr[KPT];
  uint32_t lmn = 0xffffffffu, lmx = 0u, npass = 0u;
  // 16-byte loads stay inside the row rounded up to 4 elements (score rows are padded to 16
  // bytes; candidate rows qualify only when their length is a multiple of 4); other rows load
  // element by element at clamped positions. Every load is unconditional so that all are in
  // flight together.
  const bool v4 = GATHER ? (((uintptr_t)ckeys & 15) == 0 && (Tc & 3) == 0) : vec;
  uint32_t tmx = 0u;  // threads below ntcheck: that slice's threshold key
  if (GATHER && tcheck) tmx = tcheck[min(tid, ntcheck - 1)];
  // (two separate loops: merged, the compiler would split the 16-byte loads into single words)
  if (Tc > 0 && v4) {
    const int last4 = ((Tc + 3) & ~3) - 4;
    if constexpr (GATHER) {
      uint4 w[KPT / 4];
#pragma unroll
      for (int q = 0; q < KPT / 4; ++q) w[q] = *(const uint4*)(ckeys + min(4 * (tid + NT * q), last4));
#pragma unroll
      for (int q = 0; q < KPT / 4; ++q) pr[4 * q] = w[q].x, pr[4 * q + 1] = w[q].y, pr[4 * q + 2] = w[q].z, pr[4 * q + 3] = w[q].w;
    } else {
      float4 w[KPT / 4];
#pragma unroll
      for (int q = 0; q < KPT / 4; ++q) w[q] = *(const float4*)(src + min(4 * (tid + NT * q), last4));
#pragma unroll
      for (int q = 0; q < KPT / 4; ++q) pr[4 * q] = w[q].x, pr[4 * q + 1] = w[q].y, pr[4 * q + 2] = w[q].z, pr[4 * q + 3] = w[q].w;
    }
  } else if (Tc > 0) {
#pragma unroll
    for (int q = 0; q < KPT / 4; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = min(4 * (tid + NT * q) + e, Tc - 1);
        if constexpr (GATHER) pr[4 * q + e] = ckeys[i];
        else pr[4 * q + e] = src[i];
      }
  }
  // GATHER: the positions of this thread's KPT consecutive candidates (from t * KPT, the keys its
  // compaction walks), loaded with the keys so that the output needs no dependent gather
  int32_t cp[GATHER ? KPT : 1];
  if constexpr (GATHER) {
    const int c0 = tid * KPT;
    if (Tc > 0 && v4 && ((uintptr_t)cand & 15) == 0) {
      const int last4 = ((Tc + 3) & ~3) - 4;
#pragma unroll
      for (int q = 0; q < KPT / 4; ++q) {
        const int4 w = *(const int4*)(cand + min(c0 + 4 * q, last4));
        cp[4 * q] = w.x, cp[4 * q + 1] = w.y, cp[4 * q + 2] = w.z, cp[4 * q + 3] = w.w;
      }
    } else if (Tc > 0) {
#pragma unroll
      for (int e = 0; e < KPT; ++e) cp[e] = cand[min(c0 + e, Tc - 1)];
    }
  }
  auto key_of = [&](int e) -> uint32_t {
    if constexpr (GATHER) return pr[e];
    else return float_key(pr[e]);
  };
#pragma unroll
  for (int q = 0; q < KPT / 4; ++q) {
    const int i = 4 * (tid + NT * q);
    uint32_t v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[e] = key_of(4 * q + e);
      const bool in = i + e < Tc;
      lmn = min(lmn, in ? v[e] : 0xffffffffu);
      lmx = max(lmx, in ? v[e] : 0u);
      if (thr) npass += (in && v[e] >= tkey) ? 1u : 0u;
    }
    if (i < Tc) *(uint4*)&stage[padded(i)] = make_uint4(v[0], v[1], v[2], v[3]);
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    lmn = min(lmn, (uint32_t)__shfl_xor((int)lmn, o));
    lmx = max(lmx, (uint32_t)__shfl_xor((int)lmx, o));
    if (GATHER && tcheck) tmx = max(tmx, (uint32_t)__shfl_xor((int)tmx, o));
  }
  if (thr) npass = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan(npass, lane), 63);
  if (lane == 0) {
    mm[wave] = lmn;
    mm[NW + wave] = lmx;
    mm[2 * NW + wave] = npass;
    if constexpr (GATHER) mm[3 * NW + wave] = tmx;
  }
  // (LDS only: also orders the histogram zeroing before the atomics below; GATHER's position loads
  // stay in flight)
  lds_barrier();
  uint32_t total_pass = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    lmn = min(lmn, mm[w]);
    lmx = max(lmx, mm[NW + w]);
    total_pass += mm[2 * NW + w];
    if constexpr (GATHER) tmx = max(tmx, mm[3 * NW + w]);
  }

  // ---- the parts that need no ranking ----
  if (thr) {
    if (kp > 0) kp = (int)min((uint32_t)kp, total_pass);
    for (int j = kp + wcount + tid; j < pad_to; j += NT) out[j] = -1;
    if (tid == 0 && cnt_out) *cnt_out = kp + wcount;
  }
  for (int j = tid; j < wcount; j += NT) out[kp + j] = wstart + j;
  auto map = [&](int i) -> int32_t {
    if constexpr (GATHER) return cand[i];
    else return obase + i;
  };
  // tau_out: the selection's threshold key (0, the smallest key, when every key is selected)
  if (kp <= 0 || kp >= Tc) {
    if (tau_out && tid == 0) *tau_out = 0u;
  }
  if (kp <= 0) return true;
  if (kp >= Tc) {
    for (int j = tid; j < Tc; j += NT) {
      out[j] = map(j);
      if (okeys) okeys[j] = stage[padded(j)];
    }
    return true;
  }

  // ---- 2. histogram of equal-width value bins over the range ----
  // bin(k) = clamp(floor(value(k) * s + o), 0, kBins - 1) with s = kBins / (max - min) and
  // o = -min * s: one fused multiply-add is monotone in the value, so a larger key never lands
  // in a lower bin, and equal keys share a bin. A range that is empty or not finite
  // (infinities, NaN) puts every key in bin 0. Positions past the row get bin kBins and are not
  // counted (all of them on one counter would serialise the atomics of whole waves).
  const float vmin = key_value(lmn), vmax = key_value(lmx);
  const float span = __fsub_rn(vmax, vmin);
  float scale = __fdiv_rn((float)kBins, span);
  if (!(span > 0.f) || !isfinite(span) || !isfinite(scale)) scale = 0.f;
  const float off = scale == 0.f ? 0.f : -__fmul_rn(vmin, scale);
  uint32_t kb[KPT];
#pragma unroll
  for (int q = 0; q < KPT / 4; ++q) {
    const int i = 4 * (tid + NT * q);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float x;
      if constexpr (GATHER) x = key_value(pr[4 * q + e]);
      else x = pr[4 * q + e];
      const float t = fminf(fmaxf(__fmaf_rn(x, scale, off), 0.f), (float)(kBins - 1));
      kb[4 * q + e] = i + e < Tc ? (uint32_t)t : (uint32_t)kBins;
      if (i + e < Tc) atomicAdd(&hist[kb[4 * q + e]], 1u);
    }
  }
  __syncthreads();
  find_bin<NT>(hist, (uint32_t)kp, scan, bcast);
  const uint32_t bin1 = bcast[0];
  const uint32_t c1 = bcast[2];                  // keys in bin1
  uint32_t remaining = (uint32_t)kp - bcast[1];  // rank of tau inside bin1, >= 1
  // (bcast is next written inside a find_bin, after barriers every thread passes after these
  // reads; hist is free once find_bin returns)

  uint32_t tau, take_eq;
  if (c1 <= (uint32_t)kSmall) {
    // ---- 3. gather bin1's keys (in any order) into hist, one counter update per wave; tau is
    //      the one whose counts of larger and equal keys in bin1 bracket the rank left over ----
    uint32_t* small = hist;
    uint32_t hm = 0;  // register slots of this thread's keys in bin1 (slot 4q + e: position 4u + e)
#pragma unroll
    for (int e = 0; e < KPT; ++e) hm |= (kb[e] == bin1 ? 1u : 0u) << e;
    const uint32_t cnt = (uint32_t)__popc(hm);
    const uint32_t incl = wave_incl_scan(cnt, lane);
    const uint32_t wtot = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
    if (wtot) {
      uint32_t got = 0;
      if (lane == 63) got = atomicAdd(&nsmall, wtot);
      uint32_t at = (uint32_t)__builtin_amdgcn_readlane((int)got, 63) + incl - cnt;
      while (hm) {  // the keys are read back from the staging array by position
        const int e = __builtin_ctz(hm);
        hm &= hm - 1u;
        small[at++] = stage[padded(4 * (tid + NT * (e >> 2)) + (e & 3))];
      }
    }
    __syncthreads();
    if (tid < (int)c1) {
      const uint32_t x = small[tid];
      uint32_t gt = 0, ge = 0;
      for (int j = 0; j < (int)c1; j += 16) {  // j + 15 < kSmall + 16 <= kBins
        uint4 v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = *(const uint4*)&small[j + 4 * q];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t vv[4] = {v[q].x, v[q].y, v[q].z, v[q].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const bool in = j + 4 * q + e < (int)c1;
            gt += (in && vv[e] > x) ? 1u : 0u;
            ge += (in && vv[e] >= x) ? 1u : 0u;
          }
        }
      }
      if (gt < remaining && remaining <= ge) {  // every holder of tau writes the same values
        tsel[0] = x;
        tsel[1] = remaining - gt;
      }
    }
    __syncthreads();
    tau = tsel[0];
    take_eq = tsel[1];
  } else {
    // ---- 3'. crowded bin (heavy ties, or a range stretched by outliers): three key-bit digits ----
    uint32_t prefix = 0;
    remaining = (uint32_t)kp;
#pragma unroll 1
    for (int pass = 0; pass < 3; ++pass) {
      const int shift = pass == 0 ? 21 : pass == 1 ? 10 : 0;
      const uint32_t dmask = pass == 2 ? 0x3ffu : 0x7ffu;
      const uint32_t pmask = pass == 0 ? 0u : pass == 1 ? 0xffe00000u : 0xfffffc00u;
      for (int i = tid; i < kBins; i += NT) hist[i] = 0;
      __syncthreads();
#pragma unroll
      for (int e = 0; e < KPT; ++e) {
        const uint32_t x = key_of(e);
        if (kb[e] < (uint32_t)kBins && (x & pmask) == prefix) atomicAdd(&hist[(x >> shift) & dmask], 1u);
      }
      __syncthreads();
      find_bin<NT>(hist, remaining, scan, bcast);
      prefix |= bcast[0] << shift;
      remaining -= bcast[1];
      __syncthreads();
    }
    tau = prefix;
    take_eq = remaining;  // >= 1
  }

  if (tau_out && tid == 0) *tau_out = tau;
  if (GATHER && tcheck && tau <= tmx) return false;  // tau and tmx are the same in every thread

  // ---- 4. ordered compaction over this thread's KPT consecutive keys (from t * KPT): its output
  //      slots start at the number of selected keys before its first key (a block prefix sum of
  //      its counts); the positions go to LDS in output order (over the staged keys, read for the
  //      last time before the barriers of that prefix sum) and are written out with coalesced
  //      stores ----
  const int b0 = tid * KPT;
  const int nv = min(max(Tc - b0, 0), KPT);  // valid keys of this thread
  const uint32_t vmask = nv >= 32 ? 0xffffffffu : ((1u << nv) - 1u);
  uint32_t fgt = 0, feq = 0;
#pragma unroll
  for (int c = 0; c < KPT / 4; ++c) {
    const uint4 w = *(const uint4*)&stage[padded(b0 + 4 * c)];  // stays inside the staging array
    const uint32_t kc[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      fgt |= (kc[e] > tau ? 1u : 0u) << (4 * c + e);
      feq |= (kc[e] == tau ? 1u : 0u) << (4 * c + e);
    }
  }
  fgt &= vmask;
  feq &= vmask;
  const uint32_t packed = (uint32_t)__popc(fgt) | ((uint32_t)__popc(feq) << 16);  // each <= 32768
  const uint32_t incl = wave_incl_scan(packed, lane);
  uint32_t before, total;
  block_prefix<NT>((uint32_t)__builtin_amdgcn_readlane((int)incl, 63), scan, before, total);
  const uint32_t excl = before + incl - packed;
  uint32_t ngt = excl & 0xffffu, neq = excl >> 16;
  int32_t* obuf = (int32_t*)stage;  // GATHER: the candidates' positions; else indices into the row
  if constexpr (GATHER) {
#pragma unroll
    for (int e = 0; e < KPT; ++e) {  // static register indices
      if ((fgt >> e) & 1u) {
        obuf[ngt + min(neq, take_eq)] = cp[e];
        ++ngt;
      } else if ((feq >> e) & 1u) {
        if (neq < take_eq) obuf[ngt + neq] = cp[e];
        ++neq;
      }
    }
  } else {
    uint32_t m = fgt | feq;
    while (m) {
      const int e = __builtin_ctz(m);
      m &= m - 1u;
      if ((fgt >> e) & 1u) {
        obuf[ngt + min(neq, take_eq)] = b0 + e;
        ++ngt;
      } else {
        if (neq < take_eq) obuf[ngt + neq] = b0 + e;
        ++neq;
      }
    }
  }
  __syncthreads();
  batched_copy<4>(kp, tid, NT, [&](int j) { return obuf[j]; }, [&](int j, int32_t i) {
    if constexpr (GATHER) {
      out[j] = i;
    } else {
      out[j] = obase + i;
      if (okeys) okeys[j] = float_key(src[i]);
    }
  });
  return true;
}

// The selection of a row read from global memory (rows beyond the LDS staging array that are not
// split into slices): keys float_key(src[i]), positions i, otherwise as topk_staged. Key bits
// [31:21] give the threshold bin b1; every position in b1 or above is listed in index order
// (ballot ranks), key bits [20:10] and [9:0] of tau come from histograms over the list, and the
// list filtered is the selection. A list that would not fit resolves the digits over the row.
__device__ __forceinline__ void topk_global(const float* __restrict__ src, int n, int kp, int32_t* __restrict__ out,
                                            int wcount, int wstart, bool thr, uint32_t tkey,
                                            int32_t* __restrict__ cnt_out, int pad_to) {
  __shared__ __attribute__((aligned(16))) uint32_t hist[kBins];
  __shared__ int32_t list[kList];
  __shared__ __attribute__((aligned(16))) uint32_t scan[kWaves];
  __shared__ uint32_t bcast[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int Tc = n;
  auto key_at = [&](int i) -> uint32_t { return float_key(src[i]); };
  kp = topk_prologue(key_at, [](int i) -> int32_t { return i; }, Tc, kp, out, wcount, wstart, thr, tkey, cnt_out,
                     pad_to, scan);
  if (kp == 0) return;
  // Keys of this wave for the chunk starting at `base`: wave w owns [base + w*1024, +1024), in
  // 16 slices of 64 (lane l reads the l-th key of each slice). Reads are unconditional (indices
  // clamp) so that all 16 are in flight before the first use.
  constexpr int kChunk = kThreads * kIPT;
  uint32_t kk[kIPT];
  auto load_keys = [&](int base) {
    const int w0 = base + wave * 64 * kIPT;
#pragma unroll
    for (int j = 0; j < kIPT; ++j) kk[j] = key_at(min(w0 + j * 64 + lane, Tc - 1));
  };
  const unsigned long long lt_mask = (1ull << lane) - 1ull;

  // ---- 1. the digit-1 histogram (key bits [31:21]) ----
  for (int i = tid; i < kBins; i += kThreads) hist[i] = 0;
  __syncthreads();
  batched_copy<16>(Tc, tid, kThreads, [&](int i) { return src[i]; },
                   [&](int, float v) { atomicAdd(&hist[float_key(v) >> 21], 1u); });
  __syncthreads();
  find_bin<kThreads>(hist, (uint32_t)kp, scan, bcast);
  const uint32_t bin1 = bcast[0];
  const uint32_t above = bcast[1];            // keys in bins above bin1
  const uint32_t nl = above + bcast[2];       // keys in bin1 or above
  uint32_t remaining = (uint32_t)kp - above;  // rank of tau inside bin1, >= 1

  uint32_t tau, take_eq;
  if (nl <= (uint32_t)kList) {
    // ---- 2. list every position whose key is in bin1 or above, in index order ----
    for (int i = tid; i < kBins; i += kThreads) hist[i] = 0;
    const uint32_t lo = bin1 << 21;
    uint32_t run = 0;
    for (int base = 0; base < Tc; base += kChunk) {
      load_keys(base);
      const int w0 = base + wave * 64 * kIPT;
      uint32_t cnt = 0;
#pragma unroll
      for (int j = 0; j < kIPT; ++j) cnt += (uint32_t)__popcll(__ballot(w0 + j * 64 + lane < Tc && kk[j] >= lo));
      uint32_t before, total;
      block_prefix<kThreads>(cnt, scan, before, total);
      uint32_t at = run + before;
      // the same tests as the count pass, recomputed: keeping its 16 ballots live across the
      // barrier would spill scalar registers (the empty asm hides the equality from the
      // compiler)
      uint32_t lo_w = lo;
      int tc_w = Tc;
      asm volatile("" : "+v"(lo_w), "+v"(tc_w));
#pragma unroll
      for (int j = 0; j < kIPT; ++j) {
        const int i = w0 + j * 64 + lane;
        const bool hit = i < tc_w && kk[j] >= lo_w;
        const unsigned long long m = __ballot(hit);
        if (hit) list[at + (uint32_t)__popcll(m & lt_mask)] = i;
        at += (uint32_t)__popcll(m);
      }
      run += total;
    }
    __syncthreads();
    // ---- key bits [20:10] over the listed keys of bin1, then [9:0] over those that match ----
    for (int u = tid; u < (int)nl; u += kThreads) {
      const uint32_t k = key_at(list[u]);
      if ((k >> 21) == bin1) atomicAdd(&hist[(k >> 10) & 0x7ffu], 1u);
    }
    __syncthreads();
    find_bin<kThreads>(hist, remaining, scan, bcast);
    uint32_t prefix = lo | (bcast[0] << 10);
    remaining -= bcast[1];
    for (int i = tid; i < kBins; i += kThreads) hist[i] = 0;
    __syncthreads();
    {
      constexpr int LU = kList / kThreads;
      int li[LU];
#pragma unroll
      for (int u = 0; u < LU; ++u) li[u] = list[min(tid + u * kThreads, (int)nl - 1)];
      uint32_t lk[LU];
#pragma unroll
      for (int u = 0; u < LU; ++u) lk[u] = key_at(li[u]);
#pragma unroll
      for (int u = 0; u < LU; ++u)
        if (tid + u * kThreads < (int)nl && (lk[u] & 0xfffffc00u) == prefix) atomicAdd(&hist[lk[u] & 0x3ffu], 1u);
    }
    __syncthreads();
    find_bin<kThreads>(hist, remaining, scan, bcast);
    tau = prefix | bcast[0];
    take_eq = remaining - bcast[1];
    // ---- 3. the selection is the list filtered, in list (index) order ----
    constexpr int FPT = kList / kThreads;  // list entries per thread: one pass
    uint32_t run_gt = 0, run_eq = 0;
    for (int base = 0; base < (int)nl; base += kThreads * FPT) {
      const int j0 = base + tid * FPT;
      uint32_t fgt = 0, feq = 0;
      int idx[FPT];
#pragma unroll
      for (int e = 0; e < FPT; ++e) idx[e] = list[min(j0 + e, (int)nl - 1)];
#pragma unroll
      for (int e = 0; e < FPT; ++e) {
        const uint32_t k = key_at(idx[e]);
        const bool valid = j0 + e < (int)nl;
        fgt |= (uint32_t)(valid && k > tau) << e;
        feq |= (uint32_t)(valid && k == tau) << e;
      }
      const uint32_t packed = (uint32_t)__popc(fgt) | ((uint32_t)__popc(feq) << 16);
      const uint32_t incl = wave_incl_scan(packed, lane);
      uint32_t before, total;
      block_prefix<kThreads>((uint32_t)__builtin_amdgcn_readlane((int)incl, 63), scan, before, total);
      const uint32_t excl = before + incl - packed;
      uint32_t ngt = run_gt + (excl & 0xffffu), neq = run_eq + (excl >> 16);
#pragma unroll
      for (int e = 0; e < FPT; ++e) {
        if ((fgt >> e) & 1u) {
          out[ngt + min(neq, take_eq)] = idx[e];
          ++ngt;
        } else if ((feq >> e) & 1u) {
          if (neq < take_eq) out[ngt + neq] = idx[e];
          ++neq;
        }
      }
      run_gt += total & 0xffffu;
      run_eq += total >> 16;
    }
    return;
  }

  // ---- fallback: resolve the remaining digits over the whole row ----
  uint32_t prefix = bin1 << 21;
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
    find_bin<kThreads>(hist, remaining, scan, bcast);
    prefix |= bcast[0] << shift;
    remaining -= bcast[1];
    __syncthreads();
  }
  tau = prefix;
  take_eq = remaining;  // >= 1
  // ordered compaction over the whole row: ranks inside a wave's run from ballots, the runs'
  // packed (gt, eq) totals (each at most 16384, so 16 bits apiece) exchanged per chunk
  uint32_t run_gt = 0, run_eq = 0;
  for (int base = 0; base < Tc; base += kChunk) {
    load_keys(base);
    const int w0 = base + wave * 64 * kIPT;
    uint32_t wgt = 0, weq = 0;
#pragma unroll
    for (int j = 0; j < kIPT; ++j) {
      const bool valid = w0 + j * 64 + lane < Tc;
      wgt += (uint32_t)__popcll(__ballot(valid && kk[j] > tau));
      weq += (uint32_t)__popcll(__ballot(valid && kk[j] == tau));
    }
    uint32_t before, total;
    block_prefix<kThreads>(wgt | (weq << 16), scan, before, total);
    uint32_t ngt = run_gt + (before & 0xffffu), neq = run_eq + (before >> 16);
#pragma unroll
    for (int j = 0; j < kIPT; ++j) {
      const int i = w0 + j * 64 + lane;
      const bool valid = i < Tc;
      const bool gt = valid && kk[j] > tau, eq = valid && kk[j] == tau;
      const unsigned long long mg = __ballot(gt), me = __ballot(eq);
      const uint32_t bg = ngt + (uint32_t)__popcll(mg & lt_mask);  // gt keys before i
      const uint32_t be = neq + (uint32_t)__popcll(me & lt_mask);  // eq keys before i
      if (gt) out[bg + min(be, take_eq)] = i;
      else if (eq && be < take_eq) out[bg + be] = i;
      ngt += (uint32_t)__popcll(mg);
      neq += (uint32_t)__popcll(me);
    }
    run_gt += total & 0xffffu;
    run_eq += total >> 16;
  }
}

// One row per workgroup of NT threads: rows of up to NT * KPT keys in registers (KPT > 0), longer
// rows from global memory (KPT == 0, NT = kThreads).
template <int NT, int KPT>
__global__ __launch_bounds__(NT) void topk_window_kernel(const float* __restrict__ S,
                                                               int32_t* __restrict__ sel, int Tc,
                                                               int ldS, int kp, int ctx, int n_sel,
                                                               bool vec, bool thr, uint32_t tkey,
                                                               int32_t* __restrict__ cnt) {
  const int row = blockIdx.x;
  if constexpr (KPT > 0)
    topk_rows<NT, KPT, false>(S + (size_t)row * ldS, nullptr, nullptr, Tc, kp, sel + (size_t)row * n_sel, nullptr, 0,
                          ctx - Tc, Tc, vec, thr, tkey, cnt ? cnt + row : nullptr, n_sel);
  else
    topk_global(S + (size_t)row * ldS, Tc, kp, sel + (size_t)row * n_sel, ctx - Tc, Tc, thr, tkey,
                cnt ? cnt + row : nullptr, n_sel);
}

// Rows longer than the register-resident limit: one workgroup per (row, slice of slen keys) keeps
// the m largest of its slice (ties to the lowest position) as candidates, in ascending position
// order, with their keys, and writes its threshold key (the m-th largest) to taus. With m = kp
// every element of the row's top kp is among its slice's top kp, with the lowest-index ties of the
// row's threshold key included, so the row's selection over the candidates (in ascending position
// order across slices) is exact. With m < kp (about 1.5 times a slice's expected share of the row's
// top kp) the merge checks that this still holds.
template <int NT, int KPT>
__global__ __launch_bounds__(NT) void topk_slice_kernel(const float* __restrict__ S,
                                                        int32_t* __restrict__ cand,
                                                        uint32_t* __restrict__ ckeys,
                                                        uint32_t* __restrict__ taus, int Tc, int ldS,
                                                        int m, int slen, int ns, bool vec) {
  const int row = blockIdx.x / ns, s = blockIdx.x % ns;
  const int s0 = s * slen, n = min(slen, Tc - s0);
  const size_t o = ((size_t)row * ns + s) * m;
  topk_rows<NT, KPT, false>(S + (size_t)row * ldS + s0, nullptr, nullptr, n, m, cand + o, ckeys + o, s0, 0, 0, vec,
                            false, 0u, nullptr, 0, taus + (size_t)row * ns + s);
}

// The row's selection over its slices' candidates. With m < kp the candidates may miss part of
// the row's top kp: a key a slice dropped is at most that slice's threshold key, so with T the
// largest slice threshold, a selection whose threshold key exceeds T contains no dropped key and
// misses none. That holds exactly when at least kp candidates exceed T (the kp-th largest
// candidate then exceeds T). Otherwise the row is selected from the scores themselves
// (topk_global): exact either way.
template <int KPT>
__global__ __launch_bounds__(kThreads) void topk_merge_kernel(const int32_t* __restrict__ cand,
                                                              const uint32_t* __restrict__ ckeys,
                                                              const uint32_t* __restrict__ taus,
                                                              int32_t* __restrict__ sel, int Tc, int kp,
                                                              int ns, int m, int ctx, int n_sel, bool thr,
                                                              uint32_t tkey, int32_t* __restrict__ cnt,
                                                              const float* __restrict__ S, int ldS) {
  const int row = blockIdx.x;
  const size_t o = (size_t)row * ns * m;
  // (the reduced plan keeps at most kLdsKeys / 2 candidates: merges of more keys per thread are
  // only used with m = kp, whose selection needs no check, and leave no LDS for the fallback)
  const bool check = KPT <= 16 && m < kp;
  if (!topk_rows<kThreads, KPT, true>(nullptr, cand + o, ckeys + o, ns * m, kp, sel + (size_t)row * n_sel, nullptr, 0,
                                      ctx - Tc, Tc, false, thr, tkey, cnt ? cnt + row : nullptr, n_sel, nullptr,
                                      check ? taus + (size_t)row * ns : nullptr, ns)) {
    if constexpr (KPT <= 16)
      topk_global(S + (size_t)row * ldS, Tc, kp, sel + (size_t)row * n_sel, ctx - Tc, Tc, thr, tkey,
                  cnt ? cnt + row : nullptr, n_sel);
  }
}

// Keys per thread for a register-resident row of n keys (n <= kLdsKeys).
int keys_per_thread(int n) { return n <= 4 * kThreads ? 4 : n <= 8 * kThreads ? 8 : n <= 16 * kThreads ? 16 : 32; }

}  // namespace

// Slices of a row of Tc candidates, rows rows: ns slices of *slen keys, each keeping its top *m
// (0: the row is not split). Rows up to the register-resident limit are not split. Otherwise
// (reduce, i.e. not in threshold mode) the row is cut into about one slice per CU over all rows,
// each keeping 1.5 times its expected share of the top kp (plus 32), when that fits; else into the
// fewest slices that fit, each keeping kp.
int topk_slices(int rows, int Tc, int kp, bool reduce, int* slen, int* m) {
  if (Tc <= kLdsKeys || kp <= 0) return 0;
  auto fits = [&](int ns, int mm, int* len_out) {
    const int len = (ceil_div(Tc, ns) + 3) / 4 * 4;
    const int last = Tc - (ns - 1) * len;
    if (len > kLdsKeys || last <= mm || (long)ns * mm > kLdsKeys) return false;
    *len_out = len;
    return true;
  };
  int len = 0;
  if (reduce) {
    int ns = ceil_div(256, rows > 0 ? rows : 1);
    if (ns < ceil_div(Tc, kLdsKeys)) ns = ceil_div(Tc, kLdsKeys);
    if (ns > kMaxSlices) ns = kMaxSlices;
    const int mm = (3 * ceil_div(kp, ns) / 2 + 32 + 31) / 32 * 32;
    if (mm < kp && (long)ns * mm <= kLdsKeys / 2 && fits(ns, mm, &len)) {
      if (slen) *slen = len;
      if (m) *m = mm;
      return ns;
    }
  }
  const int ns = ceil_div(Tc, kLdsKeys);
  if (!fits(ns, kp, &len)) return 0;
  if (slen) *slen = len;
  if (m) *m = kp;
  return ns;
}

size_t topk_candidate_bytes(int rows, int Tc, int kp) {
  size_t best = 0;
  for (int reduce = 0; reduce < 2; ++reduce) {
    int m = 0;
    const int ns = topk_slices(rows, Tc, kp, reduce != 0, nullptr, &m);
    // positions, then keys, then the slices' threshold keys
    const size_t b = ns ? (size_t)rows * ns * m * 8 + (size_t)rows * ns * 4 : 0;
    if (b > best) best = b;
  }
  return best;
}

uint32_t threshold_key(float tau) {
  uint32_t u;
  const float z = tau == 0.0f ? 0.0f : tau;  // -0.0 ranks as +0.0
  memcpy(&u, &z, 4);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

hipError_t launch_topk_window(const float* S, int ldS, int32_t* sel, int rows, int Tc, int kp,
                              int ctx, int n_sel, int32_t* cand, hipStream_t st, bool thr, uint32_t tkey,
                              int32_t* cnt) {
  if (rows <= 0) return hipSuccess;
  const bool vec = (ldS & 3) == 0 && ((uintptr_t)S & 15) == 0;
  int slen = 0, m = 0;
  const int ns = cand ? topk_slices(rows, Tc, kp, !thr, &slen, &m) : 0;
#define SALS_KPT_SWITCH(N, CALL) \
  switch (keys_per_thread(N)) {    \
    case 4: CALL(4); break;        \
    case 8: CALL(8); break;        \
    case 16: CALL(16); break;      \
    default: CALL(32); break;      \
  }
  if (Tc <= kShortRow) {
    // short rows: a 256-thread workgroup (up to 16 keys per thread), whose barriers and block
    // scans span 4 waves instead of 16
#define SALS_SHORT(K) \
  topk_window_kernel<kShortThreads, K><<<rows, kShortThreads, 0, st>>>(S, sel, Tc, ldS, kp, ctx, n_sel, vec, thr, tkey, cnt)
    if (Tc <= 4 * kShortThreads) SALS_SHORT(4);
    else if (Tc <= 8 * kShortThreads) SALS_SHORT(8);
    else SALS_SHORT(16);
#undef SALS_SHORT
  } else if (Tc <= kLdsKeys) {
#define SALS_ROWS(K) \
  topk_window_kernel<kThreads, K><<<rows, kThreads, 0, st>>>(S, sel, Tc, ldS, kp, ctx, n_sel, vec, thr, tkey, cnt)
    SALS_KPT_SWITCH(Tc, SALS_ROWS)
#undef SALS_ROWS
  } else if (ns > 0) {
    uint32_t* ckeys = (uint32_t*)(cand + (size_t)rows * ns * m);
    uint32_t* taus = ckeys + (size_t)rows * ns * m;
    if (slen <= kShortRow) {
#define SALS_SHORT_SLICE(K) \
  topk_slice_kernel<kShortThreads, K><<<rows * ns, kShortThreads, 0, st>>>(S, cand, ckeys, taus, Tc, ldS, m, slen, ns, vec)
      if (slen <= 4 * kShortThreads) SALS_SHORT_SLICE(4);
      else if (slen <= 8 * kShortThreads) SALS_SHORT_SLICE(8);
      else SALS_SHORT_SLICE(16);
#undef SALS_SHORT_SLICE
    } else {
#define SALS_SLICE(K) \
  topk_slice_kernel<kThreads, K><<<rows * ns, kThreads, 0, st>>>(S, cand, ckeys, taus, Tc, ldS, m, slen, ns, vec)
      SALS_KPT_SWITCH(slen, SALS_SLICE)
#undef SALS_SLICE
    }
#define SALS_MERGE(K)                                                                                  \
  topk_merge_kernel<K><<<rows, kThreads, 0, st>>>(cand, ckeys, taus, sel, Tc, kp, ns, m, ctx, n_sel, thr, tkey, \
                                                  cnt, S, ldS)
    SALS_KPT_SWITCH(ns * m, SALS_MERGE)
#undef SALS_MERGE
  } else {
    topk_window_kernel<kThreads, 0><<<rows, kThreads, 0, st>>>(S, sel, Tc, ldS, kp, ctx, n_sel, vec, thr, tkey, cnt);
  }
#undef SALS_KPT_SWITCH
  return hipGetLastError();
}

}  // namespace sals
