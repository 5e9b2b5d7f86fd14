// Per-row top-k by one workgroup with the keys in registers (the routine behind the top-k
// kernels, SALS 关键设计 items 2 and 4), shared with the key tile kernel that ranks its own
// sequence's row. Scores become order-preserving uint32 keys; ties go to the lowest position.
#pragma once

#include <type_traits>

#include "common.h"

namespace sals {
namespace tk {

constexpr int kLdsKeys = 32768;
constexpr int kBins = 2048;
constexpr int kSmall = 512;  // the largest threshold bin resolved by counting

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

// LDS word of key i in the staging layout: 4 pad words after every 32 keys, so that a thread
// reading its 32 consecutive keys as 16-byte pieces and a wave writing consecutive 16-byte pieces
// both spread over the banks.
__device__ __forceinline__ int padded(int i) { return i + ((i >> 5) << 2); }

// LDS words topk_rows<NT, KPT, false, true> takes from its caller.
__host__ __device__ constexpr int topk_ext_words(int NT, int KPT) {
  return NT * KPT / 32 * 36 + kBins + NT / 64 + 4 + 4 * (NT / 64) + 3;
}

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
template <int NT, int KPT, bool GATHER, bool EXT = false>
__device__ __forceinline__ bool topk_rows(const float* __restrict__ src, const int32_t* __restrict__ cand,
                                          const uint32_t* __restrict__ ckeys, int n, int kp,
                                          int32_t* __restrict__ out, uint32_t* __restrict__ okeys,
                                          int obase, int wcount, int wstart, bool vec, bool thr,
                                          uint32_t tkey, int32_t* __restrict__ cnt_out, int pad_to,
                                          uint32_t* __restrict__ tau_out = nullptr,
                                          const uint32_t* __restrict__ tcheck = nullptr, int ntcheck = 0,
                                          uint32_t* ext = nullptr) {
  static_assert(KPT % 4 == 0 && KPT <= 32 && NT * KPT <= kLdsKeys, "keys per thread");
  constexpr int NW = NT / 64;
  constexpr int kStage = NT * KPT / 32 * 36;  // staging words for NT * KPT keys
  // staged keys (padded layout); after the ranking, the selection's positions in output order
  // (EXT: carved in this order from the caller's LDS words ext[0 .. topk_ext_words(NT, KPT)),
  // 16-byte aligned; the selection is then left in LDS, below)
  uint32_t *stage, *hist, *scan, *bcast, *mm, *nsp, *tsel;
  if constexpr (EXT) {
    stage = ext;
    hist = stage + kStage;
    scan = hist + kBins;
    bcast = scan + NW;
    mm = bcast + 4;
    nsp = mm + 4 * NW;
    tsel = nsp + 1;
  } else {
    __shared__ __attribute__((aligned(16))) uint32_t s_stage[kStage];
    __shared__ __attribute__((aligned(16))) uint32_t s_hist[kBins];
    __shared__ __attribute__((aligned(16))) uint32_t s_scan[NW];
    __shared__ uint32_t s_bcast[4];
    __shared__ uint32_t s_mm[4 * NW];  // per-wave key minima, maxima, threshold counts, tcheck maxima
    __shared__ uint32_t s_nsmall, s_tsel[2];  // small-bin gather count; (tau, take_eq)
    stage = s_stage;
    hist = s_hist;
    scan = s_scan;
    bcast = s_bcast;
    mm = s_mm;
    nsp = &s_nsmall;
    tsel = s_tsel;
  }
  uint32_t& nsmall = *nsp;
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
  // EXT: the kp positions (row indices, or the candidates' positions) stay in LDS, ext[0 .. kp) in
  // ascending order, for the caller
  if constexpr (EXT) return true;
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

// The exact top kp of a row of n scores read from global memory by NT threads, ties to the lowest
// position: three key-bit digit passes (bits [31:21], [20:10], [9:0]) give the threshold key tau and
// how many keys equal to it are taken, then an ordered compaction over the row writes the selected
// positions to out[0 .. kp) (LDS) in ascending order. scratch: kBins + NT / 64 + 4 LDS words.
// 0 < kp < n. For rows whose candidates could not decide the selection; every thread returns
// after a barrier, with out complete.
template <int NT>
__device__ __forceinline__ void topk_row_digits(const float* __restrict__ src, int n, int kp, int32_t* out,
                                                uint32_t* scratch) {
  constexpr int NW = NT / 64, IPT = 16;
  uint32_t* hist = scratch;
  uint32_t* scan = hist + kBins;
  uint32_t* bcast = scan + NW;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  auto key_at = [&](int i) -> uint32_t { return float_key(src[i]); };
  uint32_t prefix = 0, remaining = (uint32_t)kp;
#pragma unroll 1
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : pass == 1 ? 10 : 0;
    const uint32_t dmask = pass == 2 ? 0x3ffu : 0x7ffu;
    const uint32_t pmask = pass == 0 ? 0u : pass == 1 ? 0xffe00000u : 0xfffffc00u;
    for (int i = tid; i < kBins; i += NT) hist[i] = 0;
    __syncthreads();
    batched_copy<8>(n, tid, NT, key_at, [&](int, uint32_t k) {
      if ((k & pmask) == prefix) atomicAdd(&hist[(k >> shift) & dmask], 1u);
    });
    __syncthreads();
    find_bin<NT>(hist, remaining, scan, bcast);
    prefix |= bcast[0] << shift;
    remaining -= bcast[1];
    __syncthreads();
  }
  const uint32_t tau = prefix, take_eq = remaining;  // take_eq >= 1
  // ordered compaction: wave w owns [base + w * 64 * IPT, + 64 * IPT) of each chunk, lane l the
  // l-th key of each of its IPT runs of 64; ranks inside a run come from ballots, the waves' packed
  // (gt, eq) counts (each at most NT * IPT) from a block prefix
  const unsigned long long lt_mask = (1ull << lane) - 1ull;
  uint32_t run_gt = 0, run_eq = 0;
  for (int base = 0; base < n; base += NT * IPT) {
    const int w0 = base + wave * 64 * IPT;
    uint32_t kk[IPT];
#pragma unroll
    for (int j = 0; j < IPT; ++j) kk[j] = key_at(min(w0 + j * 64 + lane, n - 1));
    uint32_t wgt = 0, weq = 0;
#pragma unroll
    for (int j = 0; j < IPT; ++j) {
      const bool valid = w0 + j * 64 + lane < n;
      wgt += (uint32_t)__popcll(__ballot(valid && kk[j] > tau));
      weq += (uint32_t)__popcll(__ballot(valid && kk[j] == tau));
    }
    uint32_t before, total;
    block_prefix<NT>(wgt | (weq << 16), scan, before, total);
    uint32_t ngt = run_gt + (before & 0xffffu), neq = run_eq + (before >> 16);
#pragma unroll
    for (int j = 0; j < IPT; ++j) {
      const int i = w0 + j * 64 + lane;
      const bool valid = i < n;
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
  __syncthreads();
}

}  // namespace tk
}  // namespace sals
