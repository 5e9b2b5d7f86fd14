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
#include "../topk_rows.h"

namespace sals {
namespace {

using tk::block_prefix;
using tk::find_bin;
using tk::kBins;
using tk::key_value;
using tk::kLdsKeys;
using tk::kSmall;
using tk::padded;
using tk::topk_rows;

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kShortThreads = 256;              // workgroup of the short-row kernel
constexpr int kShortRow = 16 * kShortThreads;   // longest short row (16 keys per thread)
constexpr int kMaxSlices = 64;                  // slices of a long row
constexpr int kIPT = 16;     // keys per lane per chunk when a wave ranks a run (16 slices of 64)
constexpr int kList = 16384; // short-list capacity of topk_global (positions)


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

int topk_rank_plan(int rows, int Tc, int kp, int* m) {
  int slen = 0, mm = 0;
  const int ns = topk_slices(rows, Tc, kp, true, &slen, &mm);
  if (ns <= 0 || mm >= kp) return 0;
  if (m) *m = mm;
  return ns;
}

hipError_t launch_topk_slices(const float* S, int ldS, int rows, int Tc, int kp, int32_t* cand, hipStream_t st) {
  int slen = 0, m = 0;
  const int ns = rows > 0 ? topk_slices(rows, Tc, kp, true, &slen, &m) : 0;
  if (ns <= 0 || m >= kp || !cand) return hipErrorInvalidValue;
  const bool vec = (ldS & 3) == 0 && ((uintptr_t)S & 15) == 0;
  uint32_t* ckeys = (uint32_t*)(cand + (size_t)rows * ns * m);
  uint32_t* taus = ckeys + (size_t)rows * ns * m;
  if (slen <= 4 * kShortThreads)
    topk_slice_kernel<kShortThreads, 4><<<rows * ns, kShortThreads, 0, st>>>(S, cand, ckeys, taus, Tc, ldS, m, slen, ns, vec);
  else if (slen <= 8 * kShortThreads)
    topk_slice_kernel<kShortThreads, 8><<<rows * ns, kShortThreads, 0, st>>>(S, cand, ckeys, taus, Tc, ldS, m, slen, ns, vec);
  else if (slen <= kShortRow)
    topk_slice_kernel<kShortThreads, 16><<<rows * ns, kShortThreads, 0, st>>>(S, cand, ckeys, taus, Tc, ldS, m, slen, ns, vec);
  else
    switch (keys_per_thread(slen)) {
      case 4: topk_slice_kernel<kThreads, 4><<<rows * ns, kThreads, 0, st>>>(S, cand, ckeys, taus, Tc, ldS, m, slen, ns, vec); break;
      case 8: topk_slice_kernel<kThreads, 8><<<rows * ns, kThreads, 0, st>>>(S, cand, ckeys, taus, Tc, ldS, m, slen, ns, vec); break;
      case 16: topk_slice_kernel<kThreads, 16><<<rows * ns, kThreads, 0, st>>>(S, cand, ckeys, taus, Tc, ldS, m, slen, ns, vec); break;
      default: topk_slice_kernel<kThreads, 32><<<rows * ns, kThreads, 0, st>>>(S, cand, ckeys, taus, Tc, ldS, m, slen, ns, vec); break;
    }
  return hipGetLastError();
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
