// Exact per-row top-k with the recent window appended (SALS 关键设计 items 2 and 4; the top-k
// index set S_{psi,k} of the VL-Cache responses, reviewer XVzL weakness 2).
//
// One workgroup of 1024 threads per row. Scores become order-preserving uint32 keys (signed
// zeros equal). The k-th largest key tau is found by an MSB-first radix select, and the row is
// read in full only twice:
//   1. one pass stages the keys in LDS (rows up to 32768 candidates) and builds a 2048-bin
//      histogram of the top 11 key bits (sign, exponent, 2 mantissa bits), from which the bin
//      b1 holding the k-th largest follows;
//   2. a second pass lists, in index order, every position whose key lies in b1 or above (the
//      keys of the higher bins plus b1's keys: a short list). Each thread tests 16 consecutive
//      keys into a 16-bit hit mask; its list position is a prefix sum of the mask counts. The
//      next 11 key bits of tau come from a histogram over the listed keys of b1, the last 10
//      from one more pass over the short list, and the selection is the list filtered by
//      (key > tau, or key == tau for the first take_eq of them), which keeps the list's index
//      order.
// If the list would not fit (heavily tied or degenerate rows, or k close to the row length),
// the remaining digits and the ordered compaction run over the whole row instead (slower).
// Every pass is branch-free over the keys and ranks come from ballots, so per-key work is a few
// VALU operations: with one row per CU the passes are bound by issue rate, not memory.
#include <string.h>

#include <type_traits>

#include "../common.h"
#include "../launch.h"

namespace sals {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kLdsKeys = 32768;
constexpr int kBins = 2048;
constexpr int kIPT = 16;  // keys per lane per chunk when a wave ranks a run (16 slices of 64)

template <bool IN_LDS>
struct TopkLds {
  // short-list capacity (positions): rows staged in LDS have positions below 32768, so their
  // list holds 16-bit entries
  static constexpr int LIST = IN_LDS ? 10240 : 16384;
  using entry = std::conditional_t<IN_LDS, uint16_t, int32_t>;
};

// Finds, in hist[0 .. kBins), the bin b holding the `remaining`-th largest item (bins ordered by
// value, highest bin = largest): bcast[0] = b, bcast[1] = items in bins above b, bcast[2] =
// items in b. Uses all threads; hist is no longer read once it returns.
__device__ __forceinline__ void find_bin(const uint32_t* hist, uint32_t remaining, uint32_t* scan,
                                         uint32_t* bcast) {
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int b0 = 2 * tid;  // each thread owns bins [2*tid, 2*tid + 2)
  const uint32_t c0 = hist[b0], c1 = hist[b0 + 1];
  const uint32_t tot = c0 + c1;
  // suffix sum over the bins: within the wave (total minus the exclusive prefix), then the
  // waves above
  const uint32_t incl = wave_incl_scan(tot, lane);
  const uint32_t wtot = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
  const uint32_t v = wtot - incl + tot;
  if (lane == 0) scan[wave] = v;
  __syncthreads();
  // the totals of all waves in four 16-byte reads, then the ones above this wave (no chain of
  // dependent LDS reads)
  uint32_t sv[kWaves];
#pragma unroll
  for (int q = 0; q < kWaves / 4; ++q) {
    const uint4 t = ((const uint4*)scan)[q];
    sv[4 * q] = t.x;
    sv[4 * q + 1] = t.y;
    sv[4 * q + 2] = t.z;
    sv[4 * q + 3] = t.w;
  }
  uint32_t above_waves = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) above_waves += w > wave ? sv[w] : 0u;
  const uint32_t suf = v + above_waves;  // items in this thread's bins and all higher bins
  const uint32_t above = suf - tot;
  if (above < remaining && remaining <= suf) {
    if (above + c1 >= remaining) {
      bcast[0] = (uint32_t)(b0 + 1);
      bcast[1] = above;
      bcast[2] = c1;
    } else {
      bcast[0] = (uint32_t)b0;
      bcast[1] = above + c1;
      bcast[2] = c0;
    }
  }
  __syncthreads();
}

// The selection of one workgroup: the kp largest of n keys, ties to the lowest position, written
// to out[0 .. kp) in ascending position order as map(position) (and, with okeys, their keys to
// okeys[0 .. kp)), followed by the window out[kp + j] = wstart + j, j < wcount. Keys are
// float_key(src[i]) with map(i) = obase + i, or (GATHER) the given keys ckeys[i] with
// map(i) = cand[i]. GATHER requires IN_LDS.
// Threshold mode (thr): only keys >= tkey may be selected, so kp becomes min(kp, #keys >= tkey)
// (counted over the raw keys before anything else); out[kp + wcount .. pad_to) is filled with -1
// and *cnt_out receives kp + wcount. For GATHER the count runs over the candidates: a row with
// fewer than kp passing keys has all of them among the candidates, otherwise at least kp pass
// there too, so min(kp, count) is the row's.
template <bool IN_LDS, bool GATHER>
__device__ __forceinline__ void topk_body(const float* __restrict__ src, const int32_t* __restrict__ cand,
                                          const uint32_t* __restrict__ ckeys, int n, int kp,
                                          int32_t* __restrict__ out, uint32_t* __restrict__ okeys,
                                          int obase, int wcount, int wstart, bool vec, bool thr,
                                          uint32_t tkey, int32_t* __restrict__ cnt_out, int pad_to) {
  static_assert(IN_LDS || !GATHER, "candidate keys are staged in LDS");
  constexpr int LIST = TopkLds<IN_LDS>::LIST;
  __shared__ __attribute__((aligned(16))) uint32_t keys[IN_LDS ? kLdsKeys : 1];
  __shared__ __attribute__((aligned(16))) uint32_t hist[kBins];
  __shared__ typename TopkLds<IN_LDS>::entry list[LIST];
  __shared__ __attribute__((aligned(16))) uint32_t scan[kWaves];
  __shared__ uint32_t bcast[4];
  __shared__ uint32_t mm[GATHER ? 2 * kWaves : 1];  // per-wave key minima and maxima
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int Tc = n;
  auto map = [&](int i) -> int32_t {
    if constexpr (GATHER) return cand[i];
    else return obase + i;
  };

  if (thr) {
    if (kp > 0) {
      uint32_t mine = 0;
      for (int i = tid; i < Tc; i += kThreads) {
        uint32_t k;
        if constexpr (GATHER) k = ckeys[i];
        else k = float_key(src[i]);
        mine += k >= tkey ? 1u : 0u;
      }
      const uint32_t wsum = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan(mine, lane), 63);
      if (lane == 0) scan[wave] = wsum;
      __syncthreads();
      uint32_t total = 0;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) total += scan[w];
      __syncthreads();  // scan is reused below
      kp = (int)min((uint32_t)kp, total);
    }
    for (int j = kp + wcount + tid; j < pad_to; j += kThreads) out[j] = -1;
    if (tid == 0 && cnt_out) *cnt_out = kp + wcount;
  }
  for (int j = tid; j < wcount; j += kThreads) out[kp + j] = wstart + j;
  if (kp <= 0) return;
  if (kp >= Tc) {
    for (int j = tid; j < Tc; j += kThreads) out[j] = map(j);
    return;
  }
  auto key_at = [&](int i) -> uint32_t {
    if constexpr (IN_LDS) return keys[i];
    else return float_key(src[i]);
  };
  // Keys of this wave for the chunk starting at `base`: wave w owns [base + w*1024, +1024), in
  // 16 slices of 64 (lane l reads the l-th key of each slice, so LDS reads are conflict-free).
  // Reads are unconditional (an LDS row never exceeds the staging array; global indices clamp)
  // so that all 16 are in flight before the first use.
  constexpr int kChunk = kThreads * kIPT;
  uint32_t kk[kIPT];
  auto load_keys = [&](int base) {
    const int w0 = base + wave * 64 * kIPT;
#pragma unroll
    for (int j = 0; j < kIPT; ++j) {
      const int i = w0 + j * 64 + lane;
      if constexpr (IN_LDS) kk[j] = keys[i];
      else kk[j] = float_key(src[min(i, Tc - 1)]);
    }
  };
  // Exclusive prefix of a per-wave count over the waves, and the block total.
  auto wave_prefix = [&](uint32_t mine, uint32_t& before, uint32_t& total) {
    if (lane == 0) scan[wave] = mine;
    __syncthreads();
    before = 0;
    total = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const uint32_t v = scan[w];
      before += (w < wave) ? v : 0u;
      total += v;
    }
    __syncthreads();
  };
  const unsigned long long lt_mask = (1ull << lane) - 1ull;

  // ---- 1. keys to LDS and the digit-1 histogram (key bits [31:21]) in one pass ----
  for (int i = tid; i < kBins; i += kThreads) hist[i] = 0;
  __syncthreads();
  if constexpr (GATHER) {
    // Candidate keys lie in a narrow range (each is among the largest of its slice), so their
    // top 11 bits would fall in a few bins (long bin searches, contended histogram atomics).
    // They are re-encoded as (key - min) << clz(max - min): strictly increasing on the range,
    // so order and ties are unchanged, and the range fills the top key bits.
    uint32_t kmn = 0xffffffffu, kmx = 0u;
    batched_copy<kLdsKeys / kThreads>(Tc, tid, kThreads, [&](int i) { return ckeys[i]; },
                                      [&](int i, uint32_t k) {
                                        keys[i] = k;
                                        kmn = min(kmn, k);
                                        kmx = max(kmx, k);
                                      });
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      kmn = min(kmn, (uint32_t)__shfl_xor((int)kmn, o));
      kmx = max(kmx, (uint32_t)__shfl_xor((int)kmx, o));
    }
    if (lane == 0) {
      mm[wave] = kmn;
      mm[kWaves + wave] = kmx;
    }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      kmn = min(kmn, mm[w]);
      kmx = max(kmx, mm[kWaves + w]);
    }
    const uint32_t range = kmx - kmn;
    const int ls = range ? __clz(range) : 0;
    for (int i = tid; i < Tc; i += kThreads) {
      const uint32_t k = (keys[i] - kmn) << ls;
      keys[i] = k;
      atomicAdd(&hist[k >> 21], 1u);
    }
  } else if constexpr (IN_LDS) {
    if (vec) {  // 16-byte loads (rows start on 16-byte boundaries); keys past Tc are never used
      const float4* s4 = (const float4*)src;
      batched_copy<kLdsKeys / 4 / kThreads>((Tc + 3) / 4, tid, kThreads, [&](int u) { return s4[u]; },
                                            [&](int u, const float4& v) {
                                              const uint32_t k0 = float_key(v.x), k1 = float_key(v.y),
                                                             k2 = float_key(v.z), k3 = float_key(v.w);
                                              *(uint4*)&keys[4 * u] = make_uint4(k0, k1, k2, k3);
                                              atomicAdd(&hist[k0 >> 21], 1u);
                                              if (4 * u + 1 < Tc) atomicAdd(&hist[k1 >> 21], 1u);
                                              if (4 * u + 2 < Tc) atomicAdd(&hist[k2 >> 21], 1u);
                                              if (4 * u + 3 < Tc) atomicAdd(&hist[k3 >> 21], 1u);
                                            });
    } else {
      batched_copy<kLdsKeys / kThreads>(Tc, tid, kThreads, [&](int i) { return src[i]; },
                                        [&](int i, float v) {
                                          const uint32_t k = float_key(v);
                                          keys[i] = k;
                                          atomicAdd(&hist[k >> 21], 1u);
                                        });
    }
  } else {
    batched_copy<16>(Tc, tid, kThreads, [&](int i) { return src[i]; },
                     [&](int, float v) { atomicAdd(&hist[float_key(v) >> 21], 1u); });
  }
  __syncthreads();
  find_bin(hist, (uint32_t)kp, scan, bcast);
  const uint32_t bin1 = bcast[0];
  const uint32_t above = bcast[1];            // keys in bins above bin1
  const uint32_t nl = above + bcast[2];       // keys in bin1 or above
  uint32_t remaining = (uint32_t)kp - above;  // rank of tau inside bin1, >= 1
  // (bcast is next written inside a find_bin, after barriers every thread passes after these
  // reads; hist is free: the zeroing below is ordered before the next atomics by barriers)

  if (nl <= (uint32_t)LIST) {
    // ---- 2. list every position whose key is in bin1 or above, in index order; the same pass
    //      builds the histogram of key bits [20:10] over bin1's keys ----
    for (int i = tid; i < kBins; i += kThreads) hist[i] = 0;
    const uint32_t lo = bin1 << 21;
    uint32_t run = 0;
    if constexpr (IN_LDS) {
      // each thread tests 16 consecutive keys (four 16-byte reads in a lane-dependent order, so
      // that the 8 lanes sharing an LDS bank row hit 8 different 16-byte slots), keeps a 16-bit
      // hit mask, and writes its hits in index order at its prefix-sum position
      for (int base = 0; base < Tc; base += kChunk) {
        const int b0 = base + tid * 16;
        uint32_t hm = 0;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int cc = ((lane >> 1) + c) & 3;
          const uint4 k4 = *(const uint4*)&keys[b0 + cc * 4];
          hm |= ((k4.x >= lo ? 1u : 0u) | (k4.y >= lo ? 2u : 0u) | (k4.z >= lo ? 4u : 0u) |
                 (k4.w >= lo ? 8u : 0u)) << (cc * 4);
        }
        const int nv = min(max(Tc - b0, 0), 16);
        hm &= nv >= 16 ? 0xffffu : ((1u << nv) - 1u);
        const uint32_t cnt = (uint32_t)__popc(hm);
        const uint32_t incl = wave_incl_scan(cnt, lane);
        uint32_t before, total;
        wave_prefix((uint32_t)__builtin_amdgcn_readlane((int)incl, 63), before, total);
        uint32_t at = run + before + incl - cnt;
        while (hm) {
          list[at++] = (uint16_t)(b0 + __builtin_ctz(hm));
          hm &= hm - 1u;
        }
        run += total;
      }
    } else {
      for (int base = 0; base < Tc; base += kChunk) {
        load_keys(base);
        const int w0 = base + wave * 64 * kIPT;
        uint32_t cnt = 0;
#pragma unroll
        for (int j = 0; j < kIPT; ++j)
          cnt += (uint32_t)__popcll(__ballot(w0 + j * 64 + lane < Tc && kk[j] >= lo));
        uint32_t before, total;
        wave_prefix(cnt, before, total);
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
    }
    __syncthreads();
    // histogram of key bits [20:10] over the listed keys of bin1
    for (int u = tid; u < (int)nl; u += kThreads) {
      const uint32_t k = key_at(list[u]);
      if ((k >> 21) == bin1) atomicAdd(&hist[(k >> 10) & 0x7ffu], 1u);
    }
    __syncthreads();
    // ---- key bits [20:10], then [9:0] over the list's keys that match so far ----
    find_bin(hist, remaining, scan, bcast);
    uint32_t prefix = lo | (bcast[0] << 10);
    remaining -= bcast[1];
    for (int i = tid; i < kBins; i += kThreads) hist[i] = 0;
    __syncthreads();
    {
      constexpr int LU = (LIST + kThreads - 1) / kThreads;
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
    find_bin(hist, remaining, scan, bcast);
    const uint32_t tau = prefix | bcast[0], take_eq = remaining - bcast[1];
    // ---- 3. the selection is the list filtered, in list (index) order ----
    constexpr int FPT = (LIST + kThreads - 1) / kThreads;  // list entries per thread: one pass
    uint32_t run_gt = 0, run_eq = 0;
    for (int base = 0; base < (int)nl; base += kThreads * FPT) {
      const int j0 = base + tid * FPT;
      uint32_t fgt = 0, feq = 0;
      int idx[FPT];
      uint32_t kv[FPT];
#pragma unroll
      for (int e = 0; e < FPT; ++e) idx[e] = list[min(j0 + e, (int)nl - 1)];
      // output values requested before the block scan, so that their loads (candidate positions)
      // are in flight while it runs
      int32_t ov[FPT];
#pragma unroll
      for (int e = 0; e < FPT; ++e) ov[e] = map(idx[e]);
#pragma unroll
      for (int e = 0; e < FPT; ++e) {
        const uint32_t k = kv[e] = key_at(idx[e]);
        const bool valid = j0 + e < (int)nl;
        fgt |= (uint32_t)(valid && k > tau) << e;
        feq |= (uint32_t)(valid && k == tau) << e;
      }
      const uint32_t packed = (uint32_t)__popc(fgt) | ((uint32_t)__popc(feq) << 16);
      const uint32_t incl = wave_incl_scan(packed, lane);
      uint32_t before, total;
      wave_prefix((uint32_t)__builtin_amdgcn_readlane((int)incl, 63), before, total);  // wave total
      const uint32_t excl = before + incl - packed;
      uint32_t ngt = run_gt + (excl & 0xffffu), neq = run_eq + (excl >> 16);
#pragma unroll
      for (int e = 0; e < FPT; ++e) {
        if ((fgt >> e) & 1u) {
          out[ngt + min(neq, take_eq)] = ov[e];
          if (okeys) okeys[ngt + min(neq, take_eq)] = kv[e];
          ++ngt;
        } else if ((feq >> e) & 1u) {
          if (neq < take_eq) {
            out[ngt + neq] = ov[e];
            if (okeys) okeys[ngt + neq] = kv[e];
          }
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
    find_bin(hist, remaining, scan, bcast);
    prefix |= bcast[0] << shift;
    remaining -= bcast[1];
    __syncthreads();
  }
  const uint32_t tau = prefix;
  const uint32_t take_eq = remaining;  // >= 1
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
    wave_prefix(wgt | (weq << 16), before, total);
    uint32_t ngt = run_gt + (before & 0xffffu), neq = run_eq + (before >> 16);
#pragma unroll
    for (int j = 0; j < kIPT; ++j) {
      const int i = w0 + j * 64 + lane;
      const bool valid = i < Tc;
      const bool gt = valid && kk[j] > tau, eq = valid && kk[j] == tau;
      const unsigned long long mg = __ballot(gt), me = __ballot(eq);
      const uint32_t bg = ngt + (uint32_t)__popcll(mg & lt_mask);  // gt keys before i
      const uint32_t be = neq + (uint32_t)__popcll(me & lt_mask);  // eq keys before i
      if (gt) {
        out[bg + min(be, take_eq)] = map(i);
        if (okeys) okeys[bg + min(be, take_eq)] = kk[j];
      } else if (eq && be < take_eq) {
        out[bg + be] = map(i);
        if (okeys) okeys[bg + be] = kk[j];
      }
      ngt += (uint32_t)__popcll(mg);
      neq += (uint32_t)__popcll(me);
    }
    run_gt += total & 0xffffu;
    run_eq += total >> 16;
  }
}

template <bool IN_LDS>
__global__ __launch_bounds__(kThreads) void topk_window_kernel(const float* __restrict__ S,
                                                               int32_t* __restrict__ sel, int Tc,
                                                               int ldS, int kp, int ctx, int n_sel,
                                                               bool vec, bool thr, uint32_t tkey,
                                                               int32_t* __restrict__ cnt) {
  const int row = blockIdx.x;
  topk_body<IN_LDS, false>(S + (size_t)row * ldS, nullptr, nullptr, Tc, kp, sel + (size_t)row * n_sel,
                           nullptr, 0, ctx - Tc, Tc, vec, thr, tkey, cnt ? cnt + row : nullptr, n_sel);
}

// Rows longer than the LDS staging array: one workgroup per (row, slice of slen keys) keeps the
// kp largest of its slice (ties to the lowest position) as candidates, in ascending position
// order, with their keys. Every element of the row's top kp is among its slice's top kp, with the
// lowest-index ties of the row's threshold key included, so the row's selection over the
// candidates (which are in ascending position order across slices) is exact.
__global__ __launch_bounds__(kThreads) void topk_slice_kernel(const float* __restrict__ S,
                                                              int32_t* __restrict__ cand,
                                                              uint32_t* __restrict__ ckeys, int Tc,
                                                              int ldS, int kp, int slen, int ns,
                                                              bool vec) {
  const int row = blockIdx.x / ns, s = blockIdx.x % ns;
  const int s0 = s * slen, n = min(slen, Tc - s0);
  const size_t o = ((size_t)row * ns + s) * kp;
  topk_body<true, false>(S + (size_t)row * ldS + s0, nullptr, nullptr, n, kp, cand + o, ckeys + o, s0, 0, 0,
                         vec, false, 0u, nullptr, 0);
}

__global__ __launch_bounds__(kThreads) void topk_merge_kernel(const int32_t* __restrict__ cand,
                                                              const uint32_t* __restrict__ ckeys,
                                                              int32_t* __restrict__ sel, int Tc, int kp,
                                                              int ns, int ctx, int n_sel, bool thr,
                                                              uint32_t tkey, int32_t* __restrict__ cnt) {
  const int row = blockIdx.x;
  const size_t o = (size_t)row * ns * kp;
  topk_body<true, true>(nullptr, cand + o, ckeys + o, ns * kp, kp, sel + (size_t)row * n_sel, nullptr, 0,
                        ctx - Tc, Tc, false, thr, tkey, cnt ? cnt + row : nullptr, n_sel);
}

}  // namespace

int topk_slices(int Tc, int kp, int* slen) {
  if (Tc <= kLdsKeys || kp <= 0) return 0;
  const int ns = ceil_div(Tc, kLdsKeys);
  const int len = (ceil_div(Tc, ns) + 3) / 4 * 4;
  const int last = Tc - (ns - 1) * len;
  if (len > kLdsKeys || last <= kp || (long)ns * kp > kLdsKeys) return 0;
  if (slen) *slen = len;
  return ns;
}

size_t topk_candidate_bytes(int rows, int Tc, int kp) {
  const int ns = topk_slices(Tc, kp, nullptr);
  return ns ? (size_t)rows * ns * kp * 8 : 0;  // positions, then keys
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
  int slen = 0;
  const int ns = cand ? topk_slices(Tc, kp, &slen) : 0;
  if (Tc <= kLdsKeys) {
    topk_window_kernel<true><<<rows, kThreads, 0, st>>>(S, sel, Tc, ldS, kp, ctx, n_sel, vec, thr, tkey, cnt);
  } else if (ns > 0) {
    uint32_t* ckeys = (uint32_t*)(cand + (size_t)rows * ns * kp);
    topk_slice_kernel<<<rows * ns, kThreads, 0, st>>>(S, cand, ckeys, Tc, ldS, kp, slen, ns, vec);
    topk_merge_kernel<<<rows, kThreads, 0, st>>>(cand, ckeys, sel, Tc, kp, ns, ctx, n_sel, thr, tkey, cnt);
  } else {
    topk_window_kernel<false><<<rows, kThreads, 0, st>>>(S, sel, Tc, ldS, kp, ctx, n_sel, vec, thr, tkey, cnt);
  }
  return hipGetLastError();
}

}  // namespace sals
