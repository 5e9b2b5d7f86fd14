// Post-prefill compaction (VL-Cache responses: reviewer KiPr W1 formula A = softmax(QK^T/sqrt(d)),
// W2 post-vision query rows, XVzL W2/W3 top-k of the importance and eviction, X8F2 Q2 once after
// prefill; PureKV abstract: no full attention matrix is formed) and plain decode attention over
// a contiguous cache (VL-Cache KiPr W6: fewer cached tokens, less HBM traffic).
//
// Importance, per (sequence b, KV head g):
//   I[t] = sum_{h of g} sum_{i < w} exp(l_{h,i,t} - m_{h,i}) / s_{h,i},   t <= p_i = ctx - w + i
// with l = Qobs . K / sqrt(d) and (m, s) the row max and softmax denominator of query (h, i).
// Pass 1 computes (m, s) per token chunk with an online update and merges the chunks; pass 2
// recomputes the logits and accumulates I. Logits are kept in base-2 units (scaled by
// log2(e) / sqrt(d)) so that every exponential is one hardware exp2; m and the merged maxima are
// in the same units. Tiles that lie wholly inside every query's causal window (all but the last
// w tokens) skip the per-element masks. Both passes are MFMA tiles of 16 tokens (A operand,
// streamed from HBM) x 16 queries (B operand, in registers), so only the last w query rows are
// ever formed, never the n x n attention matrix.
#include "../common.h"
#include "../launch.h"

namespace sals {
namespace {

constexpr int kThreads = 256;
constexpr int kChunk = SALS_IMP_CHUNK;  // tokens per workgroup
constexpr int kQG = 64;       // observation queries per workgroup (4 MFMA column blocks)
constexpr float kLog2e = 1.4426950408889634f;

template <class T, int DH>
struct Frags {
  using SG = Seg<T, DH>;  // the head dimension plays the role of the contraction length
  typename T::frag q[4][SG::KS];
};

// Query fragments of queries qg*64 + nb*16 + n16 (zero past w).
template <class T, int DH>
__device__ __forceinline__ void load_q_frags(const typename T::elem* __restrict__ Qh, int w, int qg,
                                             int lane, Frags<T, DH>& f) {
  using SG = Seg<T, DH>;
  const int n16 = lane & 15, q4 = lane >> 4;
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    const int qi = qg * kQG + nb * 16 + n16;
    u32x4 ch[SG::NCH];
    if (qi < w) {
      const u32x4* p = (const u32x4*)(Qh + (size_t)qi * DH + q4 * SG::SEG);
#pragma unroll
      for (int c = 0; c < SG::NCH; ++c) ch[c] = p[c];
    } else {
#pragma unroll
      for (int c = 0; c < SG::NCH; ++c) ch[c] = u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int kb = 0; kb < SG::KS; ++kb) f.q[nb][kb] = frag_at<T>(ch, kb);
  }
}

// K rows of one 16-token tile in the MFMA operand layout: lane (n16, q4) holds row t0 + n16
// (clamped to the last valid row), head-dimension segment q4.
template <class T, int DH>
__device__ __forceinline__ void load_k_tile(const typename T::elem* __restrict__ Kh, int t0, int ctx,
                                            int lane, u32x4 (&ch)[Seg<T, DH>::NCH]) {
  using SG = Seg<T, DH>;
  const int n16 = lane & 15, q4 = lane >> 4;
  const int t = min(t0 + n16, ctx - 1);
  const u32x4* p = (const u32x4*)(Kh + (size_t)t * DH + q4 * SG::SEG);
#pragma unroll
  for (int c = 0; c < SG::NCH; ++c) ch[c] = p[c];
}

// logits[nb][i] = K[t0 + q4*4 + i] . Qobs[qg*64 + nb*16 + n16]   (unscaled)
template <class T, int DH>
__device__ __forceinline__ void logit_tile(const u32x4 (&ch)[Seg<T, DH>::NCH], const Frags<T, DH>& f,
                                           f32x4* acc) {
  using SG = Seg<T, DH>;
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kb = 0; kb < SG::KS; ++kb) {
    const typename T::frag a = frag_at<T>(ch, kb);
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) acc[nb] = T::mma(a, f.q[nb][kb], acc[nb]);
  }
}

// A wave's tiles t = t_begin, t_begin + stride, ... < t_end with the K rows of the next D - 1
// tiles in flight while one is computed (D buffers, indexed by compile-time constants).
template <class T, int DH>
constexpr int kKDepth = sizeof(typename T::elem) == 2 ? 4 : 2;

template <class T, int DH, class StepF>
__device__ __forceinline__ void for_k_tiles(const typename T::elem* __restrict__ Kh, int ctx, int lane,
                                            int t_begin, int t_end, int stride, StepF step) {
  constexpr int D = kKDepth<T, DH>;
  u32x4 buf[D][Seg<T, DH>::NCH];
#pragma unroll
  for (int j = 0; j < D; ++j)
    if (t_begin + j * stride < t_end) load_k_tile<T, DH>(Kh, t_begin + j * stride, ctx, lane, buf[j]);
  for (int t0 = t_begin; t0 < t_end; t0 += D * stride) {
#pragma unroll
    for (int j = 0; j < D; ++j) {
      const int t = t0 + j * stride;
      if (t < t_end) {
        step(t, buf[j]);
        if (t + D * stride < t_end) load_k_tile<T, DH>(Kh, t + D * stride, ctx, lane, buf[j]);
      }
    }
  }
}

// Pass 1: per chunk (m, s) of every observation query. grid (n_chunks, H_q * n_qg, B).
template <class T, int DH>
__global__ __launch_bounds__(kThreads) void imp_stats_kernel(const typename T::elem* __restrict__ K,
                                                             const typename T::elem* __restrict__ Q,
                                                             float* __restrict__ part, int H_q,
                                                             int H_kv, int w, int ctx_cap, int ctx,
                                                             int n_chunks, int n_qg) {
  __shared__ float red[4][kQG][2];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n16 = lane & 15, q4 = lane >> 4;
  const int c = blockIdx.x, h = blockIdx.y / n_qg, qg = blockIdx.y % n_qg, b = blockIdx.z;
  const int g = h / (H_q / H_kv);
  const float scale = kLog2e / sqrtf((float)DH);
  const typename T::elem* Kh = K + ((size_t)b * H_kv + g) * ctx_cap * DH;
  Frags<T, DH> f;
  load_q_frags<T, DH>(Q + ((size_t)b * H_q + h) * w * DH, w, qg, lane, f);
  float m[4], s[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    m[nb] = -INFINITY;
    s[nb] = 0.f;
  }
  const int cbeg = c * kChunk, cend = min(ctx, cbeg + kChunk);
  // online (max, sum) per lane over its 4 tokens of each tile: the tile's own maximum first, then
  // one rescale. Branch-free: the visibility masks are combined with bitwise operators and
  // applied by selects (short-circuit conditions would compile to one divergent branch per
  // element), and a lane that has seen nothing yet (mn = -inf) rescales against 0 instead, which
  // leaves (m, s) = (-inf, 0) unchanged since every exponential is then of -inf.
  for_k_tiles<T, DH>(Kh, ctx, lane, cbeg + wave * 16, cend, 64, [&](int t0, const u32x4 (&ch)[Seg<T, DH>::NCH]) {
    f32x4 acc[4];
    logit_tile<T, DH>(ch, f, acc);
    // the whole tile is visible to every query of the group (and they all exist)
    const bool full = t0 + 16 <= cend && t0 + 15 <= ctx - w + qg * kQG && (qg + 1) * kQG <= w;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int qi = qg * kQG + nb * 16 + n16;
      const int lim = ctx - w + qi;  // last visible position of query qi
      float x[4];
      float tm = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = t0 + q4 * 4 + i;
        const bool ok = full | ((t < cend) & (t <= lim) & (qi < w));
        const float v = acc[nb][i] * scale;
        x[i] = ok ? v : -INFINITY;
        tm = fmaxf(tm, x[i]);
      }
      const float mn = fmaxf(m[nb], tm);
      const float mref = mn == -INFINITY ? 0.f : mn;
      float add = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) add += __builtin_amdgcn_exp2f(x[i] - mref);
      s[nb] = s[nb] * __builtin_amdgcn_exp2f(m[nb] - mref) + add;
      m[nb] = mn;
    }
  });
  // merge the 4 lane groups (same query), then the 4 waves
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
#pragma unroll
    for (int msk = 16; msk <= 32; msk <<= 1) {
      const float mo = __shfl_xor(m[nb], msk), so = __shfl_xor(s[nb], msk);
      const float mn = fmaxf(m[nb], mo);
      s[nb] = (mn == -INFINITY) ? 0.f : s[nb] * __builtin_amdgcn_exp2f(m[nb] - mn) + so * __builtin_amdgcn_exp2f(mo - mn);
      m[nb] = mn;
    }
    if (lane < 16) {
      red[wave][nb * 16 + lane][0] = m[nb];
      red[wave][nb * 16 + lane][1] = s[nb];
    }
  }
  __syncthreads();
  if (tid < kQG) {
    const int qi = qg * kQG + tid;
    float M = -INFINITY;
    for (int wv = 0; wv < 4; ++wv) M = fmaxf(M, red[wv][tid][0]);
    float S = 0.f;
    if (M != -INFINITY)
      for (int wv = 0; wv < 4; ++wv) S += red[wv][tid][1] * __builtin_amdgcn_exp2f(red[wv][tid][0] - M);
    if (qi < w) {
      float* p = part + ((((size_t)b * H_q + h) * w + qi) * n_chunks + c) * 2;
      p[0] = M;
      p[1] = S;
    }
  }
}

// Merge chunk partials: stats[b][h][i] = (M, S).
__global__ void imp_merge_kernel(const float* __restrict__ part, float* __restrict__ stats, int n,
                                 int n_chunks) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= n) return;
  const float* p = part + (size_t)e * n_chunks * 2;
  float M = -INFINITY;
  for (int c = 0; c < n_chunks; ++c) M = fmaxf(M, p[2 * c]);
  float S = 0.f;
  for (int c = 0; c < n_chunks; ++c)
    if (p[2 * c] != -INFINITY) S += p[2 * c + 1] * __builtin_amdgcn_exp2f(p[2 * c] - M);
  stats[2 * (size_t)e] = M;
  stats[2 * (size_t)e + 1] = S;
}

// Pass 2: I[b][g][t]. grid (n_chunks, H_kv, B). With cnt, it also counts per query head the
// causal entries of this chunk whose probability is below p_thresh (the post-vision sparsity):
// cnt[(b * H_q + h) * n_chunks + c], exact as float sums of whole numbers below 2^24.
template <class T, int DH>
__global__ __launch_bounds__(kThreads) void imp_accum_kernel(const typename T::elem* __restrict__ K,
                                                             const typename T::elem* __restrict__ Q,
                                                             const float* __restrict__ stats,
                                                             float* __restrict__ I, int H_q,
                                                             int H_kv, int w, int ctx_cap, int ctx,
                                                             float p_thresh, float* __restrict__ cnt) {
  __shared__ float acc_lds[kChunk];
  __shared__ float cnt_red[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n16 = lane & 15, q4 = lane >> 4;
  const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int nqh = H_q / H_kv;
  const float scale = kLog2e / sqrtf((float)DH);
  const typename T::elem* Kh = K + ((size_t)b * H_kv + g) * ctx_cap * DH;
  const int cbeg = c * kChunk, cend = min(ctx, cbeg + kChunk);
  for (int j = tid; j < kChunk; j += kThreads) acc_lds[j] = 0.f;
  __syncthreads();
  const int n_qg = ceil_div(w, kQG);
  const int n_chunks = gridDim.x;
  for (int hh = 0; hh < nqh; ++hh) {
    const int h = g * nqh + hh;
    float below = 0.f;  // this lane's entries under the threshold, for head h
    for (int qg = 0; qg < n_qg; ++qg) {
      Frags<T, DH> f;
      load_q_frags<T, DH>(Q + ((size_t)b * H_q + h) * w * DH, w, qg, lane, f);
      float M[4], invS[4];
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int qi = qg * kQG + nb * 16 + n16;
        if (qi < w) {
          const float* st = stats + (((size_t)b * H_q + h) * w + qi) * 2;
          M[nb] = st[0];
          invS[nb] = 1.0f / st[1];
        } else {
          M[nb] = 0.f;
          invS[nb] = 0.f;
        }
      }
      for_k_tiles<T, DH>(Kh, ctx, lane, cbeg + wave * 16, cend, 64, [&](int t0, const u32x4 (&ch)[Seg<T, DH>::NCH]) {
        f32x4 acc[4];
        logit_tile<T, DH>(ch, f, acc);
        float part[4] = {0.f, 0.f, 0.f, 0.f};
        const bool full = t0 + 15 <= ctx - w + qg * kQG && (qg + 1) * kQG <= w;
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          const int qi = qg * kQG + nb * 16 + n16;
          const int lim = ctx - w + qi;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int t = t0 + q4 * 4 + i;
            const float e = __builtin_amdgcn_exp2f(acc[nb][i] * scale - M[nb]) * invS[nb];
            const bool valid = full | ((qi < w) & (t <= lim));  // bitwise: no branch per element
            part[i] += valid ? e : 0.f;
            if (cnt) below += (valid & (e < p_thresh)) ? 1.f : 0.f;
          }
        }
        // sum over the 16 queries of the row (DPP, no LDS crossbar)
#pragma unroll
        for (int i = 0; i < 4; ++i) part[i] = row16_sum(part[i]);
        if (n16 == 0) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int t = t0 + q4 * 4 + i;
            if (t < cend) acc_lds[t - cbeg] += part[i];
          }
        }
      });
    }
    if (cnt) {  // workgroup total for head h (waves in order)
      below = wave_sum(below);
      if (lane == 0) cnt_red[wave] = below;
      __syncthreads();
      if (tid == 0) cnt[((size_t)b * H_q + h) * n_chunks + c] = ((cnt_red[0] + cnt_red[1]) + cnt_red[2]) + cnt_red[3];
      __syncthreads();
    }
  }
  __syncthreads();
  for (int j = tid; j < cend - cbeg; j += kThreads) I[((size_t)b * H_kv + g) * ctx + cbeg + j] = acc_lds[j];
}

// Kc/Vc rows: bit-exact 16-byte copies. One thread per 16-byte chunk.
__global__ void gather_rows_kernel(const u32x4* __restrict__ K, const u32x4* __restrict__ V,
                                   const int32_t* __restrict__ kept, u32x4* __restrict__ Kc,
                                   u32x4* __restrict__ Vc, long n_chunks_total, int cpr, int ctx_cap,
                                   int k_keep) {
  const long e = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= n_chunks_total) return;
  const long row = e / cpr;
  const int cc = (int)(e % cpr);
  const long bg = row / k_keep;
  const long src = (bg * ctx_cap + kept[row]) * cpr + cc;
  Kc[e] = K[src];
  Vc[e] = V[src];
}

// Dense flash-decode over a contiguous cache. A workgroup takes one split of one KV head for NG
// of its query heads (NG = 4, 2 or 1, dividing the query heads per KV head): wave w computes
// head w % NG over token phase w / NG, so with NG > 1 the waves of a CU read the same K/V rows
// at about the same time and all but the first find them in L1. Four lanes share one token row:
// load instruction i of lane l reads 16-byte piece 4i + l%4 of row l/4, so the four lanes of a
// row read 64 contiguous bytes per instruction. Each wave takes 16 tokens per step and issues the
// next step's rows before it computes on the current ones. Grid: one dimension, XCD-aware order
// with the head groups of one KV head fastest, then the split: the workgroups that read the same
// rows run on one XCD at about the same time.
template <class T, int DH>
__global__ __launch_bounds__(kThreads) void dense_decode_kernel(
    const typename T::elem* __restrict__ q, const typename T::elem* __restrict__ K,
    const typename T::elem* __restrict__ V, float* __restrict__ out, float* __restrict__ part,
    int H_q, int H_kv, int n, int stride, int split_len, int n_splits) {
  using elem = typename T::elem;
  constexpr int CW = DH / 4;                     // columns per lane
  constexpr int EPP = 16 / (int)sizeof(elem);    // elements per 16-byte piece
  constexpr int NP = CW / EPP;                   // pieces per lane and row
  __shared__ float qsh[4][DH];
  __shared__ float red[4][DH + 2];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nqh = H_q / H_kv;
  const int NG = dense_heads_per_group(nqh), NPH = 4 / NG, ngr = nqh / NG;
  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int gr = wg % ngr, sp = (wg / ngr) % n_splits, g = (wg / (ngr * n_splits)) % H_kv;
  const int b = wg / (ngr * n_splits * H_kv);
  const int myh = wave % NG, phase = wave / NG;
  const float scale = 1.0f / sqrtf((float)DH);
  for (int c = tid; c < NG * DH; c += kThreads)
    qsh[c / DH][c % DH] = T::to_f32(q[((size_t)b * H_q + g * nqh + gr * NG + c / DH) * DH + c % DH]) * scale;
  __syncthreads();
  const int lq = lane & 3;
  auto col = [&](int j) { return ((j / EPP) * 4 + lq) * EPP + j % EPP; };  // column of element j
  float qv[CW];
#pragma unroll
  for (int j = 0; j < CW; ++j) qv[j] = qsh[myh][col(j)];
  const elem* Kh = K + ((size_t)b * H_kv + g) * stride * DH;
  const elem* Vh = V + ((size_t)b * H_kv + g) * stride * DH;
  const int jbeg = sp * split_len, jend = min(n, jbeg + split_len);
  float m = -INFINITY, l = 0.f;
  float o[CW];
#pragma unroll
  for (int j = 0; j < CW; ++j) o[j] = 0.f;
  auto load = [&](int t0, u32x4 (&kr)[NP], u32x4 (&vr)[NP]) {
    const int tt = min(t0 + (lane >> 2), jend - 1);
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      kr[i] = *(const u32x4*)(Kh + (size_t)tt * DH + (4 * i + lq) * EPP);
      vr[i] = *(const u32x4*)(Vh + (size_t)tt * DH + (4 * i + lq) * EPP);
    }
  };
  auto value = [&](const u32x4 (&r)[NP], int j) {
    const uint32_t w = r[j / EPP][(j % EPP) * (int)sizeof(elem) / 4];
    if constexpr (sizeof(elem) == 2) return __uint_as_float((j & 1) ? (w & 0xffff0000u) : (w << 16));
    else return __uint_as_float(w);
  };
  auto step = [&](int t0, const u32x4 (&kr)[NP], const u32x4 (&vr)[NP]) {
    const bool ok = t0 + (lane >> 2) < jend;
    float x = 0.f;
#pragma unroll
    for (int j = 0; j < CW; ++j) x = fmaf(qv[j], value(kr, j), x);
    x += __shfl_xor(x, 1);
    x += __shfl_xor(x, 2);
    if (!ok) x = -INFINITY;
    const float tm = wave_max(x);
    const float mn = fmaxf(m, tm);
    const float corr = expf(m - mn);
    const float p = ok ? expf(x - mn) : 0.f;
    float ps = p;
    ps += __shfl_xor(ps, 4);
    ps += __shfl_xor(ps, 8);
    ps += __shfl_xor(ps, 16);
    ps += __shfl_xor(ps, 32);
    l = l * corr + ps;
    m = mn;
#pragma unroll
    for (int j = 0; j < CW; ++j) o[j] = fmaf(p, value(vr, j), o[j] * corr);
  };
  u32x4 k0[NP], v0[NP], k1[NP], v1[NP];
  const int tstep = 16 * NPH;
  int t0 = jbeg + phase * 16;
  if (t0 < jend) load(t0, k0, v0);
  for (; t0 < jend; t0 += 2 * tstep) {
    if (t0 + tstep < jend) load(t0 + tstep, k1, v1);
    step(t0, k0, v0);
    if (t0 + tstep >= jend) break;
    if (t0 + 2 * tstep < jend) load(t0 + 2 * tstep, k0, v0);
    step(t0 + tstep, k1, v1);
  }
  // reduce o over the 16 tokens of the wave (lanes with equal lane%4)
#pragma unroll
  for (int j = 0; j < CW; ++j) {
    float v = o[j];
    v += __shfl_xor(v, 4);
    v += __shfl_xor(v, 8);
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    o[j] = v;
  }
  if (lane < 4) {
#pragma unroll
    for (int j = 0; j < CW; ++j) red[wave][col(j)] = o[j];
  }
  if (lane == 0) {
    red[wave][DH] = m;
    red[wave][DH + 1] = l;
  }
  __syncthreads();
  // head e of the group: waves e, e + NG, ... (its token phases), merged in phase order
  for (int c2 = tid; c2 < NG * DH; c2 += kThreads) {
    const int e = c2 / DH, c = c2 % DH;
    float M = -INFINITY;
    for (int ph = 0; ph < NPH; ++ph) M = fmaxf(M, red[ph * NG + e][DH]);
    float L = 0.f, oc = 0.f;
    for (int ph = 0; ph < NPH; ++ph) {
      const int wv = ph * NG + e;
      const float wgt = red[wv][DH] == -INFINITY ? 0.f : expf(red[wv][DH] - M);
      L += red[wv][DH + 1] * wgt;
      oc += red[wv][c] * wgt;
    }
    const int hq = g * nqh + gr * NG + e;
    if (n_splits == 1) {
      out[((size_t)b * H_q + hq) * DH + c] = oc / L;
    } else {
      float* pp = part + (((size_t)b * H_q + hq) * n_splits + sp) * (DH + 2);
      pp[2 + c] = oc;
      if (c == 0) {
        pp[0] = M;
        pp[1] = L;
      }
    }
  }
}

}  // namespace

#define SALS_KVC_DISPATCH(dtype, d, CALL)        \
  do {                                           \
    if (dtype == 0 && d == 64) {                 \
      using TT = F32;                            \
      constexpr int DD = 64;                     \
      CALL;                                      \
    } else if (dtype == 0 && d == 128) {         \
      using TT = F32;                            \
      constexpr int DD = 128;                    \
      CALL;                                      \
    } else if (dtype == 1 && d == 64) {          \
      using TT = BF16;                           \
      constexpr int DD = 64;                     \
      CALL;                                      \
    } else if (dtype == 1 && d == 128) {         \
      using TT = BF16;                           \
      constexpr int DD = 128;                    \
      CALL;                                      \
    } else {                                     \
      return hipErrorInvalidValue;               \
    }                                            \
  } while (0)

hipError_t launch_importance_stats(int dtype, const void* K, const void* Qobs, float* stats,
                                   int B, int H_q, int H_kv, int d, int w, int ctx_cap, int ctx,
                                   hipStream_t st) {
  // stats buffer layout: [B*H_q*w*n_chunks*2] chunk partials followed by [B*H_q*w*2] merged
  const int n_chunks = ceil_div(ctx, kChunk), n_qg = ceil_div(w, kQG);
  float* part = stats + (size_t)B * H_q * w * 2;
  dim3 grid(n_chunks, H_q * n_qg, B);
  SALS_KVC_DISPATCH(dtype, d,
                    (imp_stats_kernel<TT, DD><<<grid, kThreads, 0, st>>>(
                        (const TT::elem*)K, (const TT::elem*)Qobs, part, H_q, H_kv, w, ctx_cap, ctx,
                        n_chunks, n_qg)));
  const int n = B * H_q * w;
  imp_merge_kernel<<<ceil_div(n, 256), 256, 0, st>>>(part, stats, n, n_chunks);
  return hipGetLastError();
}

// Sparsity[b][h] = (sum over chunks of cnt) / (number of causal entries of the w rows).
__global__ void sparsity_kernel(const float* __restrict__ cnt, float* __restrict__ sparsity, int n,
                                int n_chunks, double total) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= n) return;
  double s = 0.0;
  for (int c = 0; c < n_chunks; ++c) s += cnt[(size_t)e * n_chunks + c];
  sparsity[e] = (float)(s / total);
}

hipError_t launch_importance_accum(int dtype, const void* K, const void* Qobs,
                                   const float* stats, float* I, int B, int H_q, int H_kv, int d,
                                   int w, int ctx_cap, int ctx, hipStream_t st, float p_thresh,
                                   float* cnt, float* sparsity) {
  dim3 grid(ceil_div(ctx, kChunk), H_kv, B);
  SALS_KVC_DISPATCH(dtype, d,
                    (imp_accum_kernel<TT, DD><<<grid, kThreads, 0, st>>>(
                        (const TT::elem*)K, (const TT::elem*)Qobs, stats, I, H_q, H_kv, w, ctx_cap,
                        ctx, p_thresh, cnt)));
  if (cnt && sparsity) {
    const int n = B * H_q;
    const double total = (double)w * (ctx - w) + (double)w * (w + 1) / 2;
    sparsity_kernel<<<ceil_div(n, 256), 256, 0, st>>>(cnt, sparsity, n, (int)grid.x, total);
  }
  return hipGetLastError();
}

hipError_t launch_gather_rows(int dtype, const void* K, const void* V, const int32_t* kept,
                              void* Kc, void* Vc, int BG, int d, int ctx_cap, int k_keep,
                              hipStream_t st) {
  const int cpr = d * (dtype == 0 ? 4 : 2) / 16;
  const long total = (long)BG * k_keep * cpr;
  if (total <= 0) return hipSuccess;
  gather_rows_kernel<<<(unsigned)((total + 255) / 256), 256, 0, st>>>(
      (const u32x4*)K, (const u32x4*)V, kept, (u32x4*)Kc, (u32x4*)Vc, total, cpr, ctx_cap, k_keep);
  return hipGetLastError();
}

hipError_t launch_dense_decode(int dtype, const void* q, const void* K, const void* V, float* out,
                               float* part, int B, int H_q, int H_kv, int d, int n, int stride,
                               int split_len, int n_splits, hipStream_t st) {
  dim3 grid(n_splits * (H_q / dense_heads_per_group(H_q / H_kv)) * B);
  SALS_KVC_DISPATCH(dtype, d,
                    (dense_decode_kernel<TT, DD><<<grid, kThreads, 0, st>>>(
                        (const TT::elem*)q, (const TT::elem*)K, (const TT::elem*)V, out, part, H_q,
                        H_kv, n, stride, split_len, n_splits)));
  return hipGetLastError();
}

}  // namespace sals
