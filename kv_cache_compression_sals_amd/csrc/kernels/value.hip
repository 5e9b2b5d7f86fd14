// Value side of the selected attention for selection groups shared by several KV heads
// (SALS 技术框架 stage 4 over the rows selected in stage 2; the product p^T V_hat is taken in
// the latent space, p^T (L_v,sel P_v^T) = (p^T L_v,sel) P_v^T, because V carries no rotation).
//
// When one selection serves m >= 4 KV heads (e.g. G = 1 over all heads of an MHA layer), the
// fused kernel would stream the same gathered L_v rows once per KV head. Here they are read
// once per block of latent columns instead:
//   value_sum:     zpart[c][b][h][j] = w[b][h][split(c)] sum_{t in chunk c} p[b][h][t] L_v[sel[t]][j]
//                  for all query heads of the group. The selected set is cut into chunks, each a
//                  piece of one attention split, so all tokens of a chunk share that split's merge
//                  weight w = e^{m_split - M} / L. One workgroup takes one (sequence, group, chunk,
//                  column block): it stages the chunk's probabilities and gathered row pieces
//                  (transposed, tokens contiguous) in LDS and forms the (heads x tokens) .
//                  (tokens x columns) product with MFMA.
//   value_product: z[b][h] = sum_c zpart[c][b][h] (chunk order), then out[b][h][c] =
//                  sum_j P_v[kv(h) d + c][j] z[b][h][j] as an MFMA product: one workgroup per
//                  (KV head, 16 rows of P_v, up to 8 or 16 (sequence, head) columns); its four
//                  waves stage z together and split the rank, so every P_v row is read once per
//                  column tile rather than once per sequence.
// Memory reads use whole 128-byte lines where the layout allows (probabilities, z): a wave
// instruction that touches 16 rows x 64 bytes moves about half the bytes per CU cycle.
#include "../common.h"
#include "../launch.h"

namespace sals {
namespace {

constexpr int kThreads = 256;
constexpr int kLdsMax = 64512;  // value_sum dynamic LDS (with the static part: two workgroups per CU)
constexpr int kCLMax = 512;     // tokens per chunk
constexpr int kMaxHS = 128;     // query heads per selection group
constexpr int kMinChunk = 32;   // shortest chunk made by subdividing a split

// LDS layout of value_sum, in elements of the cache type, all rows of stride ts = cl + one
// 16-byte chunk (row starts then fall on different banks):
//   rowsT[CB][ts]        gathered row pieces, transposed (column-major: tokens contiguous)
//   pA[NP][hs16][ts]     probabilities of the chunk (bf16: high and low parts, NP = 2)
template <class T>
struct VSLayout {
  static constexpr int ESZ = (int)sizeof(typename T::elem);
  static constexpr int NP = T::HILO ? 2 : 1;
  __host__ __device__ static int ts(int cl) { return cl + 16 / ESZ; }
  static size_t bytes(int cb, int hs16, int cl) {
    return (size_t)(cb + NP * hs16) * ts(cl) * ESZ;
  }
};

// grid ncb * nch * B * G (XCD-aware: the chunks and column blocks of one (sequence, group) are
// consecutive, so the workgroups that split a gathered row share an L2); block 256.
template <class T, int CB>
__global__ __launch_bounds__(kThreads) void value_sum_kernel(
    const float* __restrict__ pbuf, const float* __restrict__ pstat, const int32_t* __restrict__ sel,
    const int32_t* __restrict__ cnt, const typename T::elem* __restrict__ Lv, float* __restrict__ zpart,
    int B, int H_q, int G, int r, int ctx_cap, int n_sel, int split_len, int n_splits, int nsub, int cl,
    int nch) {
  using elem = typename T::elem;
  using W = Win<T>;
  using LY = VSLayout<T>;
  constexpr int EPC = W::EPC;    // elements per 16-byte chunk
  constexpr int CPR = CB / EPC;  // 16-byte chunks per row piece
  extern __shared__ __attribute__((aligned(16))) unsigned char vs_smem[];
  __shared__ float wsh[kMaxHS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n16 = lane & 15, q4 = lane >> 4;
  const int ncb = r / CB;
  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int cb = wg % ncb, c = (wg / ncb) % nch, bs = wg / (ncb * nch);
  const int b = bs / G, s = bs % G;
  const int HS = H_q / G, hs16 = (HS + 15) / 16 * 16;
  const int sp = c / nsub, u = c % nsub;
  const int t0 = sp * split_len + u * cl;
  // a ragged (thresholded) row ends at its own count: chunks past it sum nothing
  const int t1 = min(sp * split_len + min((u + 1) * cl, split_len), cnt ? cnt[bs] : n_sel);
  const int nt = max(t1 - t0, 0);
  const int ntp = (nt + W::WLEN - 1) / W::WLEN * W::WLEN;  // whole MFMA windows
  const int ts = LY::ts(cl);
  elem* rowsT = (elem*)vs_smem;
  elem* pA = rowsT + (size_t)CB * ts;
  const int h0 = s * HS;
  const int nsp = (n_sel + 3) & ~3;  // row stride of pbuf

  // ---- 1-2. probabilities (unit: 4 tokens of one head; zero past the chunk and for padding
  //      heads) and row pieces (unit: token pair i, 16-byte chunk cc; tokens past the chunk repeat
  //      its last row, whose probabilities are zero), both staged in LDS, the pieces transposed.
  //      The first batch of every load is issued before any is consumed: the positions of this
  //      thread's pieces straight from the selection (no LDS round trip), the probabilities, then
  //      the gathered pieces; the probabilities and the split statistics are written while the
  //      pieces are in flight. ----
  const int nq = ntp / 4, npu = hs16 * nq;   // probability units
  const int np2 = ntp / 2, nru = np2 * CPR;  // row-piece units
  const int32_t* selrow = sel + (size_t)bs * n_sel + t0;
  const float* prow0 = pbuf + ((size_t)b * H_q + h0) * nsp + t0;
  const elem* vbase = Lv + (size_t)b * ctx_cap * r + cb * CB;
  auto row_pos = [&](int e0, int32_t (&pp)[4][2]) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int i = min(e0 + k * kThreads, nru - 1) % np2;
#pragma unroll
      for (int h = 0; h < 2; ++h) pp[k][h] = selrow[min(2 * i + h, nt - 1)];
    }
  };
  auto row_load = [&](int e0, const int32_t (&pp)[4][2], u32x4 (&v)[4][2]) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int cc = min(e0 + k * kThreads, nru - 1) / np2;
#pragma unroll
      for (int h = 0; h < 2; ++h) v[k][h] = *(const u32x4*)(vbase + (size_t)pp[k][h] * r + cc * EPC);
    }
  };
  auto row_store = [&](int e0, const u32x4 (&v)[4][2]) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int e = e0 + k * kThreads;
      if (e < nru) {
        const int i = e % np2, cc = e / np2;
        elem* dst = rowsT + (size_t)cc * EPC * ts + 2 * i;
        if constexpr (sizeof(elem) == 2) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            // columns 2j and 2j+1 of tokens 2i and 2i+1
            const uint32_t a = v[k][0][j], bb = v[k][1][j];
            *(uint32_t*)(dst + (size_t)(2 * j) * ts) = (a & 0xffffu) | (bb << 16);
            *(uint32_t*)(dst + (size_t)(2 * j + 1) * ts) = (a >> 16) | (bb & 0xffff0000u);
          }
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) *(uint2*)(dst + (size_t)j * ts) = make_uint2(v[k][0][j], v[k][1][j]);
        }
      }
    }
  };
  auto p_load = [&](int e0, u32x4 (&v)[4]) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int e = min(e0 + k * kThreads, npu - 1);
      const int hl = min(e / nq, HS - 1), q = min(e % nq, (nt - 1) / 4);
      v[k] = *(const u32x4*)(prow0 + (size_t)hl * nsp + 4 * q);
    }
  };
  auto p_store = [&](int e0, const u32x4 (&v)[4]) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int e = e0 + k * kThreads;
      if (e < npu) {
        const int hl = e / nq, q = e % nq;
        float x[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) x[m] = (hl < HS && 4 * q + m < nt) ? __uint_as_float(v[k][m]) : 0.f;
        elem* dst = pA + (size_t)hl * ts + 4 * q;
        if constexpr (T::HILO) {
          uint32_t hi[4], lo[4];
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            hi[m] = f32_to_bf16_bits(x[m]);
            lo[m] = f32_to_bf16_bits(x[m] - bf16_bits_to_f32(hi[m]));
          }
          *(uint2*)dst = make_uint2(hi[0] | hi[1] << 16, hi[2] | hi[3] << 16);
          *(uint2*)(dst + (size_t)hs16 * ts) = make_uint2(lo[0] | lo[1] << 16, lo[2] | lo[3] << 16);
        } else {
          *(u32x4*)dst = u32x4{__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]),
                               __float_as_uint(x[3])};
        }
      }
    }
  };
  // merge weight of this chunk's split per head (tid < HS): e^{m_split - M} / L over all splits,
  // from the split statistics held in registers (a loop over them beyond kStReg splits)
  constexpr int kStReg = 8;
  const float* st = pstat + ((size_t)b * H_q + h0 + min(tid, HS - 1)) * n_splits * 2;
  float stm[kStReg], stl[kStReg], stmine = 0.f;
  auto stats_load = [&]() {
    if (tid < HS && n_splits <= kStReg) {
#pragma unroll
      for (int k = 0; k < kStReg; ++k) {
        const int kk = min(k, n_splits - 1);
        stm[k] = st[2 * kk];
        stl[k] = st[2 * kk + 1];
      }
      stmine = st[2 * sp];
    }
  };
  auto stats_weight = [&]() {
    if (tid >= HS) return;
    float M = -INFINITY, L = 0.f;
    if (n_splits <= kStReg) {
#pragma unroll
      for (int k = 0; k < kStReg; ++k) M = k < n_splits ? fmaxf(M, stm[k]) : M;
#pragma unroll
      for (int k = 0; k < kStReg; ++k) L = k < n_splits ? L + stl[k] * expf(stm[k] - M) : L;
      wsh[tid] = expf(stmine - M) / L;
    } else {
      for (int k = 0; k < n_splits; ++k) M = fmaxf(M, st[2 * k]);
      for (int k = 0; k < n_splits; ++k) L += st[2 * k + 1] * expf(st[2 * k] - M);
      wsh[tid] = expf(st[2 * sp] - M) / L;
    }
  };
  if (nt > 0) {  // (nt = 0: no units, and the tiles below sum no window)
    int32_t pp[4][2];
    u32x4 pv[4], rv[4][2];
    row_pos(tid, pp);
    p_load(tid, pv);
    row_load(tid, pp, rv);
    stats_load();
    // every first-batch load is issued before the first LDS write (the empty asm keeps the
    // compiler from sinking the loads towards their uses)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    p_store(tid, pv);
    for (int e0 = tid + 4 * kThreads; e0 < npu; e0 += 4 * kThreads) {
      p_load(e0, pv);
      __builtin_amdgcn_sched_barrier(0);
      p_store(e0, pv);
    }
    stats_weight();
    row_store(tid, rv);
    for (int e0 = tid + 4 * kThreads; e0 < nru; e0 += 4 * kThreads) {
      row_pos(e0, pp);
      row_load(e0, pp, rv);
      __builtin_amdgcn_sched_barrier(0);
      row_store(e0, rv);
    }
  } else {
    stats_load();
    stats_weight();
  }
  __syncthreads();

  // ---- 3. MFMA tiles (head tile ht, column tile ct); wave w takes tiles w, w + 4, ... ----
  float* dstz = zpart + (size_t)c * B * H_q * r;
  const int nht = hs16 / 16;
  constexpr int NCT = CB / 16;
  for (int tile = wave; tile < nht * NCT; tile += 4) {
    const int ht = tile / NCT, ct = tile % NCT;
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    const elem* arow = pA + (size_t)(ht * 16 + n16) * ts + q4 * EPC;
    const elem* brow = rowsT + (size_t)(ct * 16 + n16) * ts + q4 * EPC;
    for (int w0 = 0; w0 < ntp; w0 += W::WLEN) {
      const u32x4 bv = *(const u32x4*)(brow + w0);
      const u32x4 av = *(const u32x4*)(arow + w0);
#pragma unroll
      for (int st = 0; st < W::KW; ++st) acc = T::mma(chunk_frag<T>(av, st), chunk_frag<T>(bv, st), acc);
      if constexpr (T::HILO) {
        const u32x4 al = *(const u32x4*)(arow + (size_t)hs16 * ts + w0);
        acc = T::mma(chunk_frag<T>(al, 0), chunk_frag<T>(bv, 0), acc);
      }
    }
    // lane (n16, q4) holds heads ht*16 + q4*4 + i of column ct*16 + n16
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hh = ht * 16 + q4 * 4 + i;
      if (hh < HS) dstz[((size_t)b * H_q + h0 + hh) * r + cb * CB + ct * 16 + n16] = acc[i] * wsh[hh];
    }
  }
}

// One workgroup per (KV head g, 16 rows of P_v[g], column tile of (sequence, head) pairs); grid
// order: row tile fastest, then column tile, then KV head (XCD-aware), so the workgroups reading
// one column tile of z share an L2. Columns of the MFMA B operand: pairs (bf16: 8 pairs as high
// parts in columns 0..7 and low parts in 8..15; fp32: 16 pairs). Wave w takes the rank windows
// w, w + 4, ...; the four partial products are added in wave order.
template <class T, int R, int DH>
__global__ __launch_bounds__(kThreads) void value_product_kernel(
    const float* __restrict__ zpart, const typename T::elem* __restrict__ Pv, float* __restrict__ out,
    int B, int H_q, int H_kv, int nch) {
  using elem = typename T::elem;
  using W = Win<T>;
  constexpr int PC = T::HILO ? 8 : 16;
  constexpr int NWV = R / W::WLEN;
  constexpr int WPW = (NWV + 3) / 4;  // windows per wave
  constexpr int ZST = R + W::EPC;
  constexpr int NRT = DH / 16;
  constexpr int NU = PC * (R / 4);    // 16-byte units of z per column tile
  __shared__ __attribute__((aligned(16))) elem zb[16 * ZST];
  __shared__ f32x4 red[4][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n16 = lane & 15, q4 = lane >> 4;
  const int nqh = H_q / H_kv, npair = B * nqh, nct = (npair + PC - 1) / PC;
  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int rt = wg % NRT, ct = (wg / NRT) % nct, g = wg / (NRT * nct);

  const elem* prow = Pv + ((size_t)g * DH + rt * 16 + n16) * R + q4 * W::EPC;
  u32x4 pa[WPW];
#pragma unroll
  for (int i = 0; i < WPW; ++i)
    if (wave + 4 * i < NWV) pa[i] = *(const u32x4*)(prow + (wave + 4 * i) * W::WLEN);
  // z of the tile's pairs: each 16-byte unit adds its nch chunk partials in chunk order
  constexpr int UZ = 4, CK = 4;
  const size_t cstride = (size_t)B * H_q * R;
  for (int e0 = tid; e0 < NU; e0 += UZ * kThreads) {
    float acc[UZ][4];
    const float* src[UZ];
#pragma unroll
    for (int v = 0; v < UZ; ++v) {
      const int e = min(e0 + v * kThreads, NU - 1);
      const int p = min(ct * PC + e / (R / 4), npair - 1);
      src[v] = zpart + ((size_t)(p / nqh) * H_q + g * nqh + p % nqh) * R + 4 * (e % (R / 4));
#pragma unroll
      for (int m = 0; m < 4; ++m) acc[v][m] = 0.f;
    }
    for (int c0 = 0; c0 < nch; c0 += CK) {
      u32x4 x[CK][UZ];
#pragma unroll
      for (int k = 0; k < CK; ++k)
#pragma unroll
        for (int v = 0; v < UZ; ++v) x[k][v] = *(const u32x4*)(src[v] + (size_t)min(c0 + k, nch - 1) * cstride);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int k = 0; k < CK; ++k)
#pragma unroll
        for (int v = 0; v < UZ; ++v)
#pragma unroll
          for (int m = 0; m < 4; ++m) acc[v][m] += c0 + k < nch ? __uint_as_float(x[k][v][m]) : 0.f;
    }
#pragma unroll
    for (int v = 0; v < UZ; ++v) {
      const int e = e0 + v * kThreads;
      if (e < NU) {
        const int j = e / (R / 4), k4 = e % (R / 4);
        const bool live = ct * PC + j < npair;
        float x[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) x[m] = live ? acc[v][m] : 0.f;
        if constexpr (T::HILO) {
          uint32_t hi[4], lo[4];
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            hi[m] = f32_to_bf16_bits(x[m]);
            lo[m] = f32_to_bf16_bits(x[m] - bf16_bits_to_f32(hi[m]));
          }
          *(uint2*)(zb + j * ZST + 4 * k4) = make_uint2(hi[0] | hi[1] << 16, hi[2] | hi[3] << 16);
          *(uint2*)(zb + (8 + j) * ZST + 4 * k4) = make_uint2(lo[0] | lo[1] << 16, lo[2] | lo[3] << 16);
        } else {
          *(u32x4*)(zb + j * ZST + 4 * k4) = u32x4{__float_as_uint(x[0]), __float_as_uint(x[1]),
                                                  __float_as_uint(x[2]), __float_as_uint(x[3])};
        }
      }
    }
  }
  __syncthreads();
  f32x4 oc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < WPW; ++i) {
    const int w = wave + 4 * i;
    if (w < NWV) {
      const u32x4 bz = *(const u32x4*)(zb + n16 * ZST + w * W::WLEN + q4 * W::EPC);
#pragma unroll
      for (int st = 0; st < W::KW; ++st) oc = T::mma(chunk_frag<T>(pa[i], st), chunk_frag<T>(bz, st), oc);
    }
  }
  red[wave][lane] = oc;
  __syncthreads();
  if (wave != 0) return;
  oc = ((red[0][lane] + red[1][lane]) + red[2][lane]) + red[3][lane];
  // lane (n16, q4) holds rows q4*4 + i of the tile for column n16
  const int p = ct * PC + (n16 % PC);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float o = oc[i];
    if constexpr (T::HILO) o += __shfl_xor(o, 8);
    if (n16 < PC && p < npair)
      out[((size_t)(p / nqh) * H_q + g * nqh + p % nqh) * DH + rt * 16 + q4 * 4 + i] = o;
  }
}

template <class T, int DH>
bool launch_product_r(const float* zpart, const void* Pv, float* out, int B, int H_q, int H_kv,
                      int r, int nch, hipStream_t st) {
  using E = typename T::elem;
  constexpr int PC = T::HILO ? 8 : 16;
  const int nct = ((H_q / H_kv) * B + PC - 1) / PC;
  const dim3 grid(H_kv * nct * (DH / 16));
#define SALS_VP_CASE(RR)                                                                        \
  case RR:                                                                                      \
    value_product_kernel<T, RR, DH><<<grid, kThreads, 0, st>>>(zpart, (const E*)Pv, out, B, H_q, \
                                                               H_kv, nch);                    \
    return true;
  switch (r) {
    SALS_VP_CASE(32)
    SALS_VP_CASE(64)
    SALS_VP_CASE(128)
    SALS_VP_CASE(256)
    SALS_VP_CASE(384)
    SALS_VP_CASE(512)
  }
#undef SALS_VP_CASE
  return false;
}

template <class T>
size_t vs_bytes(int cb, int hs16, int cl) {
  return VSLayout<T>::bytes(cb, hs16, cl);
}

}  // namespace

bool value_plan(int dtype, int B, int H_q, int H_kv, int G, int r, int n_sel, int split_len,
                int n_splits, ValuePlan* vp) {
  const int HS = H_q / G;
  const int hs16 = (HS + 15) / 16 * 16;
  if (HS > kMaxHS || split_len < 1 || n_splits < 1 || n_sel < 1) return false;
  const int cb = r >= 64 ? 64 : 32;
  const int wl = dtype == 0 ? Win<F32>::WLEN : Win<BF16>::WLEN;  // tokens per MFMA window
  auto lds = [&](int cl) { return dtype == 0 ? vs_bytes<F32>(cb, hs16, cl) : vs_bytes<BF16>(cb, hs16, cl); };
  int cl_max = kCLMax;
  while (cl_max >= wl && lds(cl_max) > (size_t)kLdsMax) cl_max -= wl;
  if (cl_max < wl) return false;
  const long base = (long)(r / cb) * B * G * n_splits;
  int nsub = (int)((256 + base - 1) / base);
  const int cap = split_len / kMinChunk > 1 ? split_len / kMinChunk : 1;
  if (nsub > cap) nsub = cap;
  const int need = (split_len + cl_max - 1) / cl_max;
  if (nsub < need) nsub = need;
  int cl = (split_len + nsub - 1) / nsub;
  cl = (cl + wl - 1) / wl * wl;
  if (cl > cl_max) cl = cl_max;
  nsub = (split_len + cl - 1) / cl;
  const long nch = (long)n_splits * nsub;
  if (nch * (r / cb) * B * G > 0x7fffffffL) return false;
  vp->cb = cb;
  vp->nsub = nsub;
  vp->cl = cl;
  vp->nch = (int)nch;
  vp->lds = lds(cl);
  return true;
}

hipError_t launch_value_sum(int dtype, const ValuePlan& vp, const float* pbuf, const float* pstat,
                            const int32_t* sel, const int32_t* cnt, const void* Lv, float* zpart, int B,
                            int H_q, int G, int r, int ctx_cap, int n_sel, int split_len, int n_splits,
                            hipStream_t st) {
  const dim3 grid((r / vp.cb) * vp.nch * B * G);
#define SALS_VS(TT, CBV)                                                                      \
  value_sum_kernel<TT, CBV><<<grid, kThreads, vp.lds, st>>>(                                 \
      pbuf, pstat, sel, cnt, (const TT::elem*)Lv, zpart, B, H_q, G, r, ctx_cap, n_sel,        \
      split_len, n_splits, vp.nsub, vp.cl, vp.nch)
  if (dtype == 0 && vp.cb == 64) SALS_VS(F32, 64);
  else if (dtype == 0) SALS_VS(F32, 32);
  else if (vp.cb == 64) SALS_VS(BF16, 64);
  else SALS_VS(BF16, 32);
#undef SALS_VS
  return hipGetLastError();
}

hipError_t launch_value_product(int dtype, const ValuePlan& vp, const float* zpart, const void* Pv,
                                float* out, int B, int H_q, int H_kv, int d, int r, hipStream_t st) {
  bool ok = false;
  const int n = vp.nch;
  if (dtype == 0 && d == 128) ok = launch_product_r<F32, 128>(zpart, Pv, out, B, H_q, H_kv, r, n, st);
  else if (dtype == 0 && d == 64) ok = launch_product_r<F32, 64>(zpart, Pv, out, B, H_q, H_kv, r, n, st);
  else if (dtype == 1 && d == 128) ok = launch_product_r<BF16, 128>(zpart, Pv, out, B, H_q, H_kv, r, n, st);
  else if (dtype == 1 && d == 64) ok = launch_product_r<BF16, 64>(zpart, Pv, out, B, H_q, H_kv, r, n, st);
  return ok ? hipGetLastError() : hipErrorInvalidValue;
}

}  // namespace sals
