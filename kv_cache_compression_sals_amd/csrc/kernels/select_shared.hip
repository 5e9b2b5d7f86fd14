// Key side of the attention when one selection serves several KV heads (SALS 技术框架 stages 3-4,
// 关键创新 3; 问题定义: RoPE after the rebuild, at true positions), bf16 cache, d = 128.
//
// With a shared selection the rebuild of all KV heads of a group is one dense product per
// sequence, L_k,sel [n_sel x r] . P_k^T [r x (heads x d)]. A workgroup computes one tile of it:
// 288 selected tokens x 2 KV heads (256 columns), so that the bytes a CU must pull in (the
// tokens' latent rows and the two heads' P_k rows, 544 KB at r = 512) are about a quarter fewer
// than one KV head over all tokens, and both operands stream the same way: the rank is cut into
// chunks of 64 (128 bytes of every row), and each chunk of both operands is copied into LDS by
// the global->LDS DMA while the previous one is multiplied. A DMA wave instruction fetches 8 rows
// x 128 bytes (whole lines); the 16-byte pieces of a row are placed at (piece XOR row) so that
// the MFMA fragment reads of 16 rows hit 8 different bank groups. Eight waves (two per SIMD)
// split the tile as 2 token groups x 4 column groups: a wave owns 9 token tiles x 4 column
// blocks in 144 accumulator registers, namely the RoPE pair of blocks (c, c + 4) of both heads,
// so that one sine/cosine serves both heads.
//
// After the last chunk each wave rotates its columns at the tokens' positions (hardware sin/cos
// of an fp64-reduced angle), forms partial logits of both heads' query heads over its 32 columns
// of each, and the four column groups are added in a fixed order. The softmax over the tile's
// tokens (one split) ends the kernel: exp(logit - m) per query head and token, and (m, l) per
// split, for the shared-selection value kernels, as in select_attend's shared-selection mode.
//
// For rows of at most 4096 candidates the kernel also makes the selection (SALS 关键设计 items 2
// and 4): every workgroup ranks its own sequence's score row with the register-resident row
// routine (topk_rows.h), its keys staged in the token buffers before their first use, while the
// first chunk's P_k rows are already being copied. All workgroups of a sequence rank the same
// row, so none waits for another and the top-k needs no launch of its own.
#include "../common.h"
#include "../launch.h"
#include "../topk_rows.h"

namespace sals {
namespace {

constexpr int kWV = 8;               // waves
constexpr int kNT = kWV * 64;        // threads
constexpr int kTT = 18;              // token tiles per workgroup
constexpr int kTOK = kTT * 16;       // 288 tokens
constexpr int kTTW = kTT / 2;        // token tiles per wave
constexpr int kDH = 128;
constexpr int kNH = 2;               // KV heads per workgroup
constexpr int kRows = kNH * kDH;     // P_k rows per workgroup
constexpr int kKC = 64;              // rank elements per chunk: 128 bytes of a row
constexpr int kAI = kTOK / 8;        // A (token rows) DMA instructions per chunk: 36
constexpr int kAIW = (kAI + kWV - 1) / kWV;  // per wave, padded: 5
constexpr int kBIW = kRows / 8 / kWV;        // B (P rows) per wave: 4
constexpr int kMaxQH = 4;
constexpr int kRankKPT = 8;          // keys per thread when the kernel ranks its own row
constexpr int kRankMax = kNT * kRankKPT;  // longest row it ranks
constexpr double kInvTwoPi = 0.15915494309189533576888376337251;

// LDS layout (bytes)
constexpr int kABytes = kTOK * 128;
constexpr int kBBytes = kRows * 128;
constexpr int kOffA = 0;                          // A[2]
constexpr int kOffB = kOffA + 2 * kABytes;        // B[2]
constexpr int kOffDummy = kOffB + 2 * kBBytes;    // target of the padding DMA instructions
constexpr int kOffPos = kOffDummy + 1024;         // int32 pos[kTOK]
constexpr int kOffQs = kOffPos + kTOK * 4;        // float qs[kNH][kMaxQH][kDH]
constexpr int kOffRed = kOffQs + kNH * kMaxQH * kDH * 4;  // double ftab[kDH / 2]
constexpr int kLds = kOffRed + kDH / 2 * 8;
static_assert(kLds <= 160 * 1024, "LDS");
static_assert(4 * kNH * kMaxQH * kTOK * 4 <= kABytes, "partial logits reuse the first A buffer");
static_assert(tk::topk_ext_words(kNT, kRankKPT) * 4 <= 2 * kABytes, "the row ranking uses the A buffers");

typedef __attribute__((address_space(3))) void* lds_ptr;

// 16 bytes from each lane's global address to LDS, lane i at lds + 16 i (gfx950 DMA).
__device__ __forceinline__ void dma16(const void* g, unsigned char* lds) {
  __builtin_amdgcn_global_load_lds(g, (lds_ptr)lds, 16, 0, 0);
}

// LDS byte offset of 16-byte piece c of row rr in a chunk buffer (rows of 128 bytes).
__device__ __forceinline__ int piece_off(int rr, int c) { return rr * 128 + ((c ^ (rr & 7)) << 4); }

__device__ __forceinline__ void rope_sincos(int pos, double frev, float* s, float* c) {
  double rv = (double)pos * frev;
  rv -= rint(rv);
  const float r = (float)rv;
  *s = __builtin_amdgcn_sinf(r);
  *c = __builtin_amdgcn_cosf(r);
}

// grid: n_splits x (H_kv / 2) x B workgroups (XCD-aware order: each XCD takes a block of
// (sequence, split) pairs x head pairs, whose token rows and P_k rows it reads several times).
// RANK: the selection is not given; every workgroup ranks its sequence's score row itself (the
// top kp of Tc scores, ties to the lowest position, then the window [Tc, ctx)), with no other
// workgroup to wait for, and the first workgroup of each (sequence, selection group) writes the
// whole selection to sel for the value kernels and the caller.
template <int R, int NQH, bool RANK>
__global__ __launch_bounds__(kNT) void shared_keys_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ Lk, const uint16_t* __restrict__ Pk,
    int32_t* __restrict__ sel, const int32_t* __restrict__ cnt, float* __restrict__ pbuf,
    float* __restrict__ pstat, int H_q, int H_kv, int G, int ctx_cap, int ctx, int n_sel, int n_splits,
    double rope_r, const float* __restrict__ S, int ldS, int Tc, int kp) {
  constexpr int NKC = R / kKC;
  __shared__ __attribute__((aligned(16))) unsigned char smem[kLds];
  int32_t* pos = (int32_t*)(smem + kOffPos);
  float* qs = (float*)(smem + kOffQs);
  double* ftab = (double*)(smem + kOffRed);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n16 = lane & 15, q4 = lane >> 4;
  const int tg = wave >> 2, cg = wave & 3;  // token group, column group (RoPE pair of blocks)
  const int npairs = H_kv / kNH;
  // logical order: groups of up to 8 head pairs, (sequence, split) pairs within a group, head
  // pairs fastest; XCD-aware, so an XCD takes a block of a few (sequence, split) pairs x up to 8
  // head pairs and its L2 serves both the token rows (shared by the head pairs) and the P_k rows
  // (shared by the sequences and splits)
  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int nbs = (int)(gridDim.x / npairs);  // (sequence, split) pairs
  const int GH = npairs < 8 ? npairs : 8;
  const int grp = wg / (GH * nbs);
  const int gh = min(GH, npairs - grp * GH);  // head pairs of this group
  const int within = wg - grp * GH * nbs;
  const int hp = grp * GH + within % gh, bsp = within / gh;
  const int sp = bsp % n_splits, b = bsp / n_splits;
  const int g0 = hp * kNH;
  const int s = (g0 * G) / H_kv;
  const int nqh = H_q / H_kv;
  const int j0 = sp * kTOK;
  // a thresholded (ragged) selection has its own count per row; a split past it holds no token
  // and leaves neutral split statistics (m = -inf, l = 0)
  const int n_row = cnt ? cnt[(size_t)b * G + s] : n_sel;
  const int n_tok = min(kTOK, n_row - j0);
  if (n_tok <= 0) {
    if (tid < kNH * nqh) {
      float* ps = pstat + (((size_t)b * H_q + (g0 + tid / nqh) * nqh + tid % nqh) * n_splits + sp) * 2;
      ps[0] = -INFINITY;
      ps[1] = 0.f;
    }
    return;
  }
  const size_t brow = (size_t)b * ctx_cap;

  // ---- DMA of one chunk of both operands (rank elements kc*64 .. +64) into buffer bsel ----
  // A instruction j: tile rows 8j + lane/8, piece (lane%8) ^ row; instructions past the tile
  // (padding, so that every wave issues the same number) reload a valid row into a dummy area.
  // B instruction j: P_k rows g0*d + 8j + lane/8 (the two heads' rows are consecutive).
  const int drow = lane >> 3, dx = lane & 7;
  auto issue_a = [&](int kc, int bsel) {
    unsigned char* abuf = smem + kOffA + bsel * kABytes;
#pragma unroll
    for (int u = 0; u < kAIW; ++u) {
      const int j = wave + kWV * u;
      const int rr = min(8 * j + drow, kTOK - 1);
      const int c = dx ^ (rr & 7);
      const uint16_t* g = Lk + (brow + pos[rr]) * R + kc * kKC + c * 8;
      dma16(g, j < kAI ? abuf + j * 1024 : smem + kOffDummy);
    }
  };
  auto issue_b = [&](int kc, int bsel) {
    unsigned char* bbuf = smem + kOffB + bsel * kBBytes;
#pragma unroll
    for (int u = 0; u < kBIW; ++u) {
      const int j = wave + kWV * u;
      const int rr = 8 * j + drow;
      const int c = dx ^ (rr & 7);
      const uint16_t* g = Pk + ((size_t)g0 * kDH + rr) * R + kc * kKC + c * 8;
      dma16(g, bbuf + j * 1024);
    }
  };
  // ---- prologue: positions, RoPE frequencies, rotated and scaled queries ----
  // The positions and this thread's query pair are loaded together, and every LDS write of the
  // prologue happens before the first copy is issued (the compiler makes an LDS write wait for
  // every global->LDS copy in flight). The first chunk's P_k rows (independent of the selection)
  // are then requested, its token rows as soon as the positions are visible to every wave.
  const int32_t* selrow = sel + ((size_t)b * G + s) * n_sel + j0;
  static_assert(kTOK <= kNT && kNH * kMaxQH * (kDH / 2) <= kNT, "one position and one query pair per thread");
  int pv = 0;
  if constexpr (!RANK) {
    if (tid < kTOK) pv = selrow[min(tid, n_tok - 1)];
  }
  const int qi = lane, qhh = wave % nqh, qh2 = wave / nqh;  // this thread's query pair (i, i + d/2)
  const bool qlive = tid < kNH * nqh * (kDH / 2);
  float x1 = 0.f, x2 = 0.f;
  if (qlive) {
    const uint16_t* qp = q + ((size_t)b * H_q + (size_t)(g0 + qh2) * nqh + qhh) * kDH;
    x1 = bf16_bits_to_f32(qp[qi]);
    x2 = bf16_bits_to_f32(qp[qi + kDH / 2]);
  }
  // theta_i / (2 pi) = rope_r^i / (2 pi) with rope_r = base^(-2/d) from the host: six fp64
  // squarings and products (relative error ~1e-15) instead of a pow per thread
  double frq = 1.0;
  {
    double bb = rope_r;
#pragma unroll
    for (int t = 0; t < 6; ++t) {
      if ((lane >> t) & 1) frq *= bb;
      bb *= bb;
    }
    frq *= kInvTwoPi;
  }
  if constexpr (RANK) {
    // the first chunk's P_k rows do not depend on the selection: requested before the ranking,
    // which stages its keys in the A buffers (free until the first token rows are copied)
    issue_b(0, 0);
    uint32_t* ext = (uint32_t*)(smem + kOffA);
    const bool ranked = kp > 0 && kp < Tc;
    if (ranked) {
      const float* srow = S + ((size_t)b * G + s) * ldS;
      const bool vec = (ldS & 3) == 0 && ((uintptr_t)S & 15) == 0;
      tk::topk_rows<kNT, kRankKPT, false, true>(srow, nullptr, nullptr, Tc, kp, nullptr, nullptr, 0, 0, 0, vec,
                                                false, 0u, nullptr, 0, nullptr, nullptr, 0, ext);
    }
    const int32_t* ranks = (const int32_t*)ext;  // ascending positions of the top kp
    auto position = [&](int j) { return j < kp ? (ranked ? ranks[j] : j) : Tc + (j - kp); };
    if (tid < kTOK) pv = position(j0 + min(tid, n_tok - 1));
    if (sp == 0 && g0 * G == s * H_kv) {
      int32_t* srow_out = sel + ((size_t)b * G + s) * n_sel;
      for (int j = tid; j < n_sel; j += kNT) srow_out[j] = position(j);
    }
  }
  if (tid < kDH / 2) ftab[tid] = frq;
  if (tid < kTOK) pos[tid] = pv;
  if (qlive) {
    const float qscale = 1.0f / sqrtf((float)kDH);
    float sn, cs;
    rope_sincos(ctx - 1, frq, &sn, &cs);
    float* dst = qs + (qh2 * kMaxQH + qhh) * kDH;
    dst[qi] = (x1 * cs - x2 * sn) * qscale;
    dst[qi + kDH / 2] = (x2 * cs + x1 * sn) * qscale;
  }
  if constexpr (!RANK) issue_b(0, 0);
  lds_barrier();  // pos visible to every wave, the ranking's LDS reads done; the copies stay in flight
  issue_a(0, 0);

  f32x4 acc[kTTW][4];
#pragma unroll
  for (int i = 0; i < kTTW; ++i)
#pragma unroll
    for (int lb = 0; lb < 4; ++lb) acc[i][lb] = f32x4{0.f, 0.f, 0.f, 0.f};
  // this wave's columns: block cg of head lb & 1 (lb < 2) and its RoPE partner cg + 4 (lb + 2)
  int brw[4];
#pragma unroll
  for (int lb = 0; lb < 4; ++lb) brw[lb] = (lb & 1) * kDH + (cg + (lb >> 1) * 4) * 16 + n16;

  for (int kc = 0; kc < NKC; ++kc) {
    // this wave's copies of chunk kc have landed; after the barrier every wave's have, and every
    // wave has finished multiplying chunk kc - 1, whose buffer the next copies overwrite
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    if (kc + 1 < NKC) {
      issue_a(kc + 1, (kc + 1) & 1);
      issue_b(kc + 1, (kc + 1) & 1);
    }
    const unsigned char* abuf = smem + kOffA + (kc & 1) * kABytes;
    const unsigned char* bbuf = smem + kOffB + (kc & 1) * kBBytes;
#pragma unroll
    for (int wi = 0; wi < 2; ++wi) {
      const int c = 4 * wi + q4;
      u32x4 bf[4];
#pragma unroll
      for (int lb = 0; lb < 4; ++lb) bf[lb] = *(const u32x4*)(bbuf + piece_off(brw[lb], c));
      // A fragments three tiles at a time (registers: the accumulators take 144)
#pragma unroll
      for (int i0 = 0; i0 < kTTW; i0 += 3) {
        u32x4 af[3];
#pragma unroll
        for (int i = 0; i < 3; ++i) af[i] = *(const u32x4*)(abuf + piece_off((tg * kTTW + i0 + i) * 16 + n16, c));
#pragma unroll
        for (int i = 0; i < 3; ++i)
#pragma unroll
          for (int lb = 0; lb < 4; ++lb)
            acc[i0 + i][lb] = BF16::mma(chunk_frag<BF16>(bf[lb], 0), chunk_frag<BF16>(af[i], 0), acc[i0 + i][lb]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
  }
  __syncthreads();  // the chunk buffers are free: the first one holds the partial logits

  // ---- RoPE at the tokens' positions, partial logits over this wave's 64 columns ----
  // acc[i][lb] holds K rows 4 q4 .. 4 q4 + 3 of column block lb for token tt * 16 + n16 (P_k is
  // the MFMA's first operand), so the RoPE pairs (c, c + 64) and the query products are in-lane;
  // only the sum over the four lane rows (q4) crosses lanes.
  float* lgp = (float*)(smem + kOffA);  // [cg][head][hh][token]
  const int c0 = cg * 16 + 4 * q4;      // first RoPE pair index of this lane (0..63)
  double frev[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) frev[e] = ftab[c0 + e];
  constexpr int NV = kTTW * kNH * NQH;  // partial logits per lane: (tile, head, query head)
  constexpr int NPT = kNH * NQH;        // per tile
  float part[NV];
  // this lane's token in tile i of the wave: tg * kTTW * 16 + i * 16 + n16
  const int32_t* posw = pos + tg * kTTW * 16 + n16;
  float* lgw = lgp + tg * kTTW * 16 + n16;
  // sum of values 4j .. 4j + 3 over the four lane rows, by two transposing swaps: lane row 0 then
  // holds the total of value 4j, row 1 of 4j + 2, row 2 of 4j + 1, row 3 of 4j + 3
  auto flush = [&](int j) {
    float v4[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v4[u] = 4 * j + u < NV ? part[4 * j + u] : 0.f;
    const float t = xor16_pair_sum(xor32_pair_sum(v4[0], v4[1]), xor32_pair_sum(v4[2], v4[3]));
    const int vi = 4 * j + ((q4 & 1) << 1) + (q4 >> 1);
    const int i = vi / NPT, h2 = (vi / NQH) % kNH, hh = vi % NQH;
    if (vi < NV && hh < nqh) lgw[((cg * kNH + h2) * kMaxQH + hh) * kTOK + i * 16] = t;
  };
#pragma unroll
  for (int i = 0; i < kTTW; ++i) {
    const double pd = (double)posw[i * 16];
#pragma unroll
    for (int v = 0; v < NPT; ++v) part[i * NPT + v] = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      double rv = pd * frev[e];
      rv -= rint(rv);
      const float sn = __builtin_amdgcn_sinf((float)rv), cs = __builtin_amdgcn_cosf((float)rv);
#pragma unroll
      for (int h2 = 0; h2 < kNH; ++h2) {
        const float x1 = acc[i][h2][e], x2 = acc[i][h2 + 2][e];
        const float r1 = x1 * cs - x2 * sn, r2 = x2 * cs + x1 * sn;
#pragma unroll
        for (int hh = 0; hh < NQH; ++hh) {
          const float* qh = qs + (h2 * kMaxQH + min(hh, nqh - 1)) * kDH + c0 + e;
          float& pv = part[(i * kNH + h2) * NQH + hh];
          pv = fmaf(qh[0], r1, fmaf(qh[kDH / 2], r2, pv));
        }
      }
    }
    // groups completed by this tile (the last, partial one after the last tile)
#pragma unroll
    for (int j = (i * NPT) / 4; j < ((i + 1) * NPT) / 4; ++j) flush(j);
    if (i == kTTW - 1 && NV % 4) flush(NV / 4);
  }
  __syncthreads();

  // ---- softmax over the split per query head: one wave per (head, query head) row ----
  const int nrows = kNH * nqh;
  const int nsp = (n_sel + 3) & ~3;
  for (int row = wave; row < nrows; row += kWV) {
    const int h2 = row / nqh, hh = row % nqh;
    constexpr int PL = (kTOK + 63) / 64;
    float x[PL];
    float m = -INFINITY;
#pragma unroll
    for (int u = 0; u < PL; ++u) {
      const int j = lane + 64 * u;
      float v = -INFINITY;
      if (j < n_tok) {  // the four column groups, in order
        v = lgp[((0 * kNH + h2) * kMaxQH + hh) * kTOK + j] + lgp[((1 * kNH + h2) * kMaxQH + hh) * kTOK + j];
        v = v + lgp[((2 * kNH + h2) * kMaxQH + hh) * kTOK + j];
        v = v + lgp[((3 * kNH + h2) * kMaxQH + hh) * kTOK + j];
      }
      x[u] = v;
      m = fmaxf(m, x[u]);
    }
    m = wave_max(m);
    float l = 0.f;
    const int h = (g0 + h2) * nqh + hh;
    float* prow = pbuf + ((size_t)b * H_q + h) * nsp + j0;
#pragma unroll
    for (int u = 0; u < PL; ++u) {
      const int j = lane + 64 * u;
      if (j < n_tok) {
        const float ev = expf(x[u] - m);
        prow[j] = ev;
        l += ev;
      }
    }
    l = wave_sum(l);
    if (lane == 0) {
      float* ps = pstat + (((size_t)b * H_q + h) * n_splits + sp) * 2;
      ps[0] = m;
      ps[1] = l;
    }
  }
}

}  // namespace

bool shared_keys_supported(int dtype, int H_q, int H_kv, int G, int d, int r) {
  const int nqh = H_q / H_kv;
  return dtype == 1 && d == kDH && (H_kv / G) % kNH == 0 && nqh >= 1 && nqh <= kMaxQH &&
         (r == 128 || r == 256 || r == 384 || r == 512);
}

int shared_keys_split() { return kTOK; }

int shared_keys_rank_max() { return kRankMax; }

hipError_t launch_shared_keys(const void* q, const void* Lk, const void* Pk, int32_t* sel,
                              const int32_t* cnt, float* pbuf, float* pstat, int B, int H_q, int H_kv, int G, int r,
                              int ctx_cap, int ctx, int n_sel, int n_splits, float rope_base,
                              hipStream_t st, hipEvent_t t_start, hipEvent_t t_stop, const float* S,
                              int ldS, int Tc, int kp) {
  const dim3 grid(n_splits * (H_kv / kNH) * B);
  const int nqh = H_q / H_kv;
  const double rope_r = pow((double)rope_base, -2.0 / kDH);  // theta_i = rope_r^i
  const auto* qq = (const uint16_t*)q;
  const auto* lk = (const uint16_t*)Lk;
  const auto* pk = (const uint16_t*)Pk;
  const bool rank = S != nullptr;
  if (rank && (cnt || Tc > kRankMax || Tc < 0 || kp < 0 || n_sel != min(kp, Tc) + (ctx - Tc)))
    return hipErrorInvalidValue;
#define SALS_SK(RR, QQ, RK)                                                                             \
  if (t_start)                                                                                          \
    hipExtLaunchKernelGGL(shared_keys_kernel<RR, QQ, RK>, grid, dim3(kNT), 0, st, t_start, t_stop, 0, qq, lk, \
                          pk, sel, cnt, pbuf, pstat, H_q, H_kv, G, ctx_cap, ctx, n_sel, n_splits, rope_r, S,  \
                          ldS, Tc, kp);                                                                 \
  else                                                                                                  \
    shared_keys_kernel<RR, QQ, RK><<<grid, kNT, 0, st>>>(qq, lk, pk, sel, cnt, pbuf, pstat, H_q, H_kv, G,     \
                                                         ctx_cap, ctx, n_sel, n_splits, rope_r, S, ldS, Tc, kp)
#define SALS_SK_Q(RR, QQ) \
  if (rank) {             \
    SALS_SK(RR, QQ, true); \
  } else {                \
    SALS_SK(RR, QQ, false); \
  }
#define SALS_SK_R(RR)  \
  if (nqh <= 1) {      \
    SALS_SK_Q(RR, 1);  \
  } else {             \
    SALS_SK_Q(RR, 4);  \
  }
  switch (r) {
    case 128: SALS_SK_R(128) break;
    case 256: SALS_SK_R(256) break;
    case 384: SALS_SK_R(384) break;
    case 512: SALS_SK_R(512) break;
    default: return hipErrorInvalidValue;
  }
#undef SALS_SK_R
#undef SALS_SK_Q
#undef SALS_SK
  return hipGetLastError();
}

}  // namespace sals
