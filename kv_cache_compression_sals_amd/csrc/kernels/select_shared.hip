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
#include "../common.h"
#include "../launch.h"

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
constexpr double kTwoPi = 6.283185307179586476925286766559;

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

// grid: n_splits x (H_kv / 2) x B workgroups (XCD-aware order: the head pairs and splits of one
// sequence, which read the same rows, share an XCD).
template <int R, int NQH>
__global__ __launch_bounds__(kNT) void shared_keys_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ Lk, const uint16_t* __restrict__ Pk,
    const int32_t* __restrict__ sel, float* __restrict__ pbuf, float* __restrict__ pstat, int H_q,
    int H_kv, int G, int ctx_cap, int ctx, int n_sel, int n_splits, float rope_base) {
  constexpr int NKC = R / kKC;
  __shared__ __attribute__((aligned(16))) unsigned char smem[kLds];
  int32_t* pos = (int32_t*)(smem + kOffPos);
  float* qs = (float*)(smem + kOffQs);
  double* ftab = (double*)(smem + kOffRed);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n16 = lane & 15, q4 = lane >> 4;
  const int tg = wave >> 2, cg = wave & 3;  // token group, column group (RoPE pair of blocks)
  const int npairs = H_kv / kNH;
  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int sp = wg % n_splits, hp = (wg / n_splits) % npairs, b = wg / (n_splits * npairs);
  const int g0 = hp * kNH;
  const int s = (g0 * G) / H_kv;
  const int nqh = H_q / H_kv;
  const int j0 = sp * kTOK;
  const int n_tok = min(kTOK, n_sel - j0);
  const size_t brow = (size_t)b * ctx_cap;

  // ---- prologue: positions, RoPE frequencies, rotated and scaled queries ----
  if (tid < kDH / 2) ftab[tid] = pow((double)rope_base, -2.0 * tid / kDH) / kTwoPi;
  {
    const int32_t* selrow = sel + ((size_t)b * G + s) * n_sel + j0;
    for (int j = tid; j < kTOK; j += kNT) pos[j] = selrow[min(j, n_tok - 1)];
  }
  __syncthreads();
  const float qscale = 1.0f / sqrtf((float)kDH);
  for (int e = tid; e < kNH * nqh * (kDH / 2); e += kNT) {
    const int i = e % (kDH / 2), hh = (e / (kDH / 2)) % nqh, h2 = e / (nqh * (kDH / 2));
    const uint16_t* qp = q + ((size_t)b * H_q + (size_t)(g0 + h2) * nqh + hh) * kDH;
    const float x1 = bf16_bits_to_f32(qp[i]), x2 = bf16_bits_to_f32(qp[i + kDH / 2]);
    float sn, cs;
    rope_sincos(ctx - 1, ftab[i], &sn, &cs);
    float* dst = qs + (h2 * kMaxQH + hh) * kDH;
    dst[i] = (x1 * cs - x2 * sn) * qscale;
    dst[i + kDH / 2] = (x2 * cs + x1 * sn) * qscale;
  }

  // ---- DMA of one chunk of both operands (rank elements kc*64 .. +64) into buffer bsel ----
  // A instruction j: tile rows 8j + lane/8, piece (lane%8) ^ row; instructions past the tile
  // (padding, so that every wave issues the same number) reload a valid row into a dummy area.
  // B instruction j: P_k rows g0*d + 8j + lane/8 (the two heads' rows are consecutive).
  const int drow = lane >> 3, dx = lane & 7;
  auto issue_chunk = [&](int kc, int bsel) {
    unsigned char* abuf = smem + kOffA + bsel * kABytes;
    unsigned char* bbuf = smem + kOffB + bsel * kBBytes;
#pragma unroll
    for (int u = 0; u < kAIW; ++u) {
      const int j = wave + kWV * u;
      const int rr = min(8 * j + drow, kTOK - 1);
      const int c = dx ^ (rr & 7);
      const uint16_t* g = Lk + (brow + pos[rr]) * R + kc * kKC + c * 8;
      dma16(g, j < kAI ? abuf + j * 1024 : smem + kOffDummy);
    }
#pragma unroll
    for (int u = 0; u < kBIW; ++u) {
      const int j = wave + kWV * u;
      const int rr = 8 * j + drow;
      const int c = dx ^ (rr & 7);
      const uint16_t* g = Pk + ((size_t)g0 * kDH + rr) * R + kc * kKC + c * 8;
      dma16(g, bbuf + j * 1024);
    }
  };

  f32x4 acc[kTTW][4];
#pragma unroll
  for (int i = 0; i < kTTW; ++i)
#pragma unroll
    for (int lb = 0; lb < 4; ++lb) acc[i][lb] = f32x4{0.f, 0.f, 0.f, 0.f};
  // this wave's columns: block cg of head lb & 1 (lb < 2) and its RoPE partner cg + 4 (lb + 2)
  int brw[4];
#pragma unroll
  for (int lb = 0; lb < 4; ++lb) brw[lb] = (lb & 1) * kDH + (cg + (lb >> 1) * 4) * 16 + n16;

  __syncthreads();  // pos visible to every wave before the first DMA addresses are formed
  issue_chunk(0, 0);
  for (int kc = 0; kc < NKC; ++kc) {
    // this wave's copies of chunk kc have landed; after the barrier every wave's have, and every
    // wave has finished multiplying chunk kc - 1, whose buffer the next copies overwrite
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    if (kc + 1 < NKC) issue_chunk(kc + 1, (kc + 1) & 1);
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
            acc[i0 + i][lb] = BF16::mma(chunk_frag<BF16>(af[i], 0), chunk_frag<BF16>(bf[lb], 0), acc[i0 + i][lb]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
  }
  __syncthreads();  // the chunk buffers are free: the first one holds the partial logits

  // ---- RoPE at the tokens' positions, partial logits over this wave's 64 columns ----
  float* lgp = (float*)(smem + kOffA);  // [cg][head][hh][token]
  const double frev = ftab[cg * 16 + n16];
  float qv[NQH][4];
#pragma unroll
  for (int hh = 0; hh < NQH; ++hh)
#pragma unroll
    for (int lb = 0; lb < 4; ++lb)
      qv[hh][lb] = qs[((lb & 1) * kMaxQH + min(hh, nqh - 1)) * kDH + (brw[lb] - (lb & 1) * kDH)];
#pragma unroll
  for (int i = 0; i < kTTW; ++i) {
    const int tt = tg * kTTW + i;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float sn, cs;
      rope_sincos(pos[tt * 16 + q4 * 4 + e], frev, &sn, &cs);
#pragma unroll
      for (int lb = 0; lb < 2; ++lb) {
        const float x1 = acc[i][lb][e], x2 = acc[i][lb + 2][e];
        acc[i][lb][e] = x1 * cs - x2 * sn;
        acc[i][lb + 2][e] = x2 * cs + x1 * sn;
      }
    }
#pragma unroll
    for (int h2 = 0; h2 < kNH; ++h2)
#pragma unroll
      for (int hh = 0; hh < NQH; ++hh) {
        float pl[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          pl[e] = row16_sum(fmaf(qv[hh][h2], acc[i][h2][e], qv[hh][h2 + 2] * acc[i][h2 + 2][e]));
        if (n16 == 0 && hh < nqh) {
#pragma unroll
          for (int e = 0; e < 4; ++e) lgp[((cg * kNH + h2) * kMaxQH + hh) * kTOK + tt * 16 + q4 * 4 + e] = pl[e];
        }
      }
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

hipError_t launch_shared_keys(const void* q, const void* Lk, const void* Pk, const int32_t* sel,
                              float* pbuf, float* pstat, int B, int H_q, int H_kv, int G, int r,
                              int ctx_cap, int ctx, int n_sel, int n_splits, float rope_base,
                              hipStream_t st, hipEvent_t t_start, hipEvent_t t_stop) {
  const dim3 grid(n_splits * (H_kv / kNH) * B);
  const int nqh = H_q / H_kv;
  const auto* qq = (const uint16_t*)q;
  const auto* lk = (const uint16_t*)Lk;
  const auto* pk = (const uint16_t*)Pk;
#define SALS_SK(RR, QQ)                                                                              \
  if (t_start)                                                                                       \
    hipExtLaunchKernelGGL(shared_keys_kernel<RR, QQ>, grid, dim3(kNT), 0, st, t_start, t_stop, 0, qq, lk, \
                          pk, sel, pbuf, pstat, H_q, H_kv, G, ctx_cap, ctx, n_sel, n_splits, rope_base);  \
  else                                                                                               \
    shared_keys_kernel<RR, QQ><<<grid, kNT, 0, st>>>(qq, lk, pk, sel, pbuf, pstat, H_q, H_kv, G,       \
                                                     ctx_cap, ctx, n_sel, n_splits, rope_base)
#define SALS_SK_R(RR) \
  if (nqh <= 1) {     \
    SALS_SK(RR, 1);   \
  } else {            \
    SALS_SK(RR, 4);   \
  }
  switch (r) {
    case 128: SALS_SK_R(128) break;
    case 256: SALS_SK_R(256) break;
    case 384: SALS_SK_R(384) break;
    case 512: SALS_SK_R(512) break;
    default: return hipErrorInvalidValue;
  }
#undef SALS_SK_R
#undef SALS_SK
  return hipGetLastError();
}

}  // namespace sals
