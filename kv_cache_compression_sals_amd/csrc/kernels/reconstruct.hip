// Full reconstruction of a latent cache range (the dense baseline that SALS avoids: its 问题定义
// and abstract describe rebuilding the whole low-rank cache so that RoPE can be applied, which
// turns the rebuild into the decode bottleneck; 技术框架 stage 3 rebuilds only the selected rows).
//   K[b, g, t, :] = RoPE_t(L_k[b, t, :] . P_k[g]^T),   V[b, g, t, :] = L_v[b, t, :] . P_v[g]^T
// for t in [t0, t0 + T), bf16 cache, d = 128, fp32 accumulation, one rounding to bf16 (nearest
// even) at the end. The output is a plain post-RoPE KV cache [B, H_kv, stride_tokens, d], which
// sals_dense_decode attends over.
//
// It is one dense product per sequence and tensor, L [T x r] . P^T [r x D]. A workgroup computes
// a tile of 256 consecutive tokens x 2 KV heads (256 columns). The rank is cut into chunks of 64
// (128 bytes of every row); each chunk of both operands is copied into LDS by the global->LDS DMA
// (a wave instruction fetches 8 whole 128-byte lines) while the previous one is multiplied, its
// 16-byte pieces at (piece XOR row) so that the fragment reads of 16 rows hit 8 different bank
// groups. Eight waves split the tile as 2 token groups x 4 column groups; a wave owns 8 token
// tiles x the RoPE pair of column blocks (c, c + 4) of both heads (128 accumulator registers),
// so that one sine/cosine per token serves both heads. The rotated tile is rounded to bf16,
// staged in LDS (rows padded against bank conflicts) and written as whole 256-byte head rows.
#include "../common.h"
#include "../launch.h"

namespace sals {
namespace {

constexpr int kWV = 8;
constexpr int kNT = kWV * 64;
constexpr int kTT = 16;              // token tiles per workgroup
constexpr int kTOK = kTT * 16;       // 256 tokens
constexpr int kTTW = kTT / 2;        // token tiles per wave
constexpr int kDH = 128;
constexpr int kNH = 2;               // KV heads per workgroup
constexpr int kRows = kNH * kDH;     // P rows per workgroup
constexpr int kKC = 64;              // rank elements per chunk
constexpr int kAIW = kTOK / 8 / kWV;   // A copy instructions per wave and chunk: 4
constexpr int kBIW = kRows / 8 / kWV;  // B copy instructions per wave and chunk: 4
constexpr double kTwoPi = 6.283185307179586476925286766559;

constexpr int kABytes = kTOK * 128;
constexpr int kBBytes = kRows * 128;
constexpr int kOffA = 0;
constexpr int kOffB = kOffA + 2 * kABytes;
constexpr int kChunkEnd = kOffB + 2 * kBBytes;       // 128 KB
constexpr int kOutRow = kDH * 2 + 16;                 // staged output row: 256 bytes + padding
constexpr int kOutEnd = kNH * kTOK * kOutRow;         // 139264 bytes
constexpr int kOffF = kOutEnd > kChunkEnd ? kOutEnd : kChunkEnd;  // double ftab[kDH / 2]
constexpr int kLds = kOffF + kDH / 2 * 8;
static_assert(kLds <= 160 * 1024, "LDS");

typedef __attribute__((address_space(3))) void* lds_ptr;

__device__ __forceinline__ void dma16(const void* g, unsigned char* lds) {
  __builtin_amdgcn_global_load_lds(g, (lds_ptr)lds, 16, 0, 0);
}

__device__ __forceinline__ int piece_off(int rr, int c) { return rr * 128 + ((c ^ (rr & 7)) << 4); }

// sin and cos of 2 pi * pos * frev (frev = theta / 2 pi), the angle reduced in fp64
__device__ __forceinline__ void rope_sincos(int pos, double frev, float* s, float* c) {
  double rv = (double)pos * frev;
  rv -= rint(rv);
  const float r = (float)rv;
  *s = __builtin_amdgcn_sinf(r);
  *c = __builtin_amdgcn_cosf(r);
}

// grid: 2 tensors x B x n_tiles x (H_kv / 2), head pair fastest (XCD-aware order: the workgroups
// that read one token tile's latent rows share an XCD). Tensor 0 is K (rotated), 1 is V.
template <int R>
__global__ __launch_bounds__(kNT) void reconstruct_kernel(
    const uint16_t* __restrict__ Lk, const uint16_t* __restrict__ Lv, const uint16_t* __restrict__ Pk,
    const uint16_t* __restrict__ Pv, uint16_t* __restrict__ Ko, uint16_t* __restrict__ Vo, int B,
    int H_kv, int ctx_cap, int t0, int T, int stride_tokens, int n_tiles, int ntens, float rope_base) {
  constexpr int NKC = R / kKC;
  __shared__ __attribute__((aligned(16))) unsigned char smem[kLds];
  double* ftab = (double*)(smem + kOffF);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n16 = lane & 15, q4 = lane >> 4;
  const int tg = wave >> 2, cg = wave & 3;
  const int npairs = H_kv / kNH;
  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int hp = wg % npairs, tile = (wg / npairs) % n_tiles, b = (wg / (npairs * n_tiles)) % B;
  const int tensor = ntens == 1 ? 0 : wg / (npairs * n_tiles * B);
  const bool rope = tensor == 0;
  const uint16_t* L = rope ? Lk : Lv;
  const uint16_t* P = rope ? Pk : Pv;
  uint16_t* O = rope ? Ko : Vo;
  const int g0 = hp * kNH;
  const int j0 = tile * kTOK;                 // first token of the tile, relative to t0
  const int n_tok = min(kTOK, T - j0);
  const size_t row0 = (size_t)b * ctx_cap + t0 + j0;

  if (tid < kDH / 2) ftab[tid] = pow((double)rope_base, -2.0 * tid / kDH) / kTwoPi;

  const int drow = lane >> 3, dx = lane & 7;
  auto issue_chunk = [&](int kc, int bsel) {
    unsigned char* abuf = smem + kOffA + bsel * kABytes;
    unsigned char* bbuf = smem + kOffB + bsel * kBBytes;
#pragma unroll
    for (int u = 0; u < kAIW; ++u) {
      const int j = wave + kWV * u;
      const int rr = 8 * j + drow;
      const int c = dx ^ (rr & 7);
      // rows past the range repeat its last row; their results are never stored
      const uint16_t* g = L + (row0 + min(rr, n_tok - 1)) * R + kc * kKC + c * 8;
      dma16(g, abuf + j * 1024);
    }
#pragma unroll
    for (int u = 0; u < kBIW; ++u) {
      const int j = wave + kWV * u;
      const int rr = 8 * j + drow;
      const int c = dx ^ (rr & 7);
      const uint16_t* g = P + ((size_t)g0 * kDH + rr) * R + kc * kKC + c * 8;
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
#pragma unroll
      for (int i0 = 0; i0 < kTTW; i0 += 4) {
        u32x4 af[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) af[i] = *(const u32x4*)(abuf + piece_off((tg * kTTW + i0 + i) * 16 + n16, c));
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int lb = 0; lb < 4; ++lb)
            acc[i0 + i][lb] = BF16::mma(chunk_frag<BF16>(af[i], 0), chunk_frag<BF16>(bf[lb], 0), acc[i0 + i][lb]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
  }
  __syncthreads();  // every wave is done with the chunk buffers: they take the staged output

  // ---- RoPE at the tokens' positions (K only), bf16 rounding, staging [head][token][column] ----
  const double frev = ftab[cg * 16 + n16];
#pragma unroll
  for (int i = 0; i < kTTW; ++i) {
    const int tt = tg * kTTW + i;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int tok = tt * 16 + q4 * 4 + e;
      if (rope) {
        float sn, cs;
        rope_sincos(t0 + j0 + tok, frev, &sn, &cs);
#pragma unroll
        for (int lb = 0; lb < 2; ++lb) {
          const float x1 = acc[i][lb][e], x2 = acc[i][lb + 2][e];
          acc[i][lb][e] = x1 * cs - x2 * sn;
          acc[i][lb + 2][e] = x2 * cs + x1 * sn;
        }
      }
#pragma unroll
      for (int lb = 0; lb < 4; ++lb) {
        const int h2 = lb & 1, col = brw[lb] - h2 * kDH;
        *(uint16_t*)(smem + (h2 * kTOK + tok) * kOutRow + col * 2) = (uint16_t)f32_to_bf16_bits(acc[i][lb][e]);
      }
    }
  }
  __syncthreads();

  // ---- whole head rows out: 16 lanes x 16 bytes per (head, token) ----
  for (int e = tid; e < kNH * n_tok * 16; e += kNT) {
    const int piece = e & 15, tok = (e >> 4) % n_tok, h2 = (e >> 4) / n_tok;
    const u32x4 v = *(const u32x4*)(smem + (h2 * kTOK + tok) * kOutRow + piece * 16);
    *(u32x4*)(O + (((size_t)b * H_kv + g0 + h2) * stride_tokens + t0 + j0 + tok) * kDH + piece * 8) = v;
  }
}

// The query rotated at one position, q_rot[b, h] = RoPE_pos(q[b, h]) rounded to bf16: one thread
// per (sequence, head, rotation pair).
__global__ __launch_bounds__(256) void rope_query_kernel(const uint16_t* __restrict__ q,
                                                         uint16_t* __restrict__ q_rot, int rows,
                                                         int pos, float rope_base) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= rows * (kDH / 2)) return;
  const int row = e / (kDH / 2), i = e % (kDH / 2);
  const double frev = pow((double)rope_base, -2.0 * i / kDH) / kTwoPi;
  float sn, cs;
  rope_sincos(pos, frev, &sn, &cs);
  const uint16_t* src = q + (size_t)row * kDH;
  const float x1 = bf16_bits_to_f32(src[i]), x2 = bf16_bits_to_f32(src[i + kDH / 2]);
  q_rot[(size_t)row * kDH + i] = (uint16_t)f32_to_bf16_bits(x1 * cs - x2 * sn);
  q_rot[(size_t)row * kDH + i + kDH / 2] = (uint16_t)f32_to_bf16_bits(x2 * cs + x1 * sn);
}

}  // namespace

hipError_t launch_rope_query(const void* q, void* q_rot, int rows, int pos, float rope_base,
                             hipStream_t st) {
  const int n = rows * (kDH / 2);
  rope_query_kernel<<<(n + 255) / 256, 256, 0, st>>>((const uint16_t*)q, (uint16_t*)q_rot, rows, pos,
                                                     rope_base);
  return hipGetLastError();
}

bool reconstruct_supported(int dtype, int H_kv, int d, int r) {
  return dtype == 1 && d == kDH && H_kv % kNH == 0 && (r == 128 || r == 256 || r == 384 || r == 512);
}

long reconstruct_grid(int B, int H_kv, int T, bool with_v) {
  const long n_tiles = (T + kTOK - 1) / kTOK;
  return (with_v ? 2 : 1) * n_tiles * (H_kv / kNH) * B;
}

hipError_t launch_reconstruct(const void* Lk, const void* Lv, const void* Pk, const void* Pv, void* K,
                              void* V, int B, int H_kv, int r, int ctx_cap, int t0, int T,
                              int stride_tokens, float rope_base, hipStream_t st) {
  const int n_tiles = (T + kTOK - 1) / kTOK;
  const int ntens = Lv ? 2 : 1;
  const dim3 grid((unsigned)reconstruct_grid(B, H_kv, T, Lv != nullptr));
  const auto* lk = (const uint16_t*)Lk;
  const auto* lv = (const uint16_t*)Lv;
  const auto* pk = (const uint16_t*)Pk;
  const auto* pv = (const uint16_t*)Pv;
  auto* ko = (uint16_t*)K;
  auto* vo = (uint16_t*)V;
#define SALS_RC(RR)                                                                              \
  reconstruct_kernel<RR><<<grid, kNT, 0, st>>>(lk, lv, pk, pv, ko, vo, B, H_kv, ctx_cap, t0, T,   \
                                               stride_tokens, n_tiles, ntens, rope_base)
  switch (r) {
    case 128: SALS_RC(128); break;
    case 256: SALS_RC(256); break;
    case 384: SALS_RC(384); break;
    case 512: SALS_RC(512); break;
    default: return hipErrorInvalidValue;
  }
#undef SALS_RC
  return hipGetLastError();
}

}  // namespace sals
