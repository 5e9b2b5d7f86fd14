// C ABI of the SALS decode path and post-prefill compaction: argument validation (all before
// any HIP call), workspace carving and the launch sequence on the caller's stream.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "../../include/sals.h"
#include "launch.h"

namespace {

thread_local int32_t g_last_hip_error = 0;

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool misaligned(const void* p) { return p != nullptr && ((uintptr_t)p & 15u) != 0; }

int elem_size(int dtype) { return dtype == SALS_F32 ? 4 : 2; }

bool rank_supported(int r) { return r == 32 || r == 64 || r == 128 || r == 256 || r == 384 || r == 512; }

sals_status check_layer_shape(const sals_shape* s) {
  if (s->dtype != SALS_F32 && s->dtype != SALS_BF16) return SALS_ERR_DTYPE;
  if (s->B < 1 || s->B > 65535 || s->H_q < 1 || s->H_kv < 1 || s->H_q % s->H_kv != 0 ||
      s->H_q / s->H_kv > 8 || s->H_kv > 65535)
    return SALS_ERR_SHAPE;
  if (s->d != 64 && s->d != 128) return SALS_ERR_SHAPE;
  if (!rank_supported(s->r)) return SALS_ERR_SHAPE;
  if ((long)s->d * s->r * elem_size(s->dtype) > 128L * 1024) return SALS_ERR_SHAPE;
  return SALS_OK;
}

sals_status check_kvc_shape(const kvc_shape* c) {
  if (c->dtype != SALS_F32 && c->dtype != SALS_BF16) return SALS_ERR_DTYPE;
  if (c->B < 1 || c->B > 65535 || c->H_q < 1 || c->H_kv < 1 || c->H_q % c->H_kv != 0 ||
      c->H_q / c->H_kv > 8 || c->H_q > 65535)
    return SALS_ERR_SHAPE;
  if (c->d != 64 && c->d != 128) return SALS_ERR_SHAPE;
  return SALS_OK;
}

sals_status hip_fail(hipError_t e) {
  g_last_hip_error = (int32_t)e;
  return SALS_ERR_HIP;
}

// A device must be present and current; checked after validation, before any launch.
sals_status device_ready() {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  return SALS_OK;
}

// ---- decode plan ---------------------------------------------------------------------------

struct DecodePlan {
  int D, nqh, Tc, ldS, kp, n_sel;
  int rb, npart;  // latent-query row block and parts per group
  int split_len, n_splits;
  bool shared;  // value side by the shared-selection kernels (one selection per >= 4 KV heads)
  bool skeys;   // key side of a shared selection by the two-head tile kernel
  sals::ValuePlan vp;
  size_t off_qpart, off_cand, off_S, off_sel, off_cnt, off_part, off_p, off_pstat, off_zp, total;
};

sals_status make_decode_plan(const sals_shape* s, const sals_select* sel, int32_t ctx,
                             DecodePlan* p) {
  if (!s || !sel) return SALS_ERR_NULL;
  sals_status st = check_layer_shape(s);
  if (st != SALS_OK) return st;
  if (sel->G < 1 || s->H_kv % sel->G != 0) return SALS_ERR_SHAPE;
  if (sel->k < 0 || sel->w < 0 || ctx < 1 || ctx > (1 << 26)) return SALS_ERR_RANGE;
  p->D = s->H_kv * s->d;
  p->nqh = s->H_q / s->H_kv;
  p->Tc = ctx > sel->w ? ctx - sel->w : 0;
  p->ldS = (p->Tc + 3) / 4 * 4;  // score rows start on 16-byte boundaries
  p->kp = sel->k < p->Tc ? sel->k : p->Tc;
  p->n_sel = p->kp + (ctx - p->Tc);
  if (p->n_sel < 1) return SALS_ERR_RANGE;  // k = w = 0 selects nothing to attend over
  const int group_rows = p->D / sel->G;
  p->rb = sals::latent_query_rows(s->H_kv, s->d, s->r, sel->G);
  p->npart = group_rows / p->rb;
  const int max_split = sals::select_attend_max_split(s->dtype, s->d, s->r, p->nqh);
  if (max_split < 16) return SALS_ERR_SHAPE;
  const long pairs = (long)s->B * s->H_kv;
  const int desired = (int)((256 + pairs - 1) / pairs);
  int split = (p->n_sel + desired - 1) / desired;
  split = (split + 15) / 16 * 16;
  if (split < 16) split = 16;
  if (split > max_split) split = max_split;
  p->split_len = split;
  p->n_splits = (p->n_sel + split - 1) / split;
  if ((long)p->n_splits * s->H_kv * s->B > 0x7fffffffL) return SALS_ERR_RANGE;  // 1-D grid
  size_t off = 0;
  p->off_qpart = off;
  off += align_up((size_t)p->npart * s->B * sel->G * s->r * 4);
  p->off_cand = off;
  off += align_up(sals::topk_candidate_bytes(s->B * sel->G, p->Tc, p->kp));
  p->off_S = off;
  off += align_up((size_t)s->B * sel->G * p->ldS * 4);
  p->off_sel = off;
  off += align_up((size_t)s->B * sel->G * p->n_sel * 4);
  p->off_cnt = off;  // per-row lengths of a thresholded selection
  off += align_up((size_t)s->B * sel->G * 4);
  p->skeys = s->H_kv / sel->G >= 4 &&
             sals::shared_keys_supported(s->dtype, s->H_q, s->H_kv, sel->G, s->d, s->r);
  if (p->skeys) {  // splits of the tile kernel's token count
    p->split_len = sals::shared_keys_split();
    p->n_splits = (p->n_sel + p->split_len - 1) / p->split_len;
  }
  p->shared = s->H_kv / sel->G >= 4 &&
              sals::value_plan(s->dtype, s->B, s->H_q, s->H_kv, sel->G, s->r, p->n_sel,
                               p->split_len, p->n_splits, &p->vp);
  if (p->skeys && !p->shared) {  // no value plan for the tile kernel's splits: the general path
    p->skeys = false;
    p->split_len = split;
    p->n_splits = (p->n_sel + split - 1) / split;
    p->shared = sals::value_plan(s->dtype, s->B, s->H_q, s->H_kv, sel->G, s->r, p->n_sel,
                                 p->split_len, p->n_splits, &p->vp);
  }
  if ((long)p->n_splits * s->H_kv * s->B > 0x7fffffffL) return SALS_ERR_RANGE;
  p->off_part = off;
  if (p->n_splits > 1 && !p->shared)
    off += align_up((size_t)s->B * s->H_q * p->n_splits * (s->r + 2) * 4);
  p->off_p = p->off_pstat = p->off_zp = off;
  if (p->shared) {
    off += align_up((size_t)s->B * s->H_q * ((p->n_sel + 3) / 4 * 4) * 4);
    p->off_pstat = off;
    off += align_up((size_t)s->B * s->H_q * p->n_splits * 2 * 4);
    p->off_zp = off;
    off += align_up((size_t)p->vp.nch * s->B * s->H_q * s->r * 4);
  }
  p->total = off;
  return SALS_OK;
}

// ---- compaction plan -----------------------------------------------------------------------

constexpr int kImpChunk = SALS_IMP_CHUNK;

struct CompactPlan {
  size_t off_stats, off_I, total;
};

sals_status make_compact_plan(const kvc_shape* c, int32_t ctx, int32_t w, int32_t k_keep,
                              CompactPlan* p) {
  if (!c) return SALS_ERR_NULL;
  sals_status st = check_kvc_shape(c);
  if (st != SALS_OK) return st;
  if (ctx < 1 || ctx > (1 << 26) || w < 1 || w > ctx || k_keep < 1 || k_keep > ctx)
    return SALS_ERR_RANGE;
  const size_t n_chunks = (ctx + kImpChunk - 1) / kImpChunk;
  const size_t nq = (size_t)c->B * c->H_q * w;
  p->off_stats = 0;
  size_t off = align_up(nq * 2 * 4 + nq * n_chunks * 2 * 4);
  p->off_I = off;
  off += align_up((size_t)c->B * c->H_kv * ctx * 4);
  p->total = off;
  return SALS_OK;
}

// ---- dense decode plan ---------------------------------------------------------------------

struct DensePlan {
  int split_len, n_splits;
  size_t total;
};

sals_status make_dense_plan(const kvc_shape* c, int32_t n, DensePlan* p) {
  if (!c) return SALS_ERR_NULL;
  sals_status st = check_kvc_shape(c);
  if (st != SALS_OK) return st;
  if (n < 1 || n > (1 << 26)) return SALS_ERR_RANGE;
  const long heads = (long)c->B * c->H_q;
  const long groups = heads / sals::dense_heads_per_group(c->H_q / c->H_kv);  // workgroups per split
  // about 4096 workgroups (16 per CU), so that each one's serial pass over its split stays short
  const int desired = (int)((4096 + groups - 1) / groups);
  int split = (n + desired - 1) / desired;
  split = (split + 63) / 64 * 64;
  if (split < 256) split = 256;
  p->split_len = split;
  p->n_splits = (n + split - 1) / split;
  if (heads * p->n_splits > 0x7fffffffL) return SALS_ERR_RANGE;  // 1-D grid
  p->total = p->n_splits > 1 ? align_up((size_t)heads * p->n_splits * (c->d + 2) * 4) : 0;
  return SALS_OK;
}

}  // namespace

namespace {

// Threshold selection (thr): a row keeps its candidates scoring at least tau, at most k of them,
// plus the window; its length goes to cnt_out (or to the workspace) and the rows of sel are
// padded with -1 to the largest length.
sals_status decode_impl(const sals_shape* s, const sals_select* sel, float rope_base, const void* q,
                        const void* Lk, const void* Lv, const void* Pk, const void* Pv,
                        int32_t ctx_cap, int32_t ctx, float* out, int32_t* sel_out, void* ws,
                        size_t ws_bytes, sals_stream_t stream, void* const* events, bool thr = false,
                        float tau = 0.f, int32_t* cnt_out = nullptr) {
  if (!s || !sel || !q || !Lk || !Lv || !Pk || !Pv || !out) return SALS_ERR_NULL;
  DecodePlan p;
  sals_status st = make_decode_plan(s, sel, ctx, &p);
  if (st != SALS_OK) return st;
  if (ctx > ctx_cap || !(rope_base > 1.0f) || !isfinite(rope_base)) return SALS_ERR_RANGE;
  if (thr && (sel->w < 1 || !isfinite(tau))) return SALS_ERR_RANGE;
  if (misaligned(q) || misaligned(Lk) || misaligned(Lv) || misaligned(Pk) || misaligned(Pv) ||
      misaligned(out) || misaligned(sel_out) || misaligned(ws) || misaligned(cnt_out))
    return SALS_ERR_ALIGN;
  if (!ws || ws_bytes < p.total) return SALS_ERR_WORKSPACE;
  if ((st = device_ready()) != SALS_OK) return st;
  hipStream_t hs = (hipStream_t)stream;
  char* w = (char*)ws;
  float* qpart = (float*)(w + p.off_qpart);
  float* S = (float*)(w + p.off_S);
  int32_t* selb = sel_out ? sel_out : (int32_t*)(w + p.off_sel);
  float* part = (float*)(w + p.off_part);
  float* pbuf = p.shared ? (float*)(w + p.off_p) : nullptr;
  float* pstat = p.shared ? (float*)(w + p.off_pstat) : nullptr;
  float* zpart = (float*)(w + p.off_zp);
  int32_t* cnt = thr ? (cnt_out ? cnt_out : (int32_t*)(w + p.off_cnt)) : nullptr;
  const int G = sel->G;
  hipError_t e = hipSuccess;
  auto mark = [&](int i) {
    if (events && e == hipSuccess) e = hipEventRecord((hipEvent_t)events[i], hs);
  };
  // scores are needed to rank a top-k, and for a threshold to test every candidate
  const bool score = p.kp > 0 && (thr || p.kp < p.Tc);
  mark(0);
  if (score && e == hipSuccess)
    e = sals::launch_latent_query(s->dtype, q, Pk, qpart, s->B, s->H_q, s->H_kv, s->d, s->r, G,
                                  p.rb, hs);
  mark(1);
  if (score && e == hipSuccess)
    e = sals::launch_latent_score(s->dtype, qpart, p.npart, Lk, S, p.ldS, s->B, G, s->r, p.Tc,
                                  ctx_cap, hs);
  mark(2);
  // with one selection shared by the key tile kernel's workgroups and rows short enough, each of
  // them ranks its own row instead of waiting for a top-k launch
  const bool rank_in_keys = p.skeys && !thr && p.Tc <= sals::shared_keys_rank_max();
  // rows long enough to be cut into checked slices: the slice kernel runs here and the attention
  // kernel's workgroups merge their own row's candidates (no merge launch)
  int rk_m = 0;
  const int rk_ns = (!p.skeys && !thr && p.kp > 0 && p.kp < p.Tc) ? sals::topk_rank_plan(s->B * G, p.Tc, p.kp, &rk_m) : 0;
  const bool rank_in_attend =
      rk_ns > 0 && sals::select_attend_rank_fits(s->dtype, s->d, s->r, p.nqh, p.split_len, rk_ns * rk_m, p.kp);
  int32_t* cand = (int32_t*)(w + p.off_cand);
  if (e == hipSuccess && rank_in_attend)
    e = sals::launch_topk_slices(S, p.ldS, s->B * G, p.Tc, p.kp, cand, hs);
  else if (e == hipSuccess && !rank_in_keys)
    e = sals::launch_topk_window(S, p.ldS, selb, s->B * G, p.Tc, p.kp, ctx, p.n_sel, cand, hs, thr,
                                 thr ? sals::threshold_key(tau) : 0u, cnt);
  // the attention kernel's own start and end (recorded by the runtime around the kernel) bound
  // its stage, so that the traced time of the dominant kernel excludes the launch gap
  hipEvent_t k0 = events ? (hipEvent_t)events[3] : nullptr, k1 = events ? (hipEvent_t)events[4] : nullptr;
  if (e == hipSuccess && p.skeys)
    e = sals::launch_shared_keys(q, Lk, Pk, selb, cnt, pbuf, pstat, s->B, s->H_q, s->H_kv, G, s->r,
                                 ctx_cap, ctx, p.n_sel, p.n_splits, rope_base, hs, k0, k1,
                                 rank_in_keys ? S : nullptr, p.ldS, p.Tc, p.kp);
  else if (e == hipSuccess)
    e = sals::launch_select_attend(s->dtype, q, Lk, Lv, Pk, Pv, selb, cnt, out, part, pbuf, pstat,
                                   s->B, s->H_q, s->H_kv, s->d, s->r, G, ctx_cap, ctx, p.n_sel,
                                   p.split_len, p.n_splits, rope_base, hs, k0, k1,
                                   rank_in_attend ? cand : nullptr, rk_ns, rk_m, S, p.ldS, p.Tc, p.kp,
                                   selb);
  if (p.shared) {
    if (e == hipSuccess)
      e = sals::launch_value_sum(s->dtype, p.vp, pbuf, pstat, selb, cnt, Lv, zpart, s->B, s->H_q, G,
                                 s->r, ctx_cap, p.n_sel, p.split_len, p.n_splits, hs);
    if (e == hipSuccess)
      e = sals::launch_value_product(s->dtype, p.vp, zpart, Pv, out, s->B, s->H_q, s->H_kv, s->d,
                                     s->r, hs);
  } else if (e == hipSuccess && p.n_splits > 1) {
    e = sals::launch_latent_combine(s->dtype, part, Pv, out, s->B, s->H_q, s->H_kv, s->d, s->r,
                                    p.n_splits, hs);
  }
  mark(5);
  return e == hipSuccess ? SALS_OK : hip_fail(e);
}

// ---- library-owned scratch for callers that cannot allocate ----------------------------------

// The decode workspace of sals_decode_step_noalloc lives here: one array per GPU, held from the
// library's first use on that GPU until the process ends. In host code `scratch` is a host-side
// stand-in for the device symbol, not a device address; the device address is looked up once per
// device with hipGetSymbolAddress and only that address is ever handed to kernels.
static __device__ __align__(256) unsigned char scratch[SALS_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array (looked up on the first call per device,
// with that device current).
sals_status scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  if (dev < 0 || dev >= kMaxDevices) return hip_fail(hipErrorInvalidDevice);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e);
    if (!ptr || ((uintptr_t)ptr & 255u) != 0) return hip_fail(hipErrorInvalidSymbol);
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return SALS_OK;
}

}  // namespace

extern "C" {

int32_t sals_abi_version(void) { return SALS_ABI_VERSION; }

const char* sals_status_string(sals_status status) {
  switch (status) {
    case SALS_OK: return "SALS_OK";
    case SALS_ERR_NULL: return "SALS_ERR_NULL: a required pointer is NULL";
    case SALS_ERR_SHAPE: return "SALS_ERR_SHAPE: unsupported or inconsistent shape";
    case SALS_ERR_DTYPE: return "SALS_ERR_DTYPE: unknown element type";
    case SALS_ERR_RANGE: return "SALS_ERR_RANGE: length or index out of range";
    case SALS_ERR_WORKSPACE: return "SALS_ERR_WORKSPACE: workspace missing or too small";
    case SALS_ERR_ALIGN: return "SALS_ERR_ALIGN: pointer not 16-byte aligned";
    case SALS_ERR_HIP: return "SALS_ERR_HIP: HIP runtime or launch failure";
  }
  return "unknown sals_status";
}

int32_t sals_last_hip_error(void) { return g_last_hip_error; }

sals_status sals_project_kv(const sals_shape* s, const void* Xk, const void* Xv, const void* Pk,
                            const void* Pv, void* Lk, void* Lv, int32_t ctx_cap, int32_t t0,
                            int32_t T, sals_stream_t stream) {
  if (!s || !Xk || !Pk || !Lk) return SALS_ERR_NULL;
  const bool with_v = Xv != nullptr;
  if (with_v != (Pv != nullptr) || with_v != (Lv != nullptr)) return SALS_ERR_NULL;
  sals_shape sk = *s;  // the projection does not involve query heads
  sk.H_q = sk.H_kv;
  sals_status st = check_layer_shape(&sk);
  if (st != SALS_OK) return st;
  if (T < 1 || t0 < 0 || ctx_cap < 1 || (long)t0 + T > ctx_cap || T > (1 << 26)) return SALS_ERR_RANGE;
  if (misaligned(Xk) || misaligned(Xv) || misaligned(Pk) || misaligned(Pv) || misaligned(Lk) ||
      misaligned(Lv))
    return SALS_ERR_ALIGN;
  if ((st = device_ready()) != SALS_OK) return st;
  hipStream_t hs = (hipStream_t)stream;
  const int D = s->H_kv * s->d;
  hipError_t e = sals::launch_project(s->dtype, Xk, Pk, Lk, s->B, T, D, s->r, ctx_cap, t0, hs);
  if (e == hipSuccess && with_v)
    e = sals::launch_project(s->dtype, Xv, Pv, Lv, s->B, T, D, s->r, ctx_cap, t0, hs);
  return e == hipSuccess ? SALS_OK : hip_fail(e);
}

sals_status sals_reconstruct_kv(const sals_shape* s, float rope_base, const void* Lk,
                               const void* Lv, const void* Pk, const void* Pv, int32_t ctx_cap,
                               int32_t t0, int32_t T, void* K, void* V, int32_t stride_tokens,
                               const void* q, void* q_rot, int32_t q_pos, sals_stream_t stream) {
  if (!s || !Lk || !Pk || !K) return SALS_ERR_NULL;
  const bool with_v = Lv != nullptr;
  if (with_v != (Pv != nullptr) || with_v != (V != nullptr)) return SALS_ERR_NULL;
  if ((q != nullptr) != (q_rot != nullptr)) return SALS_ERR_NULL;
  sals_status st = check_layer_shape(s);
  if (st != SALS_OK) return st;
  if (s->dtype != SALS_BF16) return SALS_ERR_DTYPE;
  if (!sals::reconstruct_supported(s->dtype, s->H_kv, s->d, s->r)) return SALS_ERR_SHAPE;
  if (T < 1 || t0 < 0 || ctx_cap < 1 || (long)t0 + T > ctx_cap || (long)t0 + T > stride_tokens ||
      T > (1 << 26) || (q && q_pos < 0))
    return SALS_ERR_RANGE;
  if (sals::reconstruct_grid(s->B, s->H_kv, T, with_v) > 0x7fffffffL) return SALS_ERR_RANGE;
  if (misaligned(Lk) || misaligned(Lv) || misaligned(Pk) || misaligned(Pv) || misaligned(K) ||
      misaligned(V) || misaligned(q) || misaligned(q_rot))
    return SALS_ERR_ALIGN;
  if ((st = device_ready()) != SALS_OK) return st;
  hipStream_t hs = (hipStream_t)stream;
  hipError_t e = sals::launch_reconstruct(Lk, Lv, Pk, Pv, K, V, s->B, s->H_kv, s->r, ctx_cap, t0, T,
                                          stride_tokens, rope_base, hs);
  if (e == hipSuccess && q) e = sals::launch_rope_query(q, q_rot, s->B * s->H_q, q_pos, rope_base, hs);
  return e == hipSuccess ? SALS_OK : hip_fail(e);
}

sals_status sals_decode_workspace_bytes(const sals_shape* s, const sals_select* sel, int32_t ctx,
                                        size_t* bytes) {
  if (!bytes) return SALS_ERR_NULL;
  DecodePlan p;
  sals_status st = make_decode_plan(s, sel, ctx, &p);
  if (st != SALS_OK) return st;
  *bytes = p.total;
  return SALS_OK;
}

sals_status sals_decode_step(const sals_shape* s, const sals_select* sel, float rope_base,
                             const void* q, const void* Lk, const void* Lv, const void* Pk,
                             const void* Pv, int32_t ctx_cap, int32_t ctx, float* out,
                             int32_t* sel_out, void* ws, size_t ws_bytes, sals_stream_t stream) {
  return decode_impl(s, sel, rope_base, q, Lk, Lv, Pk, Pv, ctx_cap, ctx, out, sel_out, ws,
                     ws_bytes, stream, nullptr);
}

sals_status sals_decode_step_threshold(const sals_shape* s, const sals_select* sel, float tau,
                                       float rope_base, const void* q, const void* Lk, const void* Lv,
                                       const void* Pk, const void* Pv, int32_t ctx_cap, int32_t ctx,
                                       float* out, int32_t* sel_out, int32_t* n_sel_out, void* ws,
                                       size_t ws_bytes, sals_stream_t stream) {
  return decode_impl(s, sel, rope_base, q, Lk, Lv, Pk, Pv, ctx_cap, ctx, out, sel_out, ws, ws_bytes,
                     stream, nullptr, true, tau, n_sel_out);
}

sals_status sals_decode_step_noalloc(const sals_shape* s, const sals_select* sel, float rope_base,
                                     const void* q, const void* Lk, const void* Lv, const void* Pk,
                                     const void* Pv, int32_t ctx_cap, int32_t ctx, float* out,
                                     int32_t* sel_out, sals_stream_t stream) {
  if (!s || !sel || !q || !Lk || !Lv || !Pk || !Pv || !out) return SALS_ERR_NULL;
  DecodePlan p;
  sals_status st = make_decode_plan(s, sel, ctx, &p);
  if (st != SALS_OK) return st;
  // the size limit is checked before any HIP call
  if (p.total > (size_t)SALS_NOALLOC_SCRATCH_BYTES) return SALS_ERR_WORKSPACE;
  if (ctx > ctx_cap || !(rope_base > 1.0f) || !isfinite(rope_base)) return SALS_ERR_RANGE;
  if (misaligned(q) || misaligned(Lk) || misaligned(Lv) || misaligned(Pk) || misaligned(Pv) ||
      misaligned(out) || misaligned(sel_out))
    return SALS_ERR_ALIGN;
  if ((st = device_ready()) != SALS_OK) return st;
  void* ws = nullptr;
  if ((st = scratch_of_current_device(&ws)) != SALS_OK) return st;
  // no kernel of the decode path reads workspace bytes it has not written in the same call, so
  // the array needs no clearing between calls
  return decode_impl(s, sel, rope_base, q, Lk, Lv, Pk, Pv, ctx_cap, ctx, out, sel_out, ws,
                     (size_t)SALS_NOALLOC_SCRATCH_BYTES, stream, nullptr);
}

sals_status sals_decode_step_traced(const sals_shape* s, const sals_select* sel, float rope_base,
                                    const void* q, const void* Lk, const void* Lv, const void* Pk,
                                    const void* Pv, int32_t ctx_cap, int32_t ctx, float* out,
                                    int32_t* sel_out, void* ws, size_t ws_bytes,
                                    sals_stream_t stream, void* const* events, int32_t n_events) {
  if (!events) return SALS_ERR_NULL;
  if (n_events < 6) return SALS_ERR_RANGE;
  for (int i = 0; i < 6; ++i)
    if (!events[i]) return SALS_ERR_NULL;
  return decode_impl(s, sel, rope_base, q, Lk, Lv, Pk, Pv, ctx_cap, ctx, out, sel_out, ws,
                     ws_bytes, stream, events);
}

sals_status kv_compact_workspace_bytes(const kvc_shape* c, int32_t ctx, int32_t w, int32_t k_keep,
                                       size_t* bytes) {
  if (!bytes) return SALS_ERR_NULL;
  CompactPlan p;
  sals_status st = make_compact_plan(c, ctx, w, k_keep, &p);
  if (st != SALS_OK) return st;
  *bytes = p.total;
  return SALS_OK;
}

namespace {

// Sequences per importance batch (SALS_COMPACT_BATCH_MB MiB of K per batch; 0: all sequences in
// one batch). The two importance passes read the same K, so batches small enough for the 256 MB
// Infinity Cache let the second pass find it there; measured at the compaction workload (one
// 134 MB sequence per batch), the smaller launches (512 workgroups) leave the chip underfilled
// and cost more than the cache saves (1428 vs 1292 us), so the default is one batch.
int compact_batch(const kvc_shape* c, int32_t ctx_cap) {
  if (SALS_COMPACT_BATCH_MB <= 0) return c->B;
  const double per_seq = (double)c->H_kv * ctx_cap * c->d * elem_size(c->dtype);
  const int nb = (int)((SALS_COMPACT_BATCH_MB * (double)(1 << 20)) / per_seq);
  return nb < 1 ? 1 : nb;
}

// The statistics pass (which & 1) and/or the accumulation pass (which & 2) of sequences
// [b0, b0 + nb) (clamped to B), each batch with its own region of the statistics workspace
// (merged stats, then chunk partials), so batches never overlap. With cnt / sparsity (the
// post-vision sparsity), their rows of the batch are written too.
hipError_t importance_batch(const kvc_shape* c, const void* K, const void* Qobs, int32_t w, int32_t ctx_cap,
                            int32_t ctx, int b0, int nb, float* stats, float* I, float* cnt, float* sparsity,
                            float p_thresh, hipStream_t hs, int which) {
  if (b0 + nb > c->B) nb = c->B - b0;
  const size_t es = elem_size(c->dtype);
  const size_t n_chunks = (ctx + kImpChunk - 1) / kImpChunk;
  const size_t per_seq_stats = (size_t)c->H_q * w * 2 + (size_t)c->H_q * w * n_chunks * 2;
  const char* Kb = (const char*)K + (size_t)b0 * c->H_kv * ctx_cap * c->d * es;
  const char* Qb = (const char*)Qobs + (size_t)b0 * c->H_q * w * c->d * es;
  float* st = stats + (size_t)b0 * per_seq_stats;
  float* Ib = I + (size_t)b0 * c->H_kv * ctx;
  hipError_t e = hipSuccess;
  if (which & 1) e = sals::launch_importance_stats(c->dtype, Kb, Qb, st, nb, c->H_q, c->H_kv, c->d, w, ctx_cap, ctx, hs);
  if (e == hipSuccess && (which & 2))
    e = sals::launch_importance_accum(c->dtype, Kb, Qb, st, Ib, nb, c->H_q, c->H_kv, c->d, w, ctx_cap, ctx, hs,
                                      p_thresh, cnt ? cnt + (size_t)b0 * c->H_q * n_chunks : nullptr,
                                      sparsity ? sparsity + (size_t)b0 * c->H_q : nullptr);
  return e;
}

sals_status compact_impl(const kvc_shape* c, const void* K, const void* V, const void* Qobs, int32_t w,
                         int32_t ctx_cap, int32_t ctx, int32_t k_keep, void* Kc, void* Vc, int32_t* kept,
                         float* importance, void* ws, size_t ws_bytes, sals_stream_t stream,
                         void* const* events) {
  if (!c || !K || !V || !Qobs || !Kc || !Vc || !kept) return SALS_ERR_NULL;
  CompactPlan p;
  sals_status st = make_compact_plan(c, ctx, w, k_keep, &p);
  if (st != SALS_OK) return st;
  if (ctx > ctx_cap) return SALS_ERR_RANGE;
  if (misaligned(K) || misaligned(V) || misaligned(Qobs) || misaligned(Kc) || misaligned(Vc) ||
      misaligned(kept) || misaligned(importance) || misaligned(ws))
    return SALS_ERR_ALIGN;
  if (!ws || ws_bytes < p.total) return SALS_ERR_WORKSPACE;
  if ((st = device_ready()) != SALS_OK) return st;
  hipStream_t hs = (hipStream_t)stream;
  float* stats = (float*)((char*)ws + p.off_stats);
  float* I = importance ? importance : (float*)((char*)ws + p.off_I);
  hipError_t e = hipSuccess;
  auto mark = [&](int i) {
    if (events && e == hipSuccess) e = hipEventRecord((hipEvent_t)events[i], hs);
  };
  mark(0);
  if (events) {  // traced: the two passes over all sequences, so that each has its own events
    if (e == hipSuccess) e = importance_batch(c, K, Qobs, w, ctx_cap, ctx, 0, c->B, stats, I, nullptr, nullptr, 0.f,
                                              hs, 1);
    mark(1);
    if (e == hipSuccess) e = importance_batch(c, K, Qobs, w, ctx_cap, ctx, 0, c->B, stats, I, nullptr, nullptr, 0.f,
                                              hs, 2);
  } else {
    for (int b0 = 0; b0 < c->B && e == hipSuccess; b0 += compact_batch(c, ctx_cap))
      e = importance_batch(c, K, Qobs, w, ctx_cap, ctx, b0, compact_batch(c, ctx_cap), stats, I, nullptr, nullptr,
                           0.f, hs, 3);
    mark(1);
  }
  mark(2);
  if (e == hipSuccess)
    e = sals::launch_topk_window(I, ctx, kept, c->B * c->H_kv, ctx, k_keep, ctx, k_keep, nullptr, hs);
  mark(3);
  if (e == hipSuccess)
    e = sals::launch_gather_rows(c->dtype, K, V, kept, Kc, Vc, c->B * c->H_kv, c->d, ctx_cap,
                                 k_keep, hs);
  mark(4);
  return e == hipSuccess ? SALS_OK : hip_fail(e);
}

}  // namespace

sals_status kv_compact(const kvc_shape* c, const void* K, const void* V, const void* Qobs,
                       int32_t w, int32_t ctx_cap, int32_t ctx, int32_t k_keep, void* Kc, void* Vc,
                       int32_t* kept, float* importance, void* ws, size_t ws_bytes,
                       sals_stream_t stream) {
  return compact_impl(c, K, V, Qobs, w, ctx_cap, ctx, k_keep, Kc, Vc, kept, importance, ws, ws_bytes, stream,
                      nullptr);
}

sals_status kv_compact_traced(const kvc_shape* c, const void* K, const void* V, const void* Qobs,
                              int32_t w, int32_t ctx_cap, int32_t ctx, int32_t k_keep, void* Kc, void* Vc,
                              int32_t* kept, float* importance, void* ws, size_t ws_bytes,
                              sals_stream_t stream, void* const* events, int32_t n_events) {
  if (!events) return SALS_ERR_NULL;
  if (n_events < 5) return SALS_ERR_RANGE;
  for (int i = 0; i < 5; ++i)
    if (!events[i]) return SALS_ERR_NULL;
  return compact_impl(c, K, V, Qobs, w, ctx_cap, ctx, k_keep, Kc, Vc, kept, importance, ws, ws_bytes, stream,
                      events);
}

sals_status sals_hbm_read(const void* src, size_t bytes, uint32_t* sink, int32_t blocks, sals_stream_t stream) {
  if (!src || !sink) return SALS_ERR_NULL;
  if (bytes == 0 || bytes % 16 != 0 || blocks < 1 || blocks > (1 << 20)) return SALS_ERR_RANGE;
  if (misaligned(src) || misaligned(sink)) return SALS_ERR_ALIGN;
  sals_status st = device_ready();
  if (st != SALS_OK) return st;
  hipError_t e = sals::launch_hbm_read(src, bytes, sink, blocks, (hipStream_t)stream);
  return e == hipSuccess ? SALS_OK : hip_fail(e);
}

sals_status sals_mfma_peak(int32_t blocks, int32_t iters, uint32_t* sink, sals_stream_t stream) {
  if (!sink) return SALS_ERR_NULL;
  if (blocks < 1 || blocks > (1 << 20) || iters < 1 || iters > (1 << 24)) return SALS_ERR_RANGE;
  if (misaligned(sink)) return SALS_ERR_ALIGN;
  sals_status st = device_ready();
  if (st != SALS_OK) return st;
  hipError_t e = sals::launch_mfma_peak(blocks, iters, sink, (hipStream_t)stream);
  return e == hipSuccess ? SALS_OK : hip_fail(e);
}

sals_status kv_importance_sparsity_workspace_bytes(const kvc_shape* c, int32_t ctx, int32_t w,
                                                 size_t* bytes) {
  if (!bytes) return SALS_ERR_NULL;
  CompactPlan p;
  sals_status st = make_compact_plan(c, ctx, w, 1, &p);
  if (st != SALS_OK) return st;
  const size_t n_chunks = (ctx + kImpChunk - 1) / kImpChunk;
  *bytes = p.off_I + align_up((size_t)c->B * c->H_q * n_chunks * 4);  // stats, then the counts
  return SALS_OK;
}

sals_status kv_importance_sparsity(const kvc_shape* c, const void* K, const void* Qobs, int32_t w,
                                  int32_t ctx_cap, int32_t ctx, float p_thresh, float* importance,
                                  float* sparsity, void* ws, size_t ws_bytes, sals_stream_t stream) {
  if (!c || !K || !Qobs || !importance || !sparsity) return SALS_ERR_NULL;
  CompactPlan p;
  sals_status st = make_compact_plan(c, ctx, w, 1, &p);
  if (st != SALS_OK) return st;
  if (ctx > ctx_cap || !(p_thresh >= 0.f && p_thresh <= 1.f)) return SALS_ERR_RANGE;
  if (misaligned(K) || misaligned(Qobs) || misaligned(importance) || misaligned(sparsity) || misaligned(ws))
    return SALS_ERR_ALIGN;
  size_t need = 0;
  if ((st = kv_importance_sparsity_workspace_bytes(c, ctx, w, &need)) != SALS_OK) return st;
  if (!ws || ws_bytes < need) return SALS_ERR_WORKSPACE;
  if ((st = device_ready()) != SALS_OK) return st;
  hipStream_t hs = (hipStream_t)stream;
  float* stats = (float*)((char*)ws + p.off_stats);
  float* cnt = (float*)((char*)ws + p.off_I);
  hipError_t e = hipSuccess;
  for (int b0 = 0; b0 < c->B && e == hipSuccess; b0 += compact_batch(c, ctx_cap))
    e = importance_batch(c, K, Qobs, w, ctx_cap, ctx, b0, compact_batch(c, ctx_cap), stats, importance, cnt,
                         sparsity, p_thresh, hs, 3);
  return e == hipSuccess ? SALS_OK : hip_fail(e);
}

sals_status kv_importance_budget(const kvc_shape* c, const float* importance, int32_t ctx, float mass,
                                 int32_t* n_keep, float* total, float* layer_ratio, float* layer_energy,
                                 sals_stream_t stream) {
  if (!c || !importance || !n_keep || !total) return SALS_ERR_NULL;
  sals_status st = check_kvc_shape(c);
  if (st != SALS_OK) return st;
  if (ctx < 1 || ctx > (1 << 26) || !(mass > 0.f && mass <= 1.f)) return SALS_ERR_RANGE;
  if (misaligned(importance) || misaligned(n_keep) || misaligned(total)) return SALS_ERR_ALIGN;
  if ((st = device_ready()) != SALS_OK) return st;
  hipError_t e = sals::launch_mass_budget(importance, c->B * c->H_kv, ctx, mass, n_keep, total, layer_ratio,
                                          layer_energy, (hipStream_t)stream);
  return e == hipSuccess ? SALS_OK : hip_fail(e);
}

sals_status kv_layer_budgets(const float* nonsparse, int32_t L, int64_t total, int32_t ctx,
                             int32_t* budgets) {
  if (!nonsparse || !budgets) return SALS_ERR_NULL;
  if (L < 1 || total < 0 || ctx < 1) return SALS_ERR_RANGE;
  double Z = 0.0;
  for (int l = 0; l < L; ++l) {
    if (!(nonsparse[l] >= 0.f && nonsparse[l] <= 1.f)) return SALS_ERR_RANGE;
    Z += (double)nonsparse[l];
  }
  for (int l = 0; l < L; ++l) {
    const double share = Z > 0.0 ? (double)total * (double)nonsparse[l] / Z : (double)total / L;
    double k = floor(share);
    if (k < 1.0) k = 1.0;
    if (k > ctx) k = ctx;
    budgets[l] = (int32_t)k;
  }
  return SALS_OK;
}

sals_status kv_compact_from_importance(const kvc_shape* c, const void* K, const void* V,
                                      const float* importance, int32_t ctx_cap, int32_t ctx,
                                      int32_t k_keep, void* Kc, void* Vc, int32_t* kept,
                                      sals_stream_t stream) {
  if (!c || !K || !V || !importance || !Kc || !Vc || !kept) return SALS_ERR_NULL;
  sals_status st = check_kvc_shape(c);
  if (st != SALS_OK) return st;
  if (ctx < 1 || ctx > (1 << 26) || ctx > ctx_cap || k_keep < 1 || k_keep > ctx) return SALS_ERR_RANGE;
  if (misaligned(K) || misaligned(V) || misaligned(importance) || misaligned(Kc) || misaligned(Vc) ||
      misaligned(kept))
    return SALS_ERR_ALIGN;
  if ((st = device_ready()) != SALS_OK) return st;
  hipStream_t hs = (hipStream_t)stream;
  hipError_t e = sals::launch_topk_window(importance, ctx, kept, c->B * c->H_kv, ctx, k_keep, ctx,
                                          k_keep, nullptr, hs);
  if (e == hipSuccess)
    e = sals::launch_gather_rows(c->dtype, K, V, kept, Kc, Vc, c->B * c->H_kv, c->d, ctx_cap,
                                 k_keep, hs);
  return e == hipSuccess ? SALS_OK : hip_fail(e);
}

namespace {

sals_status check_outlier(const kvc_shape* c, int32_t ctx, int32_t n_freq) {
  if (!c) return SALS_ERR_NULL;
  sals_status st = check_kvc_shape(c);
  if (st != SALS_OK) return st;
  if (c->dtype != SALS_BF16) return SALS_ERR_DTYPE;
  if (ctx < 1 || ctx > (1 << 26) || n_freq < 1 || n_freq > 64 || n_freq > ctx) return SALS_ERR_RANGE;
  if ((long)c->B * c->H_kv * 2 * ((ctx + 4095) / 4096) > 0x7fffffffL) return SALS_ERR_RANGE;
  return SALS_OK;
}

}  // namespace

sals_status kv_outlier_importance_workspace_bytes(const kvc_shape* c, int32_t ctx, int32_t n_freq,
                                                  size_t* bytes) {
  if (!bytes) return SALS_ERR_NULL;
  sals_status st = check_outlier(c, ctx, n_freq);
  if (st != SALS_OK) return st;
  *bytes = sals::outlier_workspace_bytes(c->B * c->H_kv, c->d, ctx, n_freq);
  return SALS_OK;
}

sals_status kv_outlier_importance(const kvc_shape* c, const void* K, const void* V, int32_t ctx_cap,
                                  int32_t ctx, int32_t n_freq, float* importance, void* ws,
                                  size_t ws_bytes, sals_stream_t stream) {
  if (!c || !K || !V || !importance) return SALS_ERR_NULL;
  sals_status st = check_outlier(c, ctx, n_freq);
  if (st != SALS_OK) return st;
  if (ctx > ctx_cap) return SALS_ERR_RANGE;
  if (misaligned(K) || misaligned(V) || misaligned(importance) || misaligned(ws)) return SALS_ERR_ALIGN;
  if (!ws || ws_bytes < sals::outlier_workspace_bytes(c->B * c->H_kv, c->d, ctx, n_freq))
    return SALS_ERR_WORKSPACE;
  if ((st = device_ready()) != SALS_OK) return st;
  hipError_t e = sals::launch_outlier_importance(K, V, ws, importance, c->B * c->H_kv, c->d, ctx_cap, ctx,
                                                 n_freq, (hipStream_t)stream);
  return e == hipSuccess ? SALS_OK : hip_fail(e);
}

sals_status kv_quantize_mixed(const kvc_shape* c, const void* K, const void* V, const float* importance,
                              int32_t ctx_cap, int32_t ctx, int32_t n_hi, uint8_t* codes_hi,
                              float* params_hi, int32_t* pos_hi, uint8_t* codes_lo, float* params_lo,
                              int32_t* pos_lo, sals_stream_t stream) {
  if (!c || !K || !V || !importance) return SALS_ERR_NULL;
  sals_status st = check_kvc_shape(c);
  if (st != SALS_OK) return st;
  if (c->dtype != SALS_BF16) return SALS_ERR_DTYPE;
  if (ctx < 1 || ctx > (1 << 26) || ctx > ctx_cap || n_hi < 0 || n_hi > ctx) return SALS_ERR_RANGE;
  const int n_lo = ctx - n_hi;
  if (n_hi > 0 && (!codes_hi || !params_hi || !pos_hi)) return SALS_ERR_NULL;
  if (n_lo > 0 && (!codes_lo || !params_lo || !pos_lo)) return SALS_ERR_NULL;
  if (misaligned(K) || misaligned(V) || misaligned(importance) || misaligned(codes_hi) ||
      misaligned(params_hi) || misaligned(pos_hi) || misaligned(codes_lo) || misaligned(params_lo) ||
      misaligned(pos_lo))
    return SALS_ERR_ALIGN;
  if ((st = device_ready()) != SALS_OK) return st;
  hipStream_t hs = (hipStream_t)stream;
  const int BH = c->B * c->H_kv;
  hipError_t e = hipSuccess;
  if (n_hi > 0)
    e = sals::launch_topk_window(importance, ctx, pos_hi, BH, ctx, n_hi, ctx, n_hi, nullptr, hs);
  if (e == hipSuccess)
    e = sals::launch_mixed_quant(K, V, pos_hi, codes_hi, params_hi, codes_lo, params_lo, pos_lo, BH, c->d,
                                 ctx_cap, ctx, n_hi, hs);
  return e == hipSuccess ? SALS_OK : hip_fail(e);
}

sals_status sals_dense_decode_mixed_workspace_bytes(const kvc_shape* c, int32_t n_hi, int32_t n_lo,
                                                    size_t* bytes) {
  if (!bytes) return SALS_ERR_NULL;
  if (n_hi < 0 || n_lo < 0 || (long)n_hi + n_lo > (1 << 26)) return SALS_ERR_RANGE;
  DensePlan p;
  sals_status st = make_dense_plan(c, n_hi + n_lo, &p);
  if (st != SALS_OK) return st;
  *bytes = p.total;
  return SALS_OK;
}

sals_status sals_dense_decode_mixed(const kvc_shape* c, const void* q, const uint8_t* codes_hi,
                                    const float* params_hi, int32_t n_hi, const uint8_t* codes_lo,
                                    const float* params_lo, int32_t n_lo, float* out, void* ws,
                                    size_t ws_bytes, sals_stream_t stream) {
  if (!c || !q || !out) return SALS_ERR_NULL;
  if (n_hi < 0 || n_lo < 0 || (long)n_hi + n_lo > (1 << 26)) return SALS_ERR_RANGE;
  if ((n_hi > 0 && (!codes_hi || !params_hi)) || (n_lo > 0 && (!codes_lo || !params_lo))) return SALS_ERR_NULL;
  DensePlan p;
  sals_status st = make_dense_plan(c, n_hi + n_lo, &p);
  if (st != SALS_OK) return st;
  if (c->dtype != SALS_BF16) return SALS_ERR_DTYPE;
  if (misaligned(q) || misaligned(codes_hi) || misaligned(params_hi) || misaligned(codes_lo) ||
      misaligned(params_lo) || misaligned(out) || misaligned(ws))
    return SALS_ERR_ALIGN;
  if (p.total > 0 && (!ws || ws_bytes < p.total)) return SALS_ERR_WORKSPACE;
  if ((st = device_ready()) != SALS_OK) return st;
  hipStream_t hs = (hipStream_t)stream;
  float* part = (float*)ws;
  hipError_t e = sals::launch_mixed_decode(q, codes_hi, params_hi, codes_lo, params_lo, out, part, c->B, c->H_q,
                                           c->H_kv, c->d, n_hi, n_lo, p.split_len, p.n_splits, hs);
  if (e == hipSuccess && p.n_splits > 1) e = sals::launch_combine(part, out, c->B * c->H_q, c->d, p.n_splits, hs);
  return e == hipSuccess ? SALS_OK : hip_fail(e);
}

sals_status sals_dense_decode_workspace_bytes(const kvc_shape* c, int32_t n, size_t* bytes) {
  if (!bytes) return SALS_ERR_NULL;
  DensePlan p;
  sals_status st = make_dense_plan(c, n, &p);
  if (st != SALS_OK) return st;
  *bytes = p.total;
  return SALS_OK;
}

sals_status sals_dense_decode(const kvc_shape* c, const void* q, const void* K, const void* V,
                              int32_t n, int32_t stride_tokens, float* out, void* ws,
                              size_t ws_bytes, sals_stream_t stream) {
  if (!c || !q || !K || !V || !out) return SALS_ERR_NULL;
  DensePlan p;
  sals_status st = make_dense_plan(c, n, &p);
  if (st != SALS_OK) return st;
  if (stride_tokens < n) return SALS_ERR_RANGE;
  if (misaligned(q) || misaligned(K) || misaligned(V) || misaligned(out) || misaligned(ws))
    return SALS_ERR_ALIGN;
  if (p.total > 0 && (!ws || ws_bytes < p.total)) return SALS_ERR_WORKSPACE;
  if ((st = device_ready()) != SALS_OK) return st;
  hipStream_t hs = (hipStream_t)stream;
  float* part = (float*)ws;
  hipError_t e = sals::launch_dense_decode(c->dtype, q, K, V, out, part, c->B, c->H_q, c->H_kv,
                                           c->d, n, stride_tokens, p.split_len, p.n_splits, hs);
  if (e == hipSuccess && p.n_splits > 1)
    e = sals::launch_combine(part, out, c->B * c->H_q, c->d, p.n_splits, hs);
  return e == hipSuccess ? SALS_OK : hip_fail(e);
}

}  // extern "C"
