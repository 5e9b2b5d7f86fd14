/*
 * sals.h - C ABI of the SALS decode path and post-prefill KV compaction for MI355X (gfx950).
 *
 * The method (sources cited by page title and section):
 *   "SALS: Sparse Attention in Latent Space for KV cache Compression" (arXiv 2510.24273),
 *   section 方法详解 -> 技术框架, stages 1-4: keys (before RoPE) and values are projected into a
 *   compact latent space, L = X . P; each decode query selects tokens through a RoPE-free
 *   query-key interaction in that space; only the selected tokens are rebuilt, L_sel . P^T, with
 *   RoPE applied at their true positions; standard attention runs over them. 关键设计 items 1-4:
 *   P from SVD or random, sparsity set by the number of selected tokens, top-k selection.
 *   "VL-Cache" author responses (reviewers KiPr W1/W2/W6, XVzL W2/W3, X8F2 Q2): importance from
 *   the softmax attention A = softmax(Q K^T / sqrt(d)) of the queries that follow the prompt's
 *   visual tokens, top-k of that importance, eviction once after prefill.
 *
 * Conventions shared by every entry point
 *   - Arrays are device pointers, row-major and contiguous, in the layout stated per argument.
 *     "dtype" arrays hold SALS_F32 (IEEE fp32) or SALS_BF16 (bfloat16) elements.
 *   - Every pointer must be 16-byte aligned (SALS_ERR_ALIGN otherwise).
 *   - The caller owns every buffer, workspaces included (the one exception is
 *     sals_decode_step_noalloc, whose workspace is a fixed array the library holds per GPU). The
 *     library never allocates, frees or synchronises; all work is enqueued on `stream` (NULL = the
 *     null stream) and returns asynchronously. Buffers must stay valid until that work completes.
 *   - Inputs are never written. Outputs are fully overwritten. Inputs, outputs and workspace
 *     must not overlap.
 *   - All argument checks run before any HIP call, so they cost nothing on the GPU and can be
 *     exercised on a host with no GPU. A failed HIP call returns SALS_ERR_HIP; the raw hipError_t
 *     is available from sals_last_hip_error() on the calling thread.
 *   - Inputs must be finite. Results are deterministic: the same inputs give the same bits.
 *   - Nothing is printed and no C++ exception crosses this interface. All calls are reentrant.
 */
#ifndef SALS_H
#define SALS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SALS_ABI_VERSION 1

/* A hipStream_t (same underlying type); NULL selects the null stream. */
typedef struct ihipStream_t* sals_stream_t;

typedef enum {
    SALS_OK = 0,
    SALS_ERR_NULL = 1,      /* a required pointer is NULL */
    SALS_ERR_SHAPE = 2,     /* unsupported or inconsistent shape */
    SALS_ERR_DTYPE = 3,     /* unknown element type */
    SALS_ERR_RANGE = 4,     /* a length or index argument is out of range */
    SALS_ERR_WORKSPACE = 5, /* workspace NULL or smaller than the size query returned */
    SALS_ERR_ALIGN = 6,     /* a pointer is not 16-byte aligned */
    SALS_ERR_HIP = 7        /* a HIP runtime call or kernel launch failed */
} sals_status;

typedef enum { SALS_F32 = 0, SALS_BF16 = 1 } sals_dtype;

/* Shape of one attention layer with a latent cache.
 *   B      sequences (one new token each per decode step)
 *   H_q    query heads; H_kv KV heads, H_q % H_kv == 0, H_q / H_kv <= 8
 *   d      head dimension, 64 or 128
 *   r      latent rank: 32, 64, 128, 256, 384 or 512, with d * r * elemsize <= 128 KiB
 *   dtype  element type of q, X, P and L (fp32 accumulation throughout) */
typedef struct {
    int32_t B, H_q, H_kv, d, r;
    int32_t dtype; /* sals_dtype */
} sals_shape;

/* Token selection knobs (SALS 关键设计 items 2 and 4).
 *   k  top-k over the non-window positions [0, ctx - w)
 *   w  recent window [ctx - w, ctx), always selected
 *   G  selection groups per sequence, H_kv % G == 0: KV head g belongs to group g*G/H_kv and all
 *      KV heads of a group use one token set; a group's score is the sum over its query heads
 *      of the raw latent dot products (G = 1: one set per sequence; G = H_kv: one per KV head). */
typedef struct {
    int32_t k, w, G;
} sals_select;

/* Shape of a plain (post-RoPE) KV cache for compaction and dense decode.
 * H_q % H_kv == 0, H_q / H_kv <= 8, d in {64, 128}, dtype SALS_BF16 or SALS_F32. */
typedef struct {
    int32_t B, H_q, H_kv, d;
    int32_t dtype; /* sals_dtype */
} kvc_shape;

/* Version of this interface (SALS_ABI_VERSION). */
int32_t sals_abi_version(void);

/* Static, human-readable name of a status code. Never NULL. */
const char* sals_status_string(sals_status status);

/* Raw hipError_t of the last failed HIP call on this thread (0 if none). */
int32_t sals_last_hip_error(void);

/*
 * sals_project_kv - latent projection of new cache rows (SALS 技术框架 stage 1).
 *   L[b, t0 + t, :] = X[b, t, :] . P for t in [0, T), for K and, when given, for V.
 *   X  = pre-RoPE rows of all KV heads side by side (D = H_kv * d), P = the layer's projection.
 * Args
 *   s            shape (B, H_kv, d, r, dtype used; H_q ignored)
 *   Xk, Xv       [B, T, D] dtype, read. Xv may be NULL (then Pv and Lv must be NULL too).
 *   Pk, Pv       [D, r] dtype, read.
 *   Lk, Lv       [B, ctx_cap, r] dtype; rows [t0, t0 + T) written, other rows untouched.
 *   ctx_cap      rows per sequence in L; 0 <= t0, 1 <= T, t0 + T <= ctx_cap.
 * Arithmetic: fp32 products and sums, one rounding to dtype (nearest even) at the end.
 * Errors: NULL/ALIGN/SHAPE/DTYPE/RANGE as stated above, HIP on launch failure.
 */
sals_status sals_project_kv(const sals_shape* s, const void* Xk, const void* Xv, const void* Pk,
                            const void* Pv, void* Lk, void* Lv, int32_t ctx_cap, int32_t t0,
                            int32_t T, sals_stream_t stream);

/*
 * sals_decode_workspace_bytes - exact workspace size of sals_decode_step for (s, sel, ctx).
 * Writes *bytes; returns the same argument errors sals_decode_step would.
 */
sals_status sals_decode_workspace_bytes(const sals_shape* s, const sals_select* sel, int32_t ctx,
                                        size_t* bytes);

/*
 * sals_decode_step - one decode step of one layer over a latent cache (SALS 技术框架 stages 2-4).
 *   For every sequence b and group g_s:
 *     q~      = sum over the group's query heads h of q[b, h] . P_k[kv(h)]          (fp32)
 *     S[t]    = q~ . L_k[b, t] for t in [0, T_c), T_c = max(0, ctx - w)              (fp32)
 *     Sel     = the min(k, T_c) largest S (ties to the lowest index) plus [T_c, ctx), ascending
 *   and for every query head h (KV head g = h * H_kv / H_q, group of g):
 *     K_hat   = RoPE(L_k[b, Sel] . P_k[g]^T, Sel),  V_hat = L_v[b, Sel] . P_v[g]^T
 *     out[b,h]= softmax(RoPE(q[b,h], ctx - 1) . K_hat^T / sqrt(d)) . V_hat
 *   P_x[g] = rows [g*d, (g+1)*d) of P_x. RoPE is rotate-half on pairs (i, i + d/2) with angle
 *   p * rope_base^(-2i/d); angles are reduced in fp64 before fp32 sin/cos. V_hat carries no
 *   rotation, so the value side is evaluated as (p^T L_v[b, Sel]) . P_v[g]^T (the same sum in
 *   another order, fp32): V_hat itself is never formed.
 * Args
 *   s, sel        shapes and knobs as documented on the structs; 1 <= ctx <= ctx_cap, k >= 0,
 *                 w >= 0, and at least one token selected (k > 0 or w > 0), else
 *                 SALS_ERR_RANGE.
 *   rope_base     RoPE base (> 1).
 *   q             [B, H_q, d] dtype, pre-RoPE query of the token at position ctx - 1.
 *   Lk, Lv        [B, ctx_cap, r] dtype latent caches; rows [0, ctx) are read.
 *   Pk, Pv        [D, r] dtype.
 *   out           [B, H_q, d] fp32, written.
 *   sel_out       NULL, or [B, G, n_sel] int32 written with the selected positions, ascending,
 *                 n_sel = min(k, T_c) + (ctx - T_c).
 *   ws, ws_bytes  workspace of at least sals_decode_workspace_bytes(s, sel, ctx) bytes.
 * Errors: as stated above; SALS_ERR_WORKSPACE if ws is NULL or too small.
 */
sals_status sals_decode_step(const sals_shape* s, const sals_select* sel, float rope_base,
                             const void* q, const void* Lk, const void* Lv, const void* Pk,
                             const void* Pv, int32_t ctx_cap, int32_t ctx, float* out,
                             int32_t* sel_out, void* ws, size_t ws_bytes, sals_stream_t stream);

/*
 * sals_decode_step_threshold - sals_decode_step with threshold selection instead of a fixed
 * top-k (SALS 关键设计 item 4: top-k or threshold selection of the tokens):
 *   per sequence b and group: the candidates t < T_c whose score S[t] (the raw latent score of
 *   sals_decode_step) is at least tau, at most k of them (when more pass, the k largest with ties
 *   to the lowest index), plus the window [T_c, ctx); ascending. The set's length n varies per
 *   row; attention runs over exactly its n tokens.
 * Args: as sals_decode_step (sel->k is the largest number of candidates a row may keep), plus
 *   tau          the score threshold (finite); scores are compared in fp32.
 *   sel_out      NULL, or [B, G, n_max] int32 with n_max = min(k, T_c) + (ctx - T_c): row b, g holds
 *                its n positions, then -1 up to n_max.
 *   n_sel_out    NULL, or [B, G] int32 written with each row's n.
 *   ws, ws_bytes workspace of at least sals_decode_workspace_bytes(s, sel, ctx) bytes.
 * Errors: as sals_decode_step; SALS_ERR_RANGE also when w < 1 (the window keeps every row
 *   non-empty) or tau is not finite.
 */
sals_status sals_decode_step_threshold(const sals_shape* s, const sals_select* sel, float tau,
                                       float rope_base, const void* q, const void* Lk, const void* Lv,
                                       const void* Pk, const void* Pv, int32_t ctx_cap, int32_t ctx,
                                       float* out, int32_t* sel_out, int32_t* n_sel_out, void* ws,
                                       size_t ws_bytes, sals_stream_t stream);

/*
 * sals_decode_step_noalloc - sals_decode_step for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc. It takes no
 * workspace: the library keeps one SALS_NOALLOC_SCRATCH_BYTES array of device memory per GPU (a
 * static device symbol, held from the first use on that GPU until the process ends) and runs the
 * same kernels as sals_decode_step with that array as their workspace, so the results are
 * bit-identical. It calls no hipMalloc, hipFree or other allocating routine.
 * Args: as sals_decode_step without ws / ws_bytes. The call runs on the current device.
 * Limit: the workspace sals_decode_workspace_bytes reports for (s, sel, ctx) must not exceed
 *   SALS_NOALLOC_SCRATCH_BYTES, else SALS_ERR_WORKSPACE (checked before any HIP call).
 * Concurrency: every call on one GPU shares that GPU's array, so calls that may overlap on one GPU
 *   (on different streams, or from different threads without stream ordering) race and must not
 *   be issued; calls ordered on one stream are safe. Nothing in the array must start at zero.
 * Errors: as sals_decode_step; SALS_ERR_HIP if the array's device address cannot be looked up.
 */
#define SALS_NOALLOC_SCRATCH_BYTES (16u << 20)
sals_status sals_decode_step_noalloc(const sals_shape* s, const sals_select* sel, float rope_base,
                                     const void* q, const void* Lk, const void* Lv, const void* Pk,
                                     const void* Pv, int32_t ctx_cap, int32_t ctx, float* out,
                                     int32_t* sel_out, sals_stream_t stream);

/*
 * sals_decode_step_traced - sals_decode_step that also records caller-created HIP events on
 * `stream` at its stage boundaries, for per-kernel timing without a profiler (a tracing
 * aid; the computation and results are identical to sals_decode_step):
 *   events[0] before the latent query, events[1] before the scoring, events[2] before the
 *   top-k selection, events[3] before rebuild + attention, events[4] before the split merge,
 *   events[5] after the last kernel. A stage that does not run for a shape leaves its two
 *   events back to back; when the rebuild kernel ranks the rows itself (one selection shared by
 *   at least 4 KV heads, bf16, d = 128, at most 4096 candidates, no threshold) the top-k stage
 *   is the gap before that kernel and the ranking falls in the rebuild stage; for rows past
 *   32768 candidates (bf16, d = 128, no threshold) the top-k stage holds the slice kernel and the
 *   merge of its candidates falls in the rebuild stage.
 * events: at least 6 hipEvent_t handles from hipEventCreate (owned by the caller);
 * SALS_ERR_NULL if events is NULL, SALS_ERR_RANGE if n_events < 6.
 */
sals_status sals_decode_step_traced(const sals_shape* s, const sals_select* sel, float rope_base,
                                    const void* q, const void* Lk, const void* Lv, const void* Pk,
                                    const void* Pv, int32_t ctx_cap, int32_t ctx, float* out,
                                    int32_t* sel_out, void* ws, size_t ws_bytes,
                                    sals_stream_t stream, void* const* events, int32_t n_events);

/*
 * kv_compact_workspace_bytes - exact workspace size of kv_compact for (c, ctx, w, k_keep).
 */
sals_status kv_compact_workspace_bytes(const kvc_shape* c, int32_t ctx, int32_t w, int32_t k_keep,
                                       size_t* bytes);

/*
 * kv_compact - post-prefill compaction of a plain KV cache (VL-Cache responses KiPr W1/W2,
 * XVzL W2/W3, X8F2 Q2; PureKV abstract).
 *   For every sequence b and KV head g, with observation queries at positions p_i = ctx - w + i:
 *     I[t]   = sum over query heads h of KV head g, sum over i < w, of
 *              softmax_{t' <= p_i}(Qobs[b, h, i] . K[b, g, t'] / sqrt(d))[t]          (fp32)
 *     kept   = the k_keep largest I (ties to the lowest index), ascending
 *     Kc, Vc = K[b, g, kept], V[b, g, kept]   (bit-exact copies)
 * Args
 *   c             shape; K, V and Qobs use c->dtype.
 *   K, V          [B, H_kv, ctx_cap, d] as stored (RoPE already applied), rows [0, ctx) read.
 *   Qobs          [B, H_q, w, d] queries of the last w prompt positions (RoPE applied).
 *   w             1 <= w <= ctx; ctx <= ctx_cap; 1 <= k_keep <= ctx.
 *   Kc, Vc        [B, H_kv, k_keep, d] written.
 *   kept          [B, H_kv, k_keep] int32 written.
 *   importance    NULL, or [B, H_kv, ctx] fp32 written with I.
 *   ws, ws_bytes  workspace of at least kv_compact_workspace_bytes(c, ctx, w, k_keep) bytes.
 */
sals_status kv_compact(const kvc_shape* c, const void* K, const void* V, const void* Qobs,
                       int32_t w, int32_t ctx_cap, int32_t ctx, int32_t k_keep, void* Kc, void* Vc,
                       int32_t* kept, float* importance, void* ws, size_t ws_bytes,
                       sals_stream_t stream);

/*
 * kv_compact_traced - kv_compact that also records caller-created HIP events on `stream` at its
 * stage boundaries, for per-stage timing without a profiler (results identical to kv_compact):
 * events[0] before the importance statistics pass, events[1] before the accumulation pass,
 * events[2] before the top-k, events[3] before the gather, events[4] after it.
 * events: at least 5 hipEvent_t handles (owned by the caller); SALS_ERR_NULL if events is NULL,
 * SALS_ERR_RANGE if n_events < 5.
 */
sals_status kv_compact_traced(const kvc_shape* c, const void* K, const void* V, const void* Qobs,
                              int32_t w, int32_t ctx_cap, int32_t ctx, int32_t k_keep, void* Kc, void* Vc,
                              int32_t* kept, float* importance, void* ws, size_t ws_bytes,
                              sals_stream_t stream, void* const* events, int32_t n_events);

/*
 * sals_hbm_read - a plain streaming read of `bytes` (a multiple of 16) at `src`, by `blocks`
 * workgroups of 256 threads, each writing one word to sink[block]: the measured HBM read bandwidth
 * that the kernels' fractions are also stated against (next to the 8 TB/s specification).
 * Errors: NULL, RANGE (bytes 0 or not a multiple of 16, blocks outside [1, 2^20]), ALIGN, HIP.
 */
sals_status sals_hbm_read(const void* src, size_t bytes, uint32_t* sink, int32_t blocks, sals_stream_t stream);

/*
 * sals_mfma_peak - bf16 MFMA throughput probe: `blocks` workgroups of 256 threads (4 waves), each
 * wave issuing iters x 4 independent bf16 32x32x16 MFMAs (32768 flops each) from registers, then
 * writing one word per workgroup to sink[block] (so that no result is dead). Total flops:
 * blocks * 4 * iters * 4 * 32768. The measured peak that the key rebuild is also stated against
 * (next to the 2.5 PFLOP/s specification).
 * Errors: NULL, RANGE (blocks outside [1, 2^20], iters outside [1, 2^24]), ALIGN, HIP.
 */
sals_status sals_mfma_peak(int32_t blocks, int32_t iters, uint32_t* sink, sals_stream_t stream);

/*
 * kv_importance_sparsity_workspace_bytes - workspace size of kv_importance_sparsity.
 */
sals_status kv_importance_sparsity_workspace_bytes(const kvc_shape* c, int32_t ctx, int32_t w,
                                                 size_t* bytes);

/*
 * kv_importance_sparsity - the importance of kv_compact plus the post-vision sparsity per query
 * head (VL-Cache responses: reviewer X8F2 question 1 - a sparsity Gamma per head and layer;
 * KiPr weakness 5 - taken on the post-vision attention rows; KiPr weakness 3 - a threshold p):
 *   importance[b, g, t] as in kv_compact;
 *   sparsity[b, h] = #{(i, t): t <= p_i, a_h[i, t] < p_thresh} / #{(i, t): t <= p_i},
 *   a_h[i, .] = softmax_{t <= p_i}(Qobs[b, h, i] . K[b, g, :] / sqrt(d)), p_i = ctx - w + i.
 * Args
 *   c, K, Qobs, w, ctx_cap, ctx   as for kv_compact.
 *   p_thresh       probability threshold in [0, 1].
 *   importance     [B, H_kv, ctx] fp32 written.   sparsity [B, H_q] fp32 written.
 *   ws, ws_bytes   workspace of at least kv_importance_sparsity_workspace_bytes(c, ctx, w).
 * Errors: NULL/ALIGN/SHAPE/DTYPE/RANGE/WORKSPACE as for kv_compact, RANGE for p_thresh outside
 * [0, 1], HIP on launch failure.
 */
sals_status kv_importance_sparsity(const kvc_shape* c, const void* K, const void* Qobs, int32_t w,
                                  int32_t ctx_cap, int32_t ctx, float p_thresh, float* importance,
                                  float* sparsity, void* ws, size_t ws_bytes, sals_stream_t stream);

/*
 * kv_layer_budgets - cache budgets of L layers from their non-sparse ratios nu_l = 1 - Gamma_l
 * (VL-Cache responses: reviewer X8F2 question 1 - Z, the sum of the non-sparse ratios over the
 * layers, normalises the budget; XVzL weakness 1 - the budget is layer-wise):
 *   budgets[l] = clamp(floor(total * nu_l / Z), 1, ctx),  or floor(total / L) for every layer
 *   when Z = 0. Host arithmetic in double; no GPU call.
 * Args: nonsparse [L] host floats in [0, 1]; total >= 0 tokens over all layers; ctx >= 1;
 *   budgets [L] host int32 written.
 * Errors: NULL, RANGE (L < 1, total < 0, ctx < 1, a ratio outside [0, 1]).
 */
sals_status kv_layer_budgets(const float* nonsparse, int32_t L, int64_t total, int32_t ctx,
                             int32_t* budgets);

/*
 * kv_importance_budget - dynamic budgets from an importance distribution.
 *   For every sequence b and KV head g (a row of importance[b, g, :ctx], values >= 0; negative
 *   values count as 0):
 *     total[b, g]  = sum of the row                                               (fp64 sum, fp32)
 *     n_keep[b, g] = the smallest n >= 1 whose n largest values sum to at least mass * total
 *   and for the layer (nullable single floats):
 *     layer_ratio  = sum of n_keep / (B H_kv ctx)   (ZipVL abstract: the ratio of important tokens
 *                    follows the layer's attention distribution instead of a fixed value; use
 *                    ceil(layer_ratio * ctx) as the layer's k_keep or n_hi)
 *     layer_energy = sum of total                  (FlashCache abstract: a dynamic budget decides
 *                    each layer's cache size; with the outlier importance of
 *                    kv_outlier_importance, kv_layer_budgets over E_l / max E gives budgets in
 *                    proportion to the layers' outlier energies)
 * Args: c (B, H_kv used); importance [B, H_kv, ctx] fp32; 0 < mass <= 1; n_keep [B, H_kv] int32
 *   and total [B, H_kv] fp32 written; layer_ratio, layer_energy: NULL or one device float each.
 * Sums are fp64 in a fixed order, so results are deterministic.
 * Errors: NULL/ALIGN/SHAPE/RANGE as stated above, HIP on launch failure.
 */
sals_status kv_importance_budget(const kvc_shape* c, const float* importance, int32_t ctx, float mass,
                                 int32_t* n_keep, float* total, float* layer_ratio, float* layer_energy,
                                 sals_stream_t stream);

/*
 * kv_compact_from_importance - the selection and gather of kv_compact from an importance the
 * caller supplies (PureKV abstract: attention measured on a lower layer estimates the importance
 * of the tokens of higher layers, so those layers need no attention scores of their own).
 *   kept   = the k_keep largest importance[b, g, :ctx] (ties to the lowest index), ascending
 *   Kc, Vc = K[b, g, kept], V[b, g, kept]   (bit-exact copies)
 * Args
 *   c             shape (H_q unused); K and V use c->dtype.
 *   K, V          [B, H_kv, ctx_cap, d], rows [0, ctx) read.
 *   importance    [B, H_kv, ctx] fp32 (e.g. the importance output of kv_compact on another
 *                 layer), finite values; read.
 *   ctx_cap, ctx  1 <= ctx <= ctx_cap; 1 <= k_keep <= ctx.
 *   Kc, Vc        [B, H_kv, k_keep, d] written.   kept [B, H_kv, k_keep] int32 written.
 * No workspace. Errors: NULL/ALIGN/SHAPE/DTYPE/RANGE as for kv_compact, HIP on launch failure.
 */
sals_status kv_compact_from_importance(const kvc_shape* c, const void* K, const void* V,
                                      const float* importance, int32_t ctx_cap, int32_t ctx,
                                      int32_t k_keep, void* Kc, void* Vc, int32_t* kept,
                                      sals_stream_t stream);

/*
 * kv_outlier_importance_workspace_bytes - workspace size of kv_outlier_importance.
 */
sals_status kv_outlier_importance_workspace_bytes(const kvc_shape* c, int32_t ctx, int32_t n_freq,
                                                  size_t* bytes);

/*
 * kv_outlier_importance - frequency-domain outlier importance of a plain KV cache, computed from
 * the keys and values alone, with no attention score (FlashCache page, summary and abstract: the
 * energy of the KV matrices along the tokens sits at low frequencies, a low-pass filter extracts
 * it, and the KV pairs that deviate most from it are the ones to keep):
 *   for every sequence b and KV head g, with X = K[b, g, :ctx] or V[b, g, :ctx] ([ctx, d]) and
 *   C[t, f] = a_f cos(pi (2t + 1) f / (2 ctx)) the orthonormal DCT-II basis along the tokens
 *   (a_0 = sqrt(1/ctx), a_f = sqrt(2/ctx)), X_lp = C_F C_F^T X keeps the n_freq lowest
 *   frequencies, and
 *     importance[b, g, t] = ||K[t] - K_lp[t]||^2 + ||V[t] - V_lp[t]||^2      (fp32)
 *   kv_compact_from_importance then keeps the k_keep most deviating pairs per (b, g).
 * Args
 *   c             shape; dtype must be SALS_BF16 (H_q unused).
 *   K, V          [B, H_kv, ctx_cap, d] as stored, rows [0, ctx) read.
 *   ctx_cap, ctx  1 <= ctx <= ctx_cap.
 *   n_freq        kept frequencies, 1 <= n_freq <= min(64, ctx).
 *   importance    [B, H_kv, ctx] fp32 written.
 *   ws, ws_bytes  workspace of at least kv_outlier_importance_workspace_bytes(c, ctx, n_freq).
 * Arithmetic: bf16 MFMA products with the fp32 basis values and coefficients split into high and
 * low bf16 parts, fp32 sums; angles reduced exactly in integers before the fp32 cosine.
 * Errors: NULL/ALIGN/SHAPE/RANGE/WORKSPACE as stated above, DTYPE unless bf16, HIP on launch
 * failure.
 */
sals_status kv_outlier_importance(const kvc_shape* c, const void* K, const void* V, int32_t ctx_cap,
                                  int32_t ctx, int32_t n_freq, float* importance, void* ws,
                                  size_t ws_bytes, sals_stream_t stream);

/*
 * kv_quantize_mixed - importance-based mixed-precision storage of a plain KV cache (ZipVL
 * abstract: high-bit quantization for the caches of important tokens, low-bit quantization for
 * the less important ones, to relieve the memory traffic of decoding).
 *   For every sequence b and KV head g: pos_hi = the n_hi largest importance[b, g, :ctx] (ties to
 *   the lowest index), ascending; pos_lo = the other positions of [0, ctx), ascending. The K and V
 *   rows of pos_hi are stored at 8 bits, those of pos_lo at 4 bits, per token and per group of 32
 *   channels, asymmetric and uniform: with mn, mx the group's extremes, levels = 2^bits - 1 and
 *   fp32 steps each rounded to nearest, span = mx - mn, inv = levels / span, scale = span / levels,
 *   code = clamp(floor((x - mn) * inv + 0.5), 0, levels); a group with span < 2^-96 stores code 0,
 *   scale 0, zero point mn. A value is read back as mn + code * scale.
 * Args
 *   c             shape; dtype must be SALS_BF16 (H_q unused); d in {64, 128}.
 *   K, V          [B, H_kv, ctx_cap, d] as stored, rows [0, ctx) read.
 *   importance    [B, H_kv, ctx] fp32, finite (e.g. from kv_compact or kv_outlier_importance).
 *   ctx_cap, ctx  1 <= ctx <= ctx_cap;  0 <= n_hi <= ctx;  n_lo = ctx - n_hi.
 *   codes_hi      [2, B, H_kv, n_hi, d] uint8 written (index 0 keys, 1 values).
 *   params_hi     [2, B, H_kv, n_hi, d / 32, 2] fp32 written: (scale, zero point) per group.
 *   pos_hi        [B, H_kv, n_hi] int32 written.
 *   codes_lo      [2, B, H_kv, n_lo, d / 2] uint8 written: two codes per byte, channel 2j in the
 *                 low nibble of byte j of its row.
 *   params_lo     [2, B, H_kv, n_lo, d / 32, 2] fp32 written.    pos_lo [B, H_kv, n_lo] written.
 *   The *_hi pointers may be NULL when n_hi = 0, the *_lo ones when n_lo = 0.
 * No workspace. Errors: NULL/ALIGN/SHAPE/RANGE as stated above, DTYPE unless bf16, HIP on launch
 * failure.
 */
sals_status kv_quantize_mixed(const kvc_shape* c, const void* K, const void* V, const float* importance,
                              int32_t ctx_cap, int32_t ctx, int32_t n_hi, uint8_t* codes_hi,
                              float* params_hi, int32_t* pos_hi, uint8_t* codes_lo, float* params_lo,
                              int32_t* pos_lo, sals_stream_t stream);

/*
 * sals_dense_decode_mixed_workspace_bytes - workspace size of sals_dense_decode_mixed.
 */
sals_status sals_dense_decode_mixed_workspace_bytes(const kvc_shape* c, int32_t n_hi, int32_t n_lo,
                                                    size_t* bytes);

/*
 * sals_dense_decode_mixed - one decode step of plain attention over a mixed-precision cache from
 * kv_quantize_mixed (every token of both sets; the rows were rotated before quantization, so the
 * positions play no further part):
 *   out[b, h] = softmax(q[b, h] . K_hat^T / sqrt(d)) . V_hat,  K_hat, V_hat = the dequantized rows
 *   (mn + code * scale, one fp32 fused multiply-add per value) of KV head h * H_kv / H_q.
 * Args
 *   c             shape; dtype SALS_BF16 (the query's type).
 *   q             [B, H_q, d] bf16, RoPE already applied.
 *   codes_*, params_*, n_hi, n_lo   the two sets as kv_quantize_mixed wrote them; n_hi + n_lo >= 1.
 *   out           [B, H_q, d] fp32 written.
 *   ws, ws_bytes  workspace of at least sals_dense_decode_mixed_workspace_bytes(c, n_hi, n_lo).
 */
sals_status sals_dense_decode_mixed(const kvc_shape* c, const void* q, const uint8_t* codes_hi,
                                    const float* params_hi, int32_t n_hi, const uint8_t* codes_lo,
                                    const float* params_lo, int32_t n_lo, float* out, void* ws,
                                    size_t ws_bytes, sals_stream_t stream);

/*
 * sals_dense_decode_workspace_bytes - exact workspace size of sals_dense_decode for (c, n).
 */
sals_status sals_dense_decode_workspace_bytes(const kvc_shape* c, int32_t n, size_t* bytes);

/*
 * sals_dense_decode - one decode step of plain attention over a contiguous cache, e.g. the
 * compact cache kv_compact produced (VL-Cache KiPr W1 formula, one query row):
 *   out[b, h] = softmax(q[b, h] . K[b, g, :n]^T / sqrt(d)) . V[b, g, :n],  g = h * H_kv / H_q
 * Args
 *   q             [B, H_q, d] c->dtype, RoPE already applied.
 *   K, V          [B, H_kv, stride_tokens, d] c->dtype; rows [0, n) read; 1 <= n <= stride_tokens.
 *   out           [B, H_q, d] fp32 written.
 *   ws, ws_bytes  workspace of at least sals_dense_decode_workspace_bytes(c, n) bytes.
 */
sals_status sals_dense_decode(const kvc_shape* c, const void* q, const void* K, const void* V,
                              int32_t n, int32_t stride_tokens, float* out, void* ws,
                              size_t ws_bytes, sals_stream_t stream);

/*
 * sals_reconstruct_kv - full reconstruction of latent cache rows into a plain post-RoPE KV cache:
 * the dense baseline SALS replaces (SALS 问题定义 and abstract: the whole low-rank cache must be
 * rebuilt before RoPE can be applied; 技术框架 stage 3 rebuilds only the selected rows).
 *   K[b, g, t, :] = RoPE_t(L_k[b, t, :] . P_k[g]^T),  V[b, g, t, :] = L_v[b, t, :] . P_v[g]^T
 *   for t in [t0, t0 + T), every KV head g; RoPE (rotate-half, theta_i = base^(-2i/d)) at the
 *   absolute position t. With q given, also q_rot[b, h] = RoPE_{q_pos}(q[b, h]).
 *   sals_dense_decode over K, V and q_rot then gives attention over the whole rebuilt cache.
 * Args
 *   s             shape; dtype must be SALS_BF16, d = 128, H_kv even, r in {128, 256, 384, 512}.
 *   rope_base     RoPE base (e.g. 10000).
 *   Lk, Lv        [B, ctx_cap, r] bf16, rows [t0, t0 + T) read. Lv may be NULL (then Pv and V
 *                 must be NULL too: K only).
 *   Pk, Pv        [H_kv * d, r] bf16, read.
 *   K, V          [B, H_kv, stride_tokens, d] bf16; rows [t0, t0 + T) written, others untouched.
 *   q, q_rot      [B, H_q, d] bf16, pre-RoPE query read and rotated query written; both NULL to
 *                 skip. q_pos >= 0 is the query's position.
 * Arithmetic: bf16 products, fp32 sums, rotation in fp32 with the angle reduced in fp64, one
 * rounding to bf16 (nearest even) per output element.
 * Errors: NULL (K side or the q pair incomplete), DTYPE (not bf16), SHAPE, RANGE (T < 1, t0 < 0,
 * t0 + T > ctx_cap or > stride_tokens, q_pos < 0), ALIGN, HIP on launch failure.
 */
sals_status sals_reconstruct_kv(const sals_shape* s, float rope_base, const void* Lk,
                               const void* Lv, const void* Pk, const void* Pv, int32_t ctx_cap,
                               int32_t t0, int32_t T, void* K, void* V, int32_t stride_tokens,
                               const void* q, void* q_rot, int32_t q_pos, sals_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SALS_H */
