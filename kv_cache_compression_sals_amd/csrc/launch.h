// Internal launchers (host side). Each enqueues its kernels on `st` and returns the error
// hipGetLastError reports right after the launches (hipSuccess when all were accepted).
// Shapes were validated by the C ABI layer before any of these is called.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sals {

// ---- decode path -------------------------------------------------------------------------

// Latent queries as partial sums over row blocks of P_k: qpart[part][b][s][j] = sum over the
// rows i of block `part` of group s of qsum[b][i] * P_k[i][j], where qsum[b][i] is the sum of
// q[b][h][i % d] over the query heads h that read KV head i / d. Blocks are `rb` rows long
// (rb = latent_query_rows(...), a multiple of d inside one group), so a group has
// npart = (H_kv d / G) / rb parts and q~[b][s] = sum over its parts, in part order.
constexpr int kLqMinBlocks = 192;
int latent_query_rows(int H_kv, int d, int r, int G);
hipError_t launch_latent_query(int dtype, const void* q, const void* Pk, float* qpart, int B,
                               int H_q, int H_kv, int d, int r, int G, int rb, hipStream_t st);

// S[b][s][t] = q~[b][s] . L_k[b][t], t < Tc (rows of ldS floats), with q~ the sum of the npart
// partial sums in qpart (layout above).
hipError_t launch_latent_score(int dtype, const float* qpart, int npart, const void* Lk, float* S,
                               int ldS, int B, int G, int r, int Tc, int ctx_cap, hipStream_t st);

// sel[row][0 .. kp) = top-kp of S[row][0 .. Tc) (ties to the lowest index), ascending;
// sel[row][kp .. n_sel) = Tc .. ctx-1. Rows of S are ldS floats apart. Rows longer than 32768
// candidates are split into topk_slices(...) slices whose candidates (positions, their keys and
// the slices' threshold keys: at most topk_candidate_bytes(...) bytes) go to `cand`; with cand
// null, or no valid split, one workgroup per row reads the row from memory in every pass instead.
// Threshold mode (thr): a row keeps only the candidates whose key is at least tkey
// (float_key of the threshold), at most kp of them, so its top-k count is min(kp, #passing);
// the window follows them, the rest of the row (up to n_sel) is filled with -1, and cnt[row]
// receives the row's length (count + window).
int topk_slices(int rows, int Tc, int kp, bool reduce, int* slen, int* m);
size_t topk_candidate_bytes(int rows, int Tc, int kp);
hipError_t launch_topk_window(const float* S, int ldS, int32_t* sel, int rows, int Tc, int kp,
                              int ctx, int n_sel, int32_t* cand, hipStream_t st, bool thr = false,
                              uint32_t tkey = 0, int32_t* cnt = nullptr);
uint32_t threshold_key(float tau);
// The checked candidate plan of a long row (topk_slices with reduce, each slice keeping m < kp
// candidates): ns slices, or 0 when the row is not split that way. launch_topk_slices runs only
// its slice kernel (candidates, their keys and the slices' threshold keys to cand, laid out as in
// launch_topk_window), for a consumer that ranks the candidates itself.
int topk_rank_plan(int rows, int Tc, int kp, int* m);
hipError_t launch_topk_slices(const float* S, int ldS, int rows, int Tc, int kp, int32_t* cand, hipStream_t st);

// Gather + rebuild + RoPE + attention over the selected rows, split along the selected set.
// With n_splits == 1 the normalised result goes to out; otherwise latent partials
// part[b][h][split] = (m, l, z[0 .. r)) with z = sum_j e^{logit_j - m} L_v[pos_j] go to part, for
// launch_latent_combine.
// cnt (null for a fixed n_sel) gives each selection row's own length for a ragged (thresholded)
// selection padded to n_sel; the same holds for launch_shared_keys and launch_value_sum.
// With pbuf non-null the kernel stops after the softmax and hands the probabilities to the
// shared-selection value kernels below: pbuf[b][h][j] = exp(logit_j - m_split) (rows of
// round_up(n_sel, 4) floats) and pstat[b][h][split] = (m, l).
hipError_t launch_select_attend(int dtype, const void* q, const void* Lk, const void* Lv,
                                const void* Pk, const void* Pv, const int32_t* sel, const int32_t* cnt,
                                float* out, float* part, float* pbuf, float* pstat, int B, int H_q,
                                int H_kv, int d, int r, int G, int ctx_cap, int ctx, int n_sel,
                                int split_len, int n_splits, float rope_base, hipStream_t st,
                                hipEvent_t t_start = nullptr, hipEvent_t t_stop = nullptr,
                                const int32_t* cand = nullptr, int ns = 0, int m = 0, const float* S = nullptr,
                                int ldS = 0, int Tc = 0, int kp = 0, int32_t* selw = nullptr);
// With cand non-null the kernel also makes the selection from launch_topk_slices' candidates
// (ns slices of m per row; the exact selection from the score rows S when they cannot decide it),
// every workgroup for its own row, and writes it to selw; select_attend_rank_fits tells whether a
// shape has that variant and room for it.
bool select_attend_rank_fits(int dtype, int d, int r, int nqh, int split_len, int nc, int kp);

// Key side when one selection serves several KV heads (bf16, d = 128, an even number of KV heads
// per group, at most 4 query heads per KV head, r in {128, 256, 384, 512}): the K rebuild of two
// KV heads over one split of shared_keys_split() selected tokens per workgroup, then RoPE,
// logits and the softmax over the split, written as pbuf / pstat (as select_attend's
// shared-selection mode) for the value kernels below.
// With S non-null (score rows of ldS floats, one per (sequence, selection group); Tc candidates,
// kp = min(k, Tc); a fixed n_sel = kp + ctx - Tc, no cnt; Tc <= shared_keys_rank_max()) the kernel
// also makes the selection: every workgroup ranks its own row (no top-k launch before it) and the
// selection is written to sel, which is then an output.
bool shared_keys_supported(int dtype, int H_q, int H_kv, int G, int d, int r);
int shared_keys_split();
int shared_keys_rank_max();
hipError_t launch_shared_keys(const void* q, const void* Lk, const void* Pk, int32_t* sel,
                              const int32_t* cnt, float* pbuf, float* pstat, int B, int H_q, int H_kv, int G, int r,
                              int ctx_cap, int ctx, int n_sel, int n_splits, float rope_base,
                              hipStream_t st, hipEvent_t t_start = nullptr, hipEvent_t t_stop = nullptr,
                              const float* S = nullptr, int ldS = 0, int Tc = 0, int kp = 0);

// Full reconstruction of cache rows [t0, t0 + T) into a post-RoPE KV cache [B, H_kv,
// stride_tokens, d] (bf16, d = 128, an even H_kv, r in {128, 256, 384, 512}); V (and Lv, Pv)
// may be null. launch_rope_query rotates rows of q ([rows, d], bf16) at one position.
bool reconstruct_supported(int dtype, int H_kv, int d, int r);
long reconstruct_grid(int B, int H_kv, int T, bool with_v);
hipError_t launch_reconstruct(const void* Lk, const void* Lv, const void* Pk, const void* Pv, void* K,
                              void* V, int B, int H_kv, int r, int ctx_cap, int t0, int T,
                              int stride_tokens, float rope_base, hipStream_t st);
hipError_t launch_rope_query(const void* q, void* q_rot, int rows, int pos, float rope_base,
                             hipStream_t st);

// Value side for selection groups shared by several KV heads (the group's rows are read once
// per column block instead of once per KV head):
//   zpart[c][b][h][j] = w[b][h][split(c)] sum_{t in chunk c} pbuf[b][h][t] L_v[b][sel[t]][j]
//   out[b][h][col] = sum_j P_v[kv(h) d + col][j] sum_c zpart[c][b][h][j]
// with w the log-sum-exp merge weight of the split and chunk c a piece (cl tokens) of split
// c / nsub.
struct ValuePlan {
  int cb;      // latent columns per value_sum workgroup
  int nsub;    // chunks per split
  int cl;      // tokens per chunk
  int nch;     // chunks in all (n_splits * nsub)
  size_t lds;  // dynamic LDS of value_sum
};
// false when the shape does not fit the kernels' on-chip buffers
bool value_plan(int dtype, int B, int H_q, int H_kv, int G, int r, int n_sel, int split_len,
                int n_splits, ValuePlan* vp);
hipError_t launch_value_sum(int dtype, const ValuePlan& vp, const float* pbuf, const float* pstat,
                            const int32_t* sel, const int32_t* cnt, const void* Lv, float* zpart, int B,
                            int H_q, int G, int r, int ctx_cap, int n_sel, int split_len, int n_splits,
                            hipStream_t st);
hipError_t launch_value_product(int dtype, const ValuePlan& vp, const float* zpart, const void* Pv,
                                float* out, int B, int H_q, int H_kv, int d, int r, hipStream_t st);

// LSE merge of split partials into out[b][h][:].
hipError_t launch_combine(const float* part, float* out, int BH, int d, int n_splits,
                          hipStream_t st);

// LSE merge of launch_select_attend's latent partials and the value product:
// out[b][h][c] = sum_k P_v[g*d + c][k] z[k] / L, z and L merged over the splits.
hipError_t launch_latent_combine(int dtype, const float* part, const void* Pv, float* out, int B, int H_q,
                                 int H_kv, int d, int r, int n_splits, hipStream_t st);

// Largest selected-set split that fits in on-chip memory for this shape (0 if unsupported).
int select_attend_max_split(int dtype, int d, int r, int nqh);

// ---- projection --------------------------------------------------------------------------

hipError_t launch_project(int dtype, const void* X, const void* P, void* L, int B, int T, int D,
                          int r, int ctx_cap, int t0, hipStream_t st);

// ---- compaction and dense decode ---------------------------------------------------------

// Tokens per workgroup of the two importance passes, and the size (MiB) of K the two passes
// share per batch of sequences (0: one batch of every sequence).
#ifndef SALS_IMP_CHUNK
#define SALS_IMP_CHUNK 1024
#endif
#ifndef SALS_COMPACT_BATCH_MB
#define SALS_COMPACT_BATCH_MB 0
#endif

// Per (b, g, observation query i): row max m and softmax denominator l of the causal logits.
hipError_t launch_importance_stats(int dtype, const void* K, const void* Qobs, float* stats,
                                   int B, int H_q, int H_kv, int d, int w, int ctx_cap, int ctx,
                                   hipStream_t st);

// I[b][g][t] from the stats (second pass over K).
hipError_t launch_importance_accum(int dtype, const void* K, const void* Qobs,
                                   const float* stats, float* I, int B, int H_q, int H_kv, int d,
                                   int w, int ctx_cap, int ctx, hipStream_t st,
                                   float p_thresh = 0.f, float* cnt = nullptr, float* sparsity = nullptr);

// Kc/Vc[b][g][j] = K/V[b][g][kept[b][g][j]].
hipError_t launch_gather_rows(int dtype, const void* K, const void* V, const int32_t* kept,
                              void* Kc, void* Vc, int BG, int d, int ctx_cap, int k_keep,
                              hipStream_t st);

// Frequency-domain outlier importance: I[b][g][t] = deviation energy of K and V row t from
// their low-pass (the n_freq lowest orthonormal DCT-II frequencies along the tokens), bf16 cache.
// n_freq in [1, 64]; the workspace holds the per-chunk coefficients.
int outlier_freq_pad(int n_freq);
size_t outlier_workspace_bytes(int BH, int d, int ctx, int n_freq);
hipError_t launch_outlier_importance(const void* K, const void* V, void* ws, float* I, int BH, int d,
                                     int ctx_cap, int ctx, int n_freq, hipStream_t st);

// Mixed-precision cache: rows of K and V quantized per group of 32 channels, at 8 bits for the
// positions listed in pos_hi (sorted, n_hi per pair) and at 4 bits for the rest (their positions
// written to pos_lo); bf16 input. Decode: flash-decode over both sets, partials for the combine.
hipError_t launch_mixed_quant(const void* K, const void* V, const int32_t* pos_hi, uint8_t* codes_hi,
                              float* params_hi, uint8_t* codes_lo, float* params_lo, int32_t* pos_lo, int BH, int d,
                              int ctx_cap, int ctx, int n_hi, hipStream_t st);
hipError_t launch_mixed_decode(const void* q, const uint8_t* codes_hi, const float* params_hi, const uint8_t* codes_lo,
                               const float* params_lo, float* out, float* part, int B, int H_q, int H_kv, int d,
                               int n_hi, int n_lo, int split_len, int n_splits, hipStream_t st);

// Importance-mass budgets per row of a non-negative importance [rows, ctx]: n_keep = the smallest
// count of the largest values holding `mass` of the row total, total = the row total; ratio and
// energy (nullable) = sum(n_keep) / (rows * ctx) and sum(total).
hipError_t launch_mass_budget(const float* imp, int rows, int ctx, float mass, int32_t* n_keep, float* total,
                              float* ratio, float* energy, hipStream_t st);

// Streaming read of bytes (a multiple of 16) with `blocks` workgroups of 256 threads; sink gets
// one word per workgroup.
hipError_t launch_hbm_read(const void* src, size_t bytes, uint32_t* sink, int blocks, hipStream_t st);
// blocks workgroups of 256 threads, each wave issuing iters x 4 bf16 32x32x16 MFMAs (32768 flops
// each) from registers; one word per workgroup to sink[block].
hipError_t launch_mfma_peak(int blocks, int iters, uint32_t* sink, hipStream_t st);

// Flash-decode over a contiguous cache: partials per split, or out directly (n_splits == 1).
// Query heads of one KV head that a dense-decode workgroup serves together: 4, 2 or 1.
__host__ __device__ inline int dense_heads_per_group(int nqh) { return nqh % 4 == 0 ? 4 : nqh % 2 == 0 ? 2 : 1; }
hipError_t launch_dense_decode(int dtype, const void* q, const void* K, const void* V, float* out,
                               float* part, int B, int H_q, int H_kv, int d, int n, int stride,
                               int split_len, int n_splits, hipStream_t st);

}  // namespace sals
