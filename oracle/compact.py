"""Post-prefill KV compaction oracle (VL-Cache / PureKV style) and dense decode over a cache.

TEST INFRASTRUCTURE ONLY (see the package docstring). fp64 NumPy throughout.

Sources (cited by page title and section):
  * "VL-Cache" author responses: reviewer KiPr weakness 1 (A = softmax(Q K^T / sqrt(d))),
    weakness 2 (post-vision attention: only the query rows of the language tokens after the
    vision tokens), weakness 6 (fewer KV tokens means less HBM traffic for attention);
    reviewer XVzL weakness 2 (top-k index set S_{psi,k}) and weakness 3 (scores from prefill
    attention rank the cache tokens, the unimportant ones are evicted); reviewer X8F2 question 2
    and XU5m weakness 2 (eviction happens once, after prefill).
  * "PureKV" abstract: importance estimates that stay compatible with efficient attention
    kernels (no full n x n attention matrix is formed; only the last w query rows are used).

Readings where the pages are silent:
  * the observation queries are the last w prompt positions T-w .. T-1 with a causal mask;
  * importance is the sum over those queries of the softmax probabilities; with grouped heads a
    KV head sums over the query heads that read it;
  * the top k_keep positions by importance are kept per (sequence, KV head), ties to the lowest
    index, kept positions ascending; no window is forced;
  * keys are used as stored (RoPE already applied); no rotation happens here.
"""

from __future__ import annotations

from typing import Dict

import numpy as np

from .sals import kv_head_of, stored_to_f64, topk_lowest_index


def _softmax(logits: np.ndarray) -> np.ndarray:
    m = logits.max()
    e = np.exp(logits - m)
    return e / e.sum()


def importance(Qobs: np.ndarray, K: np.ndarray, T: int) -> np.ndarray:
    """I[t] = sum_i softmax_{t' <= p_i}(Qobs[i] . K[t'] / sqrt(d))[t], p_i = T - w + i.

    One query head against one KV head: Qobs[w, d], K[>=T, d] (fp64). Returns I[T].
    """
    w, d = Qobs.shape
    I = np.zeros(T)
    for i in range(w):
        p = T - w + i
        a = _softmax(K[: p + 1] @ Qobs[i] / np.sqrt(d))
        I[: p + 1] += a
    return I


def kv_compact(K, V, Qobs, *, ctx: int, k_keep: int, H_kv: int, dtype: str = "bf16",
               pairs=None) -> Dict[str, object]:
    """Importance, per-(sequence, KV head) top-k_keep selection and gather.

    Stored K, V[B, H_kv, ctx_cap, d]; Qobs[B, H_q, w, d]. Returns ``importance[B, H_kv, ctx]``
    (fp64), ``kept[B, H_kv, k_keep]`` (ascending int64) and the compact caches
    ``Kc, Vc[B, H_kv, k_keep, d]`` holding the *stored* rows (same dtype as the input).
    ``pairs``: optional list of (b, g) to compute; the others stay NaN / -1 / zero.
    """
    Qf = stored_to_f64(Qobs, dtype)
    B, H_q, w, d = Qf.shape
    T = int(ctx)
    I = np.full((B, H_kv, T), np.nan)
    kept = np.full((B, H_kv, k_keep), -1, dtype=np.int64)
    Kc = np.zeros((B, H_kv, k_keep, d), dtype=K.dtype)
    Vc = np.zeros_like(Kc)
    todo = [(b, g) for b in range(B) for g in range(H_kv)] if pairs is None else pairs
    for b, g in todo:
        Kf = stored_to_f64(K[b, g, :T], dtype)
        acc = np.zeros(T)
        for h in range(H_q):
            if kv_head_of(h, H_q, H_kv) == g:
                acc += importance(Qf[b, h], Kf, T)
        I[b, g] = acc
        kept[b, g] = topk_lowest_index(acc, k_keep)
        Kc[b, g] = K[b, g, kept[b, g]]
        Vc[b, g] = V[b, g, kept[b, g]]
    return dict(importance=I, kept=kept, Kc=Kc, Vc=Vc)


def sparsity(Qobs: np.ndarray, K: np.ndarray, T: int, p: float):
    """Sparsity of one query head's post-vision attention (VL-Cache responses: reviewer X8F2
    question 1 - Gamma holds a sparsity per head and layer; reviewer KiPr weakness 5 - it is
    computed on the post-vision attention rows; KiPr weakness 3 - a threshold p, from 1e-4 to
    0.1). Reading: the fraction of the causal entries a[i, t] (t <= p_i = T - w + i) of the w
    observation rows whose probability is below p.
    Qobs[w, d], K[>=T, d] (fp64). Returns (Gamma, below, total, near), near = entries within
    a relative 1e-5 of p (their side of the threshold depends on rounding)."""
    w, d = Qobs.shape
    below = near = total = 0
    for i in range(w):
        pi = T - w + i
        a = _softmax(K[: pi + 1] @ Qobs[i] / np.sqrt(d))
        below += int(np.count_nonzero(a < p))
        near += int(np.count_nonzero(np.abs(a - p) <= 1e-5 * p))
        total += pi + 1
    return below / total, below, total, near


def layer_budgets(nonsparse, total: int, ctx: int) -> np.ndarray:
    """Cache budget per layer from the non-sparse ratios nu_l = 1 - Gamma_l (VL-Cache responses:
    reviewer X8F2 question 1 - Z is the sum of the non-sparse ratios over the layers, the
    normaliser of the budget; reviewer XVzL weakness 1 - the budget is layer-wise). Reading:
    k_l = floor(total * nu_l / Z), clamped to [1, ctx]; every layer gets floor(total / L) when
    Z = 0. (The pages name the allocation "skewed" without its formula; this is the plain
    proportional split.)"""
    nu = np.asarray(nonsparse, dtype=np.float64)
    L = len(nu)
    Z = float(nu.sum())
    k = np.empty(L, dtype=np.int64)
    for l in range(L):
        share = total * nu[l] / Z if Z > 0 else total / L
        k[l] = min(max(int(np.floor(share)), 1), ctx)
    return k


def compact_from_importance(K, V, importance, *, k_keep: int, pairs=None) -> Dict[str, object]:
    """Selection and gather from a given importance (the PureKV abstract: importance measured on a
    lower layer ranks the cache tokens of higher layers). importance[B, H_kv, >= T] (float), K, V
    stored [B, H_kv, ctx_cap, d]; the first T = importance.shape[2] positions are ranked.
    Returns ``kept[B, H_kv, k_keep]`` (ascending int64) and ``Kc, Vc`` (stored rows)."""
    B, H_kv, T = importance.shape
    d = K.shape[3]
    kept = np.full((B, H_kv, k_keep), -1, dtype=np.int64)
    Kc = np.zeros((B, H_kv, k_keep, d), dtype=K.dtype)
    Vc = np.zeros_like(Kc)
    todo = [(b, g) for b in range(B) for g in range(H_kv)] if pairs is None else pairs
    for b, g in todo:
        kept[b, g] = topk_lowest_index(np.asarray(importance[b, g], dtype=np.float64), k_keep)
        Kc[b, g], Vc[b, g] = K[b, g, kept[b, g]], V[b, g, kept[b, g]]
    return dict(kept=kept, Kc=Kc, Vc=Vc)


def dense_decode(q, K, V, *, n: int, H_kv: int, dtype: str = "bf16", pairs=None) -> np.ndarray:
    """o[b, h] = softmax(q[b, h] . K[b, kv(h), :n]^T / sqrt(d)) . V[b, kv(h), :n].

    Stored q[B, H_q, d] (RoPE already applied), K, V[B, H_kv, >=n, d]. fp64 result [B, H_q, d].
    (VL-Cache KiPr weakness 1 formula, one query row.) ``pairs``: optional list of (b, h).
    """
    qf = stored_to_f64(q, dtype)
    B, H_q, d = qf.shape
    out = np.full((B, H_q, d), np.nan)
    todo = [(b, h) for b in range(B) for h in range(H_q)] if pairs is None else pairs
    for b, h in todo:
        g = kv_head_of(h, H_q, H_kv)
        Kf = stored_to_f64(K[b, g, :n], dtype)
        Vf = stored_to_f64(V[b, g, :n], dtype)
        out[b, h] = _softmax(Kf @ qf[b, h] / np.sqrt(d)) @ Vf
    return out


def mass_budget(imp_row, mass: float):
    """(n, total) for one importance row (values >= 0): total = sum of the row, n = the smallest
    count whose n largest values sum to at least mass * total (at least 1). The ZipVL abstract
    sets the ratio of important tokens from the distribution of the attention scores rather than
    a fixed hyper-parameter; reading: the share of tokens that carries a fixed fraction of the
    normalized importance mass."""
    v = np.sort(np.asarray(imp_row, dtype=np.float64))[::-1]
    total = float(v.sum())
    target = mass * total
    run = 0.0
    n = 0
    while n < len(v) and run < target:
        run += v[n]
        n += 1
    return max(n, 1), total


def importance_budget(importance, *, ctx: int, mass: float):
    """Per (sequence, KV head) row of importance [B, H_kv, >= ctx]: n_keep [B, H_kv] and total
    [B, H_kv] (mass_budget), the layer's ratio = sum(n_keep) / (rows * ctx) (ZipVL: one dynamic
    ratio per layer) and the layer's energy = sum(total) (the FlashCache budget input)."""
    B, H = importance.shape[0], importance.shape[1]
    n = np.zeros((B, H), dtype=np.int64)
    tot = np.zeros((B, H))
    for b in range(B):
        for g in range(H):
            n[b, g], tot[b, g] = mass_budget(importance[b, g, :ctx], mass)
    return dict(n_keep=n, total=tot, layer_ratio=n.sum() / (B * H * ctx), layer_energy=tot.sum())


def energy_budgets(energies, total: int, ctx: int) -> np.ndarray:
    """Per-layer cache sizes from the layers' outlier energies (FlashCache page: a dynamic budget
    allocation decides each layer's KV cache size so that more outlier KVs are kept). Reading: a
    layer's share of the total budget is proportional to its outlier energy, i.e. layer_budgets
    with the ratios E_l / max E (the max cancels in the normaliser)."""
    e = np.asarray(energies, dtype=np.float64)
    top = e.max()
    return layer_budgets(e / top if top > 0 else np.zeros_like(e), total, ctx)
