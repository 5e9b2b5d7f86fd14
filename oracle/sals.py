"""SALS decode oracle: latent cache -> latent query -> RoPE-free scores -> top-k + window ->
reconstruct the selected rows -> RoPE at their positions -> softmax attention.

TEST INFRASTRUCTURE ONLY (see the package docstring). fp64 NumPy throughout.

Sources (cited by page title and section):
  * "SALS: Sparse Attention in Latent Space for KV cache Compression" (arXiv 2510.24273),
    section 方法详解 -> 技术框架 stages 1-4 (project K and V to a latent space; select tokens with
    a RoPE-free query-key interaction in that space; rebuild only the selected tokens; standard
    attention over them), 关键设计 items 1-4 (P from SVD or random; sparsity set by the number of
    selected tokens; latent size per model; top-k selection), 问题定义 and the English abstract
    (RoPE has to be applied after reconstruction, so the latent holds pre-RoPE keys).
  * "VL-Cache" author responses, reviewer KiPr weakness 1 (A = softmax(Q K^T / sqrt(d))) and
    reviewer XVzL weakness 2 (S_{psi,k}: the top-k indices under a scoring policy psi).

Readings where the pages are silent (each also listed in the design notes):
  * score reduction across heads: raw latent dot products summed over a selection group
    (G groups of consecutive KV heads; G = 1 sums all heads);
  * score: raw signed dot product, no 1/sqrt(d), no abs, no softmax (a monotone scale cannot
    change a top-k);
  * top-k runs over the non-window positions [0, T-w); the window [T-w, T) is always kept and
    is also rebuilt from the latent; ties go to the lowest index; -0.0 equals +0.0;
  * selected positions are returned ascending; the query sits at position T-1 and a key at its
    cache index;
  * RoPE is the rotate-half form on pairs (i, i + d/2) with theta_i = base^(-2i/d);
  * one P per layer over the concatenated KV heads, [D, r] row-major; KV head g uses rows
    [g*d, (g+1)*d); query head h reads KV head floor(h*H_kv/H_q); KV head g is in selection
    group floor(g*G/H_kv).
"""

from __future__ import annotations

from typing import Dict, Optional

import numpy as np


# ----------------------------------------------------------------------------------------------
# storage decode and index maps
# ----------------------------------------------------------------------------------------------

def stored_to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Stored array -> exact fp64 values. bf16 arrives as uint16 bit patterns (the upper half
    of an IEEE fp32), fp32 as float32, f64 as float64."""
    if dtype == "bf16":
        return (np.asarray(a, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if dtype == "f64":  # exact values handed in directly (used by the pins)
        return np.asarray(a, dtype=np.float64)
    raise ValueError(dtype)


def kv_head_of(h: int, H_q: int, H_kv: int) -> int:
    """KV head read by query head h: contiguous groups of H_q/H_kv query heads share one."""
    return (h * H_kv) // H_q


def group_of(g: int, H_kv: int, G: int) -> int:
    """Selection group of KV head g: contiguous groups of H_kv/G KV heads share one token set."""
    return (g * G) // H_kv


# ----------------------------------------------------------------------------------------------
# stage 1: low-rank projection into the latent space
# ----------------------------------------------------------------------------------------------

def project_kv(X: np.ndarray, P: np.ndarray) -> np.ndarray:
    """Latent rows L = X . P (SALS, 技术框架 stage 1; 关键设计 item 1 for P).

    X[..., D] pre-RoPE key (or value) rows of all KV heads side by side; P[D, r]. fp64 result,
    before any rounding to the storage type.
    """
    return np.asarray(X, dtype=np.float64) @ np.asarray(P, dtype=np.float64)


# ----------------------------------------------------------------------------------------------
# stage 2: RoPE-free query-key interaction in the latent space
# ----------------------------------------------------------------------------------------------

def latent_query(q: np.ndarray, Pk: np.ndarray, H_kv: int, G: int) -> np.ndarray:
    """q~[s] = sum over query heads h whose KV head lies in group s of q[h] . P_k[kv(h)].

    q[H_q, d] pre-RoPE (fp64), Pk[D, r] (fp64). Returns [G, r]. The dot product of q~[s] with a
    latent row equals the sum over those heads of the RoPE-free q[h] . k_hat[kv(h)], where
    k_hat = L . P^T is the key rebuilt from the latent (SALS, 技术框架 stage 2; 关键创新 2).
    """
    H_q, d = q.shape
    r = Pk.shape[1]
    qt = np.zeros((G, r))
    for h in range(H_q):
        g = kv_head_of(h, H_q, H_kv)
        s = group_of(g, H_kv, G)
        qt[s] += q[h] @ Pk[g * d:(g + 1) * d, :]
    return qt


def latent_scores(qt: np.ndarray, Lk: np.ndarray, T_c: int) -> np.ndarray:
    """S[s, t] = q~[s] . L_k[t] for the candidate positions t in [0, T_c). Returns [G, T_c]."""
    return qt @ Lk[:T_c].T


# ----------------------------------------------------------------------------------------------
# sparse token selection (top-k, plus the recent window)
# ----------------------------------------------------------------------------------------------

def topk_lowest_index(scores: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest scores, ties broken toward the lowest index, returned ascending.

    This is S_{psi,k} of the VL-Cache responses (reviewer XVzL, weakness 2) with psi = scores.
    Keys are (-score, index); NumPy compares -0.0 equal to +0.0, so signed zeros tie.
    """
    n = scores.shape[0]
    k = max(0, min(int(k), n))
    order = np.lexsort((np.arange(n), -np.asarray(scores, dtype=np.float64)))
    return np.sort(order[:k])


def select_tokens(S_row: np.ndarray, T: int, k: int, w: int) -> np.ndarray:
    """Selected positions of one group: top-min(k, T_c) over [0, T_c) plus the window [T_c, T),
    with T_c = max(0, T - w). Ascending, int64 (SALS, 关键设计 items 2 and 4)."""
    T_c = max(0, T - w)
    top = topk_lowest_index(S_row[:T_c], min(k, T_c))
    return np.concatenate([top, np.arange(T_c, T)]).astype(np.int64)


def select_tokens_threshold(S_row: np.ndarray, T: int, k: int, w: int, tau: float) -> np.ndarray:
    """Threshold selection (SALS, 关键设计 item 4 names threshold selection beside top-k): the
    candidates of [0, T_c) whose score is at least tau, at most k of them (the k largest by the
    top-k rule when more pass), plus the window [T_c, T). Ascending, int64; its length varies per
    row. Reading: tau is an absolute bound on the raw latent score, the same score top-k ranks;
    k is the capacity of the selection."""
    T_c = max(0, T - w)
    S = np.asarray(S_row[:T_c], dtype=np.float64)
    c = int(np.count_nonzero(S >= tau))
    top = topk_lowest_index(S, min(k, c))
    return np.concatenate([top, np.arange(T_c, T)]).astype(np.int64)


# ----------------------------------------------------------------------------------------------
# stage 3: rebuild the selected rows, then RoPE at their true positions
# ----------------------------------------------------------------------------------------------

def reconstruct(L_sel: np.ndarray, P_g: np.ndarray) -> np.ndarray:
    """Rebuilt pre-RoPE rows of one KV head: L_sel[n, r] . P_g^T, P_g = P[g*d:(g+1)*d] ([d, r]).
    (SALS, 技术框架 stage 3; 关键创新 3.)"""
    return L_sel @ P_g.T


def rope_theta(d: int, base: float) -> np.ndarray:
    """theta_i = base^(-2i/d), i in [0, d/2)."""
    i = np.arange(d // 2, dtype=np.float64)
    return np.float64(base) ** (-(2.0 * i) / d)


def rope(x: np.ndarray, pos, base: float) -> np.ndarray:
    """Rotate-half RoPE of rows x[n, d] at positions pos[n] (or a scalar).

    out_i = x_i cos(p theta_i) - x_{i+d/2} sin(p theta_i);
    out_{i+d/2} = x_{i+d/2} cos(p theta_i) + x_i sin(p theta_i).
    Angles are formed in fp64 and NumPy's cos/sin reduce them exactly enough at any position.
    (SALS, 问题定义 and abstract: RoPE is applied to keys after reconstruction.)
    """
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    n, d = x.shape
    half = d // 2
    p = np.broadcast_to(np.asarray(pos, dtype=np.float64), (n,))
    ang = p[:, None] * rope_theta(d, base)[None, :]
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[:, :half], x[:, half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=1)


# ----------------------------------------------------------------------------------------------
# stage 4: standard attention over the selected, rebuilt rows
# ----------------------------------------------------------------------------------------------

def _softmax(logits: np.ndarray) -> np.ndarray:
    m = logits.max()
    e = np.exp(logits - m)
    return e / e.sum()


def attend_selected(q: np.ndarray, Lk: np.ndarray, Lv: np.ndarray, Pk: np.ndarray, Pv: np.ndarray,
                    sel, T: int, base: float, H_kv: int, G: int):
    """Attention of one sequence over given selected sets (one per group).

    q[H_q, d] pre-RoPE, Lk/Lv[>=T, r], Pk/Pv[D, r] (fp64). sel: list/array of G index arrays.
    For query head h with KV head g = kv(h) and group s = grp(g):
      K_hat = RoPE(L_k[sel_s] . P_k[g]^T, sel_s);  V_hat = L_v[sel_s] . P_v[g]^T
      o_h = softmax(RoPE(q_h, T-1) . K_hat^T / sqrt(d)) . V_hat    (VL-Cache KiPr W1 formula)
    Returns (out[H_q, d], list of attention weight vectors per head).
    """
    H_q, d = q.shape
    out = np.zeros((H_q, d))
    weights = []
    for h in range(H_q):
        g = kv_head_of(h, H_q, H_kv)
        s = group_of(g, H_kv, G)
        idx = np.asarray(sel[s], dtype=np.int64)
        Kh = rope(reconstruct(Lk[idx], Pk[g * d:(g + 1) * d]), idx, base)
        Vh = reconstruct(Lv[idx], Pv[g * d:(g + 1) * d])
        qh = rope(q[h][None, :], T - 1, base)[0]
        pi = _softmax(Kh @ qh / np.sqrt(d))
        out[h] = pi @ Vh
        weights.append(pi)
    return out, weights


def decode_step(q, Lk, Lv, Pk, Pv, *, ctx: int, k: int, w: int, G: int, H_kv: int, base: float,
                dtype: str, batches: Optional[list] = None) -> Dict[str, object]:
    """One decode step of one layer, every sequence (or the listed ones).

    Stored inputs: q[B, H_q, d], Lk/Lv[B, ctx_cap, r], Pk/Pv[D, r]. Returns fp64
    ``out[B, H_q, d]``, ``sel[B, G, n_sel]`` (int64, ascending) and ``S[B, G, T_c]``
    (fp64 scores), where T_c = max(0, ctx - w) and n_sel = min(k, T_c) + ctx - T_c.
    Batches not listed in ``batches`` are left as NaN / -1.
    """
    qf = stored_to_f64(q, dtype)
    Pkf, Pvf = stored_to_f64(Pk, dtype), stored_to_f64(Pv, dtype)
    B, H_q, d = qf.shape
    T = int(ctx)
    T_c = max(0, T - w)
    n_sel = min(k, T_c) + (T - T_c)
    out = np.full((B, H_q, d), np.nan)
    sel = np.full((B, G, n_sel), -1, dtype=np.int64)
    S = np.full((B, G, T_c), np.nan)
    for b in (range(B) if batches is None else batches):
        Lkb = stored_to_f64(Lk[b, :T], dtype)
        Lvb = stored_to_f64(Lv[b, :T], dtype)
        qt = latent_query(qf[b], Pkf, H_kv, G)
        S[b] = latent_scores(qt, Lkb, T_c)
        sets = [select_tokens(S[b, s], T, k, w) for s in range(G)]
        sel[b] = np.stack(sets)
        out[b], _ = attend_selected(qf[b], Lkb, Lvb, Pkf, Pvf, sets, T, base, H_kv, G)
    return dict(out=out, sel=sel, S=S, T_c=T_c, n_sel=n_sel)


def decode_step_threshold(q, Lk, Lv, Pk, Pv, *, ctx: int, k: int, w: int, G: int, H_kv: int, base: float,
                          tau: float, dtype: str, batches: Optional[list] = None) -> Dict[str, object]:
    """decode_step with the threshold selection: per group the candidates scoring at least tau
    (at most k), plus the window. Returns ``out`` [B, H_q, d], ``sel`` (a list per sequence of G
    index arrays of varying length; None for sequences not computed), ``n_sel`` [B, G] and ``S``."""
    qf = stored_to_f64(q, dtype)
    Pkf, Pvf = stored_to_f64(Pk, dtype), stored_to_f64(Pv, dtype)
    B, H_q, d = qf.shape
    T = int(ctx)
    T_c = max(0, T - w)
    out = np.full((B, H_q, d), np.nan)
    sel = [None] * B
    n_sel = np.full((B, G), -1, dtype=np.int64)
    S = np.full((B, G, T_c), np.nan)
    for b in (range(B) if batches is None else batches):
        Lkb = stored_to_f64(Lk[b, :T], dtype)
        Lvb = stored_to_f64(Lv[b, :T], dtype)
        S[b] = latent_scores(latent_query(qf[b], Pkf, H_kv, G), Lkb, T_c)
        sel[b] = [select_tokens_threshold(S[b, s], T, k, w, tau) for s in range(G)]
        n_sel[b] = [len(x) for x in sel[b]]
        out[b], _ = attend_selected(qf[b], Lkb, Lvb, Pkf, Pvf, sel[b], T, base, H_kv, G)
    return dict(out=out, sel=sel, n_sel=n_sel, S=S, T_c=T_c)


# ----------------------------------------------------------------------------------------------
# the dense baseline the selection replaces: the whole latent cache rebuilt and rotated, then
# plain attention over every token
# ----------------------------------------------------------------------------------------------

def reconstruct_cache(L: np.ndarray, P: np.ndarray, t0: int, T: int, H_kv: int, base: Optional[float]):
    """Rows [t0, t0 + T) of one sequence rebuilt for every KV head: out[g, t - t0] = L[t] . P[g]^T,
    then rotated at the absolute position t when ``base`` is given (keys) and left as is when it is
    None (values). L[>= t0 + T, r], P[D, r] fp64; returns [H_kv, T, d].
    (SALS 问题定义 and abstract: an uncompressed attention needs every key rebuilt before RoPE;
    技术框架 stage 3 is the same product over the selected rows only.)"""
    d = P.shape[0] // H_kv
    pos = np.arange(t0, t0 + T)
    out = np.empty((H_kv, T, d))
    for g in range(H_kv):
        rows = reconstruct(L[t0:t0 + T], P[g * d:(g + 1) * d])
        out[g] = rope(rows, pos, base) if base is not None else rows
    return out


def dense_baseline(q, Lk, Lv, Pk, Pv, *, ctx: int, H_kv: int, base: float, dtype: str,
                   batches: Optional[list] = None) -> np.ndarray:
    """Attention of each query head over all ctx tokens of the rebuilt cache:
    o_h = softmax(RoPE(q_h, ctx-1) . K_g^T / sqrt(d)) . V_g with K_g, V_g = reconstruct_cache(...)
    over [0, ctx), g = kv(h). Stored inputs as in decode_step; returns fp64 out[B, H_q, d]."""
    qf = stored_to_f64(q, dtype)
    Pkf, Pvf = stored_to_f64(Pk, dtype), stored_to_f64(Pv, dtype)
    B, H_q, d = qf.shape
    out = np.full((B, H_q, d), np.nan)
    for b in (range(B) if batches is None else batches):
        K = reconstruct_cache(stored_to_f64(Lk[b, :ctx], dtype), Pkf, 0, ctx, H_kv, base)
        V = reconstruct_cache(stored_to_f64(Lv[b, :ctx], dtype), Pvf, 0, ctx, H_kv, None)
        for h in range(H_q):
            g = kv_head_of(h, H_q, H_kv)
            qh = rope(qf[b, h][None, :], ctx - 1, base)[0]
            out[b, h] = _softmax(K[g] @ qh / np.sqrt(d)) @ V[g]
    return out
