"""Frequency-domain outlier importance of a KV cache (FlashCache), fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: the FlashCache page (CVPR 2026 summary and English abstract): the energy of the KV
matrices along the token axis sits mostly at low frequencies; a low-pass filter extracts that
principal component; KV pairs that deviate strongly from it ("outlier KVs") are the ones to keep,
without any attention score, so the importance works with fused attention kernels.

Readings where the page is silent (each also listed in the design notes):
  * transform: the orthonormal DCT-II along the token axis of one (sequence, KV head) matrix
    X[T, d], C[t, f] = a_f cos(pi (2t + 1) f / (2T)), a_0 = sqrt(1/T), a_f = sqrt(2/T) (f > 0);
    the real, boundary-free form of a frequency decomposition of a finite sequence;
  * low-pass filter: keep the n_freq lowest frequencies, X_lp = C_F (C_F^T X) with C_F the first
    n_freq columns of C (per channel, every channel alike);
  * outlier score of token t: its deviation energy summed over the pair,
    I[t] = ||K[t] - K_lp[t]||^2 + ||V[t] - V_lp[t]||^2;
  * keys and values are used as stored (RoPE already applied), over the first ctx positions;
  * the kept set is the top k_keep of I (ties to the lowest index), as for kv_compact.
"""

from __future__ import annotations

import numpy as np

from .sals import stored_to_f64, topk_lowest_index


def dct_basis(T: int, n_freq: int) -> np.ndarray:
    """The first n_freq columns of the orthonormal DCT-II matrix of length T: [T, n_freq]."""
    t = np.arange(T, dtype=np.float64)[:, None]
    f = np.arange(n_freq, dtype=np.float64)[None, :]
    a = np.where(f == 0, np.sqrt(1.0 / T), np.sqrt(2.0 / T))
    return a * np.cos(np.pi * (2.0 * t + 1.0) * f / (2.0 * T))


def lowpass(X: np.ndarray, n_freq: int) -> np.ndarray:
    """Projection of X[T, d] onto its n_freq lowest DCT frequencies, per channel."""
    C = dct_basis(X.shape[0], n_freq)
    return C @ (C.T @ X)


def deviation_energy(X: np.ndarray, n_freq: int) -> np.ndarray:
    """||X[t] - X_lp[t]||^2 per token t of X[T, d]."""
    R = X - lowpass(X, n_freq)
    return (R * R).sum(axis=1)


def outlier_importance(K, V, *, ctx: int, n_freq: int, dtype: str = "bf16", pairs=None) -> np.ndarray:
    """I[b, g, t] = deviation energy of K[b, g, t] plus that of V[b, g, t] (t < ctx).

    Stored K, V [B, H_kv, ctx_cap, d]. Returns fp64 [B, H_kv, ctx]; pairs not listed in
    ``pairs`` (a list of (b, g)) stay NaN."""
    B, H_kv = K.shape[0], K.shape[1]
    I = np.full((B, H_kv, ctx), np.nan)
    todo = [(b, g) for b in range(B) for g in range(H_kv)] if pairs is None else pairs
    for b, g in todo:
        I[b, g] = (deviation_energy(stored_to_f64(K[b, g, :ctx], dtype), n_freq)
                   + deviation_energy(stored_to_f64(V[b, g, :ctx], dtype), n_freq))
    return I


def outlier_compact(K, V, *, ctx: int, n_freq: int, k_keep: int, dtype: str = "bf16", pairs=None):
    """The outlier importance, then the top k_keep per (sequence, KV head), ascending, and the
    gathered stored rows. Returns dict(importance, kept, Kc, Vc) as kv_compact does."""
    B, H_kv, _, d = K.shape
    I = outlier_importance(K, V, ctx=ctx, n_freq=n_freq, dtype=dtype, pairs=pairs)
    kept = np.full((B, H_kv, k_keep), -1, dtype=np.int64)
    Kc = np.zeros((B, H_kv, k_keep, d), dtype=K.dtype)
    Vc = np.zeros_like(Kc)
    todo = [(b, g) for b in range(B) for g in range(H_kv)] if pairs is None else pairs
    for b, g in todo:
        kept[b, g] = topk_lowest_index(I[b, g], k_keep)
        Kc[b, g], Vc[b, g] = K[b, g, kept[b, g]], V[b, g, kept[b, g]]
    return dict(importance=I, kept=kept, Kc=Kc, Vc=Vc)
