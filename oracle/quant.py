"""Importance-based mixed-precision KV cache (ZipVL) and attention over it.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: the ZipVL abstract: to ease the memory bottleneck of decoding, the KV cache is quantized
at mixed precision, with high-bit quantization for the caches of important tokens and low-bit
quantization for the less important ones. Importance comes from normalized attention scores
(here: any importance array, e.g. the one kv_compact returns).

Readings where the page is silent (each also listed in the design notes):
  * per (sequence, KV head), the n_hi most important positions (top-k, ties to the lowest index)
    are stored at 8 bits, every other position at 4 bits; both sets keep ascending positions;
  * quantization is per token, asymmetric and uniform over groups of 32 consecutive channels:
    mn, mx = the group's min and max; levels = 2^bits - 1; in fp32, with every operation rounded
    to nearest (no fused multiply-add):
        span = mx - mn;  inv = levels / span;  scale = span / levels
        code = clamp(floor((x - mn) * inv + 0.5), 0, levels)
    a group whose span is below 2^-96 (including a constant group) is stored with code 0,
    scale 0, zero point mn. The code is an integer decided in floating point, so it is fixed by
    these fp32 steps, which both sides take in the same precision;
  * dequantization: x_hat = mn + code * scale (fp64 here);
  * storage: codes_hi[2, B, H_kv, n_hi, d] (uint8, index 0 keys, 1 values),
    codes_lo[2, B, H_kv, n_lo, d / 2] (two 4-bit codes per byte, the even channel in the low
    nibble), params_*[2, B, H_kv, n, d / 32, 2] fp32 (scale, zero point), positions
    pos_hi[B, H_kv, n_hi], pos_lo[B, H_kv, n_lo] (int32, ascending);
  * decode: plain softmax attention of one query row over every stored token of both sets
    (the cache is post-RoPE, so positions play no further part).
"""

from __future__ import annotations

from typing import Dict

import numpy as np

from .sals import kv_head_of, stored_to_f64, topk_lowest_index

GROUP = 32
HI_BITS, LO_BITS = 8, 4
TINY_SPAN = np.float32(2.0 ** -96)


def quantize_group(x, bits: int):
    """Codes (int array), scale and zero point (np.float32) of one group of fp32 values."""
    x = np.asarray(x, dtype=np.float32)
    levels = np.float32((1 << bits) - 1)
    mn, mx = np.float32(x.min()), np.float32(x.max())
    span = np.float32(mx - mn)
    if not span >= TINY_SPAN:
        return np.zeros(x.shape, dtype=np.int64), np.float32(0.0), mn
    inv = np.float32(levels / span)
    scale = np.float32(span / levels)
    u = ((x - mn).astype(np.float32) * inv).astype(np.float32)
    codes = np.floor((u + np.float32(0.5)).astype(np.float32)).astype(np.int64)
    return np.clip(codes, 0, int(levels)), scale, mn


def quantize_rows(X, bits: int):
    """Per-row, per-group quantization of fp32 rows X[n, d]: codes [n, d] (int64) and params
    [n, d / 32, 2] fp32 (scale, zero point)."""
    X = np.asarray(X, dtype=np.float32)
    n, d = X.shape
    codes = np.zeros((n, d), dtype=np.int64)
    params = np.zeros((n, d // GROUP, 2), dtype=np.float32)
    for i in range(n):
        for gi in range(d // GROUP):
            c, s, z = quantize_group(X[i, gi * GROUP:(gi + 1) * GROUP], bits)
            codes[i, gi * GROUP:(gi + 1) * GROUP] = c
            params[i, gi] = (s, z)
    return codes, params


def dequantize_rows(codes, params) -> np.ndarray:
    """x_hat = zero point + code * scale, in fp64: [n, d]."""
    codes = np.asarray(codes, dtype=np.float64)
    n, d = codes.shape
    p = np.asarray(params, dtype=np.float64)
    scale = np.repeat(p[:, :, 0], GROUP, axis=1)
    zero = np.repeat(p[:, :, 1], GROUP, axis=1)
    return zero + codes * scale


def pack_nibbles(codes) -> np.ndarray:
    """4-bit codes [n, d] -> bytes [n, d / 2], channel 2j in the low nibble, 2j + 1 in the high."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(b) -> np.ndarray:
    b = np.asarray(b, dtype=np.uint8)
    out = np.empty((b.shape[0], 2 * b.shape[1]), dtype=np.int64)
    out[:, 0::2] = b & 0xF
    out[:, 1::2] = b >> 4
    return out


def split_positions(imp_row, ctx: int, n_hi: int):
    """(hi, lo): the n_hi most important of positions [0, ctx) and the rest, both ascending."""
    hi = topk_lowest_index(np.asarray(imp_row[:ctx], dtype=np.float64), n_hi)
    mask = np.ones(ctx, dtype=bool)
    mask[hi] = False
    return hi, np.nonzero(mask)[0]


def mixed_quantize(K, V, importance, *, ctx: int, n_hi: int, dtype: str = "bf16", pairs=None) -> Dict[str, object]:
    """The mixed-precision cache of stored K, V [B, H_kv, ctx_cap, d] under importance
    [B, H_kv, >= ctx] (layout in the module docstring). Pairs not listed stay zero / -1."""
    B, H, _, d = K.shape
    n_lo = ctx - n_hi
    out = dict(pos_hi=np.full((B, H, n_hi), -1, dtype=np.int64), pos_lo=np.full((B, H, n_lo), -1, dtype=np.int64),
               codes_hi=np.zeros((2, B, H, n_hi, d), dtype=np.uint8),
               params_hi=np.zeros((2, B, H, n_hi, d // GROUP, 2), dtype=np.float32),
               codes_lo=np.zeros((2, B, H, n_lo, d // 2), dtype=np.uint8),
               params_lo=np.zeros((2, B, H, n_lo, d // GROUP, 2), dtype=np.float32))
    todo = [(b, g) for b in range(B) for g in range(H)] if pairs is None else pairs
    for b, g in todo:
        hi, lo = split_positions(importance[b, g], ctx, n_hi)
        out["pos_hi"][b, g], out["pos_lo"][b, g] = hi, lo
        for x, X in enumerate((K, V)):
            rows = stored_to_f64(X[b, g, :ctx], dtype).astype(np.float32)
            c, p = quantize_rows(rows[hi], HI_BITS)
            out["codes_hi"][x, b, g], out["params_hi"][x, b, g] = c.astype(np.uint8), p
            c, p = quantize_rows(rows[lo], LO_BITS)
            out["codes_lo"][x, b, g], out["params_lo"][x, b, g] = pack_nibbles(c), p
    return out


def mixed_rows(m: Dict[str, object], x: int, b: int, g: int) -> np.ndarray:
    """Dequantized rows of tensor x (0 keys, 1 values) of pair (b, g), hi set then lo set: [n, d]."""
    hi = dequantize_rows(m["codes_hi"][x, b, g], m["params_hi"][x, b, g])
    lo = dequantize_rows(unpack_nibbles(m["codes_lo"][x, b, g]), m["params_lo"][x, b, g])
    return np.concatenate([hi, lo], axis=0)


def mixed_decode(q, m: Dict[str, object], *, H_kv: int, dtype: str = "bf16", pairs=None) -> np.ndarray:
    """o[b, h] = softmax(q[b, h] . K_hat^T / sqrt(d)) . V_hat over every token of both sets of
    KV head kv(h). Stored q [B, H_q, d] (RoPE applied). fp64 [B, H_q, d]; pairs = list of (b, h)."""
    qf = stored_to_f64(q, dtype)
    B, H_q, d = qf.shape
    out = np.full((B, H_q, d), np.nan)
    todo = [(b, h) for b in range(B) for h in range(H_q)] if pairs is None else pairs
    for b, h in todo:
        g = kv_head_of(h, H_q, H_kv)
        Kh, Vh = mixed_rows(m, 0, b, g), mixed_rows(m, 1, b, g)
        lg = Kh @ qf[b, h] / np.sqrt(d)
        e = np.exp(lg - lg.max())
        out[b, h] = (e / e.sum()) @ Vh
    return out
