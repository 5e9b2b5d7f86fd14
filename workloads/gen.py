"""Seeded input generators (shared by the HIP path's tests/bench and the oracle).

Every array is drawn from ``rng(cfg_id, layer, name)``: a PCG64 stream keyed by
(1234, config id, layer, crc32(name)), so each array is independent of the
order in which arrays are drawn and of the batch size asked for (sequence b of
a smaller batch equals sequence b of the full batch).

bf16 arrays are returned as ``uint16`` bit patterns (NumPy has no bf16 dtype);
fp32 arrays as ``float32``. The encoder below rounds fp32 to bf16 with
round-to-nearest-even; the stored bits *are* the input, so whatever rounding
happened on the way does not matter to either side.

Workload recipes follow the configurations the SALS page evaluates at (4K and
32K sequences on Llama-2-7B / Llama-3.1-8B-shaped attention layers, a 128K
long-context check) and the VL-Cache page's post-prefill compaction setting
(a VLM prompt of visual tokens followed by text). Low-rank-plus-noise key and
value rows model the SALS abstract's statement that the KV cache is low rank
along the hidden dimension.
"""

from __future__ import annotations

import zlib
from dataclasses import dataclass, replace
from typing import Dict, Optional

import numpy as np

SEED_ROOT = 1234


def rng(cfg_id: int, layer: int, name: str) -> np.random.Generator:
    """Independent PCG64 stream for one named array of one config/layer."""
    ss = np.random.SeedSequence([SEED_ROOT, int(cfg_id), int(layer), zlib.crc32(name.encode())])
    return np.random.Generator(np.random.PCG64(ss))


# ----------------------------------------------------------------------------------------------
# bf16 codec (storage format only)
# ----------------------------------------------------------------------------------------------

def f32_to_bf16_bits(x) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return the 16-bit patterns.

    Inputs must be finite (the workloads never produce NaN/Inf).
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    rounded = u + np.uint32(0x7FFF) + lsb
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _store(x, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "bf16":
        return f32_to_bf16_bits(np.asarray(x, dtype=np.float32))
    raise ValueError(dtype)


def _stored_to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_bits_to_f32(a).astype(np.float64) if dtype == "bf16" else a.astype(np.float64)


# ----------------------------------------------------------------------------------------------
# configurations
# ----------------------------------------------------------------------------------------------

@dataclass(frozen=True)
class DecodeConfig:
    """One decode workload: a latent KV cache plus one query token per sequence."""

    name: str
    cfg_id: int
    B: int
    H_q: int
    H_kv: int
    d: int
    ctx: int
    r: int
    G: int  # selection groups per sequence
    k: int  # top-k over the non-window positions
    w: int  # recent window, always kept
    dtype: str  # "f32" | "bf16"
    rank: int  # rank of the synthetic pre-RoPE K/V rows
    noise: float  # std of the additive Gaussian noise (signal entries have unit variance)
    outliers: int  # number of outlier channels (scaled x8 after noise)
    p_kind: str  # "orthonormal" (QR of a Gaussian) | "svd" (top right singular vectors of a calibration draw)
    base: float = 10000.0
    layers: int = 1
    calib_tokens: int = 4096

    @property
    def D(self) -> int:
        return self.H_kv * self.d

    def with_(self, **kw) -> "DecodeConfig":
        return replace(self, **kw)


@dataclass(frozen=True)
class CompactConfig:
    """Post-prefill compaction workload (VLM-shaped prompt: visual grid then text)."""

    name: str
    cfg_id: int
    B: int
    H_q: int
    H_kv: int
    d: int
    ctx: int
    w: int  # number of trailing observation queries
    keep_frac: float
    n_visual: int
    grid_h: int
    grid_w: int
    clusters_h: int
    clusters_w: int
    jitter: float
    dtype: str = "bf16"

    @property
    def k_keep(self) -> int:
        return int(np.floor(self.keep_frac * self.ctx))

    def with_(self, **kw) -> "CompactConfig":
        return replace(self, **kw)


C1 = DecodeConfig("c1_tiny_f32_ctx512", 0, B=1, H_q=4, H_kv=4, d=64, ctx=512, r=64, G=1, k=64, w=16,
                  dtype="f32", rank=32, noise=0.05, outliers=0, p_kind="orthonormal")
C2 = DecodeConfig("c2_llama2_7b_ctx4k", 1, B=8, H_q=32, H_kv=32, d=128, ctx=4096, r=512, G=1, k=512,
                  w=64, dtype="bf16", rank=384, noise=0.05, outliers=4, p_kind="svd")
C3 = DecodeConfig("c3_llama31_8b_ctx32k", 2, B=4, H_q=32, H_kv=8, d=128, ctx=32768, r=256, G=8,
                  k=2048, w=128, dtype="bf16", rank=192, noise=0.05, outliers=0, p_kind="svd")
C4 = CompactConfig("c4_vlm_compact_ctx16k", 3, B=16, H_q=32, H_kv=32, d=128, ctx=16384, w=64,
                   keep_frac=0.1, n_visual=14336, grid_h=112, grid_w=128, clusters_h=8, clusters_w=8,
                   jitter=0.1)
C5 = DecodeConfig("c5_llama31_8b_ctx128k_32layers", 4, B=1, H_q=32, H_kv=8, d=128, ctx=131072, r=256,
                  G=8, k=4096, w=128, dtype="bf16", rank=192, noise=0.05, outliers=0, p_kind="svd",
                  layers=32)

CONFIGS = {"c1": C1, "c2": C2, "c3": C3, "c4": C4, "c5": C5}


# ----------------------------------------------------------------------------------------------
# decode workloads
# ----------------------------------------------------------------------------------------------

def _mixing(cfg: DecodeConfig, layer: int, which: str):
    """Per-layer mixing matrix A[rank, D] ~ N(0, 1/rank) and the outlier channel indices."""
    A = rng(cfg.cfg_id, layer, f"A_{which}").standard_normal((cfg.rank, cfg.D), dtype=np.float32)
    A *= np.float32(1.0 / np.sqrt(cfg.rank))
    outl = np.sort(rng(cfg.cfg_id, layer, f"outliers_{which}").choice(cfg.D, cfg.outliers, replace=False)) \
        if cfg.outliers else np.zeros(0, dtype=np.int64)
    return A, outl


def _rows(cfg: DecodeConfig, layer: int, which: str, tag: str, n: int, A, outl) -> np.ndarray:
    """n synthetic pre-RoPE rows: Z·A + noise·N, outlier channels scaled x8 after noise (fp32)."""
    Z = rng(cfg.cfg_id, layer, f"Z_{which}/{tag}").standard_normal((n, cfg.rank), dtype=np.float32)
    X = Z @ A
    N = rng(cfg.cfg_id, layer, f"N_{which}/{tag}").standard_normal((n, cfg.D), dtype=np.float32)
    X += np.float32(cfg.noise) * N
    if len(outl):
        X[:, outl] *= np.float32(8.0)
    return X


def _projection(cfg: DecodeConfig, layer: int, which: str, A, outl) -> np.ndarray:
    """P[D, r] as stored. Orthonormal columns (sign-fixed QR) or the top-r right singular
    vectors of a calibration draw of the same rows (both options named on the SALS page)."""
    if cfg.p_kind == "orthonormal":
        g = rng(cfg.cfg_id, layer, f"P_{which}").standard_normal((cfg.D, cfg.r))
        q, rr = np.linalg.qr(g)
        q = q * np.sign(np.diag(rr))[None, :]
        P = q
    elif cfg.p_kind == "svd":
        Xc = _rows(cfg, layer, which, "calib", cfg.calib_tokens, A, outl).astype(np.float64)
        _, _, vt = np.linalg.svd(Xc, full_matrices=False)
        P = vt[: cfg.r].T
    else:
        raise ValueError(cfg.p_kind)
    return _store(P, cfg.dtype)


def decode_case(cfg: DecodeConfig, layer: int = 0, B: Optional[int] = None, ctx: Optional[int] = None,
                ctx_cap: Optional[int] = None, with_x: bool = False) -> Dict[str, object]:
    """One layer of a decode workload.

    Returns stored arrays ``q[B,H_q,d]``, ``Lk, Lv[B,ctx_cap,r]`` (rows >= ctx are zero padding
    that the path must never read into a result), ``Pk, Pv[D,r]``, plus the scalar knobs.
    The cache holds the latent of the synthetic rows under the stored P (the content an
    upstream projection leaves there); it is formed once here so both sides read the same bytes.
    ``with_x`` also returns the pre-RoPE rows ``Xk, Xv[B,ctx,D]`` (fp32) for inspection.
    """
    B = cfg.B if B is None else B
    ctx = cfg.ctx if ctx is None else ctx
    ctx_cap = ctx if ctx_cap is None else ctx_cap
    assert 1 <= ctx <= ctx_cap
    out: Dict[str, object] = dict(cfg=cfg, layer=layer, B=B, ctx=ctx, ctx_cap=ctx_cap, H_q=cfg.H_q,
                                  H_kv=cfg.H_kv, d=cfg.d, r=cfg.r, G=cfg.G, k=cfg.k, w=cfg.w,
                                  base=cfg.base, dtype=cfg.dtype)
    for which in ("k", "v"):
        A, outl = _mixing(cfg, layer, which)
        P = _projection(cfg, layer, which, A, outl)
        P64 = _stored_to_f64(P, cfg.dtype)
        L = np.zeros((B, ctx_cap, cfg.r), dtype=np.float32 if cfg.dtype == "f32" else np.uint16)
        xs = []
        for b in range(B):
            X = _rows(cfg, layer, which, f"seq{b}", ctx, A, outl)
            if cfg.dtype == "f32":
                Lb = X.astype(np.float64) @ P64
            else:
                Lb = X @ P64.astype(np.float32)
            L[b, :ctx] = _store(Lb, cfg.dtype)
            if with_x:
                xs.append(X)
        out["P" + which] = P
        out["L" + which] = L
        if with_x:
            out["X" + which] = np.stack(xs)
    q = rng(cfg.cfg_id, layer, "q").standard_normal((max(B, cfg.B), cfg.H_q, cfg.d), dtype=np.float32)[:B]
    out["q"] = _store(q, cfg.dtype)
    return out


def project_case(cfg: DecodeConfig, layer: int = 0, B: Optional[int] = None,
                 T: Optional[int] = None) -> Dict[str, object]:
    """Inputs of the projection step: stored pre-RoPE rows ``Xk, Xv[B,T,D]`` and ``Pk, Pv[D,r]``."""
    B = cfg.B if B is None else B
    T = cfg.ctx if T is None else T
    out: Dict[str, object] = dict(cfg=cfg, B=B, T=T, D=cfg.D, r=cfg.r, dtype=cfg.dtype)
    for which in ("k", "v"):
        A, outl = _mixing(cfg, layer, which)
        out["P" + which] = _projection(cfg, layer, which, A, outl)
        X = np.stack([_rows(cfg, layer, which, f"seq{b}", T, A, outl) for b in range(B)])
        out["X" + which] = _store(X, cfg.dtype)
    return out


# ----------------------------------------------------------------------------------------------
# compaction workload (VLM-shaped prompt)
# ----------------------------------------------------------------------------------------------

def _vlm_rows(cfg: CompactConfig, b: int, which: str, ctx: int) -> np.ndarray:
    """[H_kv, ctx, d] fp32 rows for sequence b.

    Visual tokens 0..n_visual-1 lie row-major on a grid_h x grid_w grid; the grid is cut into
    clusters_h x clusters_w blocks, each block one cluster with its own N(0, I) centroid per
    (sequence, head); every visual token is its centroid plus N(0, jitter^2) noise. The remaining
    tokens are i.i.d. N(0, I) text tokens.
    """
    H, d = cfg.H_kv, cfg.d
    nv = min(cfg.n_visual, ctx)
    n_cl = cfg.clusters_h * cfg.clusters_w
    cent = rng(cfg.cfg_id, b, f"centroid_{which}").standard_normal((H, n_cl, d), dtype=np.float32)
    t = np.arange(nv)
    row, col = t // cfg.grid_w, t % cfg.grid_w
    bh, bw = cfg.grid_h // cfg.clusters_h, cfg.grid_w // cfg.clusters_w
    cl = (row // bh) * cfg.clusters_w + (col // bw)
    X = np.empty((H, ctx, d), dtype=np.float32)
    jit = rng(cfg.cfg_id, b, f"jitter_{which}").standard_normal((H, nv, d), dtype=np.float32)
    X[:, :nv] = cent[:, cl, :] + np.float32(cfg.jitter) * jit
    if ctx > nv:
        X[:, nv:] = rng(cfg.cfg_id, b, f"text_{which}").standard_normal((H, ctx - nv, d), dtype=np.float32)
    return X


def compact_case(cfg: CompactConfig, B: Optional[int] = None, ctx: Optional[int] = None,
                 ctx_cap: Optional[int] = None, threads: int = 1) -> Dict[str, object]:
    """Stored ``K, V[B,H_kv,ctx_cap,d]`` (post-RoPE, as a cache holds them), observation queries
    ``Qobs[B,H_q,w,d]`` (the last w prompt positions), decode query ``q[B,H_q,d]`` (post-RoPE)."""
    B = cfg.B if B is None else B
    ctx = cfg.ctx if ctx is None else ctx
    ctx_cap = ctx if ctx_cap is None else ctx_cap
    assert 1 <= ctx <= ctx_cap
    K = np.zeros((B, cfg.H_kv, ctx_cap, cfg.d), dtype=np.uint16)
    V = np.zeros_like(K)

    def one(b):
        K[b, :, :ctx] = f32_to_bf16_bits(_vlm_rows(cfg, b, "k", ctx))
        V[b, :, :ctx] = f32_to_bf16_bits(_vlm_rows(cfg, b, "v", ctx))

    if threads > 1:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(one, range(B)))
    else:
        for b in range(B):
            one(b)
    nb = max(B, cfg.B)
    Qobs = rng(cfg.cfg_id, 0, "Qobs").standard_normal((nb, cfg.H_q, cfg.w, cfg.d), dtype=np.float32)[:B]
    q = rng(cfg.cfg_id, 0, "q_dec").standard_normal((nb, cfg.H_q, cfg.d), dtype=np.float32)[:B]
    return dict(cfg=cfg, B=B, ctx=ctx, ctx_cap=ctx_cap, H_q=cfg.H_q, H_kv=cfg.H_kv, d=cfg.d, w=cfg.w,
                k_keep=int(np.floor(cfg.keep_frac * ctx)), dtype=cfg.dtype, K=K, V=V,
                Qobs=f32_to_bf16_bits(Qobs), q=f32_to_bf16_bits(q))
