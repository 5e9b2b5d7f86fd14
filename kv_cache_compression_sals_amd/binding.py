"""Python binding of the C ABI in include/sals.h: same names, argument marshalling only.

Device tensors are torch tensors (PyTorch provides device memory and the current stream); every
step of the computation runs in the HIP kernels of libsals.so. Shapes are read from the tensors,
checked, and passed as the C structs; a non-OK status raises SalsError.
"""

from __future__ import annotations

import ctypes
from typing import Optional, Tuple

import torch

from ._lib import STATUS, KvcShape, SalsSelect, SalsShape, lib

_DTYPE = {torch.float32: 0, torch.bfloat16: 1}


class SalsError(RuntimeError):
    def __init__(self, fn: str, status: int):
        L = lib()
        msg = L.sals_status_string(status).decode()
        if status == 7:
            msg += f" (hipError_t {L.sals_last_hip_error()})"
        super().__init__(f"{fn}: {msg}")
        self.status = status
        self.name = STATUS.get(status, str(status))


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise SalsError(fn, status)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _dtype(*ts: torch.Tensor) -> int:
    dt = ts[0].dtype
    for t in ts:
        if t is not None and t.dtype != dt:
            raise ValueError(f"mixed dtypes: {dt} vs {t.dtype}")
    if dt not in _DTYPE:
        raise ValueError(f"unsupported dtype {dt}; use float32 or bfloat16")
    return _DTYPE[dt]


def _ws(nbytes: int, device, workspace: Optional[torch.Tensor]) -> torch.Tensor:
    if workspace is not None:
        return workspace
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


# ---- projection -----------------------------------------------------------------------------

def sals_project_kv(Xk: torch.Tensor, Pk: torch.Tensor, Lk: torch.Tensor, t0: int, *, d: int,
                    Xv: Optional[torch.Tensor] = None, Pv: Optional[torch.Tensor] = None,
                    Lv: Optional[torch.Tensor] = None, stream=None) -> None:
    """L[:, t0:t0+T] = X . P for K (and V). X [B, T, H_kv*d], P [H_kv*d, r], L [B, ctx_cap, r]."""
    B, T, D = Xk.shape
    r = Pk.shape[1]
    s = SalsShape(B, 1, D // d, d, r, _dtype(Xk, Pk, Lk, Xv, Pv, Lv))
    _check("sals_project_kv", lib().sals_project_kv(
        ctypes.byref(s), _ptr(Xk), _ptr(Xv), _ptr(Pk), _ptr(Pv), _ptr(Lk), _ptr(Lv), Lk.shape[1], t0, T,
        _stream(stream)))


# ---- decode step ----------------------------------------------------------------------------

def _decode_structs(q, Pk, r, k, w, G, dtype) -> Tuple[SalsShape, SalsSelect]:
    B, H_q, d = q.shape
    return SalsShape(B, H_q, Pk.shape[0] // d, d, r, dtype), SalsSelect(k, w, G)


def sals_decode_workspace_bytes(q: torch.Tensor, Pk: torch.Tensor, *, ctx: int, k: int, w: int,
                                G: int) -> int:
    s, sel = _decode_structs(q, Pk, Pk.shape[1], k, w, G, _dtype(q, Pk))
    n = ctypes.c_size_t(0)
    _check("sals_decode_workspace_bytes",
           lib().sals_decode_workspace_bytes(ctypes.byref(s), ctypes.byref(sel), ctx, ctypes.byref(n)))
    return n.value


def n_selected(ctx: int, k: int, w: int) -> int:
    T_c = max(0, ctx - w)
    return min(k, T_c) + (ctx - T_c)


def sals_decode_step(q: torch.Tensor, Lk: torch.Tensor, Lv: torch.Tensor, Pk: torch.Tensor,
                     Pv: torch.Tensor, *, ctx: int, k: int, w: int, G: int, rope_base: float = 10000.0,
                     out: Optional[torch.Tensor] = None, sel_out: Optional[torch.Tensor] = None,
                     want_sel: bool = False, workspace: Optional[torch.Tensor] = None,
                     stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """One SALS decode step. q [B, H_q, d] pre-RoPE; Lk/Lv [B, ctx_cap, r]; Pk/Pv [H_kv*d, r].
    Returns (out [B, H_q, d] fp32, sel [B, G, n_sel] int32 or None)."""
    dt = _dtype(q, Lk, Lv, Pk, Pv)
    B, H_q, d = q.shape
    s, sel = _decode_structs(q, Pk, Pk.shape[1], k, w, G, dt)
    if out is None:
        out = torch.empty((B, H_q, d), dtype=torch.float32, device=q.device)
    if sel_out is None and want_sel:
        sel_out = torch.empty((B, G, n_selected(ctx, k, w)), dtype=torch.int32, device=q.device)
    if workspace is None:
        workspace = _ws(sals_decode_workspace_bytes(q, Pk, ctx=ctx, k=k, w=w, G=G), q.device, None)
    _check("sals_decode_step", lib().sals_decode_step(
        ctypes.byref(s), ctypes.byref(sel), ctypes.c_float(rope_base), _ptr(q), _ptr(Lk), _ptr(Lv),
        _ptr(Pk), _ptr(Pv), Lk.shape[1], ctx, _ptr(out), _ptr(sel_out), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    return out, sel_out


def sals_decode_step_traced(q: torch.Tensor, Lk: torch.Tensor, Lv: torch.Tensor, Pk: torch.Tensor,
                            Pv: torch.Tensor, events, *, ctx: int, k: int, w: int, G: int,
                            rope_base: float = 10000.0, out: Optional[torch.Tensor] = None,
                            sel_out: Optional[torch.Tensor] = None, want_sel: bool = False,
                            workspace: Optional[torch.Tensor] = None,
                            stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """sals_decode_step that also records six timing events on the launch stream at its stage
    boundaries (before the latent query, the scoring, the top-k, rebuild + attention, the split
    merge, and after the last kernel). events: six torch.cuda.Event(enable_timing=True), each
    already recorded once so that its HIP event exists."""
    if len(events) != 6:
        raise ValueError("sals_decode_step_traced needs exactly 6 events")
    dt = _dtype(q, Lk, Lv, Pk, Pv)
    B, H_q, d = q.shape
    s, sel = _decode_structs(q, Pk, Pk.shape[1], k, w, G, dt)
    if out is None:
        out = torch.empty((B, H_q, d), dtype=torch.float32, device=q.device)
    if sel_out is None and want_sel:
        sel_out = torch.empty((B, G, n_selected(ctx, k, w)), dtype=torch.int32, device=q.device)
    if workspace is None:
        workspace = _ws(sals_decode_workspace_bytes(q, Pk, ctx=ctx, k=k, w=w, G=G), q.device, None)
    handles = (ctypes.c_void_p * 6)(*[e.cuda_event for e in events])
    if not all(handles):
        raise ValueError("record each event once before passing it in")
    _check("sals_decode_step_traced", lib().sals_decode_step_traced(
        ctypes.byref(s), ctypes.byref(sel), ctypes.c_float(rope_base), _ptr(q), _ptr(Lk), _ptr(Lv),
        _ptr(Pk), _ptr(Pv), Lk.shape[1], ctx, _ptr(out), _ptr(sel_out), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream), handles, 6))
    return out, sel_out


# ---- compaction -----------------------------------------------------------------------------

def kv_compact_workspace_bytes(K: torch.Tensor, Qobs: torch.Tensor, *, ctx: int, k_keep: int) -> int:
    B, H_kv, _, d = K.shape
    c = KvcShape(B, Qobs.shape[1], H_kv, d, _dtype(K, Qobs))
    n = ctypes.c_size_t(0)
    _check("kv_compact_workspace_bytes",
           lib().kv_compact_workspace_bytes(ctypes.byref(c), ctx, Qobs.shape[2], k_keep, ctypes.byref(n)))
    return n.value


def kv_compact(K: torch.Tensor, V: torch.Tensor, Qobs: torch.Tensor, *, ctx: int, k_keep: int,
               Kc: Optional[torch.Tensor] = None, Vc: Optional[torch.Tensor] = None,
               kept: Optional[torch.Tensor] = None, importance: Optional[torch.Tensor] = None,
               want_importance: bool = False, workspace: Optional[torch.Tensor] = None, stream=None):
    """K, V [B, H_kv, ctx_cap, d] post-RoPE; Qobs [B, H_q, w, d].
    Returns (Kc, Vc [B, H_kv, k_keep, d], kept [B, H_kv, k_keep] int32, importance or None)."""
    B, H_kv, ctx_cap, d = K.shape
    w = Qobs.shape[2]
    c = KvcShape(B, Qobs.shape[1], H_kv, d, _dtype(K, V, Qobs))
    dev = K.device
    if Kc is None:
        Kc = torch.empty((B, H_kv, k_keep, d), dtype=K.dtype, device=dev)
    if Vc is None:
        Vc = torch.empty((B, H_kv, k_keep, d), dtype=K.dtype, device=dev)
    if kept is None:
        kept = torch.empty((B, H_kv, k_keep), dtype=torch.int32, device=dev)
    if importance is None and want_importance:
        importance = torch.empty((B, H_kv, ctx), dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = _ws(kv_compact_workspace_bytes(K, Qobs, ctx=ctx, k_keep=k_keep), dev, None)
    _check("kv_compact", lib().kv_compact(
        ctypes.byref(c), _ptr(K), _ptr(V), _ptr(Qobs), w, ctx_cap, ctx, k_keep, _ptr(Kc), _ptr(Vc),
        _ptr(kept), _ptr(importance), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream)))
    return Kc, Vc, kept, importance


def sals_dense_decode_workspace_bytes(q: torch.Tensor, K: torch.Tensor, *, n: int) -> int:
    B, H_q, d = q.shape
    c = KvcShape(B, H_q, K.shape[1], d, _dtype(q, K))
    nb = ctypes.c_size_t(0)
    _check("sals_dense_decode_workspace_bytes",
           lib().sals_dense_decode_workspace_bytes(ctypes.byref(c), n, ctypes.byref(nb)))
    return nb.value


def sals_dense_decode(q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, *, n: Optional[int] = None,
                      out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                      stream=None) -> torch.Tensor:
    """q [B, H_q, d] post-RoPE; K, V [B, H_kv, stride, d]; attends over rows [0, n)."""
    B, H_q, d = q.shape
    stride = K.shape[2]
    n = stride if n is None else n
    c = KvcShape(B, H_q, K.shape[1], d, _dtype(q, K, V))
    if out is None:
        out = torch.empty((B, H_q, d), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = _ws(sals_dense_decode_workspace_bytes(q, K, n=n), q.device, None)
    _check("sals_dense_decode", lib().sals_dense_decode(
        ctypes.byref(c), _ptr(q), _ptr(K), _ptr(V), n, stride, _ptr(out), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


# ---- full reconstruction (the dense baseline) -------------------------------------------------

def sals_reconstruct_kv(Lk: torch.Tensor, Pk: torch.Tensor, K: torch.Tensor, *, t0: int, T: int, d: int,
                        rope_base: float = 10000.0, Lv: Optional[torch.Tensor] = None,
                        Pv: Optional[torch.Tensor] = None, V: Optional[torch.Tensor] = None,
                        q: Optional[torch.Tensor] = None, q_rot: Optional[torch.Tensor] = None,
                        q_pos: int = 0, stream=None) -> None:
    """K[:, :, t0:t0+T] = RoPE_t(L_k . P_k^T) (and V without RoPE); with q, q_rot = RoPE_{q_pos}(q).
    Lk/Lv [B, ctx_cap, r]; Pk/Pv [H_kv*d, r]; K/V [B, H_kv, stride_tokens, d]; q/q_rot [B, H_q, d]."""
    B, H_kv, stride, _ = K.shape
    H_q = q.shape[1] if q is not None else H_kv
    s = SalsShape(B, H_q, H_kv, d, Pk.shape[1], _dtype(Lk, Pk, K, Lv, Pv, V, q, q_rot))
    _check("sals_reconstruct_kv", lib().sals_reconstruct_kv(
        ctypes.byref(s), ctypes.c_float(rope_base), _ptr(Lk), _ptr(Lv), _ptr(Pk), _ptr(Pv), Lk.shape[1],
        t0, T, _ptr(K), _ptr(V), stride, _ptr(q), _ptr(q_rot), q_pos, _stream(stream)))


def kv_compact_from_importance(K: torch.Tensor, V: torch.Tensor, importance: torch.Tensor, *, k_keep: int,
                               ctx: Optional[int] = None, Kc: Optional[torch.Tensor] = None,
                               Vc: Optional[torch.Tensor] = None, kept: Optional[torch.Tensor] = None,
                               stream=None) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Keep the k_keep most important rows per (sequence, KV head) by a given importance
    [B, H_kv, ctx] fp32 (e.g. another layer's kv_compact importance). K, V [B, H_kv, ctx_cap, d].
    Returns (Kc, Vc [B, H_kv, k_keep, d], kept [B, H_kv, k_keep] int32)."""
    B, H_kv, cap, d = K.shape
    ctx = importance.shape[2] if ctx is None else ctx
    if importance.dtype != torch.float32:
        raise ValueError("importance must be float32")
    c = KvcShape(B, H_kv, H_kv, d, _dtype(K, V))
    if Kc is None:
        Kc = torch.empty((B, H_kv, k_keep, d), dtype=K.dtype, device=K.device)
    if Vc is None:
        Vc = torch.empty_like(Kc)
    if kept is None:
        kept = torch.empty((B, H_kv, k_keep), dtype=torch.int32, device=K.device)
    _check("kv_compact_from_importance", lib().kv_compact_from_importance(
        ctypes.byref(c), _ptr(K), _ptr(V), _ptr(importance), cap, ctx, k_keep, _ptr(Kc), _ptr(Vc),
        _ptr(kept), _stream(stream)))
    return Kc, Vc, kept


def kv_importance_sparsity_workspace_bytes(K: torch.Tensor, Qobs: torch.Tensor, *, ctx: int) -> int:
    B, H_kv, _, d = K.shape
    c = KvcShape(B, Qobs.shape[1], H_kv, d, _dtype(K, Qobs))
    n = ctypes.c_size_t(0)
    _check("kv_importance_sparsity_workspace_bytes",
           lib().kv_importance_sparsity_workspace_bytes(ctypes.byref(c), ctx, Qobs.shape[2], ctypes.byref(n)))
    return n.value


def kv_importance_sparsity(K: torch.Tensor, Qobs: torch.Tensor, *, ctx: int, p: float,
                           importance: Optional[torch.Tensor] = None, sparsity: Optional[torch.Tensor] = None,
                           workspace: Optional[torch.Tensor] = None, stream=None):
    """kv_compact's importance [B, H_kv, ctx] plus the post-vision sparsity [B, H_q] at threshold p.
    K [B, H_kv, ctx_cap, d]; Qobs [B, H_q, w, d]. Returns (importance, sparsity)."""
    B, H_kv, ctx_cap, d = K.shape
    H_q, w = Qobs.shape[1], Qobs.shape[2]
    c = KvcShape(B, H_q, H_kv, d, _dtype(K, Qobs))
    if importance is None:
        importance = torch.empty((B, H_kv, ctx), dtype=torch.float32, device=K.device)
    if sparsity is None:
        sparsity = torch.empty((B, H_q), dtype=torch.float32, device=K.device)
    if workspace is None:
        workspace = _ws(kv_importance_sparsity_workspace_bytes(K, Qobs, ctx=ctx), K.device, None)
    _check("kv_importance_sparsity", lib().kv_importance_sparsity(
        ctypes.byref(c), _ptr(K), _ptr(Qobs), w, ctx_cap, ctx, ctypes.c_float(p), _ptr(importance),
        _ptr(sparsity), _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))
    return importance, sparsity


def kv_layer_budgets(nonsparse, *, total: int, ctx: int):
    """Layer budgets floor(total * nu_l / sum(nu)) clamped to [1, ctx] (host arithmetic)."""
    import array
    nu = array.array("f", [float(x) for x in nonsparse])
    out = array.array("i", [0] * len(nu))
    nu_addr, _ = nu.buffer_info()
    out_addr, _ = out.buffer_info()
    _check("kv_layer_budgets", lib().kv_layer_budgets(nu_addr, len(nu), int(total), ctx, out_addr))
    return list(out)
