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


def _expect(t: Optional[torch.Tensor], name: str, shape, dtype=None) -> None:
    """ValueError unless t has exactly this shape (and dtype). The C ABI sees only pointers, so a
    tensor of the wrong size would be read or written out of bounds on the device."""
    if t is None:
        return
    if tuple(t.shape) != tuple(int(x) for x in shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(int(x) for x in shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")


def _check_decode_args(q, Lk, Lv, Pk, Pv, ctx):
    """Shapes of one decode step's inputs: q [B, H_q, d], Pk and Pv [H_kv d, r], Lk and Lv
    [B, ctx_cap, r] with ctx <= ctx_cap."""
    if q.dim() != 3 or Pk.dim() != 2 or Lk.dim() != 3:
        raise ValueError("q must be [B, H_q, d], Pk [H_kv*d, r], Lk [B, ctx_cap, r]")
    B, H_q, d = q.shape
    D, r = Pk.shape
    if D % d != 0 or D // d < 1:
        raise ValueError(f"Pk rows {D} are not a multiple of d = {d}")
    _expect(Pv, "Pv", (D, r))
    _expect(Lk, "Lk", (B, Lk.shape[1], r))
    _expect(Lv, "Lv", tuple(Lk.shape))
    if not 1 <= ctx <= Lk.shape[1]:
        raise ValueError(f"ctx = {ctx} outside [1, ctx_cap = {Lk.shape[1]}]")


# ---- projection -----------------------------------------------------------------------------

def sals_project_kv(Xk: torch.Tensor, Pk: torch.Tensor, Lk: torch.Tensor, t0: int, *, d: int,
                    Xv: Optional[torch.Tensor] = None, Pv: Optional[torch.Tensor] = None,
                    Lv: Optional[torch.Tensor] = None, stream=None) -> None:
    """L[:, t0:t0+T] = X . P for K (and V). X [B, T, H_kv*d], P [H_kv*d, r], L [B, ctx_cap, r]."""
    if Xk.dim() != 3 or Pk.dim() != 2 or Lk.dim() != 3:
        raise ValueError("Xk must be [B, T, H_kv*d], Pk [H_kv*d, r], Lk [B, ctx_cap, r]")
    B, T, D = Xk.shape
    r = Pk.shape[1]
    if D % d != 0:
        raise ValueError(f"row width {D} is not a multiple of d = {d}")
    _expect(Pk, "Pk", (D, r))
    _expect(Lk, "Lk", (B, Lk.shape[1], r))
    _expect(Xv, "Xv", tuple(Xk.shape))
    _expect(Pv, "Pv", tuple(Pk.shape))
    _expect(Lv, "Lv", tuple(Lk.shape))
    if t0 < 0 or t0 + T > Lk.shape[1]:
        raise ValueError(f"rows [{t0}, {t0 + T}) do not fit ctx_cap = {Lk.shape[1]}")
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
    _check_decode_args(q, Lk, Lv, Pk, Pv, ctx)
    B, H_q, d = q.shape
    s, sel = _decode_structs(q, Pk, Pk.shape[1], k, w, G, dt)
    _expect(out, "out", (B, H_q, d), torch.float32)
    _expect(sel_out, "sel_out", (B, G, n_selected(ctx, k, w)), torch.int32)
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


def sals_decode_step_threshold(q: torch.Tensor, Lk: torch.Tensor, Lv: torch.Tensor, Pk: torch.Tensor,
                               Pv: torch.Tensor, *, ctx: int, k: int, w: int, G: int, tau: float,
                               rope_base: float = 10000.0, out: Optional[torch.Tensor] = None,
                               sel_out: Optional[torch.Tensor] = None, n_sel_out: Optional[torch.Tensor] = None,
                               want_sel: bool = False, workspace: Optional[torch.Tensor] = None, stream=None):
    """One SALS decode step with threshold selection: per row the candidates scoring at least tau
    (at most k), plus the window. Returns (out [B, H_q, d] fp32, sel [B, G, n_max] int32 padded
    with -1 or None, n_sel [B, G] int32)."""
    dt = _dtype(q, Lk, Lv, Pk, Pv)
    _check_decode_args(q, Lk, Lv, Pk, Pv, ctx)
    B, H_q, d = q.shape
    s, sel = _decode_structs(q, Pk, Pk.shape[1], k, w, G, dt)
    n_max = n_selected(ctx, k, w)
    _expect(out, "out", (B, H_q, d), torch.float32)
    _expect(sel_out, "sel_out", (B, G, n_max), torch.int32)
    _expect(n_sel_out, "n_sel_out", (B, G), torch.int32)
    if out is None:
        out = torch.empty((B, H_q, d), dtype=torch.float32, device=q.device)
    if sel_out is None and want_sel:
        sel_out = torch.empty((B, G, n_max), dtype=torch.int32, device=q.device)
    if n_sel_out is None:
        n_sel_out = torch.empty((B, G), dtype=torch.int32, device=q.device)
    if workspace is None:
        workspace = _ws(sals_decode_workspace_bytes(q, Pk, ctx=ctx, k=k, w=w, G=G), q.device, None)
    _check("sals_decode_step_threshold", lib().sals_decode_step_threshold(
        ctypes.byref(s), ctypes.byref(sel), ctypes.c_float(tau), ctypes.c_float(rope_base), _ptr(q), _ptr(Lk),
        _ptr(Lv), _ptr(Pk), _ptr(Pv), Lk.shape[1], ctx, _ptr(out), _ptr(sel_out), _ptr(n_sel_out), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    return out, sel_out, n_sel_out


NOALLOC_SCRATCH_BYTES = 16 << 20


def sals_decode_step_noalloc(q: torch.Tensor, Lk: torch.Tensor, Lv: torch.Tensor, Pk: torch.Tensor,
                             Pv: torch.Tensor, *, ctx: int, k: int, w: int, G: int, out: torch.Tensor,
                             sel_out: Optional[torch.Tensor] = None, rope_base: float = 10000.0,
                             stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """sals_decode_step without a workspace: the library's own per-GPU scratch array serves as the
    workspace (for callers that cannot allocate). out [B, H_q, d] fp32 and sel_out (optional,
    [B, G, n_sel] int32) must be given; nothing is allocated here or in the library."""
    dt = _dtype(q, Lk, Lv, Pk, Pv)
    _check_decode_args(q, Lk, Lv, Pk, Pv, ctx)
    B, H_q, d = q.shape
    s, sel = _decode_structs(q, Pk, Pk.shape[1], k, w, G, dt)
    _expect(out, "out", (B, H_q, d), torch.float32)
    _expect(sel_out, "sel_out", (B, G, n_selected(ctx, k, w)), torch.int32)
    _check("sals_decode_step_noalloc", lib().sals_decode_step_noalloc(
        ctypes.byref(s), ctypes.byref(sel), ctypes.c_float(rope_base), _ptr(q), _ptr(Lk), _ptr(Lv),
        _ptr(Pk), _ptr(Pv), Lk.shape[1], ctx, _ptr(out), _ptr(sel_out), _stream(stream)))
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
    _check_decode_args(q, Lk, Lv, Pk, Pv, ctx)
    B, H_q, d = q.shape
    s, sel = _decode_structs(q, Pk, Pk.shape[1], k, w, G, dt)
    _expect(out, "out", (B, H_q, d), torch.float32)
    _expect(sel_out, "sel_out", (B, G, n_selected(ctx, k, w)), torch.int32)
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
    if K.dim() != 4 or Qobs.dim() != 4:
        raise ValueError("K, V must be [B, H_kv, ctx_cap, d] and Qobs [B, H_q, w, d]")
    B, H_kv, ctx_cap, d = K.shape
    w = Qobs.shape[2]
    _expect(V, "V", tuple(K.shape))
    _expect(Qobs, "Qobs", (B, Qobs.shape[1], w, d))
    _expect(Kc, "Kc", (B, H_kv, k_keep, d), K.dtype)
    _expect(Vc, "Vc", (B, H_kv, k_keep, d), K.dtype)
    _expect(kept, "kept", (B, H_kv, k_keep), torch.int32)
    _expect(importance, "importance", (B, H_kv, ctx), torch.float32)
    if not 1 <= ctx <= ctx_cap:
        raise ValueError(f"ctx = {ctx} outside [1, ctx_cap = {ctx_cap}]")
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
    if q.dim() != 3 or K.dim() != 4:
        raise ValueError("q must be [B, H_q, d] and K, V [B, H_kv, stride, d]")
    B, H_q, d = q.shape
    stride = K.shape[2]
    n = stride if n is None else n
    _expect(K, "K", (B, K.shape[1], stride, d))
    _expect(V, "V", tuple(K.shape))
    _expect(out, "out", (B, H_q, d), torch.float32)
    if not 1 <= n <= stride:
        raise ValueError(f"n = {n} outside [1, stride = {stride}]")
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
    if K.dim() != 4 or Lk.dim() != 3 or Pk.dim() != 2:
        raise ValueError("Lk must be [B, ctx_cap, r], Pk [H_kv*d, r], K [B, H_kv, stride, d]")
    B, H_kv, stride, _ = K.shape
    H_q = q.shape[1] if q is not None else H_kv
    r = Pk.shape[1]
    _expect(Pk, "Pk", (H_kv * d, r))
    _expect(K, "K", (B, H_kv, stride, d))
    _expect(Lk, "Lk", (B, Lk.shape[1], r))
    _expect(Lv, "Lv", tuple(Lk.shape))
    _expect(Pv, "Pv", tuple(Pk.shape))
    _expect(V, "V", tuple(K.shape))
    if q is not None:
        _expect(q, "q", (B, H_q, d))
        _expect(q_rot, "q_rot", tuple(q.shape))
    if t0 < 0 or t0 + T > min(Lk.shape[1], stride):
        raise ValueError(f"rows [{t0}, {t0 + T}) do not fit ctx_cap = {Lk.shape[1]} and stride = {stride}")
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
    if K.dim() != 4 or importance.dim() != 3:
        raise ValueError("K, V must be [B, H_kv, ctx_cap, d] and importance [B, H_kv, ctx]")
    B, H_kv, cap, d = K.shape
    ctx = importance.shape[2] if ctx is None else ctx
    if importance.dtype != torch.float32:
        raise ValueError("importance must be float32")
    if importance.shape[0] != B or importance.shape[1] != H_kv or importance.shape[2] < ctx:
        raise ValueError(f"importance: shape {tuple(importance.shape)}, expected ({B}, {H_kv}, >= {ctx})")
    if not importance.is_contiguous() or importance.shape[2] != ctx:
        importance = importance[:, :, :ctx].contiguous()
    _expect(V, "V", tuple(K.shape))
    _expect(Kc, "Kc", (B, H_kv, k_keep, d), K.dtype)
    _expect(Vc, "Vc", (B, H_kv, k_keep, d), K.dtype)
    _expect(kept, "kept", (B, H_kv, k_keep), torch.int32)
    if not 1 <= ctx <= cap:
        raise ValueError(f"ctx = {ctx} outside [1, ctx_cap = {cap}]")
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
    if K.dim() != 4 or Qobs.dim() != 4:
        raise ValueError("K must be [B, H_kv, ctx_cap, d] and Qobs [B, H_q, w, d]")
    B, H_kv, ctx_cap, d = K.shape
    H_q, w = Qobs.shape[1], Qobs.shape[2]
    _expect(Qobs, "Qobs", (B, H_q, w, d))
    _expect(importance, "importance", (B, H_kv, ctx), torch.float32)
    _expect(sparsity, "sparsity", (B, H_q), torch.float32)
    if not 1 <= ctx <= ctx_cap:
        raise ValueError(f"ctx = {ctx} outside [1, ctx_cap = {ctx_cap}]")
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


# ---- frequency-domain outlier importance ------------------------------------------------------

def kv_outlier_importance_workspace_bytes(K: torch.Tensor, *, ctx: int, n_freq: int) -> int:
    B, H_kv, _, d = K.shape
    c = KvcShape(B, H_kv, H_kv, d, _dtype(K))
    n = ctypes.c_size_t(0)
    _check("kv_outlier_importance_workspace_bytes",
           lib().kv_outlier_importance_workspace_bytes(ctypes.byref(c), ctx, n_freq, ctypes.byref(n)))
    return n.value


def kv_outlier_importance(K: torch.Tensor, V: torch.Tensor, *, ctx: int, n_freq: int,
                          importance: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                          stream=None) -> torch.Tensor:
    """Deviation energy of each cached (key, value) pair from the low-pass of the cache along the
    tokens (the n_freq lowest DCT-II frequencies). K, V [B, H_kv, ctx_cap, d] bf16.
    Returns importance [B, H_kv, ctx] fp32, to rank pairs with kv_compact_from_importance."""
    if K.dim() != 4:
        raise ValueError("K, V must be [B, H_kv, ctx_cap, d]")
    B, H_kv, ctx_cap, d = K.shape
    _expect(V, "V", tuple(K.shape))
    _expect(importance, "importance", (B, H_kv, ctx), torch.float32)
    if not 1 <= ctx <= ctx_cap:
        raise ValueError(f"ctx = {ctx} outside [1, ctx_cap = {ctx_cap}]")
    c = KvcShape(B, H_kv, H_kv, d, _dtype(K, V))
    if importance is None:
        importance = torch.empty((B, H_kv, ctx), dtype=torch.float32, device=K.device)
    if workspace is None:
        workspace = _ws(kv_outlier_importance_workspace_bytes(K, ctx=ctx, n_freq=n_freq), K.device, None)
    _check("kv_outlier_importance", lib().kv_outlier_importance(
        ctypes.byref(c), _ptr(K), _ptr(V), ctx_cap, ctx, n_freq, _ptr(importance), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    return importance


# ---- importance-based mixed-precision cache ---------------------------------------------------

def kv_quantize_mixed(K: torch.Tensor, V: torch.Tensor, importance: torch.Tensor, *, n_hi: int,
                      ctx: Optional[int] = None, out: Optional[dict] = None, stream=None) -> dict:
    """Stores the n_hi most important rows per (sequence, KV head) at 8 bits and the rest at 4 bits.
    K, V [B, H_kv, ctx_cap, d] bf16; importance [B, H_kv, ctx] fp32. Returns a dict with codes_hi
    [2, B, H_kv, n_hi, d] uint8, params_hi [2, B, H_kv, n_hi, d/32, 2] fp32, pos_hi [B, H_kv, n_hi]
    int32, codes_lo [2, B, H_kv, n_lo, d/2] uint8, params_lo, pos_lo (n_lo = ctx - n_hi)."""
    if K.dim() != 4 or importance.dim() != 3:
        raise ValueError("K, V must be [B, H_kv, ctx_cap, d] and importance [B, H_kv, ctx]")
    B, H_kv, cap, d = K.shape
    ctx = importance.shape[2] if ctx is None else ctx
    _expect(V, "V", tuple(K.shape))
    _expect(importance, "importance", (B, H_kv, ctx), torch.float32)
    if not 1 <= ctx <= cap or not 0 <= n_hi <= ctx:
        raise ValueError(f"need 1 <= ctx <= ctx_cap and 0 <= n_hi <= ctx (ctx {ctx}, cap {cap}, n_hi {n_hi})")
    n_lo = ctx - n_hi
    dev = K.device
    shapes = dict(codes_hi=((2, B, H_kv, n_hi, d), torch.uint8), params_hi=((2, B, H_kv, n_hi, d // 32, 2), torch.float32),
                  pos_hi=((B, H_kv, n_hi), torch.int32), codes_lo=((2, B, H_kv, n_lo, d // 2), torch.uint8),
                  params_lo=((2, B, H_kv, n_lo, d // 32, 2), torch.float32), pos_lo=((B, H_kv, n_lo), torch.int32))
    out = {} if out is None else out
    for name, (shape, dt) in shapes.items():
        if name in out:
            _expect(out[name], name, shape, dt)
        else:
            out[name] = torch.empty(shape, dtype=dt, device=dev)
    ptr = lambda name, n: _ptr(out[name]) if n > 0 else None  # noqa: E731
    c = KvcShape(B, H_kv, H_kv, d, _dtype(K, V))
    _check("kv_quantize_mixed", lib().kv_quantize_mixed(
        ctypes.byref(c), _ptr(K), _ptr(V), _ptr(importance), cap, ctx, n_hi, ptr("codes_hi", n_hi),
        ptr("params_hi", n_hi), ptr("pos_hi", n_hi), ptr("codes_lo", n_lo), ptr("params_lo", n_lo),
        ptr("pos_lo", n_lo), _stream(stream)))
    return out


def sals_dense_decode_mixed_workspace_bytes(q: torch.Tensor, H_kv: int, *, n_hi: int, n_lo: int) -> int:
    B, H_q, d = q.shape
    c = KvcShape(B, H_q, H_kv, d, _dtype(q))
    nb = ctypes.c_size_t(0)
    _check("sals_dense_decode_mixed_workspace_bytes",
           lib().sals_dense_decode_mixed_workspace_bytes(ctypes.byref(c), n_hi, n_lo, ctypes.byref(nb)))
    return nb.value


def sals_dense_decode_mixed(q: torch.Tensor, cache: dict, *, out: Optional[torch.Tensor] = None,
                            workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Attention of q [B, H_q, d] (bf16, RoPE applied) over a kv_quantize_mixed cache."""
    if q.dim() != 3:
        raise ValueError("q must be [B, H_q, d]")
    B, H_q, d = q.shape
    _, Bc, H_kv, n_hi, dc = cache["codes_hi"].shape
    n_lo = cache["codes_lo"].shape[3]
    if Bc != B or dc != d:
        raise ValueError("cache and query disagree on B or d")
    _expect(cache["params_hi"], "params_hi", (2, B, H_kv, n_hi, d // 32, 2), torch.float32)
    _expect(cache["codes_lo"], "codes_lo", (2, B, H_kv, n_lo, d // 2), torch.uint8)
    _expect(cache["params_lo"], "params_lo", (2, B, H_kv, n_lo, d // 32, 2), torch.float32)
    _expect(out, "out", (B, H_q, d), torch.float32)
    c = KvcShape(B, H_q, H_kv, d, _dtype(q))
    if out is None:
        out = torch.empty((B, H_q, d), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = _ws(sals_dense_decode_mixed_workspace_bytes(q, H_kv, n_hi=n_hi, n_lo=n_lo), q.device, None)
    p = lambda name, n: _ptr(cache[name]) if n > 0 else None  # noqa: E731
    _check("sals_dense_decode_mixed", lib().sals_dense_decode_mixed(
        ctypes.byref(c), _ptr(q), p("codes_hi", n_hi), p("params_hi", n_hi), n_hi, p("codes_lo", n_lo),
        p("params_lo", n_lo), n_lo, _ptr(out), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream)))
    return out


# ---- dynamic budgets from an importance distribution --------------------------------------------

def kv_importance_budget(importance: torch.Tensor, *, mass: float, ctx: Optional[int] = None, stream=None):
    """Per (sequence, KV head) row of importance [B, H_kv, ctx] (fp32, >= 0): the smallest number of
    tokens holding `mass` of the row's importance, and the row total; plus the layer's ratio
    (mean count / ctx) and energy (summed importance), computed on the device.
    Returns (n_keep [B, H_kv] int32, total [B, H_kv] fp32, layer_ratio [1] fp32, layer_energy [1] fp32)."""
    if importance.dim() != 3 or importance.dtype != torch.float32:
        raise ValueError("importance must be a float32 [B, H_kv, ctx] tensor")
    B, H_kv, n = importance.shape
    ctx = n if ctx is None else ctx
    if ctx != n:
        importance = importance[:, :, :ctx].contiguous()
    dev = importance.device
    n_keep = torch.empty((B, H_kv), dtype=torch.int32, device=dev)
    total = torch.empty((B, H_kv), dtype=torch.float32, device=dev)
    ratio = torch.empty((4,), dtype=torch.float32, device=dev)
    energy = torch.empty((4,), dtype=torch.float32, device=dev)
    c = KvcShape(B, H_kv, H_kv, 128, 1)
    _check("kv_importance_budget", lib().kv_importance_budget(
        ctypes.byref(c), _ptr(importance), ctx, ctypes.c_float(mass), _ptr(n_keep), _ptr(total), _ptr(ratio),
        _ptr(energy), _stream(stream)))
    return n_keep, total, ratio[:1], energy[:1]
