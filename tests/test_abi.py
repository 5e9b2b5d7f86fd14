"""The C-ABI library on the CPU: it loads, exports every declared symbol, and rejects bad
arguments with the documented status before touching HIP (no GPU needed)."""

import ctypes
import os
import re

import pytest

from kv_cache_compression_sals_amd._lib import KvcShape, SalsSelect, SalsShape, lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sals.h")

OK, NULL, SHAPE, DTYPE, RANGE, WORKSPACE, ALIGN, HIP = range(8)
P = 0x10000  # an aligned, never dereferenced stand-in pointer


def declared_functions():
    src = open(HEADER).read()
    return re.findall(r"^(?:sals_status|int32_t|const char\*)\s+(\w+)\(", src, flags=re.M)


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) == 27, names
    L = lib()
    for n in names:
        assert hasattr(L, n), n
    assert L.sals_abi_version() == 1


def test_status_strings():
    L = lib()
    for code in range(8):
        assert L.sals_status_string(code)
    assert b"unknown" in L.sals_status_string(99)


def _shape(**kw):
    base = dict(B=2, H_q=8, H_kv=4, d=128, r=256, dtype=1)
    base.update(kw)
    return SalsShape(**base)


def _ws_bytes(s, sel, ctx):
    n = ctypes.c_size_t(0)
    st = lib().sals_decode_workspace_bytes(ctypes.byref(s), ctypes.byref(sel), ctx, ctypes.byref(n))
    return st, n.value


@pytest.mark.parametrize("kw,want", [
    (dict(), OK),
    (dict(dtype=7), DTYPE),
    (dict(d=96), SHAPE),
    (dict(H_q=6, H_kv=4), SHAPE),
    (dict(H_q=32, H_kv=2), SHAPE),  # more than 8 query heads per KV head
    (dict(r=48), SHAPE),
    (dict(r=1024), SHAPE),
    (dict(r=512, dtype=0), SHAPE),  # fp32 slice of P would not fit on chip
    (dict(B=0), SHAPE),
])
def test_decode_workspace_shape_checks(kw, want):
    st, n = _ws_bytes(_shape(**kw), SalsSelect(16, 4, 2), 100)
    assert st == want
    if want == OK:
        assert n > 0


@pytest.mark.parametrize("sel,ctx,want", [
    ((16, 4, 3), 100, SHAPE),   # H_kv % G != 0
    ((16, 4, 0), 100, SHAPE),
    ((-1, 4, 2), 100, RANGE),
    ((16, -1, 2), 100, RANGE),
    ((16, 4, 2), 0, RANGE),
    ((0, 0, 2), 100, RANGE),  # k = w = 0: nothing selected to attend over
    ((0, 1, 2), 100, OK),
    ((0, 0, 1), 1, RANGE),
])
def test_decode_select_checks(sel, ctx, want):
    assert _ws_bytes(_shape(), SalsSelect(*sel), ctx)[0] == want


def _step(s=None, sel=None, base=10000.0, ptrs=None, cap=100, ctx=100, ws=P, ws_bytes=1 << 30, sel_out=None):
    s = s or _shape()
    sel = sel or SalsSelect(16, 4, 2)
    p = dict(q=P, Lk=P, Lv=P, Pk=P, Pv=P, out=P)
    p.update(ptrs or {})
    return lib().sals_decode_step(ctypes.byref(s), ctypes.byref(sel), ctypes.c_float(base), p["q"], p["Lk"],
                                  p["Lv"], p["Pk"], p["Pv"], cap, ctx, p["out"], sel_out, ws, ws_bytes, None)


def test_decode_step_argument_errors():
    assert _step(ptrs=dict(q=None)) == NULL
    assert _step(ptrs=dict(out=None)) == NULL
    assert _step(ptrs=dict(Lk=P + 8)) == ALIGN
    assert _step(sel_out=P + 4) == ALIGN
    assert _step(cap=99) == RANGE
    assert _step(base=1.0) == RANGE
    assert _step(base=float("nan")) == RANGE
    assert _step(ws=None) == WORKSPACE
    need = _ws_bytes(_shape(), SalsSelect(16, 4, 2), 100)[1]
    assert _step(ws_bytes=need - 1) == WORKSPACE
    assert _step(s=_shape(dtype=5)) == DTYPE


def test_project_argument_errors():
    L = lib()
    s = _shape()

    def call(Xk=P, Xv=P, Pk=P, Pv=P, Lk=P, Lv=P, cap=10, t0=0, T=10):
        return L.sals_project_kv(ctypes.byref(s), Xk, Xv, Pk, Pv, Lk, Lv, cap, t0, T, None)

    assert call(Xk=None) == NULL
    assert call(Xv=None) == NULL  # V pointers must be all NULL or all set
    assert call(T=0) == RANGE
    assert call(t0=5, T=6) == RANGE
    assert call(Pk=P + 2) == ALIGN


def test_compact_argument_errors():
    L = lib()
    c = KvcShape(2, 4, 4, 128, 1)

    def ws(ctx=100, w=8, k_keep=10, cc=c):
        n = ctypes.c_size_t(0)
        return L.kv_compact_workspace_bytes(ctypes.byref(cc), ctx, w, k_keep, ctypes.byref(n)), n.value

    assert ws()[0] == OK and ws()[1] > 0
    assert ws(w=0)[0] == RANGE
    assert ws(w=101)[0] == RANGE
    assert ws(k_keep=0)[0] == RANGE
    assert ws(k_keep=101)[0] == RANGE
    assert ws(cc=KvcShape(2, 4, 3, 128, 1))[0] == SHAPE
    assert ws(cc=KvcShape(2, 4, 4, 128, 9))[0] == DTYPE

    def call(K=P, Qobs=P, cap=100, ctx=100, wsp=P, wsb=1 << 30, imp=None):
        return L.kv_compact(ctypes.byref(c), K, P, Qobs, 8, cap, ctx, 10, P, P, P, imp, wsp, wsb, None)

    assert call(K=None) == NULL
    assert call(cap=50) == RANGE
    assert call(imp=P + 4) == ALIGN
    assert call(wsb=16) == WORKSPACE


def test_dense_decode_argument_errors():
    L = lib()
    c = KvcShape(2, 8, 4, 64, 1)
    assert L.sals_dense_decode(ctypes.byref(c), P, P, None, 10, 10, P, P, 1 << 20, None) == NULL
    assert L.sals_dense_decode(ctypes.byref(c), P, P, P, 11, 10, P, P, 1 << 20, None) == RANGE
    assert L.sals_dense_decode(ctypes.byref(c), P, P, P, 0, 10, P, P, 1 << 20, None) == RANGE


def test_importance_sparsity_argument_errors():
    L = lib()
    c = KvcShape(2, 8, 4, 128, 1)
    n = ctypes.c_size_t(0)
    assert L.kv_importance_sparsity_workspace_bytes(ctypes.byref(c), 100, 8, ctypes.byref(n)) == OK and n.value > 0
    assert L.kv_importance_sparsity_workspace_bytes(ctypes.byref(c), 100, 0, ctypes.byref(n)) == RANGE

    def call(K=P, imp=P, sp=P, cap=100, ctx=100, p=0.01, wsb=1 << 30):
        return L.kv_importance_sparsity(ctypes.byref(c), K, P, 8, cap, ctx, ctypes.c_float(p), imp, sp, P, wsb, None)

    assert call(sp=None) == NULL
    assert call(imp=None) == NULL
    assert call(cap=50) == RANGE
    assert call(p=-0.5) == RANGE
    assert call(p=float("nan")) == RANGE
    assert call(wsb=16) == WORKSPACE
    assert call(sp=P + 4) == ALIGN


def test_layer_budgets_match_oracle():
    """Host arithmetic: the C function and the oracle agree exactly; argument errors."""
    import numpy as np

    import kv_cache_compression_sals_amd as sals
    import oracle

    rs = np.random.default_rng(3)
    for L_ in (1, 2, 7, 32):
        for total in (0, 5, 1000, 123457):
            nu = rs.random(L_).astype(np.float32)
            if L_ > 2:
                nu[1] = 0.0
            got = sals.kv_layer_budgets(nu, total=total, ctx=4096)
            assert got == list(oracle.layer_budgets(nu.astype(np.float64), total, 4096)), (L_, total)
    assert sals.kv_layer_budgets([0.0, 0.0], total=10, ctx=100) == [5, 5]
    L = lib()
    assert L.kv_layer_budgets(None, 2, 10, 100, P) == NULL
    assert L.kv_layer_budgets(P, 0, 10, 100, P) == RANGE


def test_compact_from_importance_argument_errors():
    L = lib()

    def call(c=KvcShape(2, 4, 4, 128, 1), K=P, imp=P, cap=100, ctx=100, k=10):
        return L.kv_compact_from_importance(ctypes.byref(c), K, P, imp, cap, ctx, k, P, P, P, None)

    assert call(imp=None) == NULL
    assert call(K=None) == NULL
    assert call(ctx=101) == RANGE
    assert call(k=0) == RANGE
    assert call(k=101) == RANGE
    assert call(c=KvcShape(2, 4, 4, 96, 1)) == SHAPE
    assert call(c=KvcShape(2, 4, 4, 128, 7)) == DTYPE
    assert call(imp=P + 4) == ALIGN


def test_reconstruct_argument_errors():
    L = lib()

    def call(s=SalsShape(2, 8, 4, 128, 256, 1), Lk=P, Lv=P, Pv=P, V=P, cap=100, t0=0, T=100, stride=100,
             q=None, q_rot=None, q_pos=0):
        return L.sals_reconstruct_kv(ctypes.byref(s), ctypes.c_float(10000.0), Lk, Lv, P, Pv, cap, t0, T, P, V,
                                     stride, q, q_rot, q_pos, None)

    assert call(Lk=None) == NULL
    assert call(V=None) == NULL  # V pointers must be all NULL or all set
    assert call(q=P) == NULL     # q and q_rot come together
    assert call(s=SalsShape(2, 8, 4, 128, 256, 0)) == DTYPE
    assert call(s=SalsShape(2, 8, 4, 64, 256, 1)) == SHAPE
    assert call(s=SalsShape(2, 6, 3, 128, 256, 1)) == SHAPE   # odd number of KV heads
    assert call(s=SalsShape(2, 8, 4, 128, 64, 1)) == SHAPE
    assert call(T=0) == RANGE
    assert call(t0=1) == RANGE
    assert call(stride=99) == RANGE
    assert call(q=P, q_rot=P, q_pos=-1) == RANGE
    assert call(Lv=P + 8) == ALIGN


def _gpu_present():
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:  # noqa: BLE001
        return False


@pytest.mark.skipif(_gpu_present(), reason="stand-in pointers must never reach a real GPU")
def test_probe_argument_errors():
    L = lib()
    assert L.sals_hbm_read(None, 16, P, 1, None) == NULL
    assert L.sals_hbm_read(P, 15, P, 1, None) == RANGE
    assert L.sals_hbm_read(P, 16, P, 0, None) == RANGE
    assert L.sals_hbm_read(P + 4, 16, P, 1, None) == ALIGN
    assert L.sals_mfma_peak(1, 1, None, None) == NULL
    assert L.sals_mfma_peak(0, 1, P, None) == RANGE
    assert L.sals_mfma_peak(1, 0, P, None) == RANGE
    assert L.sals_mfma_peak(1, 1 << 25, P, None) == RANGE
    assert L.sals_mfma_peak(1, 1, P + 4, None) == ALIGN


def test_valid_call_without_device_reports_hip_error():
    assert _step() == HIP
    assert lib().sals_last_hip_error() != 0


def test_header_is_plain_c_and_links(tmp_path):
    """include/sals.h compiles as C99 with warnings as errors, and a C program that calls every
    declared function by address links against the built library."""
    import shutil
    import subprocess

    if shutil.which("gcc") is None:
        pytest.skip("no C compiler")
    names = declared_functions()
    lib_dir = os.path.join(ROOT, "kv_cache_compression_sals_amd")
    src = tmp_path / "abi.c"
    src.write_text('#include "sals.h"\ntypedef void (*fn)(void);\nint main(void) {\n  fn f[] = {'
                   + ", ".join(f"(fn)&{n}" for n in names)
                   + '};\n  for (unsigned i = 0; i < sizeof f / sizeof f[0]; ++i) if (!f[i]) return 1;\n'
                   '  return sals_abi_version() == 1 ? 0 : 2;\n}\n')
    exe = tmp_path / "abi"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
                    str(src), "-L", lib_dir, "-lsals", f"-Wl,-rpath,{lib_dir}", "-o", str(exe)], check=True)
    assert subprocess.run([str(exe)]).returncode == 0


def test_noalloc_decode_checks_before_any_hip_call():
    """The no-allocation decode entry point rejects a workspace need above its fixed array, and
    every argument error, before touching HIP."""
    L = lib()
    fn = L.sals_decode_step_noalloc
    sel = SalsSelect(2048, 128, 8)
    s = _shape(B=4, H_q=32, H_kv=8, d=128, r=256)
    args = lambda s, sel, ctx, out=P: (ctypes.byref(s), ctypes.byref(sel), ctypes.c_float(10000.0), P, P, P, P,
                                       P, 1 << 20, ctx, out, None, None)
    assert fn(*args(s, sel, 32768, out=None)) == NULL
    # a workspace above 16 MiB: 64 sequences of 128K-token score rows
    big = _shape(B=64, H_q=32, H_kv=8, d=128, r=256)
    st, need = _ws_bytes(big, sel, 131072)
    assert st == OK and need > (16 << 20)
    assert fn(*args(big, sel, 131072)) == WORKSPACE
    assert fn(*args(_shape(d=96), sel, 1000)) == SHAPE
    assert fn(*args(s, SalsSelect(-1, 4, 8), 1000)) == RANGE
    bad = (ctypes.byref(s), ctypes.byref(sel), ctypes.c_float(10000.0), P + 4, P, P, P, P, 1 << 20, 1000, P,
           None, None)
    assert fn(*bad) == ALIGN
