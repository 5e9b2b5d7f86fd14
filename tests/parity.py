"""Parity checks of the HIP path against the oracle (shared by the GPU tests).

Selection: the selected index sets must match exactly except for near-ties: candidates whose
oracle score lies within 1e-4 * max|score| of the k'-th largest score are exempt. Ties break
to the lowest index. The window is always kept, the set has exactly n_sel entries and is
strictly ascending.

Outputs: the GPU output is compared with the oracle's attention over the GPU's own selected
set (so an exempt swap cannot inflate the error). Two bounds are asserted:
  * the stated tolerance, max-abs <= 1e-4 for fp32 and 2e-2 for bf16 caches;
  * a tight bound, max-abs <= 1e-4 for every cache type. The stored inputs are exact on both
    sides (bf16 widens to fp32 exactly) and every sum on the GPU is fp32; the fp32 vectors that
    enter bf16 MFMAs as high + low bf16 parts carry about 2^-16 relative error. An output is a
    convex combination of value rows of magnitude O(1) to O(10), so the accumulated error stays
    near 1e-6; the bf16 tolerance alone would let a 1e-3 angle or value-side slip through.
"""

from __future__ import annotations

import numpy as np

import oracle

TOL = {"f32": 1e-4, "bf16": 2e-2}
TIGHT = 1e-4
EXEMPT_REL = 1e-4


def to_device(a: np.ndarray, dtype: str):
    import torch
    a = np.ascontiguousarray(a)
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    if a.dtype == np.uint16:
        raise ValueError("bf16 bits passed as f32")
    return torch.from_numpy(a).cuda()


def check_selection(S_row: np.ndarray, kp: int, T: int, w: int, sel_gpu: np.ndarray,
                    sel_ora: np.ndarray, what: str = "") -> int:
    """Asserts the set rule; returns the number of exempt candidates."""
    T_c = max(0, T - w)
    n_sel = kp + (T - T_c)
    sel_gpu = np.asarray(sel_gpu, dtype=np.int64)
    assert sel_gpu.shape == (n_sel,), (what, sel_gpu.shape, n_sel)
    assert np.all(np.diff(sel_gpu) > 0), (what, "not strictly ascending")
    assert np.array_equal(sel_gpu[kp:], np.arange(T_c, T)), (what, "window missing")
    assert sel_gpu[:kp].min(initial=0) >= 0 and sel_gpu[:kp].max(initial=-1) < T_c, (what, "out of range")
    if kp == 0 or kp == T_c:
        assert np.array_equal(sel_gpu, sel_ora), what
        return 0
    S = S_row[:T_c]
    tau = np.sort(S)[::-1][kp - 1]
    eps = EXEMPT_REL * np.abs(S).max()
    exempt = np.abs(S - tau) <= eps
    a = set(sel_gpu[:kp].tolist())
    b = set(sel_ora[:kp].tolist())
    diff = {t for t in a.symmetric_difference(b) if not exempt[t]}
    assert not diff, (what, f"{len(diff)} non-exempt mismatches, e.g. {sorted(diff)[:8]}", tau, eps)
    return int(exempt.sum())


def decode_parity(case: dict, out_gpu: np.ndarray, sel_gpu: np.ndarray, batches=None, tol=None):
    """Full check of one decode step; returns a dict of statistics."""
    dt = case["dtype"]
    tol = TOL[dt] if tol is None else tol
    T, k, w, G, H_kv = case["ctx"], case["k"], case["w"], case["G"], case["H_kv"]
    B = case["q"].shape[0]
    batches = list(range(B)) if batches is None else batches
    ora = oracle.decode_step(case["q"], case["Lk"], case["Lv"], case["Pk"], case["Pv"], ctx=T, k=k,
                             w=w, G=G, H_kv=H_kv, base=case["base"], dtype=dt, batches=batches)
    T_c = ora["T_c"]
    kp = min(k, T_c)
    qf = oracle.stored_to_f64(case["q"], dt)
    Pk, Pv = oracle.stored_to_f64(case["Pk"], dt), oracle.stored_to_f64(case["Pv"], dt)
    max_err = 0.0
    max_err_vs_ora_set = 0.0
    sq_err = sq_ref = 0.0
    exempt = 0
    for b in batches:
        for s in range(G):
            exempt += check_selection(ora["S"][b, s], kp, T, w, sel_gpu[b, s], ora["sel"][b, s], f"b{b} s{s}")
        Lk = oracle.stored_to_f64(case["Lk"][b, :T], dt)
        Lv = oracle.stored_to_f64(case["Lv"][b, :T], dt)
        ref, _ = oracle.attend_selected(qf[b], Lk, Lv, Pk, Pv, [sel_gpu[b, s] for s in range(G)], T,
                                        case["base"], H_kv, G)
        err = np.abs(out_gpu[b] - ref).max()
        max_err = max(max_err, err)
        sq_err += float(((out_gpu[b] - ref) ** 2).sum())
        sq_ref += float((ref ** 2).sum())
        max_err_vs_ora_set = max(max_err_vs_ora_set, np.abs(out_gpu[b] - ora["out"][b]).max())
    assert max_err <= tol, f"max-abs error {max_err:.3e} > {tol:.1e}"
    assert max_err <= TIGHT, f"max-abs error {max_err:.3e} > tight bound {TIGHT:.1e}"
    rel_rms = (sq_err / sq_ref) ** 0.5 if sq_ref > 0 else 0.0
    return dict(max_err=max_err, rel_rms=rel_rms, max_err_vs_oracle_set=max_err_vs_ora_set, exempt=exempt)
