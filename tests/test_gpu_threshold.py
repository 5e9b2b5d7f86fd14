"""GPU parity of sals_decode_step_threshold (threshold selection with ragged per-row lengths,
through the C ABI) against the oracle.

Set rule: a candidate may differ between the GPU's set and the oracle's only if its oracle score
lies within 1e-4 max|S| of tau or of the k-th largest score (the two places where fp32 and fp64
scores may fall on different sides); the window closes every row, ascending, and the row is
padded with -1 to its maximum length. Outputs are compared with the oracle's attention over the
GPU's own set (max-abs 1e-4 for every cache type, and the stated 1e-4 / 2e-2 tolerances)."""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - the GPU tests run on an MI355X
    pytest.skip("no GPU", allow_module_level=True)

import kv_cache_compression_sals_amd as sals  # noqa: E402
import oracle  # noqa: E402
from parity import EXEMPT_REL, TIGHT, TOL, to_device  # noqa: E402
from workloads import CONFIGS, decode_case  # noqa: E402

C1, C2, C3, C5 = CONFIGS["c1"], CONFIGS["c2"], CONFIGS["c3"], CONFIGS["c5"]


def run(case, tau):
    dt = case["dtype"]
    t = {n: to_device(case[n], dt) for n in ("q", "Lk", "Lv", "Pk", "Pv")}
    out, sel, cnt = sals.sals_decode_step_threshold(t["q"], t["Lk"], t["Lv"], t["Pk"], t["Pv"], ctx=case["ctx"],
                                                    k=case["k"], w=case["w"], G=case["G"], tau=tau,
                                                    rope_base=case["base"], want_sel=True)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64), sel.cpu().numpy(), cnt.cpu().numpy()


def check_rows(case, S, tau, sel, cnt, batches):
    T, k, w, G = case["ctx"], case["k"], case["w"], case["G"]
    T_c = max(0, T - w)
    wc = T - T_c
    n_max = min(k, T_c) + wc
    assert sel.shape[2] == n_max
    exempt_total = 0
    lengths = []
    for b in batches:
        for s in range(G):
            n = int(cnt[b, s])
            row = sel[b, s]
            assert wc <= n <= n_max, (b, s, n)
            assert np.all(row[n:] == -1), (b, s)
            got = row[:n]
            assert np.all(np.diff(got) > 0) and np.array_equal(got[n - wc:], np.arange(T_c, T)), (b, s)
            Sr = S[b, s]
            want = oracle.select_tokens_threshold(Sr, T, k, w, tau)[: -wc or None]
            eps = EXEMPT_REL * np.abs(Sr).max(initial=0.0)
            exempt = np.abs(Sr - tau) <= eps
            if 0 < k < T_c:
                exempt |= np.abs(Sr - np.sort(Sr)[::-1][k - 1]) <= eps
            diff = set(got[: n - wc].tolist()) ^ set(want.tolist())
            assert all(exempt[t] for t in diff), (b, s, sorted(t for t in diff if not exempt[t])[:8])
            exempt_total += int(exempt.sum())
            lengths.append(n)
    return exempt_total, lengths


def check(case, tau, batches=None):
    B = case["q"].shape[0]
    batches = list(range(B)) if batches is None else batches
    print(f"threshold {case['cfg'].name} B={B} ctx={case['ctx']} k={case['k']} w={case['w']} G={case['G']} "
          f"tau={tau:.6g}", flush=True)
    out, sel, cnt = run(case, tau)
    dt = case["dtype"]
    ora = oracle.decode_step_threshold(case["q"], case["Lk"], case["Lv"], case["Pk"], case["Pv"], ctx=case["ctx"],
                                       k=case["k"], w=case["w"], G=case["G"], H_kv=case["H_kv"], base=case["base"],
                                       tau=tau, dtype=dt, batches=batches)
    exempt, lengths = check_rows(case, ora["S"], tau, sel, cnt, batches)
    qf = oracle.stored_to_f64(case["q"], dt)
    Pk, Pv = oracle.stored_to_f64(case["Pk"], dt), oracle.stored_to_f64(case["Pv"], dt)
    err = 0.0
    for b in batches:
        T = case["ctx"]
        sets = [sel[b, s, : cnt[b, s]] for s in range(case["G"])]
        ref, _ = oracle.attend_selected(qf[b], oracle.stored_to_f64(case["Lk"][b, :T], dt),
                                        oracle.stored_to_f64(case["Lv"][b, :T], dt), Pk, Pv, sets, T, case["base"],
                                        case["H_kv"], case["G"])
        err = max(err, float(np.abs(out[b] - ref).max()))
    print(f"   lengths {min(lengths)}..{max(lengths)} of {sel.shape[2]}, exempt {exempt}, max-abs {err:.2e}", flush=True)
    assert err <= TOL[dt] and err <= TIGHT
    return out, sel, cnt, ora


def tau_for(case, frac):
    """A threshold between two consecutive oracle scores of sequence 0, group 0, so that about
    frac of the top-k capacity passes there (other rows get other lengths)."""
    ora = oracle.decode_step(case["q"], case["Lk"], case["Lv"], case["Pk"], case["Pv"], ctx=case["ctx"],
                             k=case["k"], w=case["w"], G=case["G"], H_kv=case["H_kv"], base=case["base"],
                             dtype=case["dtype"], batches=[0])
    S = np.sort(ora["S"][0, 0])[::-1]
    m = max(1, min(len(S) - 1, int(frac * case["k"])))
    return float((S[m - 1] + S[m]) / 2)


SMALL = [
    # name, base cfg, overrides, B, ctx, ctx_cap
    ("f32_tiny", C1, {}, 1, 512, 512),
    ("bf16_gqa_g2", C3, dict(H_q=8, H_kv=4, r=64, G=2, k=200, w=16, rank=32, calib_tokens=256), 2, 3000, 3008),
    ("bf16_long_splits", C3, dict(H_q=8, H_kv=2, r=256, G=2, k=1500, w=64, calib_tokens=512, rank=100), 2, 5000, 5000),
    ("shared_keys_g1", C2, dict(calib_tokens=1024, k=700), 2, 2000, 2000),
    ("shared_value_r384", C3, dict(H_q=16, H_kv=8, d=128, r=384, G=2, k=400, w=16, rank=200, calib_tokens=512),
     2, 1300, 1333),
]


@pytest.mark.parametrize("frac", [0.3, 0.8])
@pytest.mark.parametrize("name,cfg,ov,B,ctx,cap", SMALL, ids=[s[0] for s in SMALL])
def test_threshold_small(name, cfg, ov, B, ctx, cap, frac):
    case = decode_case(cfg.with_(**ov), B=B, ctx=ctx, ctx_cap=cap)
    check(case, tau_for(case, frac))


@pytest.mark.parametrize("name,cfg,ov,B,ctx,cap", SMALL[1:4], ids=[s[0] for s in SMALL[1:4]])
def test_threshold_cap_binding_equals_topk(name, cfg, ov, B, ctx, cap):
    """tau below every score: the cap binds on every row, so the result is the top-k step's, bit
    for bit (the same kernels with the same lengths)."""
    case = decode_case(cfg.with_(**ov), B=B, ctx=ctx, ctx_cap=cap)
    out, sel, cnt, _ = check(case, -1e30)
    dt = case["dtype"]
    t = {n: to_device(case[n], dt) for n in ("q", "Lk", "Lv", "Pk", "Pv")}
    ref, ref_sel = sals.sals_decode_step(t["q"], t["Lk"], t["Lv"], t["Pk"], t["Pv"], ctx=ctx, k=case["k"], w=case["w"],
                                         G=case["G"], rope_base=case["base"], want_sel=True)
    assert np.array_equal(sel, ref_sel.cpu().numpy()) and np.array_equal(out, ref.cpu().numpy().astype(np.float64))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_threshold_window_only_and_zero_scores(dtype):
    """tau above every score keeps only the window; q = 0 makes every score +-0: tau = -0.0 lets
    all pass (the lowest k positions are kept), tau = 1e-30 lets none pass."""
    base = C1 if dtype == "f32" else C3.with_(H_q=8, H_kv=4, r=64, G=2, rank=32, calib_tokens=256)
    case = decode_case(base.with_(k=20, w=6), B=2, ctx=400)
    _, _, cnt, _ = check(case, 1e30)
    assert np.all(cnt == 6)
    case["q"] = np.zeros_like(case["q"])
    _, sel, cnt, _ = check(case, -0.0)
    assert np.all(cnt == 26) and np.array_equal(sel[0, 0, :20], np.arange(20))
    _, _, cnt, _ = check(case, 1e-30)
    assert np.all(cnt == 6)


def test_threshold_long_rows_slice_merge():
    """Rows longer than 32768 candidates go through the slice + merge top-k."""
    case = decode_case(C5.with_(H_q=8, H_kv=2, G=2, k=1000, rank=64, calib_tokens=512), B=1, ctx=40000)
    check(case, tau_for(case, 0.5))
    check(case, -1e30)


def test_threshold_c2_full_size():
    case = decode_case(C2)
    check(case, tau_for(case, 0.5))


def test_threshold_c3_full_size():
    case = decode_case(C3)
    check(case, tau_for(case, 0.4))
