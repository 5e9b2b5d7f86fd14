"""GPU parity of kv_outlier_importance (frequency-domain outlier importance, through the C ABI)
against the oracle, and of the compaction it drives (kv_compact_from_importance)."""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - the GPU tests run on an MI355X
    pytest.skip("no GPU", allow_module_level=True)

import kv_cache_compression_sals_amd as sals  # noqa: E402
import oracle  # noqa: E402
from parity import check_selection, to_device  # noqa: E402
from workloads import CONFIGS, compact_case  # noqa: E402

C4 = CONFIGS["c4"]
# Importance error bound, relative to the largest pair energy ||K_t||^2 + ||V_t||^2 of the row:
# the cache is exact in bf16, the basis values and coefficients enter the bf16 MFMAs as high +
# low parts (2^-16 relative) and sums are fp32, so a low-pass value carries ~1e-5 relative error
# and the deviation energy about 2e-5 of the row energy.
REL = 1e-4


def _energy(K, V, ctx):
    k = oracle.stored_to_f64(K[..., :ctx, :], "bf16")
    v = oracle.stored_to_f64(V[..., :ctx, :], "bf16")
    return (k * k).sum(-1) + (v * v).sum(-1)


def check(case, n_freq, k_keep, pairs=None):
    ctx = case["ctx"]
    K, V = case["K"], case["V"]
    print(f"outlier B={K.shape[0]} H_kv={K.shape[1]} cap={K.shape[2]} d={K.shape[3]} ctx={ctx} "
          f"n_freq={n_freq} k_keep={k_keep}", flush=True)
    Kd, Vd = to_device(K, "bf16"), to_device(V, "bf16")
    imp = sals.kv_outlier_importance(Kd, Vd, ctx=ctx, n_freq=n_freq)
    Kc, Vc, kept = sals.kv_compact_from_importance(Kd, Vd, imp, k_keep=k_keep)
    torch.cuda.synchronize()
    imp, kept = imp.cpu().numpy().astype(np.float64), kept.cpu().numpy()
    Kc = Kc.view(torch.int16).cpu().numpy().view(np.uint16)
    Vc = Vc.view(torch.int16).cpu().numpy().view(np.uint16)
    ora = oracle.outlier_compact(K, V, ctx=ctx, n_freq=n_freq, k_keep=k_keep, dtype="bf16", pairs=pairs)
    B, H = K.shape[0], K.shape[1]
    todo = [(b, g) for b in range(B) for g in range(H)] if pairs is None else pairs
    worst = 0.0
    for b, g in todo:
        I = ora["importance"][b, g]
        scale = _energy(K[b, g], V[b, g], ctx).max()
        err = np.abs(imp[b, g] - I).max() / scale
        worst = max(worst, err)
        assert err <= REL, (b, g, err)
        check_selection(I, k_keep, ctx, 0, kept[b, g], ora["kept"][b, g], f"b{b} g{g}")
        assert np.array_equal(Kc[b, g], K[b, g, kept[b, g]]) and np.array_equal(Vc[b, g], V[b, g, kept[b, g]])
    print(f"   max importance error / row energy {worst:.2e}", flush=True)


SMALL = [
    # name, overrides, ctx, ctx_cap, n_freq, k_keep
    ("d128_ragged_f16", dict(B=2, H_q=3, H_kv=3, n_visual=2000, grid_h=40, grid_w=50, clusters_h=4, clusters_w=5),
     3000, 3100, 16, 300),
    ("d64_f40_three_chunks", dict(B=1, H_q=2, H_kv=2, d=64, n_visual=8000, grid_h=80, grid_w=100, clusters_h=8,
                                  clusters_w=10), 9000, 9000, 40, 900),
    ("d128_f64_short", dict(B=2, H_q=2, H_kv=2, n_visual=300, grid_h=15, grid_w=20, clusters_h=3, clusters_w=4),
     333, 340, 64, 33),
    ("dc_only", dict(B=1, H_q=2, H_kv=2, n_visual=500, grid_h=20, grid_w=25, clusters_h=2, clusters_w=5),
     700, 700, 1, 70),
]


@pytest.mark.parametrize("name,ov,ctx,cap,n_freq,k_keep", SMALL, ids=[s[0] for s in SMALL])
def test_outlier_small(name, ov, ctx, cap, n_freq, k_keep):
    check(compact_case(C4.with_(**ov), ctx=ctx, ctx_cap=cap), n_freq, k_keep)


def test_outlier_all_frequencies_kept_is_zero():
    """n_freq = ctx keeps every frequency: the low-pass is the cache itself, so every importance is
    zero up to rounding."""
    case = compact_case(C4.with_(B=1, H_q=2, H_kv=2, n_visual=40, grid_h=5, grid_w=8, clusters_h=1, clusters_w=2),
                        ctx=50, ctx_cap=56)
    imp = sals.kv_outlier_importance(to_device(case["K"], "bf16"), to_device(case["V"], "bf16"), ctx=50, n_freq=50)
    torch.cuda.synchronize()
    scale = _energy(case["K"], case["V"], 50).max()
    assert np.abs(imp.cpu().numpy()).max() <= REL * scale


def test_outlier_single_token():
    case = compact_case(C4.with_(B=2, H_q=1, H_kv=1, n_visual=1, grid_h=1, grid_w=1, clusters_h=1, clusters_w=1),
                        ctx=1, ctx_cap=4)
    check(case, 1, 1)


def test_outlier_c4_full_size_sampled():
    """The full compaction workload (B=16, 32 KV heads, ctx 16384), 10% kept, n_freq 32."""
    case = compact_case(C4, threads=16)
    check(case, 32, case["k_keep"], pairs=[(0, 0), (3, 17), (9, 5), (15, 31)])
