"""GPU parity of kv_importance_budget (importance-mass budgets, through the C ABI) against the
oracle, and the two layer-level compositions built on it: the ZipVL dynamic ratio feeding the
mixed-precision cache, and FlashCache-style per-layer budgets from outlier energies."""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - the GPU tests run on an MI355X
    pytest.skip("no GPU", allow_module_level=True)

import kv_cache_compression_sals_amd as sals  # noqa: E402
import oracle  # noqa: E402
from parity import to_device  # noqa: E402
from workloads import CONFIGS, compact_case  # noqa: E402

C4 = CONFIGS["c4"]


def _near_boundary(row, mass, n):
    """True when the cumulative mass of the n-1 or n largest values is within 1e-12 (relative) of
    the target, where fp64 sums in another order may fall on the other side."""
    c = np.cumsum(np.sort(np.asarray(row, dtype=np.float64))[::-1])
    target = mass * c[-1]
    near = [abs(c[i] - target) <= 1e-12 * max(c[-1], 1e-300) for i in (n - 2, n - 1) if 0 <= i < len(c)]
    return any(near)


def check(imp, mass, ctx=None):
    B, H, n = imp.shape
    ctx = n if ctx is None else ctx
    print(f"budget B={B} H={H} ctx={ctx} mass={mass}", flush=True)
    nk, tot, ratio, energy = sals.kv_importance_budget(torch.from_numpy(imp).cuda(), mass=mass, ctx=ctx)
    torch.cuda.synchronize()
    nk, tot = nk.cpu().numpy(), tot.cpu().numpy()
    ref = oracle.importance_budget(imp, ctx=ctx, mass=mass)
    for b in range(B):
        for g in range(H):
            if nk[b, g] != ref["n_keep"][b, g]:
                assert abs(int(nk[b, g]) - int(ref["n_keep"][b, g])) <= 1 and _near_boundary(
                    imp[b, g, :ctx], mass, int(ref["n_keep"][b, g])), (b, g, nk[b, g], ref["n_keep"][b, g])
    assert np.allclose(tot, ref["total"], rtol=1e-6, atol=0)
    # the layer ratio is the mean of the counts (checked row by row above, where a count may move
    # by one at a boundary that fp64 sums in another order cannot resolve)
    own = nk.astype(np.float64).sum() / (B * H * ctx)
    assert abs(float(ratio.item()) - own) <= 1e-6 * max(own, 1e-30)
    assert abs(float(energy.item()) - ref["layer_energy"]) <= 1e-6 * max(ref["layer_energy"], 1e-30)
    print(f"   n_keep {nk.min()}..{nk.max()}, ratio {float(ratio.item()):.4f}", flush=True)
    return nk, float(ratio.item()), float(energy.item())


@pytest.mark.parametrize("mass", [0.5, 0.9, 1.0])
def test_budget_random_rows(mass):
    rs = np.random.default_rng(int(mass * 100))
    imp = rs.exponential(size=(2, 3, 5000)).astype(np.float32) ** 3
    check(imp, mass)


def test_budget_ties_zeros_and_long_rows():
    rs = np.random.default_rng(3)
    imp = rs.integers(0, 4, size=(2, 2, 3000)).astype(np.float32)  # exact sums: heavy ties
    imp[1, 1] = 0.0  # an all-zero row keeps one token
    nk, _, _ = check(imp, 0.6)
    assert nk[1, 1] == 1
    long = rs.exponential(size=(1, 2, 40000)).astype(np.float32)  # rows past the on-chip staging
    check(long, 0.8)


def test_zipvl_ratio_feeds_mixed_cache():
    """kv_compact's importance gives the layer's dynamic ratio; the mixed-precision cache then
    keeps ceil(ratio * ctx) tokens at 8 bits per head."""
    cfg = C4.with_(B=2, H_q=4, H_kv=4, n_visual=1500, grid_h=30, grid_w=50, clusters_h=3, clusters_w=5)
    case = compact_case(cfg, ctx=2000)
    dt = "bf16"
    K, V = to_device(case["K"], dt), to_device(case["V"], dt)
    _, _, _, imp = sals.kv_compact(K, V, to_device(case["Qobs"], dt), ctx=2000, k_keep=200, want_importance=True)
    torch.cuda.synchronize()
    _, ratio, _ = check(imp.cpu().numpy(), 0.9)
    n_hi = int(np.ceil(ratio * 2000))
    m = sals.kv_quantize_mixed(K, V, imp, n_hi=n_hi)
    torch.cuda.synchronize()
    assert m["codes_hi"].shape[3] == n_hi and m["codes_lo"].shape[3] == 2000 - n_hi


def test_flashcache_layer_budgets_from_outlier_energy():
    """Three layers' outlier importance -> their energies -> per-layer budgets in proportion, equal
    to the oracle's within one token (the floor of a ratio of fp32 energies)."""
    energies, ref_e = [], []
    for layer in range(3):
        cfg = C4.with_(B=1, H_q=2, H_kv=2, n_visual=800, grid_h=20, grid_w=40, clusters_h=2, clusters_w=4,
                       cfg_id=C4.cfg_id + 100 * layer, jitter=0.1 * (layer + 1))
        case = compact_case(cfg, ctx=1000)
        imp = sals.kv_outlier_importance(to_device(case["K"], "bf16"), to_device(case["V"], "bf16"), ctx=1000,
                                         n_freq=16)
        torch.cuda.synchronize()
        _, _, e = check(imp.cpu().numpy(), 0.9)
        energies.append(e)
        ref_e.append(oracle.outlier_importance(case["K"], case["V"], ctx=1000, n_freq=16).sum())
    assert np.allclose(energies, ref_e, rtol=1e-4)
    top = max(energies)
    got = sals.kv_layer_budgets([e / top for e in energies], total=600, ctx=1000)
    want = oracle.energy_budgets(ref_e, 600, 1000)
    assert all(abs(a - b) <= 1 for a, b in zip(got, want)), (got, list(want))
