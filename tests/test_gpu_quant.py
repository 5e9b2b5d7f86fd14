"""GPU parity of kv_quantize_mixed and sals_dense_decode_mixed (the importance-based
mixed-precision cache, through the C ABI) against the oracle: positions, codes and (scale, zero
point) bit-exact, since every code is decided by the same fp32 steps on both sides; the decode
within 1e-4 max-abs of the oracle's fp64 attention over the dequantized rows."""

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
TIGHT = 1e-4


def _np(t):
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def check(case, imp, n_hi, pairs=None, heads=None):
    ctx = case["ctx"]
    K, V = case["K"], case["V"]
    B, H_kv, cap, d = K.shape
    H_q = case["H_q"]
    print(f"mixed B={B} H_q={H_q} H_kv={H_kv} d={d} cap={cap} ctx={ctx} n_hi={n_hi}", flush=True)
    Kd, Vd = to_device(K, "bf16"), to_device(V, "bf16")
    m = sals.kv_quantize_mixed(Kd, Vd, torch.from_numpy(imp).cuda(), n_hi=n_hi, ctx=ctx)
    q = to_device(case["q"], "bf16")
    out = sals.sals_dense_decode_mixed(q, m)
    torch.cuda.synchronize()
    got = {k: _np(v) for k, v in m.items()}
    out = out.cpu().numpy().astype(np.float64)
    ora = oracle.mixed_quantize(K, V, imp, ctx=ctx, n_hi=n_hi, dtype="bf16", pairs=pairs)
    todo = [(b, g) for b in range(B) for g in range(H_kv)] if pairs is None else pairs
    for b, g in todo:
        assert np.array_equal(got["pos_hi"][b, g], ora["pos_hi"][b, g]), (b, g)
        assert np.array_equal(got["pos_lo"][b, g], ora["pos_lo"][b, g]), (b, g)
        for name in ("codes_hi", "params_hi", "codes_lo", "params_lo"):
            a, r = got[name][:, b, g], ora[name][:, b, g]
            if not np.array_equal(a, r):
                bad = np.argwhere(a != r)
                raise AssertionError(f"{name} b{b} g{g}: {len(bad)} differ, first at {bad[0]}: {a[tuple(bad[0])]} vs "
                                     f"{r[tuple(bad[0])]}")
    hs = [(b, h) for b in range(B) for h in range(H_q) if (b, oracle.kv_head_of(h, H_q, H_kv)) in set(todo)]
    if heads is not None:
        hs = heads
    ref = oracle.mixed_decode(case["q"], ora, H_kv=H_kv, dtype="bf16", pairs=hs)
    err = max(np.abs(out[b, h] - ref[b, h]).max() for b, h in hs)
    print(f"   decode max-abs error {err:.2e} over {len(hs)} heads", flush=True)
    assert err <= 2e-2 and err <= TIGHT


def _tied_importance(rs, shape):
    imp = (np.round(rs.standard_normal(shape) * 4) / 4).astype(np.float32)
    imp[..., :4] = np.array([0.0, -0.0, 0.0, -0.0], dtype=np.float32)
    return imp


CASES = [
    # name, overrides, ctx, ctx_cap, n_hi
    ("d128_ragged_gqa4", dict(B=2, H_q=8, H_kv=2, n_visual=2000, grid_h=40, grid_w=50, clusters_h=4, clusters_w=5),
     3000, 3100, 300),
    ("d64_all_low", dict(B=1, H_q=3, H_kv=1, d=64, n_visual=2000, grid_h=40, grid_w=50, clusters_h=4, clusters_w=5),
     2500, 2500, 0),
    ("d128_all_high_nqh3", dict(B=1, H_q=6, H_kv=2, n_visual=500, grid_h=20, grid_w=25, clusters_h=2, clusters_w=5),
     777, 800, 777),
    ("d64_one_high", dict(B=2, H_q=2, H_kv=2, d=64, n_visual=100, grid_h=10, grid_w=10, clusters_h=2, clusters_w=2),
     129, 130, 1),
]


@pytest.mark.parametrize("name,ov,ctx,cap,n_hi", CASES, ids=[c[0] for c in CASES])
def test_mixed_small(name, ov, ctx, cap, n_hi):
    case = compact_case(C4.with_(**ov), ctx=ctx, ctx_cap=cap)
    rs = np.random.default_rng(ctx + n_hi)
    imp = _tied_importance(rs, (case["K"].shape[0], case["K"].shape[1], ctx))
    check(case, imp, n_hi)


def test_mixed_constant_groups():
    """Groups with equal values (span 0) store code 0, scale 0 and their value as zero point."""
    case = compact_case(C4.with_(B=1, H_q=2, H_kv=2, n_visual=200, grid_h=10, grid_w=20, clusters_h=2, clusters_w=2),
                        ctx=300)
    for X in (case["K"], case["V"]):
        X[0, 0, 10:40, 32:64] = X[0, 0, 10:40, 32:33]  # one constant group per row
        X[0, 1, 5, :] = X[0, 1, 5, :1]
    rs = np.random.default_rng(9)
    check(case, rs.standard_normal((1, 2, 300)).astype(np.float32), 50)


def test_mixed_from_compaction_importance():
    """The importance kv_compact returns ranks the tokens (the mixed cache of a VLM prompt)."""
    cfg = C4.with_(B=2, H_q=4, H_kv=4, n_visual=1500, grid_h=30, grid_w=50, clusters_h=3, clusters_w=5)
    case = compact_case(cfg, ctx=2000)
    dt = "bf16"
    _, _, _, imp = sals.kv_compact(to_device(case["K"], dt), to_device(case["V"], dt), to_device(case["Qobs"], dt),
                                   ctx=2000, k_keep=200, want_importance=True)
    torch.cuda.synchronize()
    check(case, imp.cpu().numpy(), 200)


def test_mixed_c4_full_size_sampled():
    """The full compaction workload (B=16, 32 heads, ctx 16384) with 10% of the tokens at 8 bits;
    four (sequence, head) pairs compared in full."""
    case = compact_case(C4, threads=16)
    rs = np.random.default_rng(12)
    imp = rs.standard_normal((16, 32, 16384)).astype(np.float32)
    check(case, imp, case["k_keep"], pairs=[(0, 0), (5, 9), (11, 20), (15, 31)])
