"""GPU parity of sals_project_kv, kv_compact and sals_dense_decode against the oracle."""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

import kv_cache_compression_sals_amd as sals  # noqa: E402
import oracle  # noqa: E402
from parity import EXEMPT_REL, check_selection, to_device  # noqa: E402
from workloads import CONFIGS, compact_case, project_case  # noqa: E402

C1, C2, C3, C4 = CONFIGS["c1"], CONFIGS["c2"], CONFIGS["c3"], CONFIGS["c4"]


def _ulp(x, dtype):
    """Spacing of the storage format at |x| (bf16: 8 significant bits, fp32: 24)."""
    ax = np.maximum(np.abs(x), np.finfo(np.float32).tiny)
    return 2.0 ** (np.floor(np.log2(ax)) - (7 if dtype == "bf16" else 23))


def _projection_bound(X, P, exact, dtype):
    """One rounding to the storage type (at most one ulp of the exact value, counting a rounding
    that crosses into the next binade) plus the forward error of an fp32 sum of D products,
    D * 2^-24 * sum_i |x_i p_i| (the products of bf16 or fp32 inputs are formed exactly or with
    one fp32 rounding each, which the same bound covers)."""
    D = X.shape[-1]
    return _ulp(exact, dtype) + D * 2.0 ** -24 * (np.abs(X) @ np.abs(P))


def _project(case, t0, cap):
    dt = case["dtype"]
    B, T = case["B"], case["T"]
    r = case["r"]
    Xk, Xv = to_device(case["Xk"], dt), to_device(case["Xv"], dt)
    Pk, Pv = to_device(case["Pk"], dt), to_device(case["Pv"], dt)
    tdt = torch.float32 if dt == "f32" else torch.bfloat16
    Lk = torch.full((B, cap, r), 7.0, dtype=tdt, device="cuda")
    Lv = torch.full((B, cap, r), 7.0, dtype=tdt, device="cuda")
    sals.sals_project_kv(Xk, Pk, Lk, t0, d=case["cfg"].d, Xv=Xv, Pv=Pv, Lv=Lv)
    torch.cuda.synchronize()
    return Lk.float().cpu().numpy(), Lv.float().cpu().numpy()


PROJ = [
    ("c1_f32", C1, 1, 512, 0, 512),
    ("c2_shape_ragged", C2.with_(calib_tokens=1024), 2, 333, 17, 400),
    ("c3_shape", C3.with_(calib_tokens=512), 2, 1000, 0, 1000),
    ("d64_r32", C3.with_(H_kv=4, d=64, r=32, rank=16, calib_tokens=256), 1, 129, 3, 200),
]


@pytest.mark.parametrize("name,cfg,B,T,t0,cap", PROJ, ids=[p[0] for p in PROJ])
def test_project_kv(name, cfg, B, T, t0, cap):
    case = project_case(cfg, B=B, T=T)
    Lk, Lv = _project(case, t0, cap)
    dt = case["dtype"]
    for X, P, L in ((case["Xk"], case["Pk"], Lk), (case["Xv"], case["Pv"], Lv)):
        Xf, Pf = oracle.stored_to_f64(X, dt), oracle.stored_to_f64(P, dt)
        exact = oracle.project_kv(Xf, Pf)
        got = L[:, t0:t0 + T]
        bound = _projection_bound(Xf, Pf, exact, dt)
        assert np.all(np.abs(got - exact) <= bound), np.max(np.abs(got - exact) / bound)
        # rows outside [t0, t0 + T) untouched
        assert np.all(L[:, :t0] == 7.0) and np.all(L[:, t0 + T:] == 7.0)


def test_project_kv_c2_full_rows():
    """Full C2 prefill (8 x 4096 rows): every output of every sequence checked."""
    case = project_case(C2, B=8, T=4096)
    Lk, _ = _project(case, 0, 4096)
    for b in range(8):
        Xf, Pf = oracle.stored_to_f64(case["Xk"][b], "bf16"), oracle.stored_to_f64(case["Pk"], "bf16")
        exact = oracle.project_kv(Xf, Pf)
        assert np.all(np.abs(Lk[b] - exact) <= _projection_bound(Xf, Pf, exact, "bf16"))


# ---- compaction ----------------------------------------------------------------------------

def _compact(case):
    dt = case["dtype"]
    K, V, Q = to_device(case["K"], dt), to_device(case["V"], dt), to_device(case["Qobs"], dt)
    Kc, Vc, kept, imp = sals.kv_compact(K, V, Q, ctx=case["ctx"], k_keep=case["k_keep"], want_importance=True)
    q = to_device(case["q"], dt)
    out = sals.sals_dense_decode(q, Kc, Vc)
    torch.cuda.synchronize()
    f = lambda t: t.cpu().numpy()  # noqa: E731
    return (f(Kc.view(torch.int16)).view(np.uint16) if dt == "bf16" else f(Kc),
            f(Vc.view(torch.int16)).view(np.uint16) if dt == "bf16" else f(Vc),
            f(kept), f(imp), f(out).astype(np.float64))


def check_compact(case, pairs):
    dt = case["dtype"]
    T, k_keep = case["ctx"], case["k_keep"]
    Kc, Vc, kept, imp, out = _compact(case)
    ora = oracle.kv_compact(case["K"], case["V"], case["Qobs"], ctx=T, k_keep=k_keep, H_kv=case["H_kv"],
                            dtype=dt, pairs=pairs)
    H_q, H_kv = case["H_q"], case["H_kv"]
    for b, g in pairs:
        I = ora["importance"][b, g]
        assert np.abs(imp[b, g] - I).max() <= EXEMPT_REL * I.max(), np.abs(imp[b, g] - I).max()
        check_selection(I, k_keep, T, 0, kept[b, g], ora["kept"][b, g], f"b{b} g{g}")
        # bit-exact gather of the GPU's own kept rows
        assert np.array_equal(Kc[b, g], case["K"][b, g, kept[b, g]])
        assert np.array_equal(Vc[b, g], case["V"][b, g, kept[b, g]])
        heads = [(b, h) for h in range(H_q) if h * H_kv // H_q == g]
        ref = oracle.dense_decode(case["q"], Kc, Vc, n=k_keep, H_kv=H_kv, dtype=dt, pairs=heads)
        for _, h in heads:
            err = np.abs(out[b, h] - ref[b, h]).max()
            # the stated bf16 tolerance, and the tight bound of exact inputs with fp32 sums
            assert err <= (2e-2 if dt == "bf16" else 1e-4), err
            assert err <= 1e-4, err


def test_compact_small_ragged():
    cfg = C4.with_(B=2, H_q=4, H_kv=4, ctx=2000, w=24, n_visual=1500, grid_h=30, grid_w=50, clusters_h=3,
                   clusters_w=5)
    case = compact_case(cfg, ctx=2000, ctx_cap=2100)
    check_compact(case, [(b, g) for b in range(2) for g in range(4)])


def test_compact_gqa_w_gt_64_f32_like_shapes():
    cfg = C4.with_(B=1, H_q=8, H_kv=2, d=64, ctx=1500, w=80, n_visual=1200, grid_h=30, grid_w=40,
                   clusters_h=3, clusters_w=4)
    case = compact_case(cfg, ctx=1500)
    check_compact(case, [(0, 0), (0, 1)])


def test_compact_keep_all_is_identity():
    cfg = C4.with_(B=1, H_q=2, H_kv=2, ctx=300, w=8, n_visual=200, grid_h=10, grid_w=20, clusters_h=2,
                   clusters_w=2)
    case = compact_case(cfg, ctx=300)
    case["k_keep"] = 300
    Kc, Vc, kept, _, _ = _compact(case)
    assert (kept == np.arange(300)).all()
    assert np.array_equal(Kc, case["K"][:, :, :300]) and np.array_equal(Vc, case["V"][:, :, :300])


def test_compact_c4_full_size():
    """The full compaction workload: every KV head of sequence 7, plus two heads elsewhere."""
    case = compact_case(C4, threads=16)
    check_compact(case, [(0, 0), (15, 31)] + [(7, g) for g in range(case["H_kv"])])


def test_dense_decode_full_cache_matches_oracle():
    cfg = C4.with_(B=2, H_q=8, H_kv=4, ctx=3000, n_visual=2000, grid_h=40, grid_w=50, clusters_h=4,
                   clusters_w=5)
    case = compact_case(cfg, ctx=3000, ctx_cap=3000)
    K, V, q = (to_device(case[n], "bf16") for n in ("K", "V", "q"))
    out = sals.sals_dense_decode(q, K, V, n=2999).cpu().numpy()
    ref = oracle.dense_decode(case["q"], case["K"], case["V"], n=2999, H_kv=4, dtype="bf16")
    assert np.abs(out - ref).max() <= 2e-2
    assert np.abs(out - ref).max() <= 1e-4  # exact inputs, fp32 sums


def _bf16_bits(x):
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


DENSE = [
    # B, H_q, H_kv, d, n, stride, dtype: query heads per KV head 4, 2, 8, 3 and 1; one token
    (2, 16, 4, 128, 5000, 5003, "bf16"),
    (1, 16, 8, 64, 3001, 3001, "bf16"),
    (2, 32, 4, 128, 1000, 1000, "bf16"),
    (1, 12, 4, 128, 777, 800, "bf16"),
    (3, 4, 4, 64, 1, 4, "bf16"),
    (1, 8, 2, 128, 2000, 2000, "f32"),
    (2, 6, 6, 64, 300, 310, "f32"),
]


@pytest.mark.parametrize("B,H_q,H_kv,d,n,stride,dt", DENSE, ids=[f"nqh{c[1] // c[2]}_n{c[4]}_{c[6]}" for c in DENSE])
def test_dense_decode_grouped_heads(B, H_q, H_kv, d, n, stride, dt):
    """Every query head against the oracle at fp32 accuracy: the inputs are exact on both sides."""
    print(f"dense B={B} H_q={H_q} H_kv={H_kv} d={d} n={n} stride={stride} {dt}", flush=True)
    rs = np.random.default_rng(B * 1000 + H_q * 10 + n)
    q = rs.standard_normal((B, H_q, d)).astype(np.float32)
    K = rs.standard_normal((B, H_kv, stride, d)).astype(np.float32) * 1.5
    V = rs.standard_normal((B, H_kv, stride, d)).astype(np.float32)
    if dt == "bf16":
        q, K, V = _bf16_bits(q), _bf16_bits(K), _bf16_bits(V)
    out = sals.sals_dense_decode(to_device(q, dt), to_device(K, dt), to_device(V, dt), n=n).cpu().numpy()
    ref = oracle.dense_decode(q, K, V, n=n, H_kv=H_kv, dtype=dt)
    err = np.abs(out - ref).max()
    print(f"   max err {err:.2e}", flush=True)
    assert err <= 1e-4


# ---- compaction from a given importance -------------------------------------------------------

FROM_IMP = [
    # B, H_kv, d, ctx, ctx_cap, k_keep, dtype (a row past 32768 positions takes the global path)
    (2, 4, 128, 3000, 3100, 300, "bf16"),
    (1, 2, 64, 40000, 40000, 4000, "bf16"),
    (2, 3, 64, 777, 800, 777, "f32"),
    (1, 1, 128, 5, 8, 1, "bf16"),
]


@pytest.mark.parametrize("B,H_kv,d,ctx,cap,k_keep,dt", FROM_IMP,
                         ids=[f"ctx{c[3]}_k{c[5]}_{c[6]}" for c in FROM_IMP])
def test_compact_from_importance_matches_oracle(B, H_kv, d, ctx, cap, k_keep, dt):
    """Heavily tied importance (multiples of 0.1, signed zeros): kept sets exact, rows bit-exact."""
    print(f"from_importance B={B} H_kv={H_kv} d={d} ctx={ctx} k_keep={k_keep} {dt}", flush=True)
    rs = np.random.default_rng(ctx + k_keep)
    imp = (np.round(rs.standard_normal((B, H_kv, ctx)) * 10) / 10).astype(np.float32)
    imp[0, 0, : min(4, ctx)] = np.array([0.0, -0.0, 0.0, -0.0], dtype=np.float32)[: min(4, ctx)]
    K = rs.standard_normal((B, H_kv, cap, d)).astype(np.float32)
    V = rs.standard_normal((B, H_kv, cap, d)).astype(np.float32)
    if dt == "bf16":
        K, V = _bf16_bits(K), _bf16_bits(V)
    Kc, Vc, kept = sals.kv_compact_from_importance(to_device(K, dt), to_device(V, dt),
                                                   torch.from_numpy(imp).cuda(), k_keep=k_keep)
    torch.cuda.synchronize()
    ref = oracle.compact_from_importance(K, V, imp, k_keep=k_keep)
    assert np.array_equal(kept.cpu().numpy(), ref["kept"])
    raw = (lambda t: t.view(torch.int16).cpu().numpy().view(np.uint16)) if dt == "bf16" else (lambda t: t.cpu().numpy())
    assert np.array_equal(raw(Kc), ref["Kc"]) and np.array_equal(raw(Vc), ref["Vc"])


def _importance_rows(kind, rows, ctx, rs):
    """Importance rows shaped to drive each path of the per-row selection: spread values (a
    small threshold bin), a range stretched by one huge value or by infinities (every key in a
    few value bins: the key-bit fallback), a narrow positive range with ties, two far clusters,
    subnormals and constant rows."""
    x = rs.standard_normal((rows, ctx)).astype(np.float32)
    if kind == "outlier":
        x[:, rs.integers(0, ctx, rows)] = np.float32(1e30)
    elif kind == "inf":
        x[:, ::97] = np.inf
        x[:, 5::89] = -np.inf
    elif kind == "narrow":
        x = (np.float32(1.0) + np.float32(2.0 ** -20) * np.round(x * 8)).astype(np.float32)
    elif kind == "clusters":
        x = np.where(rs.random((rows, ctx)) < 0.5, x * 1e-3, 1000 + x * 1e-3).astype(np.float32)
    elif kind == "subnormal":
        x = (x * np.float32(1e-39)).astype(np.float32)
    elif kind == "constant":
        x[:] = np.float32(-2.5)
    return x


IMP_KINDS = ["gauss", "outlier", "inf", "narrow", "clusters", "subnormal", "constant"]


@pytest.mark.parametrize("ctx", [4000, 16384, 32768])
@pytest.mark.parametrize("kind", IMP_KINDS)
def test_compact_from_importance_value_distributions(kind, ctx):
    """The kept sets are exact (ties to the lowest position) for every value distribution, at row
    lengths of 4, 16 and 32 keys per thread, for several k."""
    print(f"from_importance kind={kind} ctx={ctx}", flush=True)
    rs = np.random.default_rng(ctx * 31 + IMP_KINDS.index(kind))
    H_kv, d = 2, 64
    imp = _importance_rows(kind, H_kv, ctx, rs).reshape(1, H_kv, ctx)
    K = rs.standard_normal((1, H_kv, ctx, d)).astype(np.float32)
    V = rs.standard_normal((1, H_kv, ctx, d)).astype(np.float32)
    Kd, Vd, Id = torch.from_numpy(K).cuda(), torch.from_numpy(V).cuda(), torch.from_numpy(imp).cuda()
    for k_keep in (1, 37, ctx // 10, ctx // 2 + 3, ctx - 1):
        Kc, Vc, kept = sals.kv_compact_from_importance(Kd, Vd, Id, k_keep=k_keep)
        torch.cuda.synchronize()
        ref = oracle.compact_from_importance(K, V, imp, k_keep=k_keep)
        assert np.array_equal(kept.cpu().numpy(), ref["kept"]), (kind, ctx, k_keep)
        assert np.array_equal(Kc.cpu().numpy(), ref["Kc"]), (kind, ctx, k_keep)


def test_compact_higher_layer_from_lower_layer_importance():
    """The lower layer's kv_compact importance ranks a higher layer's cache (same selection rule)."""
    cfg = C4.with_(B=2, H_q=8, H_kv=4, ctx=3000, w=32, n_visual=2000, grid_h=40, grid_w=50, clusters_h=4,
                   clusters_w=5)
    low = compact_case(cfg, ctx=3000)
    high = compact_case(cfg.with_(cfg_id=cfg.cfg_id + 1000), ctx=3000)  # another layer's draw
    dt = low["dtype"]
    _, _, _, imp = sals.kv_compact(to_device(low["K"], dt), to_device(low["V"], dt), to_device(low["Qobs"], dt),
                                   ctx=3000, k_keep=300, want_importance=True)
    Kc, Vc, kept = sals.kv_compact_from_importance(to_device(high["K"], dt), to_device(high["V"], dt), imp,
                                                   k_keep=300)
    torch.cuda.synchronize()
    ref = oracle.compact_from_importance(high["K"], high["V"], imp.cpu().numpy(), k_keep=300)
    assert np.array_equal(kept.cpu().numpy(), ref["kept"])
    assert np.array_equal(Kc.view(torch.int16).cpu().numpy().view(np.uint16), ref["Kc"])


# ---- post-vision sparsity and layer budgets ---------------------------------------------------

SPARSE = [
    # cfg overrides, ctx, ctx_cap, p, heads checked ((b, h) pairs, None = all)
    (dict(B=2, H_q=8, H_kv=4, ctx=2000, w=24, n_visual=1500, grid_h=30, grid_w=50, clusters_h=3, clusters_w=5),
     2000, 2100, 1e-3, None),
    (dict(B=1, H_q=4, H_kv=4, ctx=1500, w=80, n_visual=1200, grid_h=30, grid_w=40, clusters_h=3, clusters_w=4),
     1500, 1500, 1e-2, None),
    ({}, 16384, 16384, 1e-3, [(0, 0), (7, 13), (15, 31)]),
]


@pytest.mark.parametrize("ov,ctx,cap,p,pairs", SPARSE, ids=["gqa_w24", "w80_p1e-2", "c4_full_sampled"])
def test_importance_sparsity_matches_oracle(ov, ctx, cap, p, pairs):
    """Below-threshold counts per query head within the entries the oracle finds at p (relative
    1e-5), and the importance identical to kv_compact's."""
    cfg = C4.with_(**ov)
    case = compact_case(cfg, ctx=ctx, ctx_cap=cap, threads=16)
    print(f"sparsity B={case['K'].shape[0]} H_q={case['H_q']} H_kv={case['H_kv']} ctx={ctx} p={p}", flush=True)
    dt = case["dtype"]
    K, V, Q = to_device(case["K"], dt), to_device(case["V"], dt), to_device(case["Qobs"], dt)
    imp, sp = sals.kv_importance_sparsity(K, Q, ctx=ctx, p=p)
    _, _, _, imp2 = sals.kv_compact(K, V, Q, ctx=ctx, k_keep=max(1, ctx // 10), want_importance=True)
    torch.cuda.synchronize()
    assert torch.equal(imp, imp2)
    sp = sp.cpu().numpy()
    H_q, H_kv = case["H_q"], case["H_kv"]
    B = case["K"].shape[0]
    todo = [(b, h) for b in range(B) for h in range(H_q)] if pairs is None else pairs
    Qf = oracle.stored_to_f64(case["Qobs"], dt)
    for b, h in todo:
        g = oracle.kv_head_of(h, H_q, H_kv)
        G, below, total, near = oracle.sparsity(Qf[b, h], oracle.stored_to_f64(case["K"][b, g, :ctx], dt), ctx, p)
        err = abs(float(sp[b, h]) * total - below)
        assert err <= near + 0.5 + 1e-6 * total, (b, h, float(sp[b, h]), G, near)
    print(f"   sparsity range {sp.min():.4f} .. {sp.max():.4f}", flush=True)
