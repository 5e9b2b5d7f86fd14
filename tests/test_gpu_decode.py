"""GPU parity of sals_decode_step (through the C ABI) against the oracle."""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - the GPU tests run on an MI355X
    pytest.skip("no GPU", allow_module_level=True)

import kv_cache_compression_sals_amd as sals  # noqa: E402
from parity import decode_parity, to_device  # noqa: E402
from workloads import CONFIGS, decode_case  # noqa: E402

C1, C2, C3, C5 = CONFIGS["c1"], CONFIGS["c2"], CONFIGS["c3"], CONFIGS["c5"]


def run_gpu(case):
    dt = case["dtype"]
    q, Lk, Lv = (to_device(case[n], dt) for n in ("q", "Lk", "Lv"))
    Pk, Pv = to_device(case["Pk"], dt), to_device(case["Pv"], dt)
    out, sel = sals.sals_decode_step(q, Lk, Lv, Pk, Pv, ctx=case["ctx"], k=case["k"], w=case["w"],
                                     G=case["G"], rope_base=case["base"], want_sel=True)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64), sel.cpu().numpy()


def check(case, batches=None):
    print(f"case {case['cfg'].name} B={case['B']} ctx={case['ctx']} cap={case['ctx_cap']} "
          f"k={case['k']} w={case['w']} G={case['G']} r={case['r']} d={case['d']}", flush=True)
    out, sel = run_gpu(case)
    stats = decode_parity(case, out, sel, batches=batches)
    print("  ", stats, flush=True)
    return out, sel


def test_c1_tiny_fp32_full():
    check(decode_case(C1))


SMALL = [
    # name, base cfg, overrides, B, ctx, ctx_cap
    ("c3_shape_ragged", C3, dict(calib_tokens=512), 2, 3001, 3100),
    ("c2_shape_ragged", C2, dict(calib_tokens=1024), 2, 1500, 1500),
    ("gqa_g2_d64", C3, dict(H_q=16, H_kv=8, d=64, r=128, G=2, k=50, w=8, rank=48, calib_tokens=512), 2, 777, 800),
    ("nqh8_r64", C3, dict(H_q=16, H_kv=2, d=128, r=64, G=1, k=40, w=8, rank=32, calib_tokens=256), 1, 500, 512),
    ("r32_g4", C3, dict(H_q=4, H_kv=4, d=64, r=32, G=4, k=20, w=4, rank=16, calib_tokens=256), 2, 300, 300),
    ("nqh2_r384", C3, dict(H_q=8, H_kv=4, d=128, r=384, G=4, k=100, w=16, rank=200, calib_tokens=512), 1, 1200, 1200),
    ("f32_d128_r256", C1, dict(H_q=8, H_kv=2, d=128, r=256, G=2, k=90, w=10, rank=64), 2, 700, 720),
    ("f32_gqa_d64_r128", C1, dict(H_q=8, H_kv=4, d=64, r=128, G=1, k=33, w=7, rank=40), 1, 413, 413),
    ("bf16_long_split", C3, dict(H_q=8, H_kv=2, r=256, G=2, k=1500, w=64, calib_tokens=512, rank=100), 1, 5000, 5000),
    # one selection for >= 4 KV heads: value side by the shared-selection kernels
    ("shared_r384_nqh2", C3, dict(H_q=16, H_kv=8, d=128, r=384, G=2, k=120, w=16, rank=200, calib_tokens=512), 2, 1300, 1333),
    ("shared_hs24_splits", C3, dict(H_q=24, H_kv=12, d=64, r=128, G=1, k=300, w=20, rank=48, calib_tokens=256), 2, 2000, 2100),
    ("shared_hs128", C3, dict(H_q=128, H_kv=16, d=64, r=64, G=1, k=150, w=16, rank=32, calib_tokens=256), 1, 1000, 1000),
    # the two-head key tile kernel (bf16, d = 128): r = 128 with 4 query heads per KV head over three
    # splits (the last ragged), and r = 256 whose second split holds one token
    ("skeys_r128_nqh4_ragged", C3, dict(H_q=32, H_kv=8, d=128, r=128, G=1, k=650, w=50, rank=64, calib_tokens=256), 1, 2000, 2000),
    ("skeys_r256_one_token_split", C3, dict(H_q=8, H_kv=8, d=128, r=256, G=2, k=280, w=9, rank=100, calib_tokens=256), 2, 1500, 1500),
]


@pytest.mark.parametrize("name,cfg,ov,B,ctx,cap", SMALL, ids=[s[0] for s in SMALL])
def test_small_shapes(name, cfg, ov, B, ctx, cap):
    check(decode_case(cfg.with_(**ov), B=B, ctx=ctx, ctx_cap=cap))


EDGES = [
    ("w_ge_ctx", dict(k=10, w=64), 40),
    ("k_zero", dict(k=0, w=16), 300),
    ("k_plus_w_ge_ctx", dict(k=200, w=16), 150),
    ("ctx_one", dict(k=8, w=4), 1),
    ("no_window", dict(k=25, w=0), 200),
    ("k_one", dict(k=1, w=0), 333),
]


@pytest.mark.parametrize("name,ov,ctx", EDGES, ids=[e[0] for e in EDGES])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_edge_cases(name, ov, ctx, dtype):
    base = C1 if dtype == "f32" else C3.with_(H_q=8, H_kv=4, r=64, G=2, rank=32, calib_tokens=256)
    check(decode_case(base.with_(**ov), B=2, ctx=ctx, ctx_cap=ctx + 5))


# the two-head key tile kernel ranking its own rows (bf16, d = 128, one selection for 4 KV heads):
# the same edges, where the selection needs no ranking (k = 0, k + w >= ctx, w >= ctx) or has
# massive ties (q = 0)
KEY_TILE = C3.with_(H_q=8, H_kv=4, d=128, r=128, G=1, rank=64, calib_tokens=256)


@pytest.mark.parametrize("name,ov,ctx", EDGES, ids=[e[0] for e in EDGES])
def test_edge_cases_key_tile_ranking(name, ov, ctx):
    check(decode_case(KEY_TILE.with_(**ov), B=2, ctx=ctx, ctx_cap=ctx + 5))


@pytest.mark.parametrize("Tc", [4095, 4096, 4097])
def test_key_tile_ranking_row_limit(Tc):
    """Rows of up to 4096 candidates are ranked inside the key tile kernel, longer ones by the
    top-k kernel; two selection groups of 4 KV heads, so two workgroups write selection rows."""
    case = decode_case(KEY_TILE.with_(H_q=16, H_kv=8, G=2, k=700, w=20), B=1, ctx=Tc + 20)
    check(case)


def _bf16_bits(x):
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


@pytest.mark.parametrize("kind", ["gaussian", "hot_region", "two_values"])
def test_long_row_ranked_in_attention_kernel(kind):
    """Rows past 32768 candidates with bf16 d = 128: the slice kernel keeps each slice's share and
    the attention kernel's workgroups merge their own row; with a hot region the slices' share
    cannot decide the selection and the exact digit selection over the scores takes over. The
    scores are planted: q = e_0 and P_k = I make S[t] = L_k[t][0] (bf16, so many exact ties)."""
    T, k, w = 40032, 3000, 32
    case = decode_case(C3.with_(H_q=1, H_kv=1, d=128, r=128, G=1, k=k, w=w, rank=64, calib_tokens=256), B=1,
                       ctx=T)
    rs = np.random.default_rng(11)
    sc = rs.standard_normal(T - w).astype(np.float32)
    if kind == "hot_region":
        sc[T // 3: T // 3 + 4000] += 4.0
    if kind == "two_values":
        sc = np.where(rs.random(T - w) < 0.05, 2.0, 1.0).astype(np.float32)
    case["Lk"][0, : T - w, 0] = _bf16_bits(sc)
    case["Pk"] = _bf16_bits(np.eye(128, 128, dtype=np.float32))
    q = np.zeros((1, 1, 128), dtype=np.float32)
    q[0, 0, 0] = 1.0
    case["q"] = _bf16_bits(q)
    print(f"long row ranked in the attention kernel: {kind} T={T} k={k} w={w}", flush=True)
    out, sel = run_gpu(case)
    scores = np.asarray(case["Lk"][0, : T - w, 0], dtype=np.uint32) << 16
    scores = scores.view(np.float32).astype(np.float64)
    order = np.lexsort((np.arange(T - w), -scores))  # score desc, index asc
    want = np.concatenate([np.sort(order[:k]), np.arange(T - w, T)])
    assert np.array_equal(sel[0, 0], want)
    decode_parity(case, out, sel)


@pytest.mark.parametrize("ctx", [250, 3000])
def test_zero_query_key_tile_ranking(ctx):
    case = decode_case(KEY_TILE.with_(k=20, w=6), B=2, ctx=ctx)
    case["q"] = np.zeros_like(case["q"])
    out, sel = run_gpu(case)
    want = np.concatenate([np.arange(20), np.arange(ctx - 6, ctx)])
    assert all(np.array_equal(sel[b, 0], want) for b in range(2))
    decode_parity(case, out, sel)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_exact_ties_lowest_index(dtype):
    """Latent rows drawn from 4 prototypes: scores take 4 values with massive exact ties; the
    selected set must equal the oracle's exactly (lowest indices among the threshold ties)."""
    base = C1 if dtype == "f32" else C3.with_(H_q=8, H_kv=4, r=64, G=2, rank=32, calib_tokens=256)
    case = decode_case(base.with_(k=37, w=5), B=2, ctx=400)
    rs = np.random.default_rng(5)
    for name in ("Lk", "Lv"):
        L = case[name]
        proto = L[:, :4].copy()
        pick = rs.integers(0, 4, size=L.shape[1])
        case[name] = np.ascontiguousarray(proto[:, pick])
    out, sel = run_gpu(case)
    import oracle
    ora = oracle.decode_step(case["q"], case["Lk"], case["Lv"], case["Pk"], case["Pv"], ctx=400, k=37, w=5,
                             G=case["G"], H_kv=case["H_kv"], base=case["base"], dtype=dtype)
    assert np.array_equal(sel, ora["sel"])
    decode_parity(case, out, sel)


@pytest.mark.parametrize("dtype,ctx", [("f32", 250), ("bf16", 250), ("bf16", 6000), ("bf16", 40000)])
def test_zero_query_all_ties(dtype, ctx):
    """q = 0: every score is +-0, so the selection is the lowest k positions plus the window.
    ctx 6000 ties more candidates than the short list holds; ctx 40000 exceeds the on-chip row."""
    base = C1 if dtype == "f32" else C3.with_(H_q=8, H_kv=4, r=64, G=2, rank=32, calib_tokens=256)
    case = decode_case(base.with_(k=20, w=6), B=1, ctx=ctx)
    case["q"] = np.zeros_like(case["q"])
    out, sel = run_gpu(case)
    want = np.concatenate([np.arange(20), np.arange(ctx - 6, ctx)])
    assert all(np.array_equal(sel[0, s], want) for s in range(case["G"]))
    decode_parity(case, out, sel)


def test_determinism_bitwise():
    case = decode_case(C3.with_(calib_tokens=512), B=2, ctx=2500)
    a = run_gpu(case)
    b = run_gpu(case)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_c2_full_size():
    """Every sequence and head of the 4K workload."""
    check(decode_case(C2))


def test_c3_full_size():
    """Every sequence and head of the 32K workload."""
    check(decode_case(C3))


@pytest.mark.parametrize("layer", [0, 31])
def test_c5_full_context_layer(layer):
    check(decode_case(C5, layer=layer))


def test_graph_capture_replays_match_eager():
    """A captured decode step, replayed several times with eager work and synchronisations in
    between, reproduces the eager result bit for bit on every replay."""
    case = decode_case(C3.with_(calib_tokens=512), B=2, ctx=3000)
    dt = case["dtype"]
    q, Lk, Lv, Pk, Pv = (to_device(case[n], dt) for n in ("q", "Lk", "Lv", "Pk", "Pv"))
    kw = dict(ctx=case["ctx"], k=case["k"], w=case["w"], G=case["G"], rope_base=case["base"])
    ref, ref_sel = sals.sals_decode_step(q, Lk, Lv, Pk, Pv, want_sel=True, **kw)
    torch.cuda.synchronize()
    ws = torch.empty(sals.sals_decode_workspace_bytes(q, Pk, ctx=case["ctx"], k=case["k"], w=case["w"],
                                                      G=case["G"]), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(ref)
    sel = torch.empty_like(ref_sel)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sals.sals_decode_step(q, Lk, Lv, Pk, Pv, out=out, sel_out=sel, workspace=ws, **kw)
    for rep in range(4):
        out.fill_(float("nan"))
        sel.fill_(-1)
        ws.fill_(0xAB)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref) and torch.equal(sel, ref_sel), rep
        # eager work between replays
        sals.sals_decode_step(q, Lk, Lv, Pk, Pv, **kw)
        torch.cuda.synchronize()


@pytest.mark.parametrize("name,cfg,ov,B,ctx", [
    ("shared_keys", C2, dict(calib_tokens=1024), 2, 1200),
    ("select_attend", C3, dict(calib_tokens=512), 2, 3001),
], ids=["shared_keys", "select_attend"])
def test_traced_step_matches_and_times(name, cfg, ov, B, ctx):
    """The traced entry point gives the same bytes as the plain one, and its six events are
    ordered with a positive duration for the attention kernel (timed by its own start and end)."""
    case = decode_case(cfg.with_(**ov), B=B, ctx=ctx, ctx_cap=ctx)
    print(f"traced {name} B={B} ctx={ctx}", flush=True)
    dt = case["dtype"]
    q, Lk, Lv, Pk, Pv = (to_device(case[n], dt) for n in ("q", "Lk", "Lv", "Pk", "Pv"))
    kw = dict(ctx=ctx, k=case["k"], w=case["w"], G=case["G"], rope_base=case["base"], want_sel=True)
    out0, sel0 = sals.sals_decode_step(q, Lk, Lv, Pk, Pv, **kw)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
    for e in evs:
        e.record()
    torch.cuda.synchronize()
    out1, sel1 = sals.sals_decode_step_traced(q, Lk, Lv, Pk, Pv, evs, **kw)
    torch.cuda.synchronize()
    assert torch.equal(out0, out1) and torch.equal(sel0, sel1)
    t = [evs[0].elapsed_time(e) for e in evs]
    print("   event times (ms):", [round(x, 4) for x in t], flush=True)
    assert all(t[i] <= t[i + 1] for i in range(5))
    assert evs[3].elapsed_time(evs[4]) > 0
