"""GPU parity of sals_reconstruct_kv (through the C ABI) against the oracle, and of the dense
baseline it feeds: the whole latent cache rebuilt and rotated, then sals_dense_decode.

Rebuilt rows are bf16 on both sides' terms: the GPU sums bf16 products in fp32 and rounds once,
the oracle rebuilds in fp64. An element may then differ by one bf16 step of its own magnitude
(2^-7 |x|) when the fp32 sum falls near a rounding boundary, plus fp32 noise near zero; the test
allows 2^-7 |ref| + 1e-5 max|ref|. The attention over the rounded cache is compared with the fp64
baseline at the bf16 tolerance of the decode path (2e-2 max-abs), and with the oracle's dense
decode over the GPU's own bf16 cache at fp32 accuracy (1e-4 max-abs).
"""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - the GPU tests run on an MI355X
    pytest.skip("no GPU", allow_module_level=True)

import kv_cache_compression_sals_amd as sals  # noqa: E402
import oracle.compact as OC  # noqa: E402
import oracle.sals as OS  # noqa: E402
from parity import to_device  # noqa: E402
from workloads import CONFIGS, decode_case  # noqa: E402

C2, C3 = CONFIGS["c2"], CONFIGS["c3"]
SENTINEL = 0x7F7F  # bf16 bits of a large finite value, never produced by these inputs


def bf16_to_f64(t):
    bits = t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16).astype(np.uint32)
    return (bits << 16).view(np.float32).astype(np.float64)


def rebuild_check(gpu, ref, what):
    err = np.abs(gpu - ref)
    bound = 2.0 ** -7 * np.abs(ref) + 1e-5 * np.abs(ref).max()
    worst = float((err / bound).max())
    print(f"   {what}: max err {err.max():.3e}, worst err/bound {worst:.3f}", flush=True)
    assert worst <= 1.0, what


def run(case, t0, T, stride, q_pos):
    dt = case["dtype"]
    q, Lk, Lv, Pk, Pv = (to_device(case[n], dt) for n in ("q", "Lk", "Lv", "Pk", "Pv"))
    B, H_kv, d = case["B"], case["H_kv"], case["d"]
    K = torch.full((B, H_kv, stride, d), SENTINEL, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    V = K.clone()
    q_rot = torch.empty_like(q)
    sals.sals_reconstruct_kv(Lk, Pk, K, t0=t0, T=T, d=d, rope_base=case["base"], Lv=Lv, Pv=Pv, V=V,
                             q=q, q_rot=q_rot, q_pos=q_pos)
    torch.cuda.synchronize()
    return q, K, V, q_rot


RANGES = [
    # name, cfg, overrides, B, ctx_cap, t0, T, extra stride
    ("c2_shape_ragged", C2, dict(calib_tokens=1024), 2, 1200, 37, 600, 3),
    ("c3_shape_tail", C3, dict(calib_tokens=512), 2, 1000, 0, 1000, 0),
    ("r128_one_token", C3, dict(H_q=8, H_kv=4, r=128, G=4, rank=64, calib_tokens=256), 1, 300, 299, 1, 0),
    ("r384_nqh2", C3, dict(H_q=8, H_kv=4, r=384, G=2, rank=200, calib_tokens=512), 2, 700, 100, 513, 5),
]


@pytest.mark.parametrize("name,cfg,ov,B,cap,t0,T,extra", RANGES, ids=[r[0] for r in RANGES])
def test_reconstruct_rows(name, cfg, ov, B, cap, t0, T, extra):
    case = decode_case(cfg.with_(**ov), B=B, ctx=cap, ctx_cap=cap)
    print(f"case {name} B={B} H_kv={case['H_kv']} r={case['r']} t0={t0} T={T}", flush=True)
    stride = cap + extra
    q, K, V, q_rot = run(case, t0, T, stride, q_pos=cap - 1)
    dt, H_kv = case["dtype"], case["H_kv"]
    Pk, Pv = OS.stored_to_f64(case["Pk"], dt), OS.stored_to_f64(case["Pv"], dt)
    Kg, Vg = bf16_to_f64(K), bf16_to_f64(V)
    for b in range(B):
        Lk, Lv = OS.stored_to_f64(case["Lk"][b], dt), OS.stored_to_f64(case["Lv"][b], dt)
        rebuild_check(Kg[b, :, t0:t0 + T], OS.reconstruct_cache(Lk, Pk, t0, T, H_kv, case["base"]), f"K b={b}")
        rebuild_check(Vg[b, :, t0:t0 + T], OS.reconstruct_cache(Lv, Pv, t0, T, H_kv, None), f"V b={b}")
    # rows outside [t0, t0 + T) are untouched
    raw = K.view(torch.int16).cpu().numpy().view(np.uint16)
    assert (raw[:, :, :t0] == SENTINEL).all() and (raw[:, :, t0 + T:] == SENTINEL).all()
    raw = V.view(torch.int16).cpu().numpy().view(np.uint16)
    assert (raw[:, :, :t0] == SENTINEL).all() and (raw[:, :, t0 + T:] == SENTINEL).all()
    qf = OS.stored_to_f64(case["q"], dt)
    ref_q = np.stack([OS.rope(qf[b], cap - 1, case["base"]) for b in range(B)])
    rebuild_check(bf16_to_f64(q_rot), ref_q, "q_rot")


PIPE = [
    ("c2_shape", C2, dict(calib_tokens=1024), 2, 900),
    ("c3_shape_gqa", C3, dict(calib_tokens=512), 2, 1500),
]


@pytest.mark.parametrize("name,cfg,ov,B,ctx", PIPE, ids=[p[0] for p in PIPE])
def test_dense_baseline_pipeline(name, cfg, ov, B, ctx):
    case = decode_case(cfg.with_(**ov), B=B, ctx=ctx, ctx_cap=ctx)
    print(f"case {name} B={B} H_q={case['H_q']} H_kv={case['H_kv']} r={case['r']} ctx={ctx}", flush=True)
    q, K, V, q_rot = run(case, 0, ctx, ctx, q_pos=ctx - 1)
    out = sals.sals_dense_decode(q_rot, K, V, n=ctx)
    torch.cuda.synchronize()
    out = out.cpu().numpy().astype(np.float64)
    own = lambda t: t.view(torch.int16).cpu().numpy().view(np.uint16)
    ref_own = OC.dense_decode(own(q_rot), own(K), own(V), n=ctx, H_kv=case["H_kv"], dtype="bf16")
    e_own = float(np.abs(out - ref_own).max())
    ref = OS.dense_baseline(case["q"], case["Lk"], case["Lv"], case["Pk"], case["Pv"], ctx=ctx,
                            H_kv=case["H_kv"], base=case["base"], dtype=case["dtype"])
    e = float(np.abs(out - ref).max())
    print(f"   vs dense decode over its own cache {e_own:.2e}; vs fp64 baseline {e:.2e}", flush=True)
    assert e_own <= 1e-4
    assert e <= 2e-2


SAMPLED = [("c2_full", C2), ("c3_full", C3)]


@pytest.mark.parametrize("name,cfg", SAMPLED, ids=[s[0] for s in SAMPLED])
def test_reconstruct_full_size_sampled(name, cfg):
    case = decode_case(cfg)
    ctx = case["ctx"]
    print(f"case {name} B={case['B']} H_kv={case['H_kv']} r={case['r']} ctx={ctx}", flush=True)
    q, K, V, q_rot = run(case, 0, ctx, ctx, q_pos=ctx - 1)
    dt, H_kv, d = case["dtype"], case["H_kv"], case["d"]
    Pk, Pv = OS.stored_to_f64(case["Pk"], dt), OS.stored_to_f64(case["Pv"], dt)
    rs = np.random.default_rng(5)
    for _ in range(24):
        b, g, t = int(rs.integers(case["B"])), int(rs.integers(H_kv)), int(rs.integers(ctx))
        Lk = OS.stored_to_f64(case["Lk"][b, t:t + 1], dt)
        Lv = OS.stored_to_f64(case["Lv"][b, t:t + 1], dt)
        Pg = slice(g * d, (g + 1) * d)
        ref_k = OS.rope(OS.reconstruct(Lk, Pk[Pg]), [t], case["base"])
        ref_v = OS.reconstruct(Lv, Pv[Pg])
        rebuild_check(bf16_to_f64(K[b, g, t:t + 1]), ref_k, f"K b={b} g={g} t={t}")
        rebuild_check(bf16_to_f64(V[b, g, t:t + 1]), ref_v, f"V b={b} g={g} t={t}")
    # the last tile (ragged when ctx is not a multiple of the tile) and the first token
    for t in (0, ctx - 1):
        Lk = OS.stored_to_f64(case["Lk"][0, t:t + 1], dt)
        rebuild_check(bf16_to_f64(K[0, H_kv - 1, t:t + 1]),
                      OS.rope(OS.reconstruct(Lk, Pk[(H_kv - 1) * d:]), [t], case["base"]), f"K edge t={t}")
