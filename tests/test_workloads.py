"""Seeded input generators: codec, determinism, shapes and structure (CPU only)."""

import numpy as np

from workloads import CONFIGS, bf16_bits_to_f32, compact_case, decode_case, f32_to_bf16_bits, project_case


def test_bf16_round_nearest_even():
    # exactly representable values round-trip
    x = np.array([0.0, -0.0, 1.0, -2.5, 3.140625, 65280.0, 2.0 ** -126], dtype=np.float32)
    assert np.array_equal(bf16_bits_to_f32(f32_to_bf16_bits(x)).view(np.uint32), x.view(np.uint32))
    # ties: 1 + 2^-8 is halfway between 1 and 1 + 2^-7 -> even (1.0); 1 + 3*2^-8 -> 1 + 2^-6
    t = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8)], dtype=np.float32)
    assert list(bf16_bits_to_f32(f32_to_bf16_bits(t))) == [1.0, 1 + 2 ** -6, -1.0]
    # just above half rounds up
    u = np.array([1 + 2 ** -8 + 2 ** -20], dtype=np.float32)
    assert bf16_bits_to_f32(f32_to_bf16_bits(u))[0] == 1 + 2 ** -7
    # round to nearest: error at most half a bf16 ulp, i.e. 2^-8 relative
    r = np.random.default_rng(0).standard_normal(10000).astype(np.float32)
    back = bf16_bits_to_f32(f32_to_bf16_bits(r))
    assert np.all(np.abs(back - r) <= np.abs(r) * 2.0 ** -8)


def test_decode_case_deterministic_and_prefix():
    c = CONFIGS["c3"].with_(ctx=300, B=3, calib_tokens=512)
    a = decode_case(c, B=3, ctx=300)
    b = decode_case(c, B=2, ctx=300, ctx_cap=320)
    assert a["Lk"].dtype == np.uint16 and a["Lk"].shape == (3, 300, 256)
    assert np.array_equal(a["Lk"][:2], b["Lk"][:, :300]) and np.array_equal(a["q"][:2], b["q"])
    assert np.array_equal(a["Pk"], b["Pk"]) and not np.array_equal(a["Pk"], a["Pv"])
    assert (b["Lk"][:, 300:] == 0).all()


def test_decode_case_c1_shapes_and_orthonormal_p():
    c = decode_case(CONFIGS["c1"])
    assert c["Lk"].dtype == np.float32 and c["Lk"].shape == (1, 512, 64)
    assert c["q"].shape == (1, 4, 64) and c["Pk"].shape == (256, 64)
    P = c["Pk"].astype(np.float64)
    assert np.allclose(P.T @ P, np.eye(64), atol=1e-6)
    # rows are rank-32 plus 5% noise: the latent keeps most of the energy in 32 directions
    s = np.linalg.svd(c["Lk"][0].astype(np.float64), compute_uv=False)
    assert s[31] > 5 * s[32]


def test_svd_projection_captures_signal():
    c = CONFIGS["c2"].with_(ctx=64, calib_tokens=1024, rank=48, r=64, H_kv=4, H_q=4)
    case = decode_case(c, B=1, with_x=True)
    X = case["Xk"][0].astype(np.float64)
    P = bf16_bits_to_f32(case["Pk"]).astype(np.float64)
    resid = X - (X @ P) @ P.T
    assert np.linalg.norm(resid) < 0.3 * np.linalg.norm(X)


def test_project_case_shapes():
    c = CONFIGS["c2"].with_(H_q=4, H_kv=4, r=64, rank=32, calib_tokens=256)
    p = project_case(c, B=2, T=33)
    assert p["Xk"].shape == (2, 33, 512) and p["Xk"].dtype == np.uint16 and p["Pk"].shape == (512, 64)


def test_compact_case_structure():
    c = CONFIGS["c4"]
    case = compact_case(c, B=1, ctx=c.ctx)
    K = bf16_bits_to_f32(case["K"][0, 0]).astype(np.float64)
    # tokens 0 and 1 share a cluster (same grid block): jitter-sized difference
    assert np.linalg.norm(K[0] - K[1]) < 0.25 * np.linalg.norm(K[0])
    # token 0 and token 16 lie in neighbouring blocks: different centroids
    assert np.linalg.norm(K[0] - K[16]) > 0.5 * np.linalg.norm(K[0])
    assert case["k_keep"] == 1638 and case["Qobs"].shape == (1, 32, 64, 128)
