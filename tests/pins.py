"""Pins of the oracle: each raises AssertionError when the oracle disagrees with something
other than itself (a textbook formula written with loops, a closed form, a library routine,
a hand-worked example or an invariant the mathematics fixes).

They take no arguments and call the oracle through its modules' attributes, so that
``test_oracle_mutants`` can plant a mistake in the oracle and check that some pin catches it.
"""

import math

import numpy as np
import scipy.special

import brute
import oracle.compact as OC
import oracle.outlier as OO
import oracle.quant as OQ
import oracle.sals as OS

TOL = 1e-11


def _rand(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def _orthogonal(seed, n, m=None):
    m = n if m is None else m
    q, r = np.linalg.qr(_rand(seed, n, m))
    return q * np.sign(np.diag(r))[None, :]


def _run_decode(q, Lk, Lv, Pk, Pv, T, k, w, G, H_kv, base=10000.0):
    return OS.decode_step(q[None], Lk[None], Lv[None], Pk, Pv, ctx=T, k=k, w=w, G=G, H_kv=H_kv,
                          base=base, dtype="f64")


# ---------------------------------------------------------------------------------------------
# storage decode
# ---------------------------------------------------------------------------------------------

def _ieee_value(bits: int, exp_bits: int, man_bits: int) -> float:
    """Value of a finite IEEE binary pattern from the format's definition: sign, biased exponent,
    fraction; a zero exponent field is subnormal (no implicit leading one)."""
    bias = (1 << (exp_bits - 1)) - 1
    sign = -1.0 if (bits >> (exp_bits + man_bits)) & 1 else 1.0
    e = (bits >> man_bits) & ((1 << exp_bits) - 1)
    m = bits & ((1 << man_bits) - 1)
    if e == 0:
        return sign * math.ldexp(m, 1 - bias - man_bits)
    return sign * math.ldexp((1 << man_bits) + m, e - bias - man_bits)


def pin_stored_decode():
    """bf16 bit patterns decode to the IEEE binary16-brain values (1 sign, 8 exponent, 7 fraction
    bits): named patterns, then every finite pattern against the definition; fp32 values decode
    unchanged, checked on named and random finite bit patterns."""
    named = {0x3F80: 1.0, 0xC000: -2.0, 0x0000: 0.0, 0x4049: 3.140625, 0x3EAB: 0.333984375,
             0x7F7F: (2.0 - 2.0 ** -7) * 2.0 ** 127, 0x0001: 2.0 ** -133, 0x0080: 2.0 ** -126,
             0x807F: -(127 * 2.0 ** -133)}
    got = OS.stored_to_f64(np.array(list(named), dtype=np.uint16), "bf16")
    assert got.dtype == np.float64
    assert list(got) == list(named.values()), got
    neg0 = OS.stored_to_f64(np.array([0x8000], dtype=np.uint16), "bf16")[0]
    assert neg0 == 0.0 and math.copysign(1.0, neg0) == -1.0
    pats = np.array([b for b in range(1 << 16) if (b >> 7) & 0xFF != 0xFF], dtype=np.uint16)
    ref = np.array([_ieee_value(int(b), 8, 7) for b in pats])
    assert np.array_equal(OS.stored_to_f64(pats.reshape(-1, 16), "bf16").ravel(), ref)
    rs = np.random.default_rng(11)
    u = rs.integers(0, 1 << 32, size=4000, dtype=np.uint64).astype(np.uint32)
    u = u[((u >> 23) & 0xFF) != 0xFF]
    u = np.concatenate([u, np.array([0x00000001, 0x7F7FFFFF, 0x3F800001, 0x80000000], dtype=np.uint32)])
    f = u.view(np.float32)
    ref32 = np.array([_ieee_value(int(b), 8, 23) for b in u])
    assert np.array_equal(OS.stored_to_f64(f, "f32"), ref32)
    assert np.array_equal(OS.stored_to_f64(np.array([1.5, -0.25]), "f64"), [1.5, -0.25])


# ---------------------------------------------------------------------------------------------
# RoPE
# ---------------------------------------------------------------------------------------------

def pin_rope_d2_closed_form():
    """d = 2: theta_0 = 1, so RoPE([1, 0], p) = [cos p, sin p] and RoPE([0, 1], p) = [-sin p, cos p]."""
    for p in [0, 1, 2, 7, 1000, 131071]:
        a = OS.rope(np.array([[1.0, 0.0]]), p, 10000.0)[0]
        b = OS.rope(np.array([[0.0, 1.0]]), p, 10000.0)[0]
        assert np.allclose(a, [math.cos(p), math.sin(p)], atol=1e-12, rtol=0), (p, a)
        assert np.allclose(b, [-math.sin(p), math.cos(p)], atol=1e-12, rtol=0), (p, b)


def pin_rope_complex_form():
    """Agrees with (x_i + i x_{i+d/2}) e^{i p theta_i}, theta_i = base^(-2i/d)."""
    for d, base in [(8, 10000.0), (16, 500000.0), (64, 10000.0)]:
        x = _rand(d, 5, d)
        pos = [0, 3, 511, 4095, 131071]
        got = OS.rope(x, pos, base)
        for j in range(5):
            ref = brute.rope_complex(list(x[j]), pos[j], base)
            assert np.allclose(got[j], ref, atol=1e-9, rtol=0), (d, pos[j])


def pin_rope_invariants():
    """Norm preserved; position 0 is the identity; q.k depends only on the position difference."""
    d = 16
    x = _rand(1, 4, d)
    y = OS.rope(x, [5, 17, 1000, 99999], 10000.0)
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), atol=1e-12)
    assert np.array_equal(OS.rope(x, 0, 10000.0), x)
    q, k = _rand(2, d), _rand(3, d)
    for (a, b, c) in [(10, 3, 100), (4095, 0, 12345), (7, 7, 1)]:
        l1 = OS.rope(q[None], a, 10000.0)[0] @ OS.rope(k[None], b, 10000.0)[0]
        l2 = OS.rope(q[None], a + c, 10000.0)[0] @ OS.rope(k[None], b + c, 10000.0)[0]
        assert abs(l1 - l2) < 1e-9, (a, b, c)


# ---------------------------------------------------------------------------------------------
# selection
# ---------------------------------------------------------------------------------------------

def pin_select_hand_examples():
    """Hand-worked: candidates [0.5, 2.0, -1.0, 2.0, 0.3, 2.0, 1.5, 0.0], T=10, w=2, k=2:
    three 2.0 ties -> the lowest two indices 1, 3; window 8, 9."""
    S = np.array([0.5, 2.0, -1.0, 2.0, 0.3, 2.0, 1.5, 0.0])
    assert list(OS.select_tokens(S, 10, 2, 2)) == [1, 3, 8, 9]
    assert list(OS.select_tokens(S, 10, 4, 2)) == [1, 3, 5, 6, 8, 9]
    assert list(OS.select_tokens(np.array([0.0, -0.0]), 2, 1, 0)) == [0]
    assert list(OS.select_tokens(np.array([-0.0, 0.0]), 2, 1, 0)) == [0]
    assert list(OS.select_tokens(np.array([-0.0, 0.0, 1e-300]), 3, 1, 0)) == [2]
    # k = 0: window only; w >= T: everything; k + w >= T: everything
    assert list(OS.select_tokens(S, 10, 0, 2)) == [8, 9]
    assert list(OS.select_tokens(S[:0], 5, 3, 7)) == [0, 1, 2, 3, 4]
    assert list(OS.select_tokens(S, 10, 8, 2)) == list(range(10))
    assert list(OS.select_tokens(S, 10, 100, 2)) == list(range(10))


def pin_select_bruteforce():
    """Against Python's sorted() on (-score, index) keys, with heavy ties and signed zeros."""
    rng = np.random.default_rng(7)
    for trial in range(200):
        n = int(rng.integers(1, 40))
        vals = rng.integers(-3, 4, size=n).astype(np.float64)
        vals[rng.random(n) < 0.2] = -0.0
        T = n + int(rng.integers(0, 6))
        w = T - n
        k = int(rng.integers(0, n + 3))
        S = np.concatenate([vals, np.zeros(w)])
        got = list(OS.select_tokens(S, T, k, w))
        assert got == brute.select(list(S), T, k, w), (trial, vals, k, w)


# ---------------------------------------------------------------------------------------------
# projection
# ---------------------------------------------------------------------------------------------

def pin_project_identity_orthogonal():
    X = _rand(11, 3, 5, 12)
    assert np.array_equal(OS.project_kv(X, np.eye(12)), X)
    P = _orthogonal(12, 12)
    assert np.allclose(OS.project_kv(X, P) @ P.T, X, atol=1e-12)
    Pr = _orthogonal(13, 12, 4)  # orthonormal columns: projecting rows already in span(P) is lossless
    Y = _rand(14, 6, 4)
    assert np.allclose(OS.project_kv(Y @ Pr.T, Pr), Y, atol=1e-12)


# ---------------------------------------------------------------------------------------------
# decode: scores, selection and attention against dense RoPE attention
# ---------------------------------------------------------------------------------------------

SHAPES = [  # (H_q, H_kv, G, d)
    (2, 2, 1, 8),
    (4, 2, 2, 8),
    (4, 4, 2, 4),
    (6, 3, 3, 4),
    (4, 1, 1, 8),
]


def pin_decode_dense_special_case():
    """P = I (r = H_kv*d) and k + w >= T: SALS equals dense RoPE attention over the whole cache."""
    for i, (H_q, H_kv, G, d) in enumerate(SHAPES):
        D = H_kv * d
        for T, k, w in [(1, 0, 1), (9, 4, 5), (20, 15, 5), (24, 30, 0), (17, 0, 17)]:
            rs = np.random.default_rng(100 + i * 10 + T)
            K = rs.standard_normal((T, D))
            V = rs.standard_normal((T, D))
            q = rs.standard_normal((H_q, d))
            res = _run_decode(q, K, V, np.eye(D), np.eye(D), T, k, w, G, H_kv)
            ref = brute.dense_rope_attention(q.tolist(), K.tolist(), V.tolist(), range(T), T,
                                             10000.0, H_q, H_kv, d)
            assert np.allclose(res["out"][0], ref, atol=TOL, rtol=0), (H_q, H_kv, G, d, T, k, w)
            assert all(list(res["sel"][0, s]) == list(range(T)) for s in range(G))


def _selection_case(seed, H_q, H_kv, G, d, T, lowrank):
    D = H_kv * d
    rs = np.random.default_rng(seed)
    if lowrank:  # rows in span(P) with orthonormal columns: the latent is lossless
        r = max(2, D // 2)
        P = _orthogonal(seed + 1, D, r)
        Yk, Yv = rs.standard_normal((T, r)), rs.standard_normal((T, r))
        Kpre, Vpre, Lk, Lv = Yk @ P.T, Yv @ P.T, Yk, Yv
    else:  # square orthogonal P
        P = _orthogonal(seed + 1, D)
        Kpre, Vpre = rs.standard_normal((T, D)), rs.standard_normal((T, D))
        Lk, Lv = Kpre @ P, Vpre @ P
    q = rs.standard_normal((H_q, d))
    return q, Kpre, Vpre, Lk, Lv, P


def pin_decode_selected_matches_masked_dense():
    """With a lossless projection, the latent score of group s at t is the RoPE-free logit sum
    over its heads; the selected set is its top-k (ties low) plus the window; and the output is
    dense RoPE attention restricted to that set."""
    for i, (H_q, H_kv, G, d) in enumerate(SHAPES):
        for lowrank in (False, True):
            for T, k, w in [(30, 6, 4), (41, 10, 7), (25, 1, 0), (12, 0, 3)]:
                q, Kpre, Vpre, Lk, Lv, P = _selection_case(500 + 7 * i + T, H_q, H_kv, G, d, T, lowrank)
                res = _run_decode(q, Lk, Lv, P, P, T, k, w, G, H_kv)
                T_c = max(0, T - w)
                Sb = brute.ropefree_group_scores(q.tolist(), Kpre.tolist(), T_c, H_q, H_kv, G, d)
                assert np.allclose(res["S"][0], np.array(Sb).reshape(G, T_c), atol=1e-10, rtol=0)
                for s in range(G):
                    assert list(res["sel"][0, s]) == brute.select(Sb[s], T, k, w), (i, lowrank, T, s)
                for h in range(H_q):
                    s = brute.grp_of(brute.kv_of(h, H_q, H_kv), H_kv, G)
                    pos = brute.select(Sb[s], T, k, w)
                    ref = brute.dense_rope_attention(q.tolist(), Kpre.tolist(), Vpre.tolist(), pos, T,
                                                     10000.0, H_q, H_kv, d)
                    assert np.allclose(res["out"][0, h], ref[h], atol=1e-10, rtol=0), (i, lowrank, T, h)


def pin_decode_uniform_and_single():
    """q = 0: every score and logit is 0, so the top-k is the lowest k' positions and the output
    is the plain mean of the rebuilt value rows over the selected set. ctx = 1: the output is
    the single rebuilt value row."""
    H_q, H_kv, G, d = 4, 2, 1, 8
    D = H_kv * d
    T, k, w = 20, 5, 3
    rs = np.random.default_rng(3)
    Lk, Lv = rs.standard_normal((T, 6)), rs.standard_normal((T, 6))
    Pk, Pv = rs.standard_normal((D, 6)), rs.standard_normal((D, 6))
    res = _run_decode(np.zeros((H_q, d)), Lk, Lv, Pk, Pv, T, k, w, G, H_kv)
    sel = list(range(5)) + [17, 18, 19]
    assert list(res["sel"][0, 0]) == sel
    for h in range(H_q):
        g = brute.kv_of(h, H_q, H_kv)
        Vh = np.array([[sum(Lv[t, j] * Pv[g * d + c, j] for j in range(6)) for c in range(d)] for t in sel])
        assert np.allclose(res["out"][0, h], Vh.mean(axis=0), atol=1e-12, rtol=0)
    res1 = _run_decode(rs.standard_normal((H_q, d)), Lk[:1], Lv[:1], Pk, Pv, 1, 4, 2, G, H_kv)
    for h in range(H_q):
        g = brute.kv_of(h, H_q, H_kv)
        assert np.allclose(res1["out"][0, h], Pv[g * d:(g + 1) * d] @ Lv[0], atol=1e-12, rtol=0)


def pin_decode_softmax_and_permutation():
    """Attention weights sum to 1; permuting the latent rows among unselected candidate positions
    changes neither the selected set nor the output (scores are position-free)."""
    H_q, H_kv, G, d = 4, 2, 2, 8
    D, r, T, k, w = H_kv * d, 6, 40, 8, 4
    rs = np.random.default_rng(21)
    Lk, Lv = rs.standard_normal((T, r)), rs.standard_normal((T, r))
    Pk, Pv = rs.standard_normal((D, r)), rs.standard_normal((D, r))
    q = rs.standard_normal((H_q, d))
    res = _run_decode(q, Lk, Lv, Pk, Pv, T, k, w, G, H_kv)
    sets = [res["sel"][0, s] for s in range(G)]
    _, weights = OS.attend_selected(q, Lk, Lv, Pk, Pv, sets, T, 10000.0, H_kv, G)
    for pi in weights:
        assert abs(pi.sum() - 1.0) < 1e-14 and (pi >= 0).all()
    chosen = set(np.concatenate(sets).tolist())
    free = [t for t in range(T - w) if t not in chosen]
    perm = np.array(free)[rs.permutation(len(free))]
    idx = np.arange(T)
    idx[free] = perm
    res2 = _run_decode(q, Lk[idx], Lv[idx], Pk, Pv, T, k, w, G, H_kv)
    assert np.array_equal(res2["sel"], res["sel"])
    assert np.array_equal(res2["out"], res["out"])


# ---------------------------------------------------------------------------------------------
# compaction
# ---------------------------------------------------------------------------------------------

def pin_importance_bruteforce_and_mass():
    """Causal importance against explicit loops; it is non-negative and sums to w per query head."""
    rs = np.random.default_rng(31)
    for T, w, d in [(1, 1, 4), (9, 3, 4), (23, 8, 8), (16, 16, 2)]:
        Q, K = rs.standard_normal((w, d)), rs.standard_normal((T, d))
        I = OC.importance(Q, K, T)
        assert np.allclose(I, brute.causal_importance(Q.tolist(), K.tolist(), T), atol=1e-13, rtol=0)
        assert (I >= 0).all() and abs(I.sum() - w) < 1e-12


def pin_importance_closed_forms():
    """Zero queries: every allowed key gets 1/(p_i+1), so I[t] = sum_{i: p_i >= t} 1/(p_i + 1).
    One query (w = 1) at T-1 sees every key: I equals scipy's softmax of K q / sqrt(d)."""
    T, w, d = 12, 5, 4
    I = OC.importance(np.zeros((w, d)), np.random.default_rng(0).standard_normal((T, d)), T)
    ref = [sum(1.0 / (p + 1) for p in range(T - w, T) if p >= t) for t in range(T)]
    assert np.allclose(I, ref, atol=1e-14, rtol=0)
    rs = np.random.default_rng(1)
    K, q = rs.standard_normal((T, d)), rs.standard_normal((1, d))
    assert np.allclose(OC.importance(q, K, T), scipy.special.softmax(K @ q[0] / math.sqrt(d)), atol=1e-14)


def pin_compact_identity_and_masked():
    """k_keep = T keeps every row unchanged; a dense decode over the compact cache equals
    masked attention over the full cache with the evicted positions at -inf; the dense decode
    itself equals scipy's softmax times V."""
    rs = np.random.default_rng(41)
    B, H_q, H_kv, T, w, d = 2, 4, 2, 14, 3, 4
    K, V = rs.standard_normal((B, H_kv, T, d)), rs.standard_normal((B, H_kv, T, d))
    Q = rs.standard_normal((B, H_q, w, d))
    full = OC.kv_compact(K, V, Q, ctx=T, k_keep=T, H_kv=H_kv, dtype="f64")
    assert np.array_equal(full["Kc"], K) and np.array_equal(full["Vc"], V)
    assert (full["kept"] == np.arange(T)).all()
    # importance per KV head sums over its query heads: total mass w * (H_q / H_kv)
    assert np.allclose(full["importance"].sum(axis=-1), w * H_q / H_kv, atol=1e-12)
    c = OC.kv_compact(K, V, Q, ctx=T, k_keep=5, H_kv=H_kv, dtype="f64")
    q = rs.standard_normal((B, H_q, d))
    out = OC.dense_decode(q, c["Kc"], c["Vc"], n=5, H_kv=H_kv, dtype="f64")
    for b in range(B):
        for h in range(H_q):
            g = brute.kv_of(h, H_q, H_kv)
            keep = set(c["kept"][b, g].tolist())
            ref = brute.masked_attention(q[b, h].tolist(), K[b, g].tolist(), V[b, g].tolist(), keep)
            assert np.allclose(out[b, h], ref, atol=1e-12, rtol=0)
            lib = scipy.special.softmax(K[b, g] @ q[b, h] / math.sqrt(d)) @ V[b, g]
            assert np.allclose(OC.dense_decode(q, K, V, n=T, H_kv=H_kv, dtype="f64")[b, h], lib, atol=1e-12)
            # the kept set is the top-5 of the importance (ties low), ascending
            Ib = c["importance"][b, g]
            assert sorted(c["kept"][b, g].tolist()) == sorted(sorted(range(T), key=lambda t: (-Ib[t], t))[:5])
            ref_I = np.sum([brute.causal_importance(Q[b, hh].tolist(), K[b, g].tolist(), T)
                            for hh in range(H_q) if brute.kv_of(hh, H_q, H_kv) == g], axis=0)
            assert np.allclose(Ib, ref_I, atol=1e-12)


# ---------------------------------------------------------------------------------------------
# the full-rebuild baseline
# ---------------------------------------------------------------------------------------------

def pin_reconstruct_cache_identity():
    """P = I (r = H_kv*d): the rebuilt rows of head g are its slice of the input, rotated at the
    absolute position t (complex form, loops) for keys and unchanged for values, also with t0 > 0."""
    H_kv, d, t0, T = 3, 8, 5, 7
    D = H_kv * d
    L = _rand(31, t0 + T + 2, D)
    Kc = OS.reconstruct_cache(L, np.eye(D), t0, T, H_kv, 500.0)
    Vc = OS.reconstruct_cache(L, np.eye(D), t0, T, H_kv, None)
    for g in range(H_kv):
        for j in range(T):
            row = L[t0 + j, g * d:(g + 1) * d]
            ref = brute.rope_complex(row.tolist(), t0 + j, 500.0)
            assert np.allclose(Kc[g, j], ref, atol=TOL, rtol=0), (g, j)
            assert np.array_equal(Vc[g, j], row)


def pin_dense_baseline_identity_and_full_selection():
    """P = I: the baseline is dense RoPE attention over the whole cache (loops, complex RoPE).
    With a lossy P and k + w >= T, SALS selects every token, so it equals the baseline."""
    for i, (H_q, H_kv, G, d) in enumerate(SHAPES):
        D = H_kv * d
        T = 13 + i
        rs = np.random.default_rng(700 + i)
        K, V, q = rs.standard_normal((T, D)), rs.standard_normal((T, D)), rs.standard_normal((H_q, d))
        out = OS.dense_baseline(q[None], K[None], V[None], np.eye(D), np.eye(D), ctx=T, H_kv=H_kv,
                                base=10000.0, dtype="f64")
        ref = brute.dense_rope_attention(q.tolist(), K.tolist(), V.tolist(), range(T), T, 10000.0, H_q, H_kv, d)
        assert np.allclose(out[0], ref, atol=TOL, rtol=0), (H_q, H_kv, G, d)
        r = max(2, D // 2)
        Pk, Pv = _orthogonal(710 + i, D, r), _orthogonal(720 + i, D, r)
        Lk, Lv = rs.standard_normal((T, r)), rs.standard_normal((T, r))
        base_out = OS.dense_baseline(q[None], Lk[None], Lv[None], Pk, Pv, ctx=T, H_kv=H_kv, base=10000.0,
                                     dtype="f64")
        sals_out = _run_decode(q, Lk, Lv, Pk, Pv, T, T, 3, G, H_kv)["out"]
        assert np.allclose(base_out, sals_out, atol=TOL, rtol=0), (H_q, H_kv, G, d)


def pin_compact_from_importance():
    """Against Python's sorted() on (-I, t) keys with ties and signed zeros; with the importance
    kv_compact computed for the same cache it keeps the same rows."""
    rs = np.random.default_rng(41)
    B, H, T, d, k = 2, 3, 40, 4, 11
    I = np.round(rs.standard_normal((B, H, T)), 1)  # many ties
    I[0, 0, :5] = [0.0, -0.0, 0.0, -0.0, 0.0]
    K = rs.standard_normal((B, H, T + 3, d))
    V = rs.standard_normal((B, H, T + 3, d))
    res = OC.compact_from_importance(K, V, I, k_keep=k)
    for b in range(B):
        for g in range(H):
            ref = sorted(sorted(range(T), key=lambda t: (-float(I[b, g, t]) + 0.0, t))[:k])
            assert list(res["kept"][b, g]) == ref, (b, g)
            assert np.array_equal(res["Kc"][b, g], K[b, g, ref]) and np.array_equal(res["Vc"][b, g], V[b, g, ref])
    Q = rs.standard_normal((B, 2 * H, 5, d))
    full = OC.kv_compact(K, V, Q, ctx=T, k_keep=k, H_kv=H, dtype="f64")
    again = OC.compact_from_importance(K, V, full["importance"], k_keep=k)
    assert np.array_equal(full["kept"], again["kept"]) and np.array_equal(full["Kc"], again["Kc"])


def pin_sparsity_bruteforce_and_closed_form():
    """Below-threshold counts against explicit loops with math.exp; q = 0 gives a[i, t] =
    1/(p_i + 1), so an entry counts exactly when p_i + 1 > 1/p; p above every probability counts
    all causal entries and p = 0 none."""
    rs = np.random.default_rng(53)
    T, w, d = 19, 6, 4
    Q = rs.standard_normal((w, d)) * 2.0
    K = rs.standard_normal((T + 2, d))
    for p in (0.01, 0.05, 0.2):
        G, below, total, _ = OC.sparsity(Q, K, T, p)
        cnt = tot = 0
        for i in range(w):
            pi = T - w + i
            logits = [sum(Q[i][c] * K[t][c] for c in range(d)) / math.sqrt(d) for t in range(pi + 1)]
            m = max(logits)
            e = [math.exp(v - m) for v in logits]
            z = sum(e)
            cnt += sum(1 for v in e if v / z < p)
            tot += pi + 1
        assert below == cnt and total == tot and abs(G - cnt / tot) < 1e-15, p
    G0, below0, total0, _ = OC.sparsity(np.zeros((w, d)), K, T, 0.07)
    ref = sum(T - w + i + 1 for i in range(w) if T - w + i + 1 > 1 / 0.07)
    assert below0 == ref and total0 == sum(T - w + i + 1 for i in range(w))
    assert OC.sparsity(Q, K, T, 1.5)[1] == total0 and OC.sparsity(Q, K, T, 0.0)[1] == 0
    # a probability exactly at the threshold (1/16 for the row of 16 positions) is not below it
    ref16 = sum(T - w + i + 1 for i in range(w) if T - w + i + 1 > 16)
    assert OC.sparsity(np.zeros((w, d)), K, T, 1.0 / 16)[1] == ref16


def pin_layer_budgets():
    """Proportional split: equal ratios give equal shares; shares follow the ratios and never
    exceed the total; the clamps hold; a zero normaliser splits evenly."""
    k = OC.layer_budgets([0.5, 0.5, 0.5, 0.5], 400, 1000)
    assert list(k) == [100, 100, 100, 100]
    k = OC.layer_budgets([0.1, 0.3, 0.6], 1000, 10_000)
    assert list(k) == [100, 300, 600]
    k = OC.layer_budgets([0.2, 0.7, 0.05], 777, 10_000)
    assert sum(k) <= 777 and list(k) == [int(777 * 0.2 / 0.95), int(777 * 0.7 / 0.95), int(777 * 0.05 / 0.95)]
    assert list(OC.layer_budgets([0.0, 1.0], 5000, 300)) == [1, 300]
    assert list(OC.layer_budgets([0.0, 0.0, 0.0], 90, 1000)) == [30, 30, 30]


# ---------------------------------------------------------------------------------------------
# frequency-domain outlier importance
# ---------------------------------------------------------------------------------------------

def pin_dct_basis():
    """The basis is the orthonormal DCT-II: C^T x equals scipy's dct(x, type 2, norm 'ortho'), and
    C^T C = I; a hand value: T = 2 gives [[1, 1], [1, -1]] / sqrt(2)."""
    import scipy.fft
    for T in (5, 16, 33):
        C = OO.dct_basis(T, T)
        x = _rand(T, T, 3)
        assert np.allclose(C.T @ x, scipy.fft.dct(x, type=2, norm="ortho", axis=0), atol=1e-12, rtol=0), T
        assert np.allclose(C.T @ C, np.eye(T), atol=1e-12), T
    assert np.allclose(OO.dct_basis(2, 2), np.array([[1.0, 1.0], [1.0, -1.0]]) / math.sqrt(2.0), atol=1e-15)


def pin_outlier_closed_forms():
    """Closed forms of the deviation energy: zero when every frequency is kept, zero for a
    constant (DC) signal, zero for a mode below the cutoff and its full energy for one at or above
    it; the total equals the energy of the dropped coefficients (Parseval); and the explicit
    per-token loops of the definition on a tiny input."""
    T, d = 24, 3
    X = _rand(7, T, d)
    assert np.abs(OO.deviation_energy(X, T)).max() < 1e-20
    Xc = np.tile(_rand(8, 1, d), (T, 1))
    assert np.abs(OO.deviation_energy(Xc, 1)).max() < 1e-20
    t = np.arange(T)
    for f0, F in ((3, 4), (3, 3), (10, 2)):
        col = math.sqrt(2.0 / T) * np.cos(np.pi * (2 * t + 1) * f0 / (2 * T))
        Xm = np.outer(col, [2.0, -1.0, 0.5])
        got = OO.deviation_energy(Xm, F)
        want = np.zeros(T) if f0 < F else (col ** 2) * (4.0 + 1.0 + 0.25)
        assert np.allclose(got, want, atol=1e-12, rtol=0), (f0, F)
    for F in (1, 5, 17):
        import scipy.fft
        coef = scipy.fft.dct(X, type=2, norm="ortho", axis=0)
        assert abs(OO.deviation_energy(X, F).sum() - (coef[F:] ** 2).sum()) < 1e-10, F
    # brute force: explicit loops with math.cos
    T, F = 9, 3
    Xs = _rand(9, T, 2)
    ref = []
    for tt in range(T):
        e = 0.0
        for c in range(2):
            lp = 0.0
            for f in range(F):
                a = math.sqrt((1.0 if f == 0 else 2.0) / T)
                coef = sum(a * math.cos(math.pi * (2 * u + 1) * f / (2 * T)) * Xs[u, c] for u in range(T))
                lp += a * math.cos(math.pi * (2 * tt + 1) * f / (2 * T)) * coef
            e += (Xs[tt, c] - lp) ** 2
        ref.append(e)
    assert np.allclose(OO.deviation_energy(Xs, F), ref, atol=1e-12, rtol=0)


def pin_outlier_importance_pairs():
    """The importance of a pair is the deviation energy of its key plus that of its value (a zero
    value contributes nothing); the kept set is the top-k of it with lowest-index ties, and the
    gathered rows are the stored rows."""
    B, H, T, d, F = 2, 3, 40, 4, 6
    rs = np.random.default_rng(3)
    K = rs.standard_normal((B, H, T + 2, d))
    V = rs.standard_normal((B, H, T + 2, d))
    I = OO.outlier_importance(K, V, ctx=T, n_freq=F, dtype="f64")
    for b in range(B):
        for g in range(H):
            want = OO.deviation_energy(K[b, g, :T], F) + OO.deviation_energy(V[b, g, :T], F)
            assert np.allclose(I[b, g], want, atol=1e-12)
    I0 = OO.outlier_importance(K, np.zeros_like(V), ctx=T, n_freq=F, dtype="f64")
    assert np.allclose(I0[1, 2], OO.deviation_energy(K[1, 2, :T], F), atol=1e-12)
    r = OO.outlier_compact(K, V, ctx=T, n_freq=F, k_keep=7, dtype="f64")
    for b in range(B):
        for g in range(H):
            order = sorted(range(T), key=lambda t: (-I[b, g, t], t))[:7]
            assert list(r["kept"][b, g]) == sorted(order)
            assert np.array_equal(r["Kc"][b, g], K[b, g, r["kept"][b, g]])
            assert np.array_equal(r["Vc"][b, g], V[b, g, r["kept"][b, g]])


# ---------------------------------------------------------------------------------------------
# mixed-precision cache
# ---------------------------------------------------------------------------------------------

def pin_quant_group():
    """Groups whose values sit exactly on the grid decode exactly (4 bits: zero point 0.5, step
    1/16; 8 bits: zero point -1, step 1/128); a constant group, or one whose span is below 2^-96,
    has code 0, scale 0 and its minimum as zero point; and for random groups every code is in
    [0, 2^bits - 1] and within 1/2 step (plus fp32 rounding) of its value."""
    q4 = np.array([0, 15, 3, 7, 8, 1, 14, 2] * 4)
    x4 = (0.5 + q4 / 16.0).astype(np.float32)
    c, sc, z = OQ.quantize_group(x4, 4)
    assert list(c) == list(q4) and sc == np.float32(1 / 16) and z == np.float32(0.5)
    q8 = np.array([0, 255, 128, 127, 1, 254, 64, 200] * 4)
    x8 = (-1.0 + q8 / 128.0).astype(np.float32)
    c, sc, z = OQ.quantize_group(x8, 8)
    assert list(c) == list(q8) and sc == np.float32(1 / 128) and z == np.float32(-1.0)
    assert np.array_equal(OQ.dequantize_rows(c[None], np.array([[[sc, z]]])), x8[None].astype(np.float64))
    c, sc, z = OQ.quantize_group(np.full(32, 0.75, dtype=np.float32), 8)
    assert not c.any() and sc == 0.0 and z == np.float32(0.75)
    tiny = np.zeros(32, dtype=np.float32)
    tiny[5] = np.float32(2.0 ** -110)
    c, sc, z = OQ.quantize_group(tiny, 4)
    assert not c.any() and sc == 0.0 and z == 0.0
    rs = np.random.default_rng(21)
    for bits in (4, 8):
        for _ in range(200):
            x = (rs.standard_normal(32) * rs.uniform(0.01, 30)).astype(np.float32)
            c, sc, z = OQ.quantize_group(x, bits)
            assert c.min() >= 0 and c.max() <= (1 << bits) - 1
            assert c[np.argmin(x)] == 0 and c[np.argmax(x)] == (1 << bits) - 1
            xh = float(z) + c * float(sc)
            step = (float(x.max()) - float(x.min())) / ((1 << bits) - 1)
            assert np.all(np.abs(xh - x) <= 0.5 * step * (1 + 1e-5) + 2.0 ** -21 * np.abs(x).max()), bits


def pin_quant_layout_and_split():
    """Nibble packing puts the even channel in the low nibble (hand example, round trip); the
    important set is the top n_hi by (-importance, position), the rest is its complement, both
    ascending; rows are quantized at 8 and 4 bits in their own sets."""
    assert OQ.pack_nibbles(np.array([[1, 2, 3, 4]])).tolist() == [[0x21, 0x43]]
    c = np.random.default_rng(2).integers(0, 16, size=(5, 64))
    assert np.array_equal(OQ.unpack_nibbles(OQ.pack_nibbles(c)), c)
    imp = np.array([0.3, 2.0, -1.0, 2.0, 0.0, -0.0, 5.0, 0.3, 1.0])
    hi, lo = OQ.split_positions(imp, 9, 4)
    assert list(hi) == [1, 3, 6, 8] and list(lo) == [0, 2, 4, 5, 7]
    B, H, T, d = 1, 2, 40, 64
    rs = np.random.default_rng(4)
    K = rs.standard_normal((B, H, T, d))
    V = rs.standard_normal((B, H, T, d))
    I = rs.standard_normal((B, H, T))
    m = OQ.mixed_quantize(K, V, I, ctx=T, n_hi=7, dtype="f64")
    for g in range(H):
        order = sorted(range(T), key=lambda t: (-I[0, g, t], t))
        assert list(m["pos_hi"][0, g]) == sorted(order[:7]) and list(m["pos_lo"][0, g]) == sorted(order[7:])
        rows_hi = K[0, g, m["pos_hi"][0, g]].astype(np.float32)
        c8, p8 = OQ.quantize_rows(rows_hi, 8)
        assert np.array_equal(m["codes_hi"][0, 0, g], c8) and np.array_equal(m["params_hi"][0, 0, g], p8)
        rows_lo = V[0, g, m["pos_lo"][0, g]].astype(np.float32)
        c4, p4 = OQ.quantize_rows(rows_lo, 4)
        assert np.array_equal(OQ.unpack_nibbles(m["codes_lo"][1, 0, g]), c4)
        assert np.array_equal(m["params_lo"][1, 0, g], p4)


def pin_mixed_decode():
    """On grid-exact data (every 32-channel group spans -1 .. 127/128 in steps of 1/128) with every
    position at 8 bits, the decode equals plain attention over the original cache; in general it
    equals plain attention over the dequantized rows put back at their positions."""
    B, H_q, H_kv, T, d = 1, 4, 2, 30, 64
    rs = np.random.default_rng(6)
    qv = rs.integers(0, 256, size=(2, B, H_kv, T, d))
    qv[..., 0] = 0
    qv[..., 32] = 255
    qv[..., 1] = 255
    qv[..., 33] = 0
    K, V = -1.0 + qv[0] / 128.0, -1.0 + qv[1] / 128.0
    q = rs.standard_normal((B, H_q, d))
    I = rs.standard_normal((B, H_kv, T))
    m = OQ.mixed_quantize(K, V, I, ctx=T, n_hi=T, dtype="f64")
    ref = OC.dense_decode(q, K, V, n=T, H_kv=H_kv, dtype="f64")
    assert np.allclose(OQ.mixed_decode(q, m, H_kv=H_kv, dtype="f64"), ref, atol=1e-13, rtol=0)
    K, V = rs.standard_normal((B, H_kv, T, d)), rs.standard_normal((B, H_kv, T, d))
    for n_hi in (0, 11, T):
        m = OQ.mixed_quantize(K, V, I, ctx=T, n_hi=n_hi, dtype="f64")
        Kh, Vh = np.zeros_like(K), np.zeros_like(V)
        for g in range(H_kv):
            pos = np.concatenate([m["pos_hi"][0, g], m["pos_lo"][0, g]])
            Kh[0, g, pos], Vh[0, g, pos] = OQ.mixed_rows(m, 0, 0, g), OQ.mixed_rows(m, 1, 0, g)
        ref = OC.dense_decode(q, Kh, Vh, n=T, H_kv=H_kv, dtype="f64")
        assert np.allclose(OQ.mixed_decode(q, m, H_kv=H_kv, dtype="f64"), ref, atol=1e-12, rtol=0), n_hi


def pin_select_threshold():
    """Threshold selection, hand-worked on candidates [0.5, 2.0, -1.0, 2.0, 0.3, 2.0, 1.5, 0.0],
    T = 10, w = 2: tau 1.5, k 4 keeps every score >= 1.5 (1, 3, 5, 6); tau 1.6, k 2 caps three
    passing 2.0 ties at the lowest two; a score equal to tau passes; tau above every score keeps
    only the window; tau -inf is plain top-k; k = 0 keeps the window. Random rows: equal to a
    filter-then-sort written with sorted()."""
    S = np.array([0.5, 2.0, -1.0, 2.0, 0.3, 2.0, 1.5, 0.0, 9.0, 9.0])
    f = OS.select_tokens_threshold
    assert list(f(S, 10, 4, 2, 1.5)) == [1, 3, 5, 6, 8, 9]
    assert list(f(S, 10, 2, 2, 1.6)) == [1, 3, 8, 9]
    assert list(f(S, 10, 9, 2, 0.3)) == [0, 1, 3, 4, 5, 6, 8, 9]
    assert list(f(S, 10, 4, 2, 3.0)) == [8, 9]
    assert list(f(S, 10, 0, 2, -5.0)) == [8, 9]
    assert list(f(np.array([0.0, -0.0, 1.0]), 3, 5, 0, -0.0)) == [0, 1, 2]
    rs = np.random.default_rng(8)
    for _ in range(100):
        T = int(rs.integers(1, 60))
        w = int(rs.integers(0, 5))
        k = int(rs.integers(0, 40))
        S = np.round(rs.standard_normal(T) * 3) / 2
        tau = float(np.round(rs.standard_normal() * 3) / 2)
        assert list(f(S, T, k, w, -np.inf)) == list(OS.select_tokens(S, T, k, w))
        T_c = max(0, T - w)
        passing = [t for t in range(T_c) if S[t] >= tau]
        keep = sorted(sorted(passing, key=lambda t: (-S[t], t))[:k])
        assert list(f(S, T, k, w, tau)) == keep + list(range(T_c, T)), (T, w, k, tau)


def pin_decode_threshold():
    """The threshold decode attends over its own ragged sets: equal to attend_selected over them,
    and to the top-k decode when tau lies below every score."""
    H_q, H_kv, G, d, r, T = 4, 2, 2, 8, 6, 40
    rs = np.random.default_rng(14)
    q = rs.standard_normal((H_q, d))
    Lk, Lv = rs.standard_normal((T, r)), rs.standard_normal((T, r))
    Pk, Pv = rs.standard_normal((H_kv * d, r)), rs.standard_normal((H_kv * d, r))
    kw = dict(ctx=T, k=9, w=3, G=G, H_kv=H_kv, base=10000.0, dtype="f64")
    th = OS.decode_step_threshold(q[None], Lk[None], Lv[None], Pk, Pv, tau=0.5, **kw)
    S = th["S"][0]
    for s in range(G):
        want = OS.select_tokens_threshold(S[s], T, 9, 3, 0.5)
        assert np.array_equal(th["sel"][0][s], want) and th["n_sel"][0, s] == len(want)
    ref, _ = OS.attend_selected(q, Lk, Lv, Pk, Pv, th["sel"][0], T, 10000.0, H_kv, G)
    assert np.allclose(th["out"][0], ref, atol=1e-12)
    low = OS.decode_step_threshold(q[None], Lk[None], Lv[None], Pk, Pv, tau=-1e300, **kw)
    top = OS.decode_step(q[None], Lk[None], Lv[None], Pk, Pv, **kw)
    assert np.allclose(low["out"], top["out"], atol=1e-12)
    assert all(np.array_equal(low["sel"][0][s], top["sel"][0, s]) for s in range(G))


def pin_mass_budget():
    """Hand-worked: [4, 3, 2, 1] holds 10; 70% needs 4 + 3 (n = 2), 71% needs three values; ties
    [2, 2, 2, 2] at 50% need two; a row of zeros keeps one; order does not matter; random rows
    against a cumulative sum of the sorted values."""
    assert OC.mass_budget([1.0, 4.0, 2.0, 3.0], 0.7) == (2, 10.0)
    assert OC.mass_budget([4.0, 3.0, 2.0, 1.0], 0.71)[0] == 3
    assert OC.mass_budget([2.0, 2.0, 2.0, 2.0], 0.5)[0] == 2
    assert OC.mass_budget([0.0, 0.0, 0.0], 0.9) == (1, 0.0)
    assert OC.mass_budget([5.0, 0.0, 0.0], 1.0)[0] == 1
    assert OC.mass_budget([1.0, 1.0, 1.0], 1.0)[0] == 3
    rs = np.random.default_rng(10)
    for _ in range(50):
        v = rs.exponential(size=int(rs.integers(1, 200)))
        m = float(rs.uniform(0.05, 1.0))
        c = np.cumsum(np.sort(v)[::-1])
        assert OC.mass_budget(v, m)[0] == int(np.argmax(c >= m * v.sum() - 1e-12)) + 1
    I = rs.exponential(size=(2, 3, 50))
    r = OC.importance_budget(I, ctx=40, mass=0.5)
    assert r["n_keep"][1, 2] == OC.mass_budget(I[1, 2, :40], 0.5)[0]
    assert abs(r["layer_ratio"] - r["n_keep"].sum() / (6 * 40)) < 1e-15
    assert abs(r["layer_energy"] - I[:, :, :40].sum()) < 1e-9


def pin_energy_budgets():
    """Budgets follow the energies: equal energies split evenly, 1:4 splits 1:4, a zero-energy
    layer gets the minimum of one token, the clamp to ctx holds."""
    assert list(OC.energy_budgets([2.0, 2.0], 100, 1000)) == [50, 50]
    assert list(OC.energy_budgets([1.0, 4.0], 500, 1000)) == [100, 400]
    assert list(OC.energy_budgets([0.0, 5.0], 100, 60)) == [1, 60]


PINS = [
    pin_stored_decode,
    pin_rope_d2_closed_form,
    pin_rope_complex_form,
    pin_rope_invariants,
    pin_select_hand_examples,
    pin_select_bruteforce,
    pin_project_identity_orthogonal,
    pin_decode_dense_special_case,
    pin_decode_selected_matches_masked_dense,
    pin_decode_uniform_and_single,
    pin_decode_softmax_and_permutation,
    pin_importance_bruteforce_and_mass,
    pin_importance_closed_forms,
    pin_compact_identity_and_masked,
    pin_reconstruct_cache_identity,
    pin_dense_baseline_identity_and_full_selection,
    pin_compact_from_importance,
    pin_sparsity_bruteforce_and_closed_form,
    pin_layer_budgets,
    pin_dct_basis,
    pin_outlier_closed_forms,
    pin_outlier_importance_pairs,
    pin_quant_group,
    pin_quant_layout_and_split,
    pin_mixed_decode,
    pin_select_threshold,
    pin_decode_threshold,
    pin_mass_budget,
    pin_energy_budgets,
]
