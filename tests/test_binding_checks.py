"""The Python binding rejects mis-shaped tensors with ValueError before any pointer reaches the C
ABI (which sees only pointers, so a wrong size would mean out-of-bounds device accesses). CPU
tensors are enough: the shape checks run before the device check."""

import pytest
import torch

import kv_cache_compression_sals_amd as sals

bf = torch.bfloat16


def _decode_inputs(B=2, H_q=8, H_kv=4, d=64, r=64, cap=100):
    q = torch.zeros(B, H_q, d, dtype=bf)
    Lk = torch.zeros(B, cap, r, dtype=bf)
    Pk = torch.zeros(H_kv * d, r, dtype=bf)
    return q, Lk, Lk.clone(), Pk, Pk.clone()


DECODE_BAD = [
    ("Lv", lambda a: a.__setitem__(2, torch.zeros(2, 99, 64, dtype=bf))),
    ("Lv", lambda a: a.__setitem__(2, torch.zeros(2, 100, 32, dtype=bf))),
    ("Pv", lambda a: a.__setitem__(4, torch.zeros(256, 32, dtype=bf))),
    ("Lk", lambda a: a.__setitem__(1, torch.zeros(3, 100, 64, dtype=bf))),
    ("multiple of d", lambda a: a.__setitem__(3, torch.zeros(100, 64, dtype=bf))),
    ("ctx", None),
]


@pytest.mark.parametrize("what,mut", DECODE_BAD, ids=[f"{i}_{b[0]}" for i, b in enumerate(DECODE_BAD)])
def test_decode_rejects_bad_inputs(what, mut):
    a = list(_decode_inputs())
    ctx = 50
    if mut is None:
        ctx = 101
    else:
        mut(a)
    with pytest.raises(ValueError, match=what):
        sals.sals_decode_step(*a, ctx=ctx, k=10, w=4, G=2)


def test_decode_rejects_bad_outputs():
    a = _decode_inputs()
    with pytest.raises(ValueError, match="out"):
        sals.sals_decode_step(*a, ctx=50, k=10, w=4, G=2, out=torch.zeros(2, 8, 32))
    with pytest.raises(ValueError, match="out"):
        sals.sals_decode_step(*a, ctx=50, k=10, w=4, G=2, out=torch.zeros(2, 8, 64, dtype=bf))
    with pytest.raises(ValueError, match="sel_out"):
        sals.sals_decode_step(*a, ctx=50, k=10, w=4, G=2, sel_out=torch.zeros(2, 2, 15, dtype=torch.int32))
    with pytest.raises(ValueError, match="sel_out"):
        sals.sals_decode_step(*a, ctx=50, k=10, w=4, G=1, sel_out=torch.zeros(2, 2, 14, dtype=torch.int32))


def test_decode_good_shapes_reach_the_device_check():
    with pytest.raises(ValueError, match="GPU"):
        sals.sals_decode_step(*_decode_inputs(), ctx=50, k=10, w=4, G=2,
                              out=torch.zeros(2, 8, 64), sel_out=torch.zeros(2, 2, 14, dtype=torch.int32))


def test_compact_rejects_bad_shapes():
    K = torch.zeros(2, 4, 100, 64, dtype=bf)
    Q = torch.zeros(2, 8, 8, 64, dtype=bf)
    with pytest.raises(ValueError, match="V"):
        sals.kv_compact(K, torch.zeros(2, 4, 99, 64, dtype=bf), Q, ctx=90, k_keep=10)
    with pytest.raises(ValueError, match="Qobs"):
        sals.kv_compact(K, K, torch.zeros(2, 8, 8, 32, dtype=bf), ctx=90, k_keep=10)
    with pytest.raises(ValueError, match="Kc"):
        sals.kv_compact(K, K, Q, ctx=90, k_keep=10, Kc=torch.zeros(2, 4, 11, 64, dtype=bf))
    with pytest.raises(ValueError, match="kept"):
        sals.kv_compact(K, K, Q, ctx=90, k_keep=10, kept=torch.zeros(2, 4, 10, dtype=torch.int64))
    with pytest.raises(ValueError, match="importance"):
        sals.kv_compact(K, K, Q, ctx=90, k_keep=10, importance=torch.zeros(2, 4, 100))
    with pytest.raises(ValueError, match="ctx"):
        sals.kv_compact(K, K, Q, ctx=101, k_keep=10)


def test_dense_decode_and_reconstruct_reject_bad_shapes():
    q = torch.zeros(2, 8, 64, dtype=bf)
    K = torch.zeros(2, 4, 100, 64, dtype=bf)
    with pytest.raises(ValueError, match="V"):
        sals.sals_dense_decode(q, K, torch.zeros(2, 4, 100, 32, dtype=bf))
    with pytest.raises(ValueError, match="out"):
        sals.sals_dense_decode(q, K, K, out=torch.zeros(2, 8, 65))
    with pytest.raises(ValueError, match="n = "):
        sals.sals_dense_decode(q, K, K, n=101)
    Lk = torch.zeros(2, 100, 64, dtype=bf)
    with pytest.raises(ValueError, match="Pk"):
        sals.sals_reconstruct_kv(Lk, torch.zeros(200, 64, dtype=bf), K, t0=0, T=100, d=64)
    with pytest.raises(ValueError, match="rows"):
        sals.sals_reconstruct_kv(Lk, torch.zeros(256, 64, dtype=bf), K, t0=10, T=100, d=64)


def test_from_importance_and_sparsity_reject_bad_shapes():
    K = torch.zeros(2, 4, 100, 64, dtype=bf)
    with pytest.raises(ValueError, match="importance"):
        sals.kv_compact_from_importance(K, K, torch.zeros(2, 3, 100), k_keep=5)
    with pytest.raises(ValueError, match="Vc"):
        sals.kv_compact_from_importance(K, K, torch.zeros(2, 4, 100), k_keep=5, Vc=torch.zeros(2, 4, 5, 64))
    with pytest.raises(ValueError, match="sparsity"):
        sals.kv_importance_sparsity(K, torch.zeros(2, 8, 8, 64, dtype=bf), ctx=100, p=1e-3,
                                    sparsity=torch.zeros(2, 4))


def test_project_rejects_bad_shapes():
    X = torch.zeros(2, 10, 256, dtype=bf)
    P = torch.zeros(256, 64, dtype=bf)
    with pytest.raises(ValueError, match="Lk"):
        sals.sals_project_kv(X, P, torch.zeros(2, 100, 32, dtype=bf), 0, d=64)
    with pytest.raises(ValueError, match="rows"):
        sals.sals_project_kv(X, P, torch.zeros(2, 100, 64, dtype=bf), 95, d=64)
    with pytest.raises(ValueError, match="Xv"):
        sals.sals_project_kv(X, P, torch.zeros(2, 100, 64, dtype=bf), 0, d=64, Xv=torch.zeros(2, 9, 256, dtype=bf),
                             Pv=P, Lv=torch.zeros(2, 100, 64, dtype=bf))
