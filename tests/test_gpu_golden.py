"""The stored selection cases on the GPU, through the C ABI: latent inputs are built so that the
device's scores are exactly the stored candidate scores (P_k = identity, query = e_0, so
S[t] = L_k[t, 0]); the selected set must equal the stored one and the output the oracle's."""

import json
import os

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - the GPU tests run on an MI355X
    pytest.skip("no GPU", allow_module_level=True)

import kv_cache_compression_sals_amd as sals  # noqa: E402
import oracle  # noqa: E402

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "selection_cases.json")
with open(GOLDEN) as f:
    CASES = json.load(f)["cases"]


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_golden_selection_on_device(case):
    d = r = 64
    T, w, k = case["T"], case["w"], case["k"]
    rs = np.random.default_rng(7)
    Lk = (0.1 * rs.standard_normal((1, T, r))).astype(np.float32)
    Lv = rs.standard_normal((1, T, r)).astype(np.float32)
    Lk[0, : len(case["scores"]), 0] = np.asarray(case["scores"], dtype=np.float32)
    P = np.eye(d, r, dtype=np.float32)
    q = np.zeros((1, 1, d), dtype=np.float32)
    q[0, 0, 0] = 1.0
    print(f"golden {case['name']} T={T} w={w} k={k}", flush=True)
    dev = {n: torch.from_numpy(a).cuda() for n, a in dict(q=q, Lk=Lk, Lv=Lv, P=P).items()}
    out, sel = sals.sals_decode_step(dev["q"], dev["Lk"], dev["Lv"], dev["P"], dev["P"], ctx=T, k=k, w=w,
                                     G=1, rope_base=10000.0, want_sel=True)
    torch.cuda.synchronize()
    assert sel.cpu().numpy()[0, 0].tolist() == case["sel"]
    ora = oracle.decode_step(q, Lk, Lv, P, P, ctx=T, k=k, w=w, G=1, H_kv=1, base=10000.0, dtype="f32")
    assert ora["sel"][0, 0].tolist() == case["sel"]
    err = np.abs(out.cpu().numpy().astype(np.float64) - ora["out"]).max()
    assert err <= 1e-4, err
