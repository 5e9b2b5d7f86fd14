"""The no-allocation decode entry point (sals_decode_step_noalloc, through the C ABI) gives the
same bits as sals_decode_step with a caller workspace, on two calls in a row, the second with a
smaller input, so the library's scratch array is reused with stale contents from the first."""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - the GPU tests run on an MI355X
    pytest.skip("no GPU", allow_module_level=True)

import kv_cache_compression_sals_amd as sals  # noqa: E402
from parity import decode_parity, to_device  # noqa: E402
from workloads import CONFIGS, decode_case  # noqa: E402

C2, C3 = CONFIGS["c2"], CONFIGS["c3"]

CASES = [
    # a shared selection for all KV heads (key tile kernel + value kernels), then a smaller
    # per-KV-head selection (attention kernel + split merge)
    ("shared_then_grouped", (C2.with_(calib_tokens=1024), 2, 3000), (C3.with_(calib_tokens=512), 1, 1000)),
    # the same path twice, the second call smaller
    ("grouped_twice", (C3.with_(calib_tokens=512), 2, 4000), (C3.with_(calib_tokens=512), 1, 700)),
]


def _inputs(cfg, B, ctx):
    case = decode_case(cfg, B=B, ctx=ctx, ctx_cap=ctx + 8)
    dt = case["dtype"]
    return case, {n: to_device(case[n], dt) for n in ("q", "Lk", "Lv", "Pk", "Pv")}


@pytest.mark.parametrize("name,first,second", CASES, ids=[c[0] for c in CASES])
def test_noalloc_matches_workspace_entry_point(name, first, second):
    for cfg, B, ctx in (first, second):
        print(f"noalloc {name}: B={B} ctx={ctx} H_q={cfg.H_q} H_kv={cfg.H_kv} G={cfg.G} r={cfg.r}", flush=True)
        case, t = _inputs(cfg, B, ctx)
        kw = dict(ctx=ctx, k=cfg.k, w=cfg.w, G=cfg.G, rope_base=cfg.base)
        ref, ref_sel = sals.sals_decode_step(t["q"], t["Lk"], t["Lv"], t["Pk"], t["Pv"], want_sel=True, **kw)
        out = torch.full_like(ref, float("nan"))
        sel = torch.full_like(ref_sel, -1)
        sals.sals_decode_step_noalloc(t["q"], t["Lk"], t["Lv"], t["Pk"], t["Pv"], out=out, sel_out=sel, **kw)
        torch.cuda.synchronize()
        assert torch.equal(out, ref) and torch.equal(sel, ref_sel)
        # and the result is right, not only equal
        stats = decode_parity(case, out.cpu().numpy().astype(np.float64), sel.cpu().numpy())
        print("   ", stats, flush=True)

