"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check that some pin fails.

Each mutant rewrites one snippet of an oracle source file, loads the result as a fresh module
and swaps its functions into ``oracle.sals`` / ``oracle.compact`` for the duration of one test.
A pin "catches" a mutant when it raises (an AssertionError, or any error the mistake causes).
"""

import os
import types

import pytest

import oracle.compact as OC
import oracle.outlier as OO
import oracle.quant as OQ
import oracle.sals as OS
from pins import PINS

ORACLE_DIR = os.path.dirname(OS.__file__)

MUTANTS = [
    # (file, original snippet, mutated snippet, what the mistake is)
    ("compact.py", "    while n < len(v) and run < target:", "    while n < len(v) and run <= target:",
     "mass budget takes one token past the target"),
    ("compact.py", "v = np.sort(np.asarray(imp_row, dtype=np.float64))[::-1]", "v = np.asarray(imp_row, dtype=np.float64)",
     "mass budget in position order instead of by size"),
    ("compact.py", "return layer_budgets(e / top if top > 0 else np.zeros_like(e), total, ctx)",
     "return layer_budgets(1.0 - e / top if top > 0 else np.zeros_like(e), total, ctx)", "budget falls with energy"),
    ("sals.py", "c = int(np.count_nonzero(S >= tau))", "c = int(np.count_nonzero(S > tau))",
     "a score equal to the threshold fails it"),
    ("sals.py", "top = topk_lowest_index(S, min(k, c))", "top = topk_lowest_index(S, c)", "threshold set not capped at k"),
    ("sals.py", "S = np.asarray(S_row[:T_c], dtype=np.float64)\n    c = int(np.count_nonzero(S >= tau))",
     "S = np.asarray(S_row[:T_c], dtype=np.float64)\n    c = int(np.count_nonzero(np.asarray(S_row[:T]) >= tau))",
     "threshold count includes the window"),
    ("quant.py", "codes = np.floor((u + np.float32(0.5)).astype(np.float32)).astype(np.int64)",
     "codes = np.floor(u).astype(np.int64)", "codes truncated instead of rounded"),
    ("quant.py", "levels = np.float32((1 << bits) - 1)", "levels = np.float32(1 << bits)", "2^bits levels"),
    ("quant.py", "return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)",
     "return (c[:, 1::2] | (c[:, 0::2] << 4)).astype(np.uint8)", "nibbles swapped"),
    ("quant.py", "hi = topk_lowest_index(np.asarray(imp_row[:ctx], dtype=np.float64), n_hi)",
     "hi = topk_lowest_index(-np.asarray(imp_row[:ctx], dtype=np.float64), n_hi)", "least important tokens at 8 bits"),
    ("quant.py", "return zero + codes * scale", "return codes * scale", "dequantization drops the zero point"),
    ("quant.py", "HI_BITS, LO_BITS = 8, 4", "HI_BITS, LO_BITS = 4, 8", "bit widths swapped"),
    ("quant.py", "scale = np.float32(span / levels)", "scale = np.float32(span / (levels + 1))", "step off by one level"),
    ("quant.py", "out[:, 1::2] = b >> 4", "out[:, 1::2] = b & 0xF", "high nibble lost"),
    ("outlier.py", "a = np.where(f == 0, np.sqrt(1.0 / T), np.sqrt(2.0 / T))",
     "a = np.sqrt(2.0 / T) + 0.0 * f", "DCT DC column not normalised"),
    ("outlier.py", "np.cos(np.pi * (2.0 * t + 1.0) * f / (2.0 * T))", "np.cos(np.pi * (2.0 * t) * f / (2.0 * T))",
     "DCT phase: 2t instead of 2t + 1"),
    ("outlier.py", "C = dct_basis(X.shape[0], n_freq)", "C = dct_basis(X.shape[0], n_freq + 1)",
     "low-pass keeps one frequency too many"),
    ("outlier.py", "return (R * R).sum(axis=1)", "return np.abs(R).sum(axis=1)", "deviation measured as an L1 norm"),
    ("outlier.py", "+ deviation_energy(stored_to_f64(V[b, g, :ctx], dtype), n_freq))",
     "+ 0.0 * deviation_energy(stored_to_f64(V[b, g, :ctx], dtype), n_freq))", "value deviation dropped"),
    ("outlier.py", "kept[b, g] = topk_lowest_index(I[b, g], k_keep)", "kept[b, g] = topk_lowest_index(-I[b, g], k_keep)",
     "keeps the least deviating pairs"),
    ("sals.py", "return (np.asarray(a, dtype=np.uint16).astype(np.uint32) << 16)",
     "return ((np.asarray(a, dtype=np.uint16) << 16).astype(np.uint32))", "bf16 bits shifted before widening"),
    ("sals.py", "return (np.asarray(a, dtype=np.uint16).astype(np.uint32) << 16)",
     "return (np.asarray(a, dtype=np.uint16).astype(np.uint32) << 15)", "bf16 bits shifted by 15"),
    ("sals.py", "return (np.asarray(a, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)",
     "return np.asarray(a, dtype=np.uint16).view(np.float16).astype(np.float64)", "bf16 bits read as IEEE half"),
    ("sals.py", "return np.asarray(a, dtype=np.float32).astype(np.float64)",
     "return np.asarray(a, dtype=np.float16).astype(np.float64)", "fp32 decoded through half precision"),
    ("sals.py", "return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=1)",
     "return np.concatenate([x1 * c + x2 * s, x2 * c - x1 * s], axis=1)", "RoPE rotates the wrong way"),
    ("sals.py", "** (-(2.0 * i) / d)", "** (-(1.0 * i) / d)", "RoPE frequency exponent"),
    ("sals.py", "x1, x2 = x[:, :half], x[:, half:]", "x1, x2 = x[:, 0::2], x[:, 1::2]",
     "RoPE pairs interleaved instead of halves"),
    ("sals.py", "return (h * H_kv) // H_q", "return h % H_kv", "query-head to KV-head map"),
    ("sals.py", "return (g * G) // H_kv", "return g % G", "KV-head to group map"),
    ("sals.py", "qt[s] += q[h] @ Pk[g * d:(g + 1) * d, :]",
     "qt[s] += q[h] @ Pk[((g + 1) % H_kv) * d:((g + 1) % H_kv + 1) * d, :]", "latent query uses another head's P"),
    ("sals.py", "order = np.lexsort((np.arange(n), -np.asarray(", "order = np.lexsort((-np.arange(n), -np.asarray(",
     "ties go to the highest index"),
    ("sals.py", "top = topk_lowest_index(S_row[:T_c], min(k, T_c))",
     "top = topk_lowest_index(S_row[:T_c], min(k + 1, T_c))", "one token too many"),
    ("sals.py", "top = topk_lowest_index(S_row[:T_c], min(k, T_c))",
     "top = topk_lowest_index(S_row[:T], min(k, T))[:min(k, T_c)]", "top-k also ranks window positions"),
    ("sals.py", "pi = _softmax(Kh @ qh / np.sqrt(d))", "pi = _softmax(Kh @ qh)", "attention scale dropped"),
    ("sals.py", "qh = rope(q[h][None, :], T - 1, base)[0]", "qh = rope(q[h][None, :], T, base)[0]",
     "query rotated at T instead of T-1"),
    ("sals.py", "Kh = rope(reconstruct(Lk[idx], Pk[g * d:(g + 1) * d]), idx, base)",
     "Kh = rope(reconstruct(Lk[idx], Pk[g * d:(g + 1) * d]), np.arange(len(idx)), base)",
     "keys rotated at their slot, not their position"),
    ("sals.py", "Kh = rope(reconstruct(Lk[idx], Pk[g * d:(g + 1) * d]), idx, base)",
     "Kh = reconstruct(Lk[idx], Pk[g * d:(g + 1) * d])", "keys not rotated"),
    ("sals.py", "Vh = reconstruct(Lv[idx], Pv[g * d:(g + 1) * d])",
     "Vh = reconstruct(Lv[idx], Pk[g * d:(g + 1) * d])", "values rebuilt with P_k"),
    ("sals.py", "return np.asarray(X, dtype=np.float64) @ np.asarray(P, dtype=np.float64)",
     "return np.asarray(X, dtype=np.float64) @ np.asarray(P, dtype=np.float64).T", "projection transposed"),
    ("sals.py", "    e = np.exp(logits - m)\n    return e / e.sum()", "    e = np.exp(logits - m)\n    return e",
     "softmax not normalised"),
    ("sals.py", "pos = np.arange(t0, t0 + T)", "pos = np.arange(T)", "rebuilt keys rotated relative to t0"),
    ("sals.py", "out[g] = rope(rows, pos, base) if base is not None else rows",
     "out[g] = rope(rows, pos, base if base is not None else 10000.0)", "rebuilt values rotated"),
    ("sals.py", "qh = rope(qf[b, h][None, :], ctx - 1, base)[0]", "qh = qf[b, h]", "baseline query not rotated"),
    ("sals.py", "V = reconstruct_cache(stored_to_f64(Lv[b, :ctx], dtype), Pvf, 0, ctx, H_kv, None)",
     "V = reconstruct_cache(stored_to_f64(Lv[b, :ctx], dtype), Pkf, 0, ctx, H_kv, None)", "baseline values from P_k"),
    ("compact.py", "topk_lowest_index(np.asarray(importance[b, g], dtype=np.float64), k_keep)",
     "topk_lowest_index(-np.asarray(importance[b, g], dtype=np.float64), k_keep)",
     "given importance ranked upside down"),
    ("compact.py", "Kc[b, g], Vc[b, g] = K[b, g, kept[b, g]], V[b, g, kept[b, g]]",
     "Kc[b, g], Vc[b, g] = K[b, g, kept[b, g]], K[b, g, kept[b, g]]", "given-importance values gathered from K"),
    ("compact.py", "below += int(np.count_nonzero(a < p))", "below += int(np.count_nonzero(a <= p))",
     "sparsity counts entries equal to p"),
    ("compact.py", "total += pi + 1", "total += pi", "sparsity total misses the diagonal"),
    ("compact.py", "a = _softmax(K[: pi + 1] @ Qobs[i] / np.sqrt(d))", "a = _softmax(K[:T] @ Qobs[i] / np.sqrt(d))",
     "sparsity ignores the causal mask"),
    ("compact.py", "share = total * nu[l] / Z if Z > 0 else total / L", "share = total * nu[l] / L if Z > 0 else total / L",
     "budgets not normalised by Z"),
    ("compact.py", "a = _softmax(K[: p + 1] @ Qobs[i] / np.sqrt(d))\n        I[: p + 1] += a",
     "a = _softmax(K[:T] @ Qobs[i] / np.sqrt(d))\n        I[:T] += a", "causal mask dropped"),
    ("compact.py", "p = T - w + i", "p = T - w + i + 1 if i < w - 1 else T - 1", "observation positions shifted"),
    ("compact.py", "a = _softmax(K[: p + 1] @ Qobs[i] / np.sqrt(d))", "a = _softmax(K[: p + 1] @ Qobs[i])",
     "importance scale dropped"),
    ("compact.py", "out[b, h] = _softmax(Kf @ qf[b, h] / np.sqrt(d)) @ Vf", "out[b, h] = _softmax(Kf @ qf[b, h]) @ Vf",
     "dense decode scale dropped"),
    ("compact.py", "if kv_head_of(h, H_q, H_kv) == g:", "if h == g:", "importance ignores grouped heads"),
    ("compact.py", "Vc[b, g] = V[b, g, kept[b, g]]", "Vc[b, g] = K[b, g, kept[b, g]]", "values gathered from K"),
    ("compact.py", "    e = np.exp(logits - m)\n    return e / e.sum()", "    e = np.exp(logits - m)\n    return e / e.max()",
     "importance softmax normalised by the max"),
]


def _load(fname, old, new):
    path = os.path.join(ORACLE_DIR, fname)
    src = open(path).read()
    assert src.count(old) == 1, (fname, old)
    src = src.replace(old, new).replace("from .sals import", "from oracle.sals import")
    mod = types.ModuleType("oracle_mutant_" + fname[:-3])
    exec(compile(src, path + " (mutant)", "exec"), mod.__dict__)
    return mod


def _patch(monkeypatch, mod, target):
    for name, obj in vars(mod).items():
        if isinstance(obj, types.FunctionType) and obj.__module__ == mod.__name__ and hasattr(target, name):
            monkeypatch.setattr(target, name, obj)
            if target is OS and hasattr(OC, name):
                monkeypatch.setattr(OC, name, obj)


@pytest.mark.parametrize("mutant", MUTANTS, ids=[m[3] for m in MUTANTS])
def test_some_pin_catches(mutant, monkeypatch):
    fname, old, new, what = mutant
    mod = _load(fname, old, new)
    _patch(monkeypatch, mod, {"sals.py": OS, "compact.py": OC, "outlier.py": OO, "quant.py": OQ}[fname])
    caught = []
    for pin in PINS:
        try:
            pin()
        except Exception:  # noqa: BLE001 - any failure of a pin counts as catching the mutant
            caught.append(pin.__name__)
    assert caught, f"no pin catches: {what}"


def test_unmutated_copy_passes(monkeypatch):
    """Loading the sources through the same path without a change passes every pin."""
    for fname, target in (("sals.py", OS), ("compact.py", OC), ("outlier.py", OO), ("quant.py", OQ)):
        _patch(monkeypatch, _load(fname, "import numpy as np", "import numpy as np"), target)
    for pin in PINS:
        pin()
