"""Writes selection_cases.json: selection worked examples whose expected sets come from the
oracle only (run: python tests/golden/make_fixtures.py from the repository root).

The pages print no worked example, so the inputs here are small hand-built score rows that
exercise each rule of the selection step: the top-k over the non-window positions plus the
always-kept recent window ("SALS: Sparse Attention in Latent Space for KV cache Compression",
方法详解 -> 关键设计 items 2 and 4: sparsity set by the number of selected tokens, top-k
selection; the index set S_{psi,k} of the VL-Cache author responses, reviewer XVzL weakness 2),
with ties going to the lowest index and -0.0 equal to +0.0 (the readings this build fixes where
the pages are silent). Expected sets are whatever oracle.select_tokens returns; the hand-worked
values of the first cases are checked against it separately (tests/test_golden.py).
"""

import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import numpy as np  # noqa: E402

import oracle  # noqa: E402

CASES = [
    # name, candidate scores (positions [0, T - w)), T, w, k
    ("three_way_tie_at_threshold", [0.5, 2.0, -1.0, 2.0, 0.3, 2.0, 1.5, 0.0], 10, 2, 2),
    ("signed_zeros_tie", [0.0, -0.0], 2, 0, 1),
    ("all_equal", [1.0, 1.0, 1.0, 1.0, 1.0], 7, 2, 3),
    ("k_covers_all_candidates", [3.0, 1.0, 2.0], 5, 2, 5),
    ("window_covers_context", [], 3, 5, 2),
    ("negative_scores_with_tie", [-3.0, -1.0, -2.0, -1.0], 4, 0, 2),
    ("k_zero_window_only", [5.0, 4.0], 4, 2, 0),
    ("descending_scores", [9.0, 8.0, 7.0, 6.0, 5.0, 4.0, 3.0, 2.0, 1.0], 12, 3, 4),
    ("ascending_scores", [1.0, 2.0, 3.0, 4.0, 5.0, 6.0, 7.0, 8.0, 9.0], 12, 3, 4),
    ("tie_straddles_threshold", [4.0, 3.0, 3.0, 3.0, 3.0, 1.0, 5.0], 8, 1, 4),
]


def main():
    out = []
    for name, scores, T, w, k in CASES:
        sel = oracle.select_tokens(np.asarray(scores, dtype=np.float64), T, k, w)
        out.append(dict(name=name, scores=scores, T=T, w=w, k=k, sel=[int(x) for x in sel]))
    doc = dict(
        source="oracle.select_tokens (see make_fixtures.py for the rules and their citations)",
        cases=out,
    )
    with open(os.path.join(HERE, "selection_cases.json"), "w") as f:
        json.dump(doc, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()
