"""The stored selection cases (tests/golden/selection_cases.json) against the oracle and against
values worked out by hand from the selection rules (top-k over [0, T - w), ties to the lowest
index, -0.0 equal to +0.0, the window [T - w, T) always kept, positions ascending)."""

import json
import os

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "selection_cases.json")

# worked by hand, independently of any implementation
HAND = {
    "three_way_tie_at_threshold": [1, 3, 8, 9],  # 2.0 at 1, 3, 5: the two lowest; window 8, 9
    "signed_zeros_tie": [0],                     # 0.0 and -0.0 tie: lowest index
    "all_equal": [0, 1, 2, 5, 6],                # all tie: first three; window 5, 6
    "k_covers_all_candidates": [0, 1, 2, 3, 4],  # k >= T - w keeps everything
    "window_covers_context": [0, 1, 2],          # w >= T: no candidates, all in the window
    "negative_scores_with_tie": [1, 3],          # -1.0 at 1 and 3 are the two largest
    "k_zero_window_only": [2, 3],
    "descending_scores": [0, 1, 2, 3, 9, 10, 11],
    "ascending_scores": [5, 6, 7, 8, 9, 10, 11],
    "tie_straddles_threshold": [0, 1, 2, 6, 7],  # 5.0@6, 4.0@0, then 3.0 at 1, 2 of 1..4
}


def load():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


def test_fixture_matches_hand_worked_values():
    cases = load()
    assert {c["name"] for c in cases} == set(HAND)
    for c in cases:
        assert c["sel"] == HAND[c["name"]], c["name"]


def test_fixture_matches_oracle():
    for c in load():
        sel = oracle.select_tokens(np.asarray(c["scores"], dtype=np.float64), c["T"], c["k"], c["w"])
        assert sel.tolist() == c["sel"], c["name"]
        assert len(c["scores"]) == max(0, c["T"] - c["w"])
