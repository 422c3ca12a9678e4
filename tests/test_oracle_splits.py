"""Pins of the oracle's split scan (CPU only).

- the hand-worked toys A-F in tests/golden/toys.json (exact rational gains);
- brute force: every candidate's sums recomputed from rows, no prefix scan,
  and the chosen gain checked against exact rational arithmetic;
- the tie-break order (feature, bin, right-before-left).
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from histogram_gradient_boosted_amd import synth

from bruteforce import best_split_by_rows

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "toys.json")
TOYS = json.load(open(GOLDEN))["toys"]


def _run_toy(t):
    bins = np.array(t["bins"], dtype=np.uint8)
    g = np.array(t["grad"], dtype=np.float32)
    h = np.array(t["hess"], dtype=np.float32)
    qg, kg = oracle.quantize(g, False)
    qh, kh = oracle.quantize(h, True)
    hist = oracle.build_hist(bins, t["n_bins"], t["has_missing"], qg, qh)
    sp = oracle.find_splits(hist, t["n_bins"], t["has_missing"], kg, kh, t["lambda"], t["gamma"])
    return sp[0], kg, kh


@pytest.mark.parametrize("t", TOYS, ids=[t["name"] for t in TOYS])
def test_toy(t):
    rec, kg, kh = _run_toy(t)
    e = t["expect"]
    assert int(rec["feature"]) == e["feature"]
    assert int(rec["bin"]) == e["bin"]
    assert int(rec["default_left"]) == e["default_left"]
    if e["gain"] == "-inf":
        assert math.isinf(rec["gain"]) and rec["gain"] < 0
    else:
        exact = Fraction(e["gain"])
        assert abs(Fraction(float(rec["gain"])) - exact) <= abs(exact) * Fraction(1, 10 ** 15)
    for key, k in (("g_left", kg), ("h_left", kh), ("g_total", kg), ("h_total", kh)):
        assert math.ldexp(int(rec[key]), -k) == float(e[key])


def test_toy_e_other_candidates_tie():
    """b0/right and b1/right tie exactly at 1/12 (checked by brute force)."""
    t = next(x for x in TOYS if x["name"] == "E")
    bins = np.array(t["bins"], dtype=np.uint8)
    qg, kg = oracle.quantize(np.array(t["grad"], np.float32), False)
    qh, kh = oracle.quantize(np.array(t["hess"], np.float32), True)
    _, cands = best_split_by_rows(bins, 2, True, qg, qh, np.arange(3), kg, kh, 1.0, 0.0)
    got = {(b, d): v for (_, b, d, v) in cands}
    for oc in t["other_candidates"]:
        assert got[(oc["bin"], oc["default_left"])] == Fraction(oc["gain"])
    assert got[(0, 1)] == Fraction(43, 12)
    assert (1, 1) not in got


CASES = [(s, n, F, B, m) for s, (n, F, B, m) in enumerate([
    (12, 1, 2, False), (40, 3, 8, False), (40, 3, 8, True), (64, 2, 5, True),
    (7, 3, 3, True), (64, 3, 8, False), (30, 2, 6, True), (64, 1, 8, True),
])]


@pytest.mark.parametrize("seed,n,F,B,missing", CASES)
@pytest.mark.parametrize("lam,gamma", [(1.0, 0.0), (0.5, 0.25), (3.0, 0.0)])
def test_brute_force_split(seed, n, F, B, missing, lam, gamma):
    w = synth.random_small(seed, n, F, B, missing, 0)
    qg, kg = oracle.quantize(w.grad, False)
    qh, kh = oracle.quantize(w.hess, True)
    hist = oracle.build_hist(w.bins, B, missing, qg, qh)
    rec = oracle.find_splits(hist, B, missing, kg, kh, lam, gamma)[0]
    ref, cands = best_split_by_rows(w.bins, B, missing, qg, qh, np.arange(n), kg, kh, lam, gamma)
    for key in ("feature", "bin", "default_left", "g_left", "h_left", "g_total", "h_total"):
        assert int(rec[key]) == int(ref[key]), key
    assert rec["gain"] == ref["gain"] or (math.isinf(rec["gain"]) and math.isinf(ref["gain"]))
    if cands:
        best_exact = max(c[3] for c in cands)
        assert abs(Fraction(float(rec["gain"])) - best_exact) <= abs(best_exact) * Fraction(1, 10 ** 12) + Fraction(1, 10 ** 300)


def test_brute_force_split_on_level_nodes():
    w = synth.random_small(21, 64, 3, 6, True, 6)
    qg, kg = oracle.quantize(w.grad, False)
    qh, kh = oracle.quantize(w.hess, True)
    L = w.level
    hist = oracle.build_hist(w.bins, 6, True, qg, qh, L.children_row_index, L.children_offsets)
    recs = oracle.find_splits(hist, 6, True, kg, kh, 1.0, 0.0)
    for c in range(6):
        rows = L.children_row_index[L.children_offsets[c]: L.children_offsets[c + 1]]
        ref, _ = best_split_by_rows(w.bins, 6, True, qg, qh, rows, kg, kh, 1.0, 0.0)
        for key in ("feature", "bin", "default_left", "g_left", "h_left", "g_total", "h_total"):
            assert int(recs[c][key]) == int(ref[key])
        assert recs[c]["gain"] == ref["gain"] or math.isinf(ref["gain"])


def test_no_missing_rows_reports_right():
    """With a missing slot but no missing rows, L ties R exactly and R is kept."""
    bins = np.array([[0, 0, 1, 1]], dtype=np.uint8)
    qg, kg = oracle.quantize(np.array([1, 1, -1, -1], np.float32), False)
    qh, kh = oracle.quantize(np.ones(4, np.float32), True)
    hist = oracle.build_hist(bins, 2, True, qg, qh)
    rec = oracle.find_splits(hist, 2, True, kg, kh)[0]
    assert (int(rec["feature"]), int(rec["bin"]), int(rec["default_left"])) == (0, 0, 0)


def test_empty_node_no_split():
    hist = np.zeros((2, 3, 9, 2), dtype=np.int64)
    recs = oracle.find_splits(hist, 8, True, 29, 29)
    assert (recs["feature"] == -1).all() and np.isneginf(recs["gain"]).all()


def test_feature_permutation_moves_winner():
    w = synth.random_small(33, 64, 4, 8, False, 0)
    qg, kg = oracle.quantize(w.grad, False)
    qh, kh = oracle.quantize(w.hess, True)
    a = oracle.find_splits(oracle.build_hist(w.bins, 8, False, qg, qh), 8, False, kg, kh)[0]
    perm = np.array([2, 3, 0, 1])
    b = oracle.find_splits(oracle.build_hist(np.ascontiguousarray(w.bins[perm]), 8, False, qg, qh),
                           8, False, kg, kh)[0]
    assert perm[int(b["feature"])] == int(a["feature"])
    assert int(a["bin"]) == int(b["bin"]) and a["gain"] == b["gain"]
