"""Brute-force checkers for the oracle (test infrastructure, CPU only).

They compute the same quantities as the oracle by a different route: each
histogram cell by a boolean mask over the node's rows (slot-major, not the
oracle's feature -> row walk), and each split candidate's left/right sums
directly from rows (no prefix scan).
"""
from fractions import Fraction

import numpy as np


def hist_by_mask(bins, n_bins, has_missing, qg, qh, rows):
    """[F][S][2] int64 histogram of one node, cell by cell."""
    F = bins.shape[0]
    S = n_bins + (1 if has_missing else 0)
    rows = np.asarray(rows, dtype=np.int64)
    g = qg[rows].astype(np.int64)
    h = qh[rows].astype(np.int64)
    out = np.zeros((F, S, 2), dtype=np.int64)
    for f in range(F):
        col = bins[f, rows].astype(np.int64)
        for s in range(S):
            m = col == s
            out[f, s, 0] = int(g[m].sum())
            out[f, s, 1] = int(h[m].sum())
    return out


def best_split_by_rows(bins, n_bins, has_missing, qg, qh, rows, k_g, k_h, lam, gamma):
    """Every candidate from rows; fp64 gain; strict '>' in (f, b, right-then-left) order.

    Returns (record dict, list of (f, b, d, exact Fraction gain) for every
    valid candidate)."""
    rows = np.asarray(rows, dtype=np.int64)
    g = qg[rows].astype(np.int64)
    h = qh[rows].astype(np.int64)
    G, H = int(g.sum()), int(h.sum())
    sg, sh = 2.0 ** -k_g, 2.0 ** -k_h
    best = dict(feature=-1, bin=-1, default_left=0, gain=float("-inf"), g_left=0, h_left=0,
                g_total=G, h_total=H)
    cands = []
    for f in range(bins.shape[0]):
        col = bins[f, rows].astype(np.int64)
        miss = col == n_bins
        for b in range(n_bins):
            for d in ((0, 1) if has_missing else (0,)):
                left = (col <= b) & ~miss
                if d:
                    left = left | miss
                GL, HL = int(g[left].sum()), int(h[left].sum())
                GR, HR = int(g[~left].sum()), int(h[~left].sum())
                if not (HL > 0 and HR > 0):
                    continue
                gl, hl, gr, hr = float(GL) * sg, float(HL) * sh, float(GR) * sg, float(HR) * sh
                gt, ht = float(G) * sg, float(H) * sh
                gain = gl * gl / (hl + lam) + gr * gr / (hr + lam) - gt * gt / (ht + lam) - gamma
                FL, FHL = Fraction(GL) * Fraction(2) ** -k_g, Fraction(HL) * Fraction(2) ** -k_h
                FR, FHR = Fraction(GR) * Fraction(2) ** -k_g, Fraction(HR) * Fraction(2) ** -k_h
                FG, FH = Fraction(G) * Fraction(2) ** -k_g, Fraction(H) * Fraction(2) ** -k_h
                FLAM, FGAM = Fraction(lam), Fraction(gamma)
                exact = FL * FL / (FHL + FLAM) + FR * FR / (FHR + FLAM) - FG * FG / (FH + FLAM) - FGAM
                cands.append((f, b, d, exact))
                if gain > best["gain"]:
                    best.update(feature=f, bin=b, default_left=d, gain=gain, g_left=GL, h_left=HL)
    return best, cands
