"""Seeded synthetic inputs for the level histogram build.

This module only draws random inputs and lays out node row lists; it holds
none of the method's arithmetic (no quantization, histogram, subtraction or
gain).  Both the HIP path and the CPU oracle are fed from it.

Five workloads, each shaped like a case the pages describe:

  c1  tiny root:        4,096 x 8, u8 bins uniform in [0, 255], root only.
  c2  depth-6 level:    1,000,000 x 100, u8; features 0-79 uniform, 80-99
                        skewed (90% of rows in one hot bin); 32 nodes with
                        Dirichlet(1) sizes; build the smaller of each pair.
  c3  tall narrow:      10,000,000 x 28, u8 quantile-binned Gaussian features
                        (exactly uniform over 256 bins); logistic-loss grad/hess
                        from random labels and N(0,1) margins; a whole tree,
                        levels 0..7.
  c4  wide:             131,072 x 16,384, u8 uniform; root, then the 8 nodes
                        of level 3 from a uniform random partition.
  c5  high cardinality: 2,000,000 x 50, u16 over 1,024 bins with 40% of the
                        entries set to the missing sentinel (value 1,024);
                        128 nodes with Dirichlet(1) sizes.

Unless stated otherwise grad ~ N(0, 1) and hess ~ U(0.1, 1) in fp32,
lambda = 1 and gamma = 0.  Every array is drawn from its own stream,
numpy default_rng(SeedSequence(seed).spawn(...)).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

CONFIGS = ("c1", "c2", "c3", "c4", "c5")

FULL_SHAPES = {
    # name: (n_rows, n_features)
    "c1": (4_096, 8),
    "c2": (1_000_000, 100),
    "c3": (10_000_000, 28),
    "c4": (131_072, 16_384),
    "c5": (2_000_000, 50),
}


@dataclass
class Level:
    """One level of sibling pairs: children 2i and 2i+1 share parent i.

    children_*    row lists of all 2P children, node order 0..2P-1.
    built_*       row lists of the children that are built from rows, in pair
                  order (the other child of each pair comes from subtraction).
    parent_*      row lists of the P parents (union of each pair, ascending).
    built_is_right[i] = 1 when child 2i+1 is the built one.
    """
    children_row_index: np.ndarray
    children_offsets: np.ndarray
    built_is_right: np.ndarray
    built_row_index: np.ndarray
    built_offsets: np.ndarray
    parent_row_index: np.ndarray
    parent_offsets: np.ndarray

    @property
    def n_pairs(self) -> int:
        return int(self.built_is_right.shape[0])

    @property
    def built_slots(self) -> np.ndarray:
        """Child slot that each built histogram lands in (2i + built_is_right[i])."""
        return (2 * np.arange(self.n_pairs) + self.built_is_right).astype(np.int32)


@dataclass
class Workload:
    name: str
    bins: np.ndarray            # [F][n] uint8 or uint16, feature-major
    n_bins: int                 # value bins per feature
    has_missing: bool           # sentinel value n_bins marks a missing entry
    grad: np.ndarray            # fp32 [n]
    hess: np.ndarray            # fp32 [n]
    lam: float = 1.0
    gamma: float = 0.0
    kind: str = "root"          # "root", "level", "tree", "root+level"
    level: Optional[Level] = None
    depth: int = 0              # levels 0..depth-1 for kind == "tree"
    notes: dict = field(default_factory=dict)
    margin: Optional[np.ndarray] = None   # fp32 [n] raw scores, where the recipe has them
    label: Optional[np.ndarray] = None    # fp32 [n] labels, where the recipe has them

    @property
    def n_rows(self) -> int:
        return int(self.bins.shape[1])

    @property
    def n_features(self) -> int:
        return int(self.bins.shape[0])

    @property
    def n_slots(self) -> int:
        return self.n_bins + (1 if self.has_missing else 0)


def _streams(seed: int, k: int):
    return [np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(k)]


def _grad_hess_normal_uniform(rng_g, rng_h, n):
    grad = rng_g.standard_normal(n, dtype=np.float32)
    hess = rng_h.uniform(0.1, 1.0, n).astype(np.float32)
    return grad, hess


def smaller_is_right(n_left: np.ndarray, n_right: np.ndarray) -> np.ndarray:
    """Which child of each pair is built from rows: the one with fewer rows,
    the left one on a tie (harness planning rule)."""
    return (n_right < n_left).astype(np.uint8)


def level_from_node_ids(node_id: np.ndarray, n_children: int) -> Level:
    """Row lists of a level from a per-row child id (ascending rows per child)."""
    assert n_children % 2 == 0
    order = np.argsort(node_id, kind="stable").astype(np.int32)
    counts = np.bincount(node_id, minlength=n_children).astype(np.int64)
    offsets = np.zeros(n_children + 1, dtype=np.int64)
    np.cumsum(counts, out=offsets[1:])
    return level_from_lists(order, offsets)


def level_from_lists(children_row_index: np.ndarray, children_offsets: np.ndarray) -> Level:
    """Pair up children (2i, 2i+1); choose the built child; derive parents."""
    off = np.asarray(children_offsets, dtype=np.int64)
    ri = np.asarray(children_row_index, dtype=np.int32)
    n_children = off.shape[0] - 1
    P = n_children // 2
    counts = np.diff(off)
    bir = smaller_is_right(counts[0::2], counts[1::2])
    built_lists, parent_lists = [], []
    for i in range(P):
        left = ri[off[2 * i]: off[2 * i + 1]]
        right = ri[off[2 * i + 1]: off[2 * i + 2]]
        built_lists.append(right if bir[i] else left)
        parent_lists.append(np.sort(np.concatenate([left, right]), kind="stable"))

    def cat(lists):
        o = np.zeros(len(lists) + 1, dtype=np.int64)
        np.cumsum([len(x) for x in lists], out=o[1:])
        r = np.concatenate(lists).astype(np.int32) if lists else np.zeros(0, np.int32)
        return r, o

    b_ri, b_off = cat(built_lists)
    p_ri, p_off = cat(parent_lists)
    return Level(ri, off, bir, b_ri, b_off, p_ri, p_off)


def make(name: str, seed: int = 0, n_rows: Optional[int] = None,
         n_features: Optional[int] = None) -> Workload:
    """Build workload `name` (c1..c5).  n_rows / n_features shrink it for tests."""
    if name not in FULL_SHAPES:
        raise ValueError(f"unknown workload {name!r}; expected one of {CONFIGS}")
    n0, f0 = FULL_SHAPES[name]
    n = int(n_rows or n0)
    F = int(n_features or f0)
    s = _streams(seed, 8)

    if name == "c1":
        bins = s[0].integers(0, 256, size=(F, n), dtype=np.uint8)
        grad, hess = _grad_hess_normal_uniform(s[1], s[2], n)
        return Workload(name, bins, 256, False, grad, hess, kind="root")

    if name == "c2":
        bins = s[0].integers(0, 256, size=(F, n), dtype=np.uint8)
        n_uniform = (F * 80) // 100
        skew = np.arange(n_uniform, F)
        if skew.size:
            hot = s[3].integers(0, 256, size=skew.size, dtype=np.uint8)
            is_hot = s[4].random((skew.size, n)) < 0.9
            sub = bins[skew]
            bins[skew] = np.where(is_hot, hot[:, None], sub)
        grad, hess = _grad_hess_normal_uniform(s[1], s[2], n)
        p = s[5].dirichlet(np.ones(32))
        node_id = s[6].choice(32, size=n, p=p)
        lvl = level_from_node_ids(node_id, 32)
        return Workload(name, bins, 256, False, grad, hess, kind="level", level=lvl,
                        notes={"hot_features": skew.tolist()})

    if name == "c3":
        # floor(256 * Phi(x)) of a Gaussian x is exactly uniform over 0..255.
        bins = s[0].integers(0, 256, size=(F, n), dtype=np.uint8)
        margin = s[1].standard_normal(n)
        label = (s[2].random(n) < 0.5).astype(np.float64)
        prob = 1.0 / (1.0 + np.exp(-margin))
        grad = (prob - label).astype(np.float32)
        hess = (prob * (1.0 - prob)).astype(np.float32)
        return Workload(name, bins, 256, False, grad, hess, kind="tree", depth=8,
                        margin=margin.astype(np.float32), label=label.astype(np.float32))

    if name == "c4":
        bins = s[0].integers(0, 256, size=(F, n), dtype=np.uint8)
        grad, hess = _grad_hess_normal_uniform(s[1], s[2], n)
        node_id = s[3].integers(0, 8, size=n)
        lvl = level_from_node_ids(node_id, 8)
        return Workload(name, bins, 256, False, grad, hess, kind="root+level", level=lvl)

    # c5
    n_bins = 1024
    vals = s[0].integers(0, n_bins, size=(F, n), dtype=np.uint16)
    missing = s[3].random((F, n)) < 0.4
    vals[missing] = n_bins
    grad, hess = _grad_hess_normal_uniform(s[1], s[2], n)
    p = s[5].dirichlet(np.ones(128))
    node_id = s[6].choice(128, size=n, p=p)
    lvl = level_from_node_ids(node_id, 128)
    return Workload(name, vals, n_bins, True, grad, hess, kind="level", level=lvl)


def random_small(seed: int, n_rows: int, n_features: int, n_bins: int,
                 has_missing: bool, n_children: int = 0, wide_grad: bool = False,
                 u16: Optional[bool] = None) -> Workload:
    """Tiny random case for brute-force checks.  n_children = 0 gives a root.

    wide_grad spreads |grad| over 40 binary orders of magnitude so that any
    reordering or truncation of a sum shows in the low bits."""
    s = _streams(seed, 6)
    hi = n_bins + (1 if has_missing else 0)
    use16 = (hi > 256) if u16 is None else u16
    dt = np.uint16 if use16 else np.uint8
    bins = s[0].integers(0, hi, size=(n_features, n_rows)).astype(dt)
    if wide_grad:
        mant = s[1].uniform(1.0, 2.0, n_rows)
        expo = s[2].integers(-40, 1, n_rows)
        sign = np.where(s[3].random(n_rows) < 0.5, -1.0, 1.0)
        grad = (sign * np.ldexp(mant, expo)).astype(np.float32)
    else:
        grad = s[1].standard_normal(n_rows, dtype=np.float32)
    hess = s[4].uniform(0.1, 1.0, n_rows).astype(np.float32)
    if n_children == 0:
        return Workload(f"small{seed}", bins, n_bins, has_missing, grad, hess, kind="root")
    node_id = s[5].integers(0, n_children, size=n_rows)
    lvl = level_from_node_ids(node_id, n_children)
    return Workload(f"small{seed}", bins, n_bins, has_missing, grad, hess,
                    kind="level", level=lvl)


def objective_inputs(seed: int, n: int, kind: str, weighted: bool = False):
    """Scores, labels and (optionally) weights, fp32 [n], for loss `kind`.

    Scores are N(0, 2^2) for 90% of the rows and spread uniformly over a wide
    range for the rest (+-60 for squared and logistic, so that the logistic
    probability saturates; +-20 for Poisson, whose exp must stay finite in
    fp32).  Labels: N(0, 1) for squared, Bernoulli(0.5) in {0, 1} for logistic,
    Poisson counts with rate e^N(0,1) for Poisson.  Weights U(0.5, 2)."""
    if kind not in ("squared", "logistic", "poisson"):
        raise ValueError(f"unknown objective {kind!r}")
    s = _streams(seed, 5)
    wide = 20.0 if kind == "poisson" else 60.0
    margin = s[0].normal(0.0, 2.0, n)
    far = s[1].random(n) < 0.1
    margin[far] = s[2].uniform(-wide, wide, int(far.sum()))
    if kind == "squared":
        label = s[3].standard_normal(n)
    elif kind == "logistic":
        label = (s[3].random(n) < 0.5).astype(np.float64)
    else:
        label = s[3].poisson(np.exp(s[3].standard_normal(n))).astype(np.float64)
    weight = s[4].uniform(0.5, 2.0, n).astype(np.float32) if weighted else None
    return margin.astype(np.float32), label.astype(np.float32), weight
