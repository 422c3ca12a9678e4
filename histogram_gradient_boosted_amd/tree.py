"""Level driver over the C ABI: one level, or a whole depthwise tree.

Per level the device does build_level (the built siblings), subtract_siblings
(the other siblings) and find_splits, all enqueued on the context's stream.
Between levels the host partitions rows by the found splits (a stable
left/right split of each node's row list); that step is plain host logic over
the caller's copy of the bins and is not part of the device path.

A tree is first grown once with the host partition (`plan_tree`), which fixes
every level's row lists; `replay_tree` then enqueues the whole device path of
that tree with every input already resident, which is what a timing loop
repeats.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

from .binding import SPLIT_BYTES, Context, splits_to_numpy


@dataclass
class LevelPlan:
    """Device-resident description of one level.

    depth 0 is the root (row_index None).  For depth >= 1 the level has
    2 * n_pairs child nodes; pair i's parent is node parent_slot[i] of the
    previous level, its built child is node 2i + built_is_right[i]."""
    depth: int
    n_nodes: int
    row_index: Optional[object] = None         # CUDA int32, built children's rows
    offsets: Optional[np.ndarray] = None       # int32 [n_built + 1]
    out_slot: Optional[np.ndarray] = None      # int32 [n_built]
    built_is_right: Optional[np.ndarray] = None
    parent_slot: Optional[np.ndarray] = None
    hist: Optional[object] = None              # CUDA int64 [n_nodes][F][S][2]
    splits: Optional[object] = None            # CUDA uint8 [n_nodes * 56]
    built_rows: int = 0                        # rows in built nodes (the cells are rows x F)
    children_rows: Optional[np.ndarray] = None  # host: every child's row list, concatenated
    children_offsets: Optional[np.ndarray] = None

    @property
    def n_pairs(self) -> int:
        return 0 if self.built_is_right is None else int(self.built_is_right.shape[0])


@dataclass
class Objective:
    """Scores and labels (CUDA fp32 tensors, optional weights) from which
    begin_tree_objective derives each row's (g, h) on the device.  Wherever a
    driver below takes `grad, hess`, an Objective may stand for grad (hess is
    then None)."""
    kind: str
    margin: object
    label: object
    weight: Optional[object] = None


def begin(ctx: Context, grad, hess=None):
    """Start a tree from (grad, hess) tensors or from an Objective."""
    if isinstance(grad, Objective):
        ctx.begin_tree_objective(grad.kind, grad.margin, grad.label, grad.weight)
    else:
        ctx.begin_tree(grad, hess)


def _choose_built(counts: np.ndarray) -> np.ndarray:
    """Build the child with fewer rows; the left one on a tie."""
    return (counts[1::2] < counts[0::2]).astype(np.uint8)


def partition_host(bins: np.ndarray, n_bins: int, rows: Optional[np.ndarray],
                   offsets: Optional[np.ndarray], splits: np.ndarray):
    """Stable left/right split of each node's rows by its split record.

    Returns (children_rows, children_offsets, parent_slot): the children of the
    j-th node with a valid split are 2j (left) and 2j+1 (right)."""
    n = bins.shape[1]
    if rows is None:
        rows = np.arange(n, dtype=np.int32)
        offsets = np.array([0, n], dtype=np.int64)
    lists, parent_slot = [], []
    for node in range(len(offsets) - 1):
        sp = splits[node]
        if int(sp["feature"]) < 0:
            continue
        r = rows[offsets[node]:offsets[node + 1]]
        v = bins[int(sp["feature"]), r]
        left = np.where(v == n_bins, bool(sp["default_left"]), v <= int(sp["bin"]))
        lists.append(r[left])
        lists.append(r[~left])
        parent_slot.append(node)
    offs = np.zeros(len(lists) + 1, dtype=np.int64)
    np.cumsum([len(x) for x in lists], out=offs[1:])
    cat = np.concatenate(lists).astype(np.int32) if lists else np.zeros(0, np.int32)
    return cat, offs, np.array(parent_slot, dtype=np.int32)


def level_plan_from_children(ctx: Context, depth: int, children_rows: np.ndarray,
                             children_offsets: np.ndarray, parent_slot: np.ndarray) -> LevelPlan:
    """Allocate and upload one non-root level from its children's row lists."""
    import torch
    dev = torch.device("cuda", ctx.device)
    counts = np.diff(children_offsets)
    bir = _choose_built(counts)
    P = bir.shape[0]
    built_lists = []
    for i in range(P):
        c = 2 * i + int(bir[i])
        built_lists.append(children_rows[children_offsets[c]:children_offsets[c + 1]])
    boffs = np.zeros(P + 1, dtype=np.int64)
    np.cumsum([len(x) for x in built_lists], out=boffs[1:])
    brows = np.concatenate(built_lists).astype(np.int32) if built_lists else np.zeros(0, np.int32)
    n_nodes = 2 * P
    return LevelPlan(
        depth=depth, n_nodes=n_nodes,
        row_index=torch.from_numpy(brows).to(dev) if brows.size else torch.zeros(1, dtype=torch.int32, device=dev),
        offsets=boffs.astype(np.int32),
        out_slot=(2 * np.arange(P) + bir).astype(np.int32),
        built_is_right=bir, parent_slot=np.asarray(parent_slot, dtype=np.int32),
        hist=torch.empty((max(n_nodes, 1), ctx.n_features, ctx.n_slots, 2), dtype=torch.int64, device=dev),
        splits=torch.empty(max(n_nodes, 1) * SPLIT_BYTES, dtype=torch.uint8, device=dev),
        built_rows=int(boffs[-1]),
        children_rows=children_rows, children_offsets=children_offsets)


def root_plan(ctx: Context) -> LevelPlan:
    import torch
    dev = torch.device("cuda", ctx.device)
    return LevelPlan(
        depth=0, n_nodes=1,
        hist=torch.empty((1, ctx.n_features, ctx.n_slots, 2), dtype=torch.int64, device=dev),
        splits=torch.empty(SPLIT_BYTES, dtype=torch.uint8, device=dev),
        built_rows=ctx.n_rows)


def run_root(ctx: Context, plan: LevelPlan, lam: float, gamma: float):
    ctx.build_level(plan.hist)
    ctx.find_splits(plan.hist, 1, lam, gamma, plan.splits)


def run_level(ctx: Context, plan: LevelPlan, parent_hist, lam: float, gamma: float):
    """Build the smaller siblings, then subtract for the others and find every
    split in one pass."""
    if plan.n_nodes == 0:
        return
    ctx.build_level(plan.hist, plan.row_index, plan.offsets, plan.out_slot)
    ctx.subtract_find_splits(parent_hist, plan.hist, plan.built_is_right, lam, gamma, plan.splits,
                             plan.parent_slot)


def plan_tree(ctx: Context, bins_host: np.ndarray, n_bins: int, grad, hess, depth: int,
              lam: float, gamma: float) -> List[LevelPlan]:
    """Grow levels 0..depth-1 on the device, partitioning rows on the host."""
    begin(ctx, grad, hess)
    plans = [root_plan(ctx)]
    run_root(ctx, plans[0], lam, gamma)
    rows, offs = None, None
    for d in range(1, depth):
        prev = plans[-1]
        sp = splits_to_numpy(prev.splits)[: prev.n_nodes]
        rows, offs, parent_slot = partition_host(bins_host, n_bins, rows, offs, sp)
        plan = level_plan_from_children(ctx, d, rows, offs, parent_slot)
        run_level(ctx, plan, prev.hist, lam, gamma)
        plans.append(plan)
        if plan.n_nodes == 0:
            break
    ctx.sync()
    return plans


def replay_tree(ctx: Context, plans: List[LevelPlan], grad, hess, lam: float, gamma: float):
    """Enqueue the device path of a planned tree (begin_tree + every level)."""
    begin(ctx, grad, hess)
    run_root(ctx, plans[0], lam, gamma)
    for prev, plan in zip(plans[:-1], plans[1:]):
        run_level(ctx, plan, prev.hist, lam, gamma)


@dataclass
class DeviceLevel:
    """One level grown entirely on the device (grow_tree_device)."""
    depth: int
    n_nodes: int
    rows: Optional[object]                 # CUDA int32: the nodes' rows (None: the root)
    offsets: Optional[np.ndarray]          # host int32 [n_nodes + 1] (None: the root)
    hist: object                           # CUDA int64 [n_nodes][F][S][2]
    splits: object                         # CUDA uint8 [n_nodes * 56]
    built_rows: int = 0


def grow_tree_device(ctx: Context, grad, hess, depth: int, lam: float, gamma: float,
                     sync: bool = True, fused: bool = True) -> List[DeviceLevel]:
    """Grow levels 0..depth-1 with the rows partitioned on the device.

    Each level: hgb_partition_level lays out the children of the previous
    level's split nodes (pair j = children 2j, 2j + 1); build_level builds the
    smaller child of each pair from that layout (the other node's slot is -1,
    so its rows are skipped); subtract_find_splits derives the other and scores
    every child.  Only the child sizes and each pair's parent come back
    to the host (to size and plan the next level).  fused: the three calls of
    a level as one hgb_grow_level (nothing runs on the host between them);
    otherwise one call each, with the choice of the built children here.
    sync: wait for the tree at the end (hgb_sync, which also reports a bad row
    index); without it the caller syncs later."""
    import torch
    dev = torch.device("cuda", ctx.device)
    F, S = ctx.n_features, ctx.n_slots
    begin(ctx, grad, hess)
    hist = torch.empty((1, F, S, 2), dtype=torch.int64, device=dev)
    sp = torch.empty(SPLIT_BYTES, dtype=torch.uint8, device=dev)
    ctx.build_level(hist)
    ctx.find_splits(hist, 1, lam, gamma, sp)
    levels = [DeviceLevel(0, 1, None, None, hist, sp, ctx.n_rows)]
    for d in range(1, depth):
        prev = levels[-1]
        total = ctx.n_rows if prev.rows is None else int(prev.offsets[-1])
        out = torch.empty(max(total, 1), dtype=torch.int32, device=dev)
        if fused:
            # room for every child of every parent: the level's size is known
            # only once the rows are partitioned, inside the call
            hist = torch.empty((2 * prev.n_nodes, F, S, 2), dtype=torch.int64, device=dev)
            sp = torch.empty(2 * prev.n_nodes * SPLIT_BYTES, dtype=torch.uint8, device=dev)
            child, _, _, built_rows = ctx.grow_level(prev.hist, prev.splits, prev.rows, prev.offsets, out,
                                                     hist, sp, lam, gamma)
            n_nodes = int(child.shape[0]) - 1
            if n_nodes == 0:
                break
            levels.append(DeviceLevel(d, n_nodes, out, child, hist[:n_nodes], sp[: n_nodes * SPLIT_BYTES],
                                      built_rows))
            continue
        child, split_nodes = ctx.partition_level(prev.splits, out, prev.rows, prev.offsets)
        n_nodes = int(child.shape[0]) - 1
        if n_nodes == 0:
            break
        counts = np.diff(child)
        bir = _choose_built(counts)
        P = n_nodes // 2
        slots = np.full(n_nodes, -1, dtype=np.int32)
        built = 2 * np.arange(P) + bir
        slots[built] = built
        hist = torch.empty((n_nodes, F, S, 2), dtype=torch.int64, device=dev)
        sp = torch.empty(n_nodes * SPLIT_BYTES, dtype=torch.uint8, device=dev)
        ctx.build_level(hist, out, child, slots)
        ctx.subtract_find_splits(prev.hist, hist, bir, lam, gamma, sp, split_nodes.astype(np.int32))
        levels.append(DeviceLevel(d, n_nodes, out, child, hist, sp, int(counts[built].sum())))
    if sync:
        ctx.sync()
    return levels


def grow_oblivious_tree_device(ctx: Context, grad, hess, depth: int, lam: float,
                               gamma: float, sync: bool = True, fused: bool = True) -> List[DeviceLevel]:
    """Grow an oblivious (symmetric) tree of levels 0..depth-1 on the device:
    every node of a level takes the level's one (feature, bin, direction) from
    find_level_split, so every node of a split level gets two children (one
    may be empty).  Per level: partition_level with the node records,
    build_level of the smaller child of each pair, subtract_siblings for the
    other, find_level_split over all children.  Each level's `splits` holds
    n_nodes + 1 records, the last one the level's.  sync, fused: as for
    grow_tree_device."""
    import torch
    dev = torch.device("cuda", ctx.device)
    F, S = ctx.n_features, ctx.n_slots
    begin(ctx, grad, hess)
    hist = torch.empty((1, F, S, 2), dtype=torch.int64, device=dev)
    sp = torch.empty(2 * SPLIT_BYTES, dtype=torch.uint8, device=dev)
    ctx.build_level(hist)
    ctx.find_level_split(hist, 1, lam, gamma, sp)
    levels = [DeviceLevel(0, 1, None, None, hist, sp, ctx.n_rows)]
    for d in range(1, depth):
        prev = levels[-1]
        total = ctx.n_rows if prev.rows is None else int(prev.offsets[-1])
        out = torch.empty(max(total, 1), dtype=torch.int32, device=dev)
        if fused:
            hist = torch.empty((2 * prev.n_nodes, F, S, 2), dtype=torch.int64, device=dev)
            sp = torch.empty((2 * prev.n_nodes + 1) * SPLIT_BYTES, dtype=torch.uint8, device=dev)
            child, _, _, built_rows = ctx.grow_level(prev.hist, prev.splits, prev.rows, prev.offsets, out,
                                                     hist, sp, lam, gamma, oblivious=True)
            n_nodes = int(child.shape[0]) - 1
            if n_nodes == 0:
                break
            levels.append(DeviceLevel(d, n_nodes, out, child, hist[:n_nodes], sp[: (n_nodes + 1) * SPLIT_BYTES],
                                      built_rows))
            continue
        child, split_nodes = ctx.partition_level(prev.splits, out, prev.rows, prev.offsets)
        n_nodes = int(child.shape[0]) - 1
        if n_nodes == 0:
            break
        counts = np.diff(child)
        bir = _choose_built(counts)
        P = n_nodes // 2
        slots = np.full(n_nodes, -1, dtype=np.int32)
        built = 2 * np.arange(P) + bir
        slots[built] = built
        hist = torch.empty((n_nodes, F, S, 2), dtype=torch.int64, device=dev)
        sp = torch.empty((n_nodes + 1) * SPLIT_BYTES, dtype=torch.uint8, device=dev)
        ctx.build_level(hist, out, child, slots)
        ctx.subtract_siblings(prev.hist, hist, bir, split_nodes.astype(np.int32))
        ctx.find_level_split(hist, n_nodes, lam, gamma, sp)
        levels.append(DeviceLevel(d, n_nodes, out, child, hist, sp, int(counts[built].sum())))
    if sync:
        ctx.sync()
    return levels
