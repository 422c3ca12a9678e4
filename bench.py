#!/usr/bin/env python3
"""Level histogram build benchmark on one MI355X.

A step is one pass of the whole device path over one batch of synthetic input:
begin_tree (quantize), then every level's build_level + subtract_siblings +
find_splits.  The default workload is the tall-narrow case: 10,000,000 rows x
28 u8 features, one depthwise tree, levels 0..7, whose (g, h) are the logistic
loss's, derived on the device from resident scores and labels
(begin_tree_objective).  Its row lists per level are fixed once before timing
(the host partition is not part of the device path), so the timed steps replay
the same tree with every input resident in HBM; --grow partitions on the
device instead.

Prints one JSON line:  value = built cells (rows x features of every node
built from rows) per second over the timed steps, in G cell-updates/s.
"""
from __future__ import annotations

import argparse
import gc
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
# The fill class timed for the roofline: the LDS fill kernels and the merge of
# split nodes' partial histograms (bracketed together by the library's events
# on its stream).
FILL_KERNELS = "k_fill_root / k_fill_root_il / k_fill_rows / k_fill_cols + k_merge"
METRIC = "level histogram build G cell-updates/s (rows x features) + % of HBM peak"

WORKLOAD_NAMES = {
    "c1": "tiny root 4,096 x 8 u8 (256 bins), root build + split",
    "c2": "depth-6 level 1,000,000 x 100 u8 (80 uniform + 20 skewed features), 32 Dirichlet nodes: build 16 smaller + subtract + split",
    "c3": "tall narrow 10,000,000 x 28 u8 (256 bins), logistic grad/hess, one depthwise tree levels 0-7",
    "c4": "wide 131,072 x 16,384 u8 (256 bins), root + level 3 (8 nodes): build + subtract + split",
    "c5": "high-cardinality 2,000,000 x 50 u16 (1,024 bins + 40% missing), 128 Dirichlet nodes: build 64 smaller + subtract + split",
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Plan:
    """What one step enqueues, and its work accounting."""

    def __init__(self):
        self.levels = []          # (kind, LevelPlan, parent_hist)
        self.cells = 0            # built rows x features per step
        self.all_cells = 0        # rows x features of every node of every level (built or derived)
        self.fill_bytes = 0       # algorithmic bytes of the build kernels per step
        self.root_bytes = 0       # ... of the root's fill
        self.level_bytes = 0      # ... of the fills below the root
        self.root_rows = 0        # rows of the root build per step
        self.level_notes = []


def fill_alg_bytes(w, built_rows: int, n_built_nodes: int, root: bool) -> int:
    """Algorithmic bytes of one build: bins w*cells, (g,h) 8 B/row (+4 B row
    index below the root), and one 16 B write per output slot."""
    wbytes = w.bins.dtype.itemsize
    per_row = 8 if root else 12
    return (wbytes * built_rows * w.n_features + per_row * built_rows
            + 16 * w.n_features * w.n_slots * n_built_nodes)


def resolve_objective(w, objective: str):
    """"auto" is the workload's own loss (logistic for c3, whose recipe has
    scores and labels), else "none"; None if the workload cannot take it."""
    if objective == "auto":
        return "logistic" if w.margin is not None else "none"
    if objective != "none" and w.margin is None:
        return None
    return objective


def step_inputs(w, objective: str, torch):
    """The resident inputs a step starts a tree from: (Objective, None) for a
    device objective, else the (g, h) tensors."""
    if objective != "none":
        from histogram_gradient_boosted_amd import tree
        return tree.Objective(objective, torch.from_numpy(w.margin).cuda(),
                              torch.from_numpy(w.label).cuda()), None
    return torch.from_numpy(w.grad).cuda(), torch.from_numpy(w.hess).cuda()


def prepare(ctx, w, g, h, torch):
    """g may be a tree.Objective (h None): the tree then starts from the device objective."""
    from histogram_gradient_boosted_amd import tree
    plan = Plan()
    if w.kind == "tree":
        plans = tree.plan_tree(ctx, w.bins, w.n_bins, g, h, w.depth, w.lam, w.gamma)
        plan.tree = plans
        for lp in plans:
            nb = 1 if lp.depth == 0 else lp.n_pairs
            plan.cells += lp.built_rows * w.n_features
            level_rows = w.n_rows if lp.depth == 0 else int(lp.children_offsets[-1])
            plan.all_cells += level_rows * w.n_features
            b = fill_alg_bytes(w, lp.built_rows, nb, lp.depth == 0)
            plan.fill_bytes += b
            if lp.depth == 0:
                plan.root_bytes += b
                plan.root_rows += lp.built_rows
            else:
                plan.level_bytes += b
            plan.level_notes.append({"depth": lp.depth, "nodes": lp.n_nodes, "built_rows": lp.built_rows})
        return plan
    plan.tree = None
    tree.begin(ctx, g, h)
    dev = torch.device("cuda", ctx.device)
    if w.kind in ("root", "root+level"):
        rp = tree.root_plan(ctx)
        plan.levels.append(("root", rp, None))
        plan.cells += w.n_rows * w.n_features
        plan.all_cells += w.n_rows * w.n_features
        b = fill_alg_bytes(w, w.n_rows, 1, True)
        plan.fill_bytes += b
        plan.root_bytes += b
        plan.root_rows += w.n_rows
        plan.level_notes.append({"depth": 0, "nodes": 1, "built_rows": w.n_rows})
    if w.kind in ("level", "root+level"):
        L = w.level
        parents = torch.empty((L.n_pairs, w.n_features, w.n_slots, 2), dtype=torch.int64, device=dev)
        ctx.build_level(parents, torch.from_numpy(L.parent_row_index).to(dev),
                        L.parent_offsets.astype(np.int32))
        lp = tree.level_plan_from_children(ctx, 1, L.children_row_index, L.children_offsets,
                                           np.arange(L.n_pairs, dtype=np.int32))
        plan.levels.append(("level", lp, parents))
        plan.cells += lp.built_rows * w.n_features
        plan.all_cells += int(L.children_offsets[-1]) * w.n_features
        b = fill_alg_bytes(w, lp.built_rows, lp.n_pairs, False)
        plan.fill_bytes += b
        plan.level_bytes += b
        plan.level_notes.append({"nodes": lp.n_nodes, "built_rows": lp.built_rows})
    ctx.sync()
    return plan


def step(ctx, w, plan, g, h):
    from histogram_gradient_boosted_amd import tree
    # (grown trees: the library's error word is checked by the hgb_sync that
    # follows the timed steps, as for the replayed ones)
    if getattr(plan, "oblivious", False):
        tree.grow_oblivious_tree_device(ctx, g, h, w.depth, w.lam, w.gamma, sync=False)
        return
    if getattr(plan, "grow", False):
        # the whole level loop on the device: partition, build, subtract, split
        tree.grow_tree_device(ctx, g, h, w.depth, w.lam, w.gamma, sync=False)
        return
    if plan.tree is not None:
        tree.replay_tree(ctx, plan.tree, g, h, w.lam, w.gamma)
        return
    tree.begin(ctx, g, h)
    for kind, lp, parents in plan.levels:
        if kind == "root":
            tree.run_root(ctx, lp, w.lam, w.gamma)
        else:
            tree.run_level(ctx, lp, parents, w.lam, w.gamma)


def _oracle_pass(w, budget_s: float, objective: str = "none"):
    """One step of the oracle, as it stands, on the host: (the objective's
    gradients,) quantize, builds of the built nodes, subtraction, split scan,
    the tree grown with its own (untimed) partition.  Returns (built cells,
    timed seconds, sample)."""
    import oracle
    t_work = 0.0
    cells = 0

    def timed(fn, *a):
        nonlocal t_work
        t0 = time.perf_counter()
        r = fn(*a)
        t_work += time.perf_counter() - t0
        return r

    if objective != "none":
        grad, hess = timed(oracle.objective, objective, w.margin, w.label)
    else:
        grad, hess = w.grad, w.hess
    qg, kg = timed(oracle.quantize, grad, False)
    qh, kh = timed(oracle.quantize, hess, True)
    B, M = w.n_bins, w.has_missing
    sample = "full step"
    if w.kind in ("root", "root+level", "tree"):
        hist = timed(oracle.build_hist, w.bins, B, M, qg, qh)
        cells += w.n_rows * w.n_features
        sp = timed(oracle.find_splits, hist, B, M, kg, kh, w.lam, w.gamma)
    if w.kind == "tree":
        rows, offs = None, None
        parent = hist
        for d in range(1, w.depth):
            if t_work > budget_s:
                sample = f"levels 0..{d - 1} of the tree (time budget)"
                break
            rows, offs = oracle.partition(w.bins, B, rows, offs, sp)   # untimed host step
            if len(offs) == 1:
                break
            counts = np.diff(offs)
            bir = (counts[1::2] < counts[0::2]).astype(np.uint8)
            P = len(bir)
            blist = [rows[offs[2 * i + bir[i]]:offs[2 * i + bir[i] + 1]] for i in range(P)]
            boffs = np.zeros(P + 1, np.int64)
            np.cumsum([len(x) for x in blist], out=boffs[1:])
            brows = np.concatenate(blist).astype(np.int32)
            built = timed(oracle.build_hist, w.bins, B, M, qg, qh, brows, boffs)
            cells += int(boffs[-1]) * w.n_features
            child = np.zeros((2 * P,) + built.shape[1:], np.int64)
            child[2 * np.arange(P) + bir] = built
            # parents of this level are the previous level's split nodes, in order
            split_nodes = np.nonzero(sp["feature"] >= 0)[0]
            timed(oracle.subtract, parent[split_nodes], child, bir)
            sp = timed(oracle.find_splits, child, B, M, kg, kh, w.lam, w.gamma)
            parent = child
    if w.kind in ("level", "root+level"):
        L = w.level
        parents = oracle.build_hist(w.bins, B, M, qg, qh, L.parent_row_index, L.parent_offsets)
        built = timed(oracle.build_hist, w.bins, B, M, qg, qh, L.built_row_index, L.built_offsets)
        cells += int(L.built_offsets[-1]) * w.n_features
        child = np.zeros((2 * L.n_pairs,) + built.shape[1:], np.int64)
        child[L.built_slots] = built
        timed(oracle.subtract, parents, child, L.built_is_right)
        timed(oracle.find_splits, child, B, M, kg, kh, w.lam, w.gamma)
    return cells, t_work, sample


def host_cpu() -> dict:
    """The host the oracle ran on: CPU model and the CPUs this process may use."""
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count() or 0
    return {"cpu_model": model, "nproc": usable}


def cpu_baseline(w, objective: str = "none", min_s: float = 10.0, max_reps: int = 30,
                 budget_s: float = 20.0):
    """The oracle timed on one host core: whole steps repeated until about
    min_s seconds of timed work (a step larger than budget_s is cut after the
    level that crosses it)."""
    import oracle
    oracle.build()
    cells = 0
    t_work = 0.0
    reps = 0
    sample = ""
    while reps < max_reps and (reps == 0 or t_work < min_s):
        c, t, sample = _oracle_pass(w, budget_s, objective)
        cells += c
        t_work += t
        reps += 1
    return {"value": cells / t_work / 1e9, "unit": "G cell-updates/s", "cores": 1,
            "kind": "oracle", "seconds": round(t_work, 3), "host": host_cpu(),
            "sample": f"{reps} x ({sample}) of workload {w.name}: serial C oracle (gcc -O2), "
                      f"1 thread, {cells} built cells"}


def lds_rates(device: int = 0):
    """LDS atomic-add rates (lane-ops/s) from the microbenchmark library
    (csrc/lds_rate.hip): u64 adds at uniformly random bins with 1, 2 and 16
    lane-interleaved copies (the fill's layout), and conflict-free u64 adds
    (every lane a distinct word).  None if the library is missing."""
    import ctypes
    path = os.path.join(ROOT, "histogram_gradient_boosted_amd", "liblds_rate.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    fn = lib.lds_rate_measure
    fn.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_double),
                   ctypes.POINTER(ctypes.c_int)]
    fn.restype = ctypes.c_int
    out = {}
    n_cu = ctypes.c_int(0)
    for name, kind, copies in (("u64_random_bins_1_copy", 0, 1), ("u64_random_bins_2_copies", 0, 2),
                               ("u64_random_bins_16_copies", 0, 16), ("u64_conflict_free", 1, 1),
                               ("u64_interleaved_tile_fill_shape", 3, 1), ("u32_conflict_free", 4, 1),
                               ("u32_random_bins_16_copies", 2, 16)):
        r = ctypes.c_double(0.0)
        if fn(device, kind, copies, ctypes.byref(r), ctypes.byref(n_cu)) != 0:
            return None
        out[name] = r.value
    out["n_cu"] = n_cu.value
    if hasattr(lib, "gather_rate_measure"):
        g = lib.gather_rate_measure
        g.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_double)]
        g.restype = ctypes.c_int
        r = ctypes.c_double(0.0)
        if g(device, ctypes.byref(r)) == 0:
            out["random_lines_per_s"] = r.value
    return out


def counters_record(config: str, precision: int, mode: str = ""):
    """The rocprofv3 counter record bench_counters.py wrote for this workload
    and step (mode "" is the replayed depthwise tree that bench_counters.py
    drives; grown and oblivious trees have no record): HBM traffic per kernel
    (FETCH_SIZE, WRITE_SIZE, calibrated against a copy of known size).  None
    when there is no record or the kernel sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"counters_{config}{mode}_p{precision}.json")
    if not os.path.exists(path):
        return None
    try:
        import bench_counters
        with open(path) as f:
            rec = json.load(f)
        if rec.get("source_hash") != bench_counters.source_hash():
            return None
        return rec
    except Exception:
        return None


def dominant_roofline(prof, plan, steps: int, counters):
    """The roofline of the step's dominant build kernel: the level fill
    (k_fill_rows / k_fill_cols, every level below the root) or the root fill
    (k_fill_root / k_fill_root_il), whichever takes longer, each timed by the
    library's events around its own launches.  achieved = its algorithmic bytes
    per launch / its average launch duration."""
    parts = {"fill_level": ("k_fill_rows / k_fill_cols (levels below the root)", plan.level_bytes),
             "fill_root": ("k_fill_root / k_fill_root_il (the root)", plan.root_bytes)}
    name = max(parts, key=lambda k: prof[k][0])
    ms, launches = prof[name]
    if launches == 0 or ms <= 0:
        return None
    kernel, alg_bytes = parts[name]
    per_launch_bytes = alg_bytes / (launches / steps)
    avg_s = ms * 1e-3 / launches
    achieved = per_launch_bytes / avg_s / 1e9
    traffic = None
    if counters is not None:
        kk = counters.get("per_step", {})
        names = ("k_fill_rows", "k_fill_cols") if name == "fill_level" else ("k_fill_root", "k_fill_root_il")
        tb = sum(int(kk[k]["FETCH_SIZE"]["bytes"]) + int(kk[k]["WRITE_SIZE"]["bytes"]) for k in names if k in kk)
        dispatches = sum(int(kk[k]["FETCH_SIZE"]["dispatches"]) for k in names if k in kk)
        if dispatches:
            traffic = int(round(tb / dispatches))
    return {"bound": "hbm", "kernel": kernel, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
            "traffic_unit": "HBM bytes per launch (fetch + write, calibrated counters)",
            "alg_bytes_per_launch": int(round(per_launch_bytes)),
            "launches_per_step": launches // steps, "avg_launch_us": round(avg_s * 1e6, 3)}


# untimed steps of the set-up before the warm-up: at least this many, for at
# least this long
SETTLE_STEPS = 10
SETTLE_S = 0.05


def spin_until_done(torch):
    """Poll an event recorded after the queued work until the device has done
    it, so that the blocking synchronize after it returns at once (its
    wake-up latency is then not part of the timed region)."""
    ev = torch.cuda.Event()
    ev.record()
    while not ev.query():
        pass


def measure(config: str, precision: int, steps: int, warmup: int, seed: int, objective_arg: str,
            grow: bool, oblivious: bool, flush_mib: int, cpu: bool, cpu_min_s: float = 10.0):
    """Set up one workload, time `steps` steps after `warmup`, and return its
    record (value, ms per step, the rooflines, optionally the oracle's rate)."""
    import torch
    from histogram_gradient_boosted_amd import binding, synth

    t0 = time.time()
    w = synth.make(config, seed=seed)
    log(f"[bench] workload {config}: {w.n_rows} x {w.n_features}, generated in {time.time() - t0:.1f}s")
    ctx = binding.Context(0)
    ctx.set_precision(precision)
    # begin_tree enqueues its passes and returns: no host round trip between
    # a tree's start and its first level (the check of the maxima happens at
    # the next sync)
    ctx.set_async_begin(True)
    ctx.upload_bins(w.bins, w.n_bins, w.has_missing)
    objective = resolve_objective(w, objective_arg)
    if objective is None:
        print(f"--objective {objective_arg} needs a workload with scores and labels (c3)", file=sys.stderr)
        sys.exit(2)
    g, h = step_inputs(w, objective, torch)
    plan = prepare(ctx, w, g, h, torch)
    if grow or oblivious:
        if plan.tree is None:
            print("--grow / --oblivious need a tree workload (c3)", file=sys.stderr)
            sys.exit(2)
        plan.grow = True
    if oblivious:
        # the oblivious tree differs from the planned depthwise one: count its
        # built cells from one untimed growth
        from histogram_gradient_boosted_amd import tree
        plan.oblivious = True
        levels = tree.grow_oblivious_tree_device(ctx, g, h, w.depth, w.lam, w.gamma)
        plan.cells = sum(lv.built_rows for lv in levels) * w.n_features
        plan.all_cells = sum(w.n_rows if lv.depth == 0 else int(lv.offsets[-1]) for lv in levels) * w.n_features
        plan.root_rows = sum(lv.built_rows for lv in levels if lv.depth == 0)
        plan.root_bytes = sum(fill_alg_bytes(w, lv.built_rows, 1, True) for lv in levels if lv.depth == 0)
        plan.level_bytes = sum(fill_alg_bytes(w, lv.built_rows, lv.n_nodes // 2, False)
                               for lv in levels if lv.depth > 0)
        plan.fill_bytes = plan.root_bytes + plan.level_bytes
        plan.level_notes = [{"depth": lv.depth, "nodes": lv.n_nodes, "built_rows": lv.built_rows}
                            for lv in levels]
        del levels
    log(f"[bench] plan ready: {plan.cells} built cells per step, levels {plan.level_notes}")

    # The set-up made millions of Python objects (torch's own, the workload);
    # a full collection of them in the middle of the timed steps stalls the
    # host for tens of milliseconds.  Freeze them out of the collector.
    gc.collect()
    gc.freeze()
    # Settle, as part of the set-up: untimed steps for at least SETTLE_S and
    # SETTLE_STEPS.  A few steps of a sub-millisecond tree do not reach the
    # steady state of a fit (131,072 x 16,384 after 3 steps: its first timed
    # pass ran 1.52 ms a step against 1.46 ms for every later one; after 30,
    # 1.46 ms from the first).  Then the W warm-up steps.
    settle_steps = 0
    t_settle = time.perf_counter()
    while settle_steps < SETTLE_STEPS or time.perf_counter() - t_settle < SETTLE_S:
        step(ctx, w, plan, g, h)
        settle_steps += 1
        if settle_steps % 8 == 0:
            ctx.sync()   # keeps the host within a few trees of the device
    ctx.sync()
    for _ in range(warmup):
        step(ctx, w, plan, g, h)
    ctx.sync()

    # The timed steps, back to back, with nothing else on the stream, between
    # two device synchronizations; the library's own check of the steps (its
    # error word, the trees' maxima) follows outside the timed region.
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for _ in range(steps):
        step(ctx, w, plan, g, h)
    spin_until_done(torch)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    ctx.sync()

    # The same steps with an event on the library's stream (torch's current
    # stream) between consecutive steps, for the median and spread of the
    # per-step times beside the mean (each marker adds a little host and
    # device time of its own).
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    marks[0].record()
    for i in range(steps):
        step(ctx, w, plan, g, h)
        marks[i + 1].record()
    ctx.sync()
    torch.cuda.synchronize()
    per_step = np.array([marks[i].elapsed_time(marks[i + 1]) for i in range(steps)])

    # The same steps again with the library's per-kernel events (recorded on
    # its own stream around each kernel class), for the breakdown and the fill
    # kernels' duration.  Before each of these steps a scratch buffer larger
    # than the 256 MB Infinity Cache is written, so the kernels start without
    # the previous step's data in that cache (the write is not a library
    # kernel, so no event brackets it).
    flush = torch.empty(flush_mib << 18, dtype=torch.float32, device="cuda") if flush_mib else None
    ctx.profile_enable(True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(steps):
        if flush is not None:
            flush.fill_(1.0)
        step(ctx, w, plan, g, h)
    ctx.sync()
    torch.cuda.synchronize()
    wall_prof = time.perf_counter() - t1
    del flush
    prof = {k: ctx.profile_query(k) for k in binding.KERNELS}
    ctx.profile_enable(False)

    ms_per_step = wall * 1e3 / steps
    value = plan.cells * steps / wall / 1e9
    fill_ms, fill_launches = prof["fill"]
    fill_ms_step = fill_ms / steps
    achieved = plan.fill_bytes / (fill_ms_step * 1e-3) / 1e9 if fill_ms_step > 0 else 0.0
    breakdown = {k: round(v[0] / steps, 4) for k, v in prof.items()}
    log(f"[bench] per-step device ms by kernel class: {breakdown}; launches {{{', '.join(f'{k}: {v[1] // steps}' for k, v in prof.items())}}}")
    log(f"[bench] wall ms/step {ms_per_step:.3f} (timed, events off; median {np.median(per_step):.3f}), "
        f"{wall_prof * 1e3 / steps:.3f} (events on)")

    counters = counters_record(config, precision,
                               "_oblivious" if oblivious else "_grow" if grow else "")
    traffic = int(counters["fill_traffic"]["bytes_per_step"]) if counters else None
    result = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "G cell-updates/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "settle_steps": settle_steps,
        "ms_per_step": round(ms_per_step, 4),
        # per-step spans from events between consecutive steps (a second pass)
        "ms_per_step_stats": {"median": round(float(np.median(per_step)), 4),
                              "min": round(float(per_step.min()), 4),
                              "p10": round(float(np.percentile(per_step, 10)), 4),
                              "p90": round(float(np.percentile(per_step, 90)), 4),
                              "max": round(float(per_step.max()), 4),
                              "mean": round(float(per_step.mean()), 4)},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int64",
        "data": "synthetic",
        "config": {"workload": WORKLOAD_NAMES[config], "name": config,
                   "rows": w.n_rows, "features": w.n_features, "bins": w.n_bins,
                   "built_cells_per_step": plan.cells, "levels": plan.level_notes},
        # every node's histogram per second, the derived siblings included
        # (what the subtraction buys: cells that were never added)
        "effective_gcells_per_s": round(plan.all_cells * steps / wall / 1e9, 3),
        "build_only_gcells_per_s": round(plan.cells / (fill_ms_step + breakdown["gather"] + breakdown["zero"]) / 1e6, 3)
        if fill_ms_step > 0 else None,
        "ms_per_step_events_on": round(wall_prof * 1e3 / steps, 4),
        "event_pass": f"per-kernel events, {flush_mib} MiB written before each step"
        if flush_mib else "per-kernel events",
        "kernel_ms_per_step": breakdown,
        "roofline": dominant_roofline(prof, plan, steps, counters),
        # the whole build class (every fill launch and the merges), the unit the
        # level build's bandwidth target speaks of
        "fill_class_roofline": {"bound": "hbm", "kernel": FILL_KERNELS, "achieved": round(achieved, 1),
                                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                                "traffic": traffic,
                                "traffic_unit": "HBM bytes per step (fetch + write, calibrated counters)",
                                # the bytes the fill class actually moves, per second of its time
                                "traffic_gbs": round(traffic / (fill_ms_step * 1e-3) / 1e9, 1)
                                if traffic and fill_ms_step > 0 else None,
                                "alg_bytes_per_step": plan.fill_bytes,
                                "launches_per_step": fill_launches // max(steps, 1),
                                "avg_launch_us": round(fill_ms * 1e3 / max(fill_launches, 1), 3)},
        "precision_bits": precision,
        "gradients": "device objective: " + objective + " loss from resident scores and labels"
        if objective != "none" else "resident fp32 (g, h) arrays",
        "step": "oblivious: partition + build + subtract + level split per level, on the device"
        if oblivious else
        "grow: partition + build + subtract + split per level, on the device" if grow
        else "replay: build + subtract + split per level on fixed row lists",
    }
    ctx.close()
    # the LDS ceiling: each fill's atomic adds per step (two per cell in wide
    # mode, P > 19; one in packed mode) against the microbenchmark's rates
    rates = lds_rates(0)
    per_cell = 2 if precision > 19 else 1
    if rates:
        def lds(cells, ms):
            a = cells * per_cell / (ms * 1e-3) if ms > 0 else 0.0
            return {"atomics_per_step": cells * per_cell, "achieved": round(a / 1e9, 1),
                    "frac": round(a / rates["u64_conflict_free"], 4)}
        root_cells = plan.root_rows * w.n_features
        result["lds_roofline"] = {
            "kernel": FILL_KERNELS, "unit": "u64 LDS atomic adds (lane-ops)/s",
            **lds(plan.cells, fill_ms_step),
            "peak": round(rates["u64_conflict_free"] / 1e9, 1),
            "peak_kind": "measured: conflict-free u64 LDS atomic adds, whole chip (csrc/lds_rate.hip)",
            "root_fill": lds(root_cells, breakdown["fill_root"]) if root_cells else None,
            "level_fill": lds(plan.cells - root_cells, breakdown["fill_level"]) if plan.cells > root_cells else None,
            "random_bins": {k: round(v / 1e9, 1) for k, v in rates.items() if k.startswith("u64_random")},
            # the fills' own pattern and launch shape: two lanes per bank pair,
            # 16 waves per CU (the ceiling a 1024-thread fill block can reach)
            "interleaved_tile_fill_shape": round(rates["u64_interleaved_tile_fill_shape"] / 1e9, 1),
            # u32 adds, for a cell split into 32-bit halves (four adds instead of two)
            "u32": {k: round(rates[k] / 1e9, 1) for k in ("u32_conflict_free", "u32_random_bins_16_copies")},
            "scale": "G lane-ops/s", "n_cu": rates["n_cu"]}
        # The level fill of a narrow matrix reads its built rows and their (g, h)
        # scattered: its ceiling is the rate of scattered 128-byte line fetches
        # (every read the L2 sends to memory is a whole line), measured by the
        # same library.  Lines per step from the counters' read requests.
        kk = (counters or {}).get("read_requests_per_step", {})
        lines = sum(kk[k]["requests"] for k in ("k_fill_rows", "k_fill_cols") if k in kk)
        if "random_lines_per_s" in rates and breakdown["fill_level"] > 0:
            # (achieved and frac null when the committed counters are not of these sources)
            ach = lines / (breakdown["fill_level"] * 1e-3) if lines > 0 else None
            result["gather_roofline"] = {
                "kernel": "k_fill_rows / k_fill_cols (levels below the root)",
                "unit": "128-byte line fetches/s", "lines_per_step": int(lines) if lines > 0 else None,
                "achieved": round(ach / 1e9, 2) if ach else None,
                "peak": round(rates["random_lines_per_s"] / 1e9, 2),
                "frac": round(ach / rates["random_lines_per_s"], 4) if ach else None, "scale": "G lines/s",
                "peak_kind": "measured: random 128-byte line reads, 8 in flight per thread, 640 MiB buffer "
                             "(csrc/lds_rate.hip gather_rate_measure)"}
        log(f"[bench] LDS atomics {plan.cells * per_cell / (fill_ms_step * 1e-3) / 1e9:.0f} G/s in the fill; "
            f"microbenchmark { {k: round(v / 1e9) for k, v in rates.items() if k != 'n_cu'} } G/s")
    if cpu:
        log(f"[bench] timing the oracle on the host ({config}) ...")
        result["cpu_baseline"] = cpu_baseline(w, objective, min_s=cpu_min_s)
    del w, plan, g, h
    gc.unfreeze()
    gc.collect()
    torch.cuda.empty_cache()
    return result


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed steps first (default 3; 25 for --grow / --oblivious, whose "
                         "first few dozen trees run slower while the allocator and the device warm up)")
    ap.add_argument("--config", default="c3", choices=sorted(WORKLOAD_NAMES))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-targets", action="store_true",
                    help="skip the second measured workload (the wide 131,072 x 16,384 case, "
                         "measured after the default one in the same process)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--grow", action="store_true",
                    help="tree workloads: grow the tree each step with the device partition "
                         "(the level loop closed on the device) instead of replaying fixed row lists")
    ap.add_argument("--flush-mib", type=int, default=512,
                    help="MiB of scratch written before each event-timed step (0: none)")
    ap.add_argument("--oblivious", action="store_true",
                    help="tree workloads: grow an oblivious tree (one split per level, "
                         "find_level_split) on the device each step")
    ap.add_argument("--objective", default="auto", choices=["auto", "none", "logistic"],
                    help="start each tree from the device objective (logistic: the c3 recipe's "
                         "loss, from its scores and labels) or from resident (g, h) arrays (none); "
                         "auto = logistic for c3, none otherwise")
    ap.add_argument("--precision", type=int, default=30,
                    help="fixed-point bits P (k = P - e); 30 is the int64-cell default, "
                         "P <= 19 selects the packed one-atomic fill")
    args = ap.parse_args()

    if args.warmup is None:
        args.warmup = 25 if (args.grow or args.oblivious) else 3
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch
    from histogram_gradient_boosted_amd import binding

    if not torch.cuda.is_available() or not binding.available():
        print("no HIP device available", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    result = measure(args.config, args.precision, args.steps, args.warmup, args.seed, args.objective,
                     args.grow, args.oblivious, args.flush_mib, not args.no_cpu_baseline)
    # The default run also measures the wide case (the other workload the
    # bandwidth target names), in the same process after the headline one,
    # with its own warm-up and a one-step oracle sample.
    if (not args.no_targets and args.config == "c3" and not args.grow and not args.oblivious):
        wide = measure("c4", args.precision, args.steps, 3, args.seed, "auto", False, False,
                       args.flush_mib, not args.no_cpu_baseline, cpu_min_s=0.0)
        keep = ("value", "unit", "ms_per_step", "ms_per_step_stats", "steps", "warmup", "settle_steps", "config",
                "kernel_ms_per_step", "roofline", "fill_class_roofline", "lds_roofline", "cpu_baseline",
                "precision_bits", "effective_gcells_per_s", "gather_roofline")
        result["targets"] = {"c4": {k: wide[k] for k in keep if k in wide}}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
