"""GPU parity of the device partition (hgb_partition_level) and of levels grown
with it, against the oracle's partition and tree.  Row lists and offsets must
be identical (the partition is stable, so there is exactly one answer)."""
import numpy as np
import pytest

import oracle
from histogram_gradient_boosted_amd import synth

from test_gpu_parity import assert_splits, oracle_quantized, oracle_tree, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    import torch as _torch
    from histogram_gradient_boosted_amd import binding
    if not _torch.cuda.is_available() or not binding.available():
        pytest.skip("no HIP device")
    return _torch


@pytest.fixture(scope="module")
def hgb(torch):
    from histogram_gradient_boosted_amd import binding
    return binding


def splits_dev(torch, sp):
    return torch.from_numpy(np.ascontiguousarray(sp).view(np.uint8).copy()).cuda()


def gpu_partition(hgb, torch, w, sp, rows=None, offs=None):
    ctx = hgb.Context(0)
    ctx.upload_bins(w.bins, w.n_bins, w.has_missing)
    total = w.n_rows if rows is None else int(offs[-1])
    out = torch.full((max(total, 1),), -5, dtype=torch.int32, device="cuda")
    ri = None if rows is None else torch.from_numpy(np.ascontiguousarray(rows, dtype=np.int32)).cuda()
    child, parent = ctx.partition_level(splits_dev(torch, sp), out, ri,
                                        None if offs is None else np.asarray(offs, dtype=np.int32))
    ctx.close()
    assert np.array_equal(parent, np.nonzero(np.asarray(sp)["feature"] >= 0)[0])
    return out.cpu().numpy()[: int(child[-1])], child


SMALL = [
    # seed, n, F, B, missing, children, u16
    (60, 1, 2, 3, False, 0, None), (61, 5000, 4, 16, False, 0, None), (62, 9000, 3, 64, True, 0, None),
    (63, 20000, 5, 256, False, 8, None), (64, 30000, 4, 300, True, 12, True),
    (65, 17, 2, 4, True, 6, None), (66, 70000, 3, 1024, True, 6, True),
]


@pytest.mark.parametrize("seed,n,F,B,missing,children,u16", SMALL)
def test_partition_vs_oracle(hgb, torch, seed, n, F, B, missing, children, u16):
    """Splits from the oracle (some nodes forced to have none); the device
    partition must reproduce the oracle's row lists and offsets exactly."""
    say("partition", seed, n, F, B, missing, children)
    w = synth.random_small(seed, n, F, B, missing, children, u16=u16)
    qg, qh, kg, kh = oracle_quantized(w)
    if children == 0:
        rows, offs = None, None
        hist = oracle.build_hist(w.bins, w.n_bins, w.has_missing, qg, qh)
    else:
        rows, offs = w.level.children_row_index, w.level.children_offsets
        hist = oracle.build_hist(w.bins, w.n_bins, w.has_missing, qg, qh, rows, offs)
    sp = oracle.find_splits(hist, w.n_bins, w.has_missing, kg, kh, w.lam, w.gamma)
    if children >= 4:
        sp["feature"][1] = -1   # a node without a split: its rows are dropped
        sp["feature"][children - 1] = -1
    want_rows, want_offs = oracle.partition(w.bins, w.n_bins, rows, offs, sp)
    got_rows, got_offs = gpu_partition(hgb, torch, w, sp, rows, offs)
    assert np.array_equal(got_offs.astype(np.int64), want_offs)
    assert np.array_equal(got_rows, want_rows)


@pytest.mark.parametrize("n_nodes", [4096, 4097])
def test_partition_many_nodes(hgb, torch, n_nodes):
    """Levels of 4,096 nodes (the scan held in LDS) and 4,097 (the scan in
    global memory), with empty nodes, nodes without a split and nodes of one
    row, against the oracle's partition."""
    say("partition many nodes", n_nodes)
    rng = np.random.default_rng(n_nodes)
    w = synth.random_small(70, 60_000, 3, 16, True, 0)
    node = rng.integers(0, n_nodes, w.n_rows)
    node[node % 97 == 5] = 0   # some nodes left empty
    rows = np.argsort(node, kind="stable").astype(np.int32)
    offs = np.concatenate([[0], np.cumsum(np.bincount(node, minlength=n_nodes))]).astype(np.int32)
    sp = np.zeros(n_nodes, dtype=oracle.SPLIT_DTYPE)
    sp["feature"] = rng.integers(0, 3, n_nodes)
    sp["bin"] = rng.integers(0, 16, n_nodes)
    sp["default_left"] = rng.integers(0, 2, n_nodes)
    sp["feature"][rng.random(n_nodes) < 0.1] = -1
    want_rows, want_offs = oracle.partition(w.bins, w.n_bins, rows, offs, sp)
    got_rows, got_offs = gpu_partition(hgb, torch, w, sp, rows, offs)
    assert np.array_equal(got_offs.astype(np.int64), want_offs)
    assert np.array_equal(got_rows, want_rows)


def test_partition_every_direction(hgb, torch):
    """Splits chosen by hand on every feature and bin edge, both default
    directions, including bin n_bins - 1 (everything left) and missing rows."""
    say("partition directions")
    w = synth.random_small(67, 12_000, 3, 8, True, 18)
    rows, offs = w.level.children_row_index, w.level.children_offsets
    sp = np.zeros(18, dtype=oracle.SPLIT_DTYPE)
    for i in range(18):   # every (feature, bin, default) of 3 x 3 x 2
        sp[i]["feature"] = i % 3
        sp[i]["bin"] = [0, 3, 7][(i // 3) % 3]
        sp[i]["default_left"] = i // 9
    want_rows, want_offs = oracle.partition(w.bins, w.n_bins, rows, offs, sp)
    got_rows, got_offs = gpu_partition(hgb, torch, w, sp, rows, offs)
    assert np.array_equal(got_offs.astype(np.int64), want_offs)
    assert np.array_equal(got_rows, want_rows)


def test_partition_no_splits(hgb, torch):
    say("partition no splits")
    w = synth.random_small(68, 3000, 2, 16, False, 4)
    sp = np.zeros(4, dtype=oracle.SPLIT_DTYPE)
    sp["feature"] = -1
    rows, offs = w.level.children_row_index, w.level.children_offsets
    got_rows, got_offs = gpu_partition(hgb, torch, w, sp, rows, offs)
    assert got_offs.tolist() == [0] and got_rows.size == 0


def test_partition_bad_row_index(hgb, torch):
    say("partition bad row index")
    w = synth.random_small(69, 1000, 2, 16, False, 0)
    sp = np.zeros(1, dtype=oracle.SPLIT_DTYPE)
    sp["feature"] = 0
    sp["bin"] = 7
    rows = np.arange(1000, dtype=np.int32)
    rows[500] = 5000
    with pytest.raises(hgb.HGBError) as e:
        gpu_partition(hgb, torch, w, sp, rows, np.array([0, 1000]))
    assert e.value.status == hgb.HGB_E_INVALID


def test_build_level_skips_slot_minus_one(hgb, torch):
    """Nodes with output slot -1 are not built and their slots not written."""
    say("skip slots")
    w = synth.random_small(70, 40_000, 4, 64, True, 8)
    L = w.level
    ctx = hgb.Context(0)
    ctx.upload_bins(w.bins, w.n_bins, w.has_missing)
    g = torch.from_numpy(w.grad).cuda()
    h = torch.from_numpy(w.hess).cuda()
    ctx.begin_tree(g, h)
    slots = np.array([0, -1, 2, -1, -1, 5, 6, -1], dtype=np.int32)
    t = torch.full((8, 4, 65, 2), -9, dtype=torch.int64, device="cuda")
    ctx.build_level(t, torch.from_numpy(L.children_row_index).cuda(),
                    L.children_offsets.astype(np.int32), slots)
    ctx.sync()
    got = t.cpu().numpy()
    ctx.close()
    qg, qh, _, _ = oracle_quantized(w)
    want = oracle.build_hist(w.bins, w.n_bins, True, qg, qh, L.children_row_index, L.children_offsets)
    for i, s in enumerate(slots):
        if s >= 0:
            assert np.array_equal(got[s], want[i]), f"node {i}"
        else:
            assert (got[i] == -9).all(), f"slot {i} was written"


@pytest.mark.parametrize("n,bits,fused", [(300_000, 30, True), (300_000, 30, False), (300_000, 19, True),
                                          (None, 30, True)])
def test_c3_tree_device_partition(hgb, torch, n, bits, fused):
    """A whole c3 tree grown with the device partition equals the oracle's tree:
    row lists, offsets, histograms and splits at every level (fused: each
    level one hgb_grow_level; else partition, build and tail called apart)."""
    say("c3 device tree", n, bits, fused)
    from histogram_gradient_boosted_amd import tree
    w = synth.make("c3", n_rows=n)
    ctx = hgb.Context(0)
    ctx.set_precision(bits)
    ctx.upload_bins(w.bins, w.n_bins, w.has_missing)
    g = torch.from_numpy(w.grad).cuda()
    h = torch.from_numpy(w.hess).cuda()
    levels = tree.grow_tree_device(ctx, g, h, w.depth, w.lam, w.gamma, fused=fused)
    want = oracle_tree(w, w.depth, bits)
    assert len(levels) == len(want)
    for d, (lv, (rows, offs, hist, sp)) in enumerate(zip(levels, want)):
        say("c3 device level", d)
        if d > 0:
            assert np.array_equal(lv.offsets.astype(np.int64), offs)
            assert np.array_equal(lv.rows.cpu().numpy()[: int(offs[-1])], rows)
        assert np.array_equal(lv.hist.cpu().numpy(), hist), f"level {d} histograms differ"
        assert_splits(hgb.splits_to_numpy(lv.splits)[: lv.n_nodes], sp, f"level {d}")
    ctx.close()


@pytest.mark.parametrize("case", ["hot_u8", "c5"])
def test_tree_device_partition_hot_slots(hgb, torch, case):
    """A tree grown with the device partition on matrices whose stored bins are
    rotated (a hot slot exists: constant, skewed and mostly-missing features,
    or c5's 40% missing): the partition compares real bin values, and every
    level equals the oracle's."""
    say("device tree hot slots", case)
    from histogram_gradient_boosted_amd import tree
    from test_gpu_parity import with_hot_slots
    if case == "hot_u8":
        w = with_hot_slots(synth.random_small(123, 60_000, 6, 16, True, 0), 9)
        depth = 6
    else:
        w = synth.make("c5", n_rows=200_000)
        depth = 6
    ctx = hgb.Context(0)
    ctx.upload_bins(w.bins, w.n_bins, w.has_missing)
    g = torch.from_numpy(w.grad).cuda()
    h = torch.from_numpy(w.hess).cuda()
    levels = tree.grow_tree_device(ctx, g, h, depth, w.lam, w.gamma)
    want = oracle_tree(w, depth, 30)
    assert len(levels) == len(want)
    for d, (lv, (rows, offs, hist, sp)) in enumerate(zip(levels, want)):
        if d > 0:
            assert np.array_equal(lv.offsets.astype(np.int64), offs), f"level {d} offsets"
            assert np.array_equal(lv.rows.cpu().numpy()[: int(offs[-1])], rows), f"level {d} rows"
        assert np.array_equal(lv.hist.cpu().numpy(), hist), f"level {d} histograms differ"
        assert_splits(hgb.splits_to_numpy(lv.splits)[: lv.n_nodes], sp, f"level {d}")
    ctx.close()


def test_grow_level_without_splits(hgb, torch):
    """hgb_grow_level on parents none of which has a split: no children, and
    nothing is built (the output buffers keep their poison)."""
    say("grow level, no splits")
    w = synth.random_small(71, 5_000, 3, 16, False, 4)
    rows, offs = w.level.children_row_index, w.level.children_offsets
    F, S = w.n_features, w.n_slots
    ctx = hgb.Context(0)
    ctx.upload_bins(w.bins, w.n_bins, w.has_missing)
    g = torch.from_numpy(w.grad).cuda()
    h = torch.from_numpy(w.hess).cuda()
    ctx.begin_tree(g, h)
    sp = np.zeros(4, dtype=oracle.SPLIT_DTYPE)
    sp["feature"] = -1
    parent_hist = torch.zeros((4, F, S, 2), dtype=torch.int64, device="cuda")
    child_hist = torch.full((8, F, S, 2), -9, dtype=torch.int64, device="cuda")
    child_sp = torch.full((8 * hgb.SPLIT_BYTES,), 7, dtype=torch.uint8, device="cuda")
    out = torch.full((int(offs[-1]),), -5, dtype=torch.int32, device="cuda")
    child, bir, parents, built = ctx.grow_level(parent_hist, splits_dev(torch, sp),
                                                torch.from_numpy(np.ascontiguousarray(rows, dtype=np.int32)).cuda(),
                                                offs, out, child_hist, child_sp, w.lam, w.gamma)
    ctx.sync()
    assert child.tolist() == [0] and bir.size == 0 and parents.size == 0 and built == 0
    assert (child_hist.cpu().numpy() == -9).all() and (child_sp.cpu().numpy() == 7).all()
    ctx.close()


@pytest.mark.parametrize("fused", [True, False], ids=["one call per level", "three calls per level"])
def test_many_trees_on_one_context(hgb, torch, fused):
    """Twelve grown trees of eight levels on one context, queued without a
    wait between trees: the launch plans' staging slots are reused many
    times behind the library's stream markers, and the maxima and node
    records are read back through the sequence words (each level's records
    must be that level's, not the previous one's).  Every tree equals the
    first, level by level, and the first equals the oracle's."""
    say("many trees, one context", "fused" if fused else "apart")
    from histogram_gradient_boosted_amd import tree
    w = synth.make("c3", n_rows=200_000)
    ctx = hgb.Context(0)
    ctx.set_async_begin(True)
    ctx.upload_bins(w.bins, w.n_bins, w.has_missing)
    g = torch.from_numpy(w.grad).cuda()
    h = torch.from_numpy(w.hess).cuda()
    trees = [tree.grow_tree_device(ctx, g, h, w.depth, w.lam, w.gamma, sync=False, fused=fused) for _ in range(12)]
    ctx.sync()
    want = oracle_tree(w, w.depth, 30)
    first = trees[0]
    assert len(first) == len(want)
    for d, (lv, (rows, offs, hist, sp)) in enumerate(zip(first, want)):
        if d > 0:
            assert np.array_equal(lv.offsets.astype(np.int64), offs), f"level {d} offsets"
        assert np.array_equal(lv.hist.cpu().numpy(), hist), f"level {d} histograms differ"
        assert_splits(hgb.splits_to_numpy(lv.splits)[: lv.n_nodes], sp, f"level {d}")
    for t, levels in enumerate(trees[1:], 1):
        assert len(levels) == len(first), f"tree {t}"
        for d, (a, b) in enumerate(zip(first, levels)):
            assert a.n_nodes == b.n_nodes, f"tree {t} level {d}"
            if d > 0:
                assert np.array_equal(a.offsets, b.offsets), f"tree {t} level {d} offsets"
                assert torch.equal(a.rows[: int(a.offsets[-1])], b.rows[: int(b.offsets[-1])]), f"tree {t} level {d} rows"
            assert torch.equal(a.hist, b.hist), f"tree {t} level {d} histograms"
            assert torch.equal(a.splits, b.splits), f"tree {t} level {d} splits"
    ctx.close()


def test_two_contexts_on_two_streams(hgb, torch):
    """Two contexts, each on a stream of its own, grow trees of different
    matrices (one-byte bins, and two-byte bins with a missing slot and hot
    slots) with their work queued together on the device: each tree equals
    its oracle's, so nothing of one context (staging, scratch, sequence
    words, launch attributes) leaks into the other."""
    say("two contexts, two streams")
    from histogram_gradient_boosted_amd import tree
    wa = synth.make("c3", n_rows=150_000)
    wb = synth.make("c5", n_rows=60_000)
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    ca, cb = hgb.Context(0, sa), hgb.Context(0, sb)
    ca.set_async_begin(True)
    cb.set_async_begin(True)
    ga, ha = torch.from_numpy(wa.grad).cuda(), torch.from_numpy(wa.hess).cuda()
    gb, hb = torch.from_numpy(wb.grad).cuda(), torch.from_numpy(wb.hess).cuda()
    torch.cuda.synchronize()
    ca.upload_bins(wa.bins, wa.n_bins, wa.has_missing)
    cb.upload_bins(wb.bins, wb.n_bins, wb.has_missing)
    got = {"a": [], "b": []}
    for _ in range(3):   # alternate whole trees: each queues behind the other's on the device
        with torch.cuda.stream(sa):
            got["a"].append(tree.grow_tree_device(ca, ga, ha, 6, wa.lam, wa.gamma, sync=False))
        with torch.cuda.stream(sb):
            got["b"].append(tree.grow_tree_device(cb, gb, hb, 6, wb.lam, wb.gamma, sync=False))
    ca.sync()
    cb.sync()
    for key, w in (("a", wa), ("b", wb)):
        want = oracle_tree(w, 6, 30)
        for t, levels in enumerate(got[key]):
            assert len(levels) == len(want), f"{key} tree {t}"
            for d, (lv, (rows, offs, hist, sp)) in enumerate(zip(levels, want)):
                if d > 0:
                    assert np.array_equal(lv.offsets.astype(np.int64), offs), f"{key} tree {t} level {d} offsets"
                assert np.array_equal(lv.hist.cpu().numpy(), hist), f"{key} tree {t} level {d} histograms"
                assert_splits(hgb.splits_to_numpy(lv.splits)[: lv.n_nodes], sp, f"{key} tree {t} level {d}")
    ca.close()
    cb.close()


def test_grow_level_errors(hgb, torch):
    """hgb_grow_level's own checks, through the C ABI: null outputs and a
    parent count outside [1, 32767] are HGB_E_INVALID, before any work."""
    say("grow level errors")
    import ctypes
    w = synth.random_small(72, 2_000, 2, 8, False, 0)
    ctx = hgb.Context(0)
    ctx.upload_bins(w.bins, w.n_bins, w.has_missing)
    g = torch.from_numpy(w.grad).cuda()
    h = torch.from_numpy(w.hess).cuda()
    ctx.begin_tree(g, h)
    lib = hgb.load()
    F, S = w.n_features, w.n_slots
    ph = torch.zeros((1, F, S, 2), dtype=torch.int64, device="cuda")
    ps = torch.zeros(hgb.SPLIT_BYTES, dtype=torch.uint8, device="cuda")
    cr = torch.zeros(w.n_rows, dtype=torch.int32, device="cuda")
    ch = torch.zeros((2, F, S, 2), dtype=torch.int64, device="cuda")
    cs = torch.zeros(3 * hgb.SPLIT_BYTES, dtype=torch.uint8, device="cuda")
    offs = np.zeros(3, dtype=np.int32)
    bir = np.zeros(1, dtype=np.uint8)
    nc = ctypes.c_int32(0)
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    def call(n_parents, hist_out=True):
        return lib.hgb_grow_level(ctx._h, p(ph), p(ps), None, None, n_parents, p(cr),
                                  p(ch) if hist_out else None, p(cs), offs.ctypes.data_as(ctypes.c_void_p),
                                  ctypes.byref(nc), bir.ctypes.data_as(ctypes.c_void_p), None, None,
                                  ctypes.c_double(1.0), ctypes.c_double(0.0), 0)
    assert call(1, hist_out=False) == hgb.HGB_E_INVALID
    assert call(0) == hgb.HGB_E_INVALID
    assert call(32768) == hgb.HGB_E_INVALID
    ctx.sync()
    ctx.close()
