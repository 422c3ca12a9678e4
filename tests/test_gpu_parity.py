"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Histograms, split features, bins and directions must be bit-exact; gains are
held to 1e-6 relative (and, separately, checked for exact equality: both sides
evaluate the same fp64 expression with one rounding per operation).
"""
import math
import sys

import numpy as np
import pytest

import oracle
from histogram_gradient_boosted_amd import synth

pytestmark = pytest.mark.gpu

GAIN_RTOL = 1e-6


def say(*a):
    print("[gpu-parity]", *a, flush=True)
    sys.stdout.flush()


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


# ---------------------------------------------------------------- helpers ---

def oracle_quantized(w, bits=30):
    qg, kg = oracle.quantize(w.grad, False, bits)
    qh, kh = oracle.quantize(w.hess, True, bits)
    return qg, qh, kg, kh


def new_ctx(hgb, w, torch, bits=30):
    ctx = hgb.Context(0)
    ctx.set_precision(bits)
    ctx.upload_bins(w.bins, w.n_bins, w.has_missing)
    g = torch.from_numpy(w.grad).cuda()
    h = torch.from_numpy(w.hess).cuda()
    ctx.begin_tree(g, h)
    return ctx, g, h


def assert_splits(got, want, where=""):
    assert got.shape == want.shape, where
    for key in ("feature", "bin", "default_left", "g_left", "h_left", "g_total", "h_total", "pad"):
        bad = np.nonzero(got[key] != want[key])[0]
        assert bad.size == 0, f"{where} {key} differs at nodes {bad[:8]}: {got[key][bad[:4]]} vs {want[key][bad[:4]]}"
    gg, wg = got["gain"], want["gain"]
    both_inf = np.isneginf(gg) & np.isneginf(wg)
    fin = ~both_inf
    assert np.isfinite(gg[fin]).all() and np.isfinite(wg[fin]).all(), where
    rel = np.abs(gg[fin] - wg[fin]) / np.maximum(np.abs(wg[fin]), 1e-300)
    assert (rel <= GAIN_RTOL).all(), f"{where} gain rel err {rel.max()}"


def gpu_splits(hgb, ctx, hist_t, n_nodes, lam, gamma, torch):
    out = torch.empty(max(n_nodes, 1) * hgb.SPLIT_BYTES, dtype=torch.uint8, device="cuda")
    ctx.find_splits(hist_t, n_nodes, lam, gamma, out)
    ctx.sync()
    return hgb.splits_to_numpy(out)[:n_nodes]


def run_level_both(hgb, torch, w, check_exact_gain=False, bits=30, fused=False):
    """Parents + built children + subtraction + splits on the GPU vs the oracle
    (fused: subtraction and splits through subtract_find_splits)."""
    L = w.level
    ctx, g, h = new_ctx(hgb, w, torch, bits)
    qg, qh, kg, kh = oracle_quantized(w, bits)
    assert ctx.get_scales() == (kg, kh)
    F, S = w.n_features, w.n_slots
    P = L.n_pairs
    dev = torch.device("cuda")
    par_t = torch.empty((P, F, S, 2), dtype=torch.int64, device=dev)
    ctx.build_level(par_t, torch.from_numpy(L.parent_row_index).to(dev),
                    L.parent_offsets.astype(np.int32))
    ch_t = torch.empty((2 * P, F, S, 2), dtype=torch.int64, device=dev)
    ch_t.fill_(-7)   # poison: every slot must be written
    ctx.build_level(ch_t, torch.from_numpy(L.built_row_index).to(dev),
                    L.built_offsets.astype(np.int32), L.built_slots)
    if fused:
        out = torch.empty(2 * P * hgb.SPLIT_BYTES, dtype=torch.uint8, device=dev)
        ctx.subtract_find_splits(par_t, ch_t, L.built_is_right, w.lam, w.gamma, out)
        ctx.sync()
        sp = hgb.splits_to_numpy(out)[: 2 * P]
    else:
        ctx.subtract_siblings(par_t, ch_t, L.built_is_right)
        sp = gpu_splits(hgb, ctx, ch_t, 2 * P, w.lam, w.gamma, torch)
    got_par = par_t.cpu().numpy()
    got_ch = ch_t.cpu().numpy()
    ctx.close()

    want_par = oracle.build_hist(w.bins, w.n_bins, w.has_missing, qg, qh,
                                 L.parent_row_index, L.parent_offsets)
    want_ch = oracle.build_hist(w.bins, w.n_bins, w.has_missing, qg, qh,
                                L.children_row_index, L.children_offsets)
    want_sp = oracle.find_splits(want_ch, w.n_bins, w.has_missing, kg, kh, w.lam, w.gamma)
    assert np.array_equal(got_par, want_par), "parent histograms differ"
    assert np.array_equal(got_ch, want_ch), "child histograms differ"
    assert_splits(sp, want_sp, w.name)
    if check_exact_gain:
        assert np.array_equal(sp["gain"].view(np.int64), want_sp["gain"].view(np.int64))
    return sp


def run_root_both(hgb, torch, w, bits=30):
    ctx, g, h = new_ctx(hgb, w, torch, bits)
    qg, qh, kg, kh = oracle_quantized(w, bits)
    assert ctx.get_scales() == (kg, kh)
    t = torch.full((1, w.n_features, w.n_slots, 2), -3, dtype=torch.int64, device="cuda")
    ctx.build_level(t)
    sp = gpu_splits(hgb, ctx, t, 1, w.lam, w.gamma, torch)
    got = t.cpu().numpy()
    ctx.close()
    want = oracle.build_hist(w.bins, w.n_bins, w.has_missing, qg, qh)
    assert np.array_equal(got, want), "root histogram differs"
    want_sp = oracle.find_splits(want, w.n_bins, w.has_missing, kg, kh, w.lam, w.gamma)
    assert_splits(sp, want_sp, w.name)
    assert np.array_equal(sp["gain"].view(np.int64), want_sp["gain"].view(np.int64))
    return sp


# ------------------------------------------------------------------ tests ---

def test_quantization_one_row_per_bin(hgb, torch):
    """Each row alone in its own bin: every cell is that row's (qg, qh)."""
    say("quantization one row per bin")
    rng = np.random.default_rng(1)
    n = 256
    step = 2.0 ** -29
    g = rng.standard_normal(n).astype(np.float32) * 0.5
    g[0] = 1.0                                            # M = 1 -> k = 29
    g[1:9] = np.array([0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 3.5, 1e-38]) * step
    h = rng.uniform(0, 1, n).astype(np.float32)
    h[3] = -0.0
    h[4] = 0.0
    bins = np.arange(n, dtype=np.uint8)[None, :].copy()
    w = synth.Workload("q", bins, 256, False, g, h)
    ctx, _, _ = new_ctx(hgb, w, torch)
    t = torch.empty((1, 1, 256, 2), dtype=torch.int64, device="cuda")
    ctx.build_level(t)
    got = t.cpu().numpy()[0, 0]
    qg, kg = oracle.quantize(g, False)
    qh, kh = oracle.quantize(h, True)
    assert ctx.get_scales() == (kg, kh)
    ctx.close()
    assert np.array_equal(got[:, 0], qg.astype(np.int64))
    assert np.array_equal(got[:, 1], qh.astype(np.int64))


SMALL = [
    # seed, n, F, B, missing, children, u16
    (0, 17, 1, 2, False, 0, None), (1, 64, 3, 8, False, 0, None), (2, 64, 3, 8, True, 0, None),
    (3, 50, 2, 5, False, 4, None), (4, 63, 3, 7, True, 6, None), (5, 1, 2, 3, True, 2, None),
    (6, 40, 3, 8, False, 8, None), (7, 64, 3, 4, True, 2, None), (8, 1000, 5, 300, True, 6, True),
    (9, 3000, 7, 255, True, 10, False), (10, 5000, 20, 256, False, 16, False),
    (11, 777, 3, 1024, True, 4, True), (12, 9, 1, 4095, True, 2, True),
]


@pytest.mark.parametrize("seed,n,F,B,missing,children,u16", SMALL)
@pytest.mark.parametrize("wide,bits", [(False, 30), (True, 30), (False, 19), (True, 12)])
def test_small_random(hgb, torch, seed, n, F, B, missing, children, u16, wide, bits):
    say("small", seed, n, F, B, missing, children, u16, wide, bits)
    w = synth.random_small(seed, n, F, B, missing, children, wide_grad=wide, u16=u16)
    if children == 0:
        run_root_both(hgb, torch, w, bits)
    else:
        run_level_both(hgb, torch, w, check_exact_gain=True, bits=bits)


@pytest.mark.parametrize("name,n,F", [("c2", 300_000, 100), ("c5", 300_000, 50),
                                      ("c4", 8_192, 1_024), ("c1", None, None)])
def test_packed_precision_configs(hgb, torch, name, n, F):
    """Precision 19 selects packed (g, h) accumulation in the root fill, and
    in the level fills where no wide plan with lane pairs fits (the 2-byte,
    1,025-slot matrix)."""
    say("packed", name, n, F)
    w = synth.make(name, n_rows=n, n_features=F)
    if w.level is not None:
        run_level_both(hgb, torch, w, check_exact_gain=True, bits=19)
    if w.kind in ("root", "root+level"):
        run_root_both(hgb, torch, w, bits=19)


@pytest.mark.parametrize("case", ["small8", "small9", "small10", "small11", "small12", "c2", "c5", "c4"])
def test_subtract_find_splits(hgb, torch, case):
    """The fused level tail equals subtract_siblings + find_splits (the oracle's
    subtraction and scan); small12's 4,095 bins take the two-pass fallback."""
    say("fused tail", case)
    if case.startswith("small"):
        row = [r for r in SMALL if r[0] == int(case[5:])][0]
        seed, n, F, B, missing, children, u16 = row
        w = synth.random_small(seed, n, F, B, missing, children, u16=u16)
    elif case == "c4":
        w = synth.make("c4", n_rows=8_192, n_features=1_024)
    else:
        w = synth.make(case, n_rows=200_000)
    run_level_both(hgb, torch, w, check_exact_gain=True, fused=True)


@pytest.mark.parametrize("F,B,missing,fused", [(17, 64, True, True), (32, 255, False, True),
                                               (33, 64, True, True), (32, 1024, True, True),
                                               (31, 100, True, False), (33, 100, False, False)])
def test_split_feature_counts(hgb, torch, F, B, missing, fused):
    """Feature counts around a wave block's width (4 features per block of the
    split grid), lane slot counts 1, 2, 4 and 16, with and without missing
    values, through the fused tail and the two-pass path."""
    say("split block boundary", F, B, missing, fused)
    w = synth.random_small(90 + F, 30_000, F, B, missing, 10, u16=B > 255)
    run_level_both(hgb, torch, w, check_exact_gain=True, fused=fused)


@pytest.mark.parametrize("F,n_const", [(16_400, 0), (16_400, 16_000), (200, 0), (200, 150), (256, 255)])
def test_split_reduce_wide_ties(hgb, torch, F, n_const):
    """F identical features, so the root's per-feature winners all tie on
    gain: the smallest feature wins.  16,400 features run the node's
    reduction on 1,024 threads with several entries each; 200 and 256
    features (50 and 64 entries of four features) run it on one wave with
    lane exchanges.  With the first n_const features made constant (no valid
    split) the first of the others wins (256 and 255: only the last lane's
    entry is valid)."""
    say("split reduce ties", F, n_const)
    rng = np.random.default_rng(77)
    n = 2048
    col = rng.integers(0, 256, n).astype(np.uint8)
    bins = np.tile(col, (F, 1))
    bins[:n_const] = 7
    g = rng.standard_normal(n).astype(np.float32)
    h = rng.uniform(0.1, 1.0, n).astype(np.float32)
    sp = run_root_both(hgb, torch, synth.Workload("ties", bins, 256, False, g, h, kind="root"))
    assert int(sp["feature"][0]) == n_const


@pytest.mark.parametrize("B", [32, 600])
def test_split_calls_in_a_row(hgb, torch, B):
    """One context, its split scratch reused across calls: find_splits and
    subtract_find_splits over node counts that grow and shrink (3,000, 1,000,
    3,000 nodes; 1,500 then 200 pairs), each against the oracle.  600 bins
    take the sliced scan (one block per feature)."""
    say("split calls in a row", B)
    rng = np.random.default_rng(B)
    n, F, N = 40_000, 6, 3_000
    w = synth.random_small(7 + B, n, F, B, True, 0, u16=B > 255)
    node = rng.integers(0, N, n)
    ri = np.argsort(node, kind="stable").astype(np.int32)
    offs = np.concatenate([[0], np.cumsum(np.bincount(node, minlength=N))]).astype(np.int64)
    qg, qh, kg, kh = oracle_quantized(w)
    hist = oracle.build_hist(w.bins, w.n_bins, w.has_missing, qg, qh, ri, offs)
    ctx, g, h = new_ctx(hgb, w, torch)
    hist_t = torch.from_numpy(hist).cuda()
    for m in (N, 1_000, N):
        sp = gpu_splits(hgb, ctx, hist_t, m, w.lam, w.gamma, torch)
        want = oracle.find_splits(hist[:m], w.n_bins, w.has_missing, kg, kh, w.lam, w.gamma)
        assert_splits(sp, want, f"find_splits {m} nodes")
    for P in (1_500, 200):
        parent = hist[:P] + hist[P:2 * P]   # pair i's parent: nodes i and P + i together
        child = np.empty((2 * P,) + hist.shape[1:], dtype=np.int64)
        bir = rng.integers(0, 2, P).astype(np.uint8)
        for i in range(P):
            child[2 * i + int(bir[i])] = hist[i]
        ch_t = torch.from_numpy(child).cuda()
        out = torch.empty(2 * P * hgb.SPLIT_BYTES, dtype=torch.uint8, device="cuda")
        ctx.subtract_find_splits(torch.from_numpy(parent).cuda(), ch_t, bir, w.lam, w.gamma, out)
        ctx.sync()
        sp = hgb.splits_to_numpy(out)[: 2 * P]
        want_ch = oracle.subtract(parent, child.copy(), bir)
        assert np.array_equal(ch_t.cpu().numpy(), want_ch), f"{P} pairs: children differ"
        want = oracle.find_splits(want_ch, w.n_bins, w.has_missing, kg, kh, w.lam, w.gamma)
        assert_splits(sp, want, f"subtract_find_splits {P} pairs")
    ctx.close()


def test_c1_full(hgb, torch):
    say("c1 full")
    run_root_both(hgb, torch, synth.make("c1"))


@pytest.mark.parametrize("n,F", [(200_000, 100), (None, None)])
def test_c2(hgb, torch, n, F):
    say("c2", n, F)
    run_level_both(hgb, torch, synth.make("c2", n_rows=n, n_features=F), check_exact_gain=True)


@pytest.mark.parametrize("n,F", [(200_000, 50), (None, None)])
def test_c5(hgb, torch, n, F):
    say("c5", n, F)
    run_level_both(hgb, torch, synth.make("c5", n_rows=n, n_features=F), check_exact_gain=True)


@pytest.mark.parametrize("n,F,bits", [(8_192, 2_048, 30), (None, None, 30), (None, None, 19)])
def test_c4(hgb, torch, n, F, bits):
    """131,072 x 16,384 (and a slice of it): the root and the level of 8
    nodes; at P = 19 the root takes the packed interleaved tile."""
    say("c4", n, F, bits)
    w = synth.make("c4", n_rows=n, n_features=F)
    run_root_both(hgb, torch, w, bits=bits)
    run_level_both(hgb, torch, w, check_exact_gain=True, bits=bits)


@pytest.mark.parametrize("missing,bits", [(True, 30), (False, 19)])
def test_feature_major_levels(hgb, torch, missing, bits):
    """Rows wider than the row-major copy's limit (64 KiB: here 33,000 u16
    features) are filled from the feature-major matrix."""
    F, u16 = 33_000, True
    say("feature-major levels", F, missing, u16, bits)
    w = synth.random_small(44, 1_200, F, 256, missing, 6, u16=u16)
    run_level_both(hgb, torch, w, check_exact_gain=True, bits=bits)


def with_hot_slots(w, seed):
    """The workload with hot slots planted: feature 0 constant, feature 1 with
    90% of rows in bin 0, feature 2 with 90% in the last value bin, and (with
    missing values) feature 3 with 60% missing -- so that the fills skip each
    feature's most frequent slot and recover its cell by subtraction."""
    import dataclasses
    rng = np.random.default_rng(seed)
    b = w.bins.copy()
    n = b.shape[1]
    b[0, :] = 3 % w.n_bins
    b[1, rng.random(n) < 0.9] = 0
    b[2, rng.random(n) < 0.9] = w.n_bins - 1
    if w.has_missing and b.shape[0] > 3:
        b[3, rng.random(n) < 0.6] = w.n_bins
    return dataclasses.replace(w, bins=b)


@pytest.mark.parametrize("case", ["rows_u8", "rows_u16", "cols_u16"])
@pytest.mark.parametrize("bits", [30, 19])
def test_hot_slots(hgb, torch, case, bits):
    """Matrices with hot slots (constant, skewed and mostly-missing features):
    root and level histograms and splits equal the oracle's, through the
    row-major fill (u8 and u16) and the feature-major fill."""
    say("hot slots", case, bits)
    if case == "rows_u8":
        w = synth.random_small(120, 40_000, 6, 16, True, 8)
    elif case == "rows_u16":
        w = synth.random_small(121, 30_000, 5, 1024, True, 6, u16=True)
    else:
        w = synth.random_small(122, 1_200, 33_000, 64, True, 6, u16=True)
    w = with_hot_slots(w, 7)
    run_level_both(hgb, torch, w, check_exact_gain=True, bits=bits)
    if case != "cols_u16":
        run_root_both(hgb, torch, w, bits=bits)


def oracle_tree(w, depth, bits=30):
    qg, qh, kg, kh = oracle_quantized(w, bits)
    levels = []
    hist = oracle.build_hist(w.bins, w.n_bins, w.has_missing, qg, qh)
    sp = oracle.find_splits(hist, w.n_bins, w.has_missing, kg, kh, w.lam, w.gamma)
    levels.append((None, None, hist, sp))
    rows, offs = None, None
    for _ in range(1, depth):
        rows, offs = oracle.partition(w.bins, w.n_bins, rows, offs, sp)
        if len(offs) == 1:
            break
        hist = oracle.build_hist(w.bins, w.n_bins, w.has_missing, qg, qh, rows, offs)
        sp = oracle.find_splits(hist, w.n_bins, w.has_missing, kg, kh, w.lam, w.gamma)
        levels.append((rows, offs, hist, sp))
    return levels


@pytest.mark.parametrize("n,bits", [(300_000, 30), (None, 30), (300_000, 19), (None, 19)])
def test_c3_tree(hgb, torch, n, bits):
    say("c3 tree", n, bits)
    from histogram_gradient_boosted_amd import tree
    w = synth.make("c3", n_rows=n)
    ctx = hgb.Context(0)
    ctx.set_precision(bits)
    ctx.upload_bins(w.bins, w.n_bins, w.has_missing)
    g = torch.from_numpy(w.grad).cuda()
    h = torch.from_numpy(w.hess).cuda()
    plans = tree.plan_tree(ctx, w.bins, w.n_bins, g, h, w.depth, w.lam, w.gamma)
    want = oracle_tree(w, w.depth, bits)
    assert len(plans) == len(want) == 8
    for d, (plan, (rows, offs, hist, sp)) in enumerate(zip(plans, want)):
        say("c3 level", d)
        if d > 0:
            assert np.array_equal(plan.children_offsets, offs)
            assert np.array_equal(plan.children_rows, rows)
        got = plan.hist.cpu().numpy()[: plan.n_nodes]
        assert np.array_equal(got, hist), f"level {d} histograms differ"
        assert_splits(hgb.splits_to_numpy(plan.splits)[: plan.n_nodes], sp, f"level {d}")
    ctx.close()


def test_run_to_run_identity(hgb, torch):
    say("run-to-run identity")
    w = synth.make("c2", n_rows=300_000, n_features=40)
    L = w.level
    ctx, g, h = new_ctx(hgb, w, torch)
    outs = []
    for _ in range(3):
        t = torch.empty((2 * L.n_pairs, w.n_features, w.n_slots, 2), dtype=torch.int64, device="cuda")
        ctx.build_level(t, torch.from_numpy(L.children_row_index).cuda(),
                        L.children_offsets.astype(np.int32))
        outs.append(t.cpu().numpy())
    ctx.close()
    assert all(np.array_equal(outs[0], o) for o in outs[1:])


def test_ragged_and_empty_nodes(hgb, torch):
    say("ragged nodes")
    w = synth.random_small(40, 70_001, 9, 256, False, 0)
    rng = np.random.default_rng(3)
    # nodes of sizes 0, 1, 2, 511, 512, 513, 4097, rest; rows shuffled within nodes
    sizes = [0, 1, 2, 511, 512, 513, 4097]
    sizes.append(w.n_rows - sum(sizes))
    perm = rng.permutation(w.n_rows).astype(np.int32)
    offs = np.zeros(len(sizes) + 1, dtype=np.int64)
    np.cumsum(sizes, out=offs[1:])
    ctx, g, h = new_ctx(hgb, w, torch)
    t = torch.full((len(sizes), 9, 256, 2), 5, dtype=torch.int64, device="cuda")
    ctx.build_level(t, torch.from_numpy(perm).cuda(), offs.astype(np.int32))
    ctx.sync()
    got = t.cpu().numpy()
    ctx.close()
    qg, qh, _, _ = oracle_quantized(w)
    want = oracle.build_hist(w.bins, 256, False, qg, qh, perm, offs)
    assert np.array_equal(got, want)
    assert not got[0].any()


def test_out_slots_scattered(hgb, torch):
    say("scattered output slots")
    w = synth.random_small(41, 20_000, 4, 64, True, 6)
    L = w.level
    ctx, g, h = new_ctx(hgb, w, torch)
    slots = np.array([5, 0, 3, 1, 4, 2], dtype=np.int32)
    t = torch.empty((6, 4, 65, 2), dtype=torch.int64, device="cuda")
    ctx.build_level(t, torch.from_numpy(L.children_row_index).cuda(),
                    L.children_offsets.astype(np.int32), slots)
    ctx.sync()
    got = t.cpu().numpy()
    ctx.close()
    qg, qh, _, _ = oracle_quantized(w)
    want = oracle.build_hist(w.bins, 64, True, qg, qh, L.children_row_index, L.children_offsets)
    assert np.array_equal(got[slots], want)


@pytest.mark.parametrize("n_pairs", [1, 256, 257, 600])
def test_subtract_plan_sizes(hgb, torch, n_pairs):
    """Small plans travel in the kernel's arguments, larger ones are uploaded:
    both against the oracle's subtraction, with parents taken out of order."""
    say("subtract plan sizes", n_pairs)
    w = synth.random_small(43, 1_000, 3, 16, False, 0)
    F, S = w.n_features, w.n_slots
    rng = np.random.default_rng(n_pairs)
    parent = rng.integers(-2**40, 2**40, size=(n_pairs + 3, F, S, 2), dtype=np.int64)
    child = rng.integers(-2**40, 2**40, size=(2 * n_pairs, F, S, 2), dtype=np.int64)
    bir = rng.integers(0, 2, size=n_pairs).astype(np.uint8)
    pslot = rng.permutation(n_pairs + 3)[:n_pairs].astype(np.int32)
    ctx = hgb.Context(0)
    ctx.upload_bins(w.bins, w.n_bins, w.has_missing)
    par_t = torch.from_numpy(parent).cuda()
    ch_t = torch.from_numpy(child).cuda()
    ctx.subtract_siblings(par_t, ch_t, bir, pslot)
    ctx.sync()
    got = ch_t.cpu().numpy()
    ctx.close()
    want = oracle.subtract(parent[pslot], child.copy(), bir)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("n_pairs", [1, 300])
def test_subtract_five_argument_form(hgb, torch, n_pairs):
    """hgb_subtract_siblings called with exactly the five arguments of its
    prototype (ctypes, no wrapper): pair i's parent is slot i.  Against the
    oracle's subtraction."""
    import ctypes
    say("five-argument subtract", n_pairs)
    w = synth.random_small(44, 1_000, 3, 16, True, 0)
    F, S = w.n_features, w.n_slots
    rng = np.random.default_rng(100 + n_pairs)
    parent = rng.integers(-2**40, 2**40, size=(n_pairs, F, S, 2), dtype=np.int64)
    child = rng.integers(-2**40, 2**40, size=(2 * n_pairs, F, S, 2), dtype=np.int64)
    bir = rng.integers(0, 2, size=n_pairs).astype(np.uint8)
    ctx = hgb.Context(0)
    ctx.upload_bins(w.bins, w.n_bins, w.has_missing)
    par_t = torch.from_numpy(parent).cuda()
    ch_t = torch.from_numpy(child).cuda()
    lib = hgb.load()
    st = lib.hgb_subtract_siblings(ctx._h, ctypes.c_void_p(par_t.data_ptr()), ctypes.c_void_p(ch_t.data_ptr()),
                                   bir.ctypes.data_as(ctypes.c_void_p), ctypes.c_int32(n_pairs))
    assert st == hgb.HGB_OK
    ctx.sync()
    got = ch_t.cpu().numpy()
    ctx.close()
    want = oracle.subtract(parent, child.copy(), bir)
    assert np.array_equal(got, want)


# ----------------------------------------------------------------- errors ---

def test_error_paths(hgb, torch):
    say("error paths")
    E = hgb
    ctx = hgb.Context(0)
    t = torch.empty((1, 2, 4, 2), dtype=torch.int64, device="cuda")
    with pytest.raises(hgb.HGBError) as e:
        ctx._check(ctx._lib.hgb_begin_tree(ctx._h, None, None), "begin_tree")
    assert e.value.status == E.HGB_E_STATE
    bins = np.array([[0, 1, 2, 3], [3, 2, 1, 0]], dtype=np.uint8)
    with pytest.raises(hgb.HGBError) as e:
        ctx.upload_bins(bins, 3, False)         # value 3 is not a slot
    assert e.value.status == E.HGB_E_INVALID
    with pytest.raises(hgb.HGBError) as e:
        ctx.upload_bins(np.zeros((1, 4), np.uint16), 5000, True)
    assert e.value.status == E.HGB_E_UNSUPPORTED
    ctx.upload_bins(bins, 4, False)
    with pytest.raises(hgb.HGBError) as e:
        ctx.build_level(t)                      # before begin_tree
    assert e.value.status == E.HGB_E_STATE
    g = torch.tensor([1.0, float("nan"), 0.0, 1.0], device="cuda")
    h = torch.ones(4, device="cuda")
    with pytest.raises(hgb.HGBError) as e:
        ctx.begin_tree(g, h)
    assert e.value.status == E.HGB_E_NONFINITE
    g = torch.ones(4, device="cuda")
    with pytest.raises(hgb.HGBError) as e:
        ctx.begin_tree(g, torch.tensor([1.0, -1e-30, 0.0, 1.0], device="cuda"))
    assert e.value.status == E.HGB_E_NONFINITE
    with pytest.raises(hgb.HGBError) as e:
        ctx.begin_tree(g, torch.tensor([1.0, float("inf"), 0.0, 1.0], device="cuda"))
    assert e.value.status == E.HGB_E_NONFINITE
    ctx.begin_tree(g, torch.tensor([1.0, -0.0, 0.0, 1.0], device="cuda"))
    ri = torch.tensor([0, 1, 2, 3], dtype=torch.int32, device="cuda")
    t2 = torch.empty((2, 2, 4, 2), dtype=torch.int64, device="cuda")
    with pytest.raises(hgb.HGBError) as e:
        ctx.build_level(t2, ri, np.array([0, 3, 2], np.int32))   # decreasing
    assert e.value.status == E.HGB_E_INVALID
    with pytest.raises(hgb.HGBError) as e:
        ctx.build_level(t2, ri, np.array([1, 3, 4], np.int32))   # not starting at 0
    assert e.value.status == E.HGB_E_INVALID
    with pytest.raises(hgb.HGBError) as e:
        ctx.build_level(t2, ri, np.array([0, 2, 4], np.int32), np.array([1, 1], np.int32))
    assert e.value.status == E.HGB_E_INVALID
    out = torch.empty(56, dtype=torch.uint8, device="cuda")
    with pytest.raises(hgb.HGBError) as e:
        ctx.find_splits(t, 1, -1.0, 0.0, out)
    assert e.value.status == E.HGB_E_INVALID
    with pytest.raises(hgb.HGBError) as e:
        ctx.find_splits(t, 1, float("nan"), 0.0, out)
    assert e.value.status == E.HGB_E_INVALID
    # a row index outside [0, n) is skipped on the device and reported by sync
    bad = torch.tensor([0, 7, -1, 3], dtype=torch.int32, device="cuda")
    ctx.build_level(t, bad, np.array([0, 4], np.int32))
    with pytest.raises(hgb.HGBError) as e:
        ctx.sync()
    assert e.value.status == E.HGB_E_INVALID
    ctx.sync()      # flag cleared
    got = t.cpu().numpy()[0]
    assert got[0, 0, 0] == 2 ** 29 and got[0, 3, 0] == 2 ** 29   # rows 0 and 3 only
    # binding-level size checks never reach a kernel
    with pytest.raises(ValueError):
        ctx.build_level(torch.empty(3, dtype=torch.int64, device="cuda"))
    ctx.close()


def test_unaligned_gradient_views(hgb, torch):
    """Gradient tensors that start 4 bytes into an allocation take the scalar path."""
    say("unaligned gradients")
    w = synth.random_small(50, 10_003, 3, 64, False, 0)
    big_g = torch.zeros(w.n_rows + 1, dtype=torch.float32, device="cuda")
    big_h = torch.zeros(w.n_rows + 1, dtype=torch.float32, device="cuda")
    big_g[1:] = torch.from_numpy(w.grad).cuda()
    big_h[1:] = torch.from_numpy(w.hess).cuda()
    ctx = hgb.Context(0)
    ctx.upload_bins(w.bins, w.n_bins, w.has_missing)
    ctx.begin_tree(big_g[1:], big_h[1:])
    t = torch.empty((1, 3, 64, 2), dtype=torch.int64, device="cuda")
    ctx.build_level(t)
    ctx.sync()
    got = t.cpu().numpy()
    qg, qh, kg, kh = oracle_quantized(w)
    assert ctx.get_scales() == (kg, kh)
    ctx.close()
    assert np.array_equal(got, oracle.build_hist(w.bins, 64, False, qg, qh))


@pytest.mark.parametrize("B,missing", [(64, False), (255, True), (1024, True)])
def test_splits_unaligned_histograms(hgb, torch, B, missing):
    """A histogram buffer 8 bytes off a 16-byte boundary takes the scan that
    reads slots from memory; aligned ones keep a lane's slots in registers.
    Both against the oracle."""
    say("split alignment", B, missing)
    w = synth.random_small(51, 20_000, 5, B, missing, 6)
    L = w.level
    ctx, g, h = new_ctx(hgb, w, torch)
    qg, qh, kg, kh = oracle_quantized(w)
    N = 2 * L.n_pairs
    elems = N * w.n_features * w.n_slots * 2
    big = torch.zeros(elems + 2, dtype=torch.int64, device="cuda")
    want_h = oracle.build_hist(w.bins, w.n_bins, w.has_missing, qg, qh,
                               L.children_row_index, L.children_offsets)
    want = oracle.find_splits(want_h, w.n_bins, w.has_missing, kg, kh, w.lam, w.gamma)
    for off in (2, 1):   # 16-byte aligned, then 8 bytes off
        view = big[off:off + elems]
        view.copy_(torch.from_numpy(want_h.reshape(-1)).cuda())
        sp = gpu_splits(hgb, ctx, view, N, w.lam, w.gamma, torch)
        assert_splits(sp, want, f"offset {off}")
        assert np.array_equal(sp["gain"].view(np.int64), want["gain"].view(np.int64))
    ctx.close()
