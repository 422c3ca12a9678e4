"""begin_tree without the host wait (hgb_set_async_begin): the same
histograms, scales and splits as the waiting form, on plain gradients and on
the device objective; a non-finite gradient or negative hessian reported by
the next sync (and by get_scales), once, and a later good tree unaffected."""
import sys

import numpy as np
import pytest

import oracle
from histogram_gradient_boosted_amd import synth

pytestmark = pytest.mark.gpu


def say(*a):
    print("[gpu-async]", *a, flush=True)
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


def level_pass(hgb, torch, w, asyn, objective=None):
    """Root and one level (build, fused subtract + split) of workload w;
    returns (root hist, child hist, split records, scales)."""
    L = w.level
    ctx = hgb.Context(0)
    ctx.set_async_begin(asyn)
    ctx.upload_bins(w.bins, w.n_bins, w.has_missing)
    if objective is None:
        ctx.begin_tree(torch.from_numpy(w.grad).cuda(), torch.from_numpy(w.hess).cuda())
    else:
        m, y = objective
        ctx.begin_tree_objective("logistic", torch.from_numpy(m).cuda(), torch.from_numpy(y).cuda())
    F, S, P = w.n_features, w.n_slots, L.n_pairs
    root = torch.empty((1, F, S, 2), dtype=torch.int64, device="cuda")
    ctx.build_level(root)
    par = torch.empty((P, F, S, 2), dtype=torch.int64, device="cuda")
    ctx.build_level(par, torch.from_numpy(L.parent_row_index).cuda(), L.parent_offsets.astype(np.int32))
    ch = torch.empty((2 * P, F, S, 2), dtype=torch.int64, device="cuda")
    ctx.build_level(ch, torch.from_numpy(L.built_row_index).cuda(), L.built_offsets.astype(np.int32),
                    L.built_slots)
    out = torch.empty(2 * P * hgb.SPLIT_BYTES, dtype=torch.uint8, device="cuda")
    ctx.subtract_find_splits(par, ch, L.built_is_right, w.lam, w.gamma, out)
    sp1 = torch.empty(hgb.SPLIT_BYTES, dtype=torch.uint8, device="cuda")
    ctx.find_splits(root, 1, w.lam, w.gamma, sp1)
    ctx.sync()
    scales = ctx.get_scales()
    res = (root.cpu().numpy(), ch.cpu().numpy(), out.cpu().numpy(), sp1.cpu().numpy(), scales)
    ctx.close()
    return res


@pytest.mark.parametrize("case", [(61, 60_000, 10, 256, False, 8), (62, 40_000, 6, 1024, True, 6)])
def test_async_equals_waiting(hgb, torch, case):
    w = synth.random_small(*case)
    say("case", case)
    a = level_pass(hgb, torch, w, False)
    b = level_pass(hgb, torch, w, True)
    for x, y in zip(a[:4], b[:4]):
        assert np.array_equal(x, y)
    assert a[4] == b[4]
    qg, kg = oracle.quantize(w.grad, False)
    qh, kh = oracle.quantize(w.hess, True)
    assert b[4] == (kg, kh)
    assert np.array_equal(b[0], oracle.build_hist(w.bins, w.n_bins, w.has_missing, qg, qh))


def test_async_objective_equals_waiting(hgb, torch):
    w = synth.random_small(63, 50_000, 8, 256, False, 4)
    m, y, _ = synth.objective_inputs(5, w.n_rows, "logistic")
    a = level_pass(hgb, torch, w, False, (m, y))
    b = level_pass(hgb, torch, w, True, (m, y))
    for x, z in zip(a[:4], b[:4]):
        assert np.array_equal(x, z)
    assert a[4] == b[4]


def test_async_nonfinite_reported_by_sync_once(hgb, torch):
    w = synth.random_small(64, 10_000, 4, 64, False, 0)
    ctx = hgb.Context(0)
    ctx.set_async_begin(True)
    ctx.upload_bins(w.bins, w.n_bins, w.has_missing)
    h = torch.from_numpy(w.hess).cuda()
    g = torch.from_numpy(w.grad).cuda()
    bad_g = g.clone()
    bad_g[777] = float("nan")
    ctx.begin_tree(bad_g, h)                      # returns at once
    t = torch.empty((1, 4, 64, 2), dtype=torch.int64, device="cuda")
    ctx.build_level(t)                            # enqueued behind it (meaningless sums)
    with pytest.raises(hgb.HGBError) as e:
        ctx.get_scales()
    assert e.value.status == hgb.HGB_E_NONFINITE
    with pytest.raises(hgb.HGBError) as e:
        ctx.sync()
    assert e.value.status == hgb.HGB_E_NONFINITE
    ctx.sync()                                    # reported once
    # a negative hessian, then a good tree before the next sync: the sync
    # reports the bad one, and the good tree's results stand
    bad_h = h.clone()
    bad_h[5] = -1e-3
    ctx.begin_tree(g, bad_h)
    ctx.begin_tree(g, h)
    ctx.build_level(t)
    with pytest.raises(hgb.HGBError) as e:
        ctx.sync()
    assert e.value.status == hgb.HGB_E_NONFINITE
    qg, kg = oracle.quantize(w.grad, False)
    qh, kh = oracle.quantize(w.hess, True)
    assert ctx.get_scales() == (kg, kh)
    assert np.array_equal(t.cpu().numpy(), oracle.build_hist(w.bins, w.n_bins, w.has_missing, qg, qh))
    # the waiting form again: the error comes back from begin_tree itself
    ctx.set_async_begin(False)
    with pytest.raises(hgb.HGBError) as e:
        ctx.begin_tree(bad_g, h)
    assert e.value.status == hgb.HGB_E_NONFINITE
    ctx.sync()
    ctx.close()


@pytest.mark.parametrize("asyn", [False, True])
def test_consecutive_trees_codes(hgb, torch, asyn):
    """Trees one after another on one context, with scales that repeat and
    that change (the max pass encodes the rows at the previous tree's scales
    and the quantize pass re-encodes them only when the scales differ): every
    tree's codes and root histogram equal the oracle's."""
    w = synth.random_small(65, 30_001, 5, 64, False, 0)
    ctx = hgb.Context(0)
    ctx.set_async_begin(asyn)
    ctx.upload_bins(w.bins, w.n_bins, w.has_missing)
    t = torch.empty((1, 5, 64, 2), dtype=torch.int64, device="cuda")
    q = torch.empty((w.n_rows, 2), dtype=torch.int32, device="cuda")
    plan = [(1.0, 1.0, 30), (1.0, 1.0, 30), (8.0, 1.0, 30), (8.0, 1.0, 30), (8.0, 0.25, 30),
            (8.0, 0.25, 20), (8.0, 0.25, 20), (1.0, 1.0, 30)]
    for i, (sg, sh, bits) in enumerate(plan):
        say("tree", i, sg, sh, bits)
        ctx.set_precision(bits)
        grad = (w.grad * np.float32(sg)).astype(np.float32)
        hess = (w.hess * np.float32(sh)).astype(np.float32)
        ctx.begin_tree(torch.from_numpy(grad).cuda(), torch.from_numpy(hess).cuda())
        ctx.copy_quantized(q)
        ctx.build_level(t)
        ctx.sync()
        qg, kg = oracle.quantize(grad, False, bits)
        qh, kh = oracle.quantize(hess, True, bits)
        assert ctx.get_scales() == (kg, kh)
        got = q.cpu().numpy()
        assert np.array_equal(got[:, 0], qg) and np.array_equal(got[:, 1], qh), f"tree {i}"
        assert np.array_equal(t.cpu().numpy(), oracle.build_hist(w.bins, w.n_bins, w.has_missing, qg, qh))
    ctx.close()


@pytest.mark.parametrize("asyn", [False, True])
def test_consecutive_objective_trees_codes(hgb, torch, asyn):
    """The same on the device objective, whose max pass writes the codes at
    the previous tree's scales: weighted squared and logistic trees whose
    scales repeat and change (weights x1, x1, x8, x8, logistic, logistic, P
    = 21); every tree's codes and root histogram equal the oracle's."""
    w = synth.random_small(66, 20_003, 4, 32, False, 0)
    m, y, _ = synth.objective_inputs(6, w.n_rows, "squared")
    ml, yl, _ = synth.objective_inputs(7, w.n_rows, "logistic")
    ones = np.ones(w.n_rows, np.float32)
    ctx = hgb.Context(0)
    ctx.set_async_begin(asyn)
    ctx.upload_bins(w.bins, w.n_bins, w.has_missing)
    t = torch.empty((1, 4, 32, 2), dtype=torch.int64, device="cuda")
    q = torch.empty((w.n_rows, 2), dtype=torch.int32, device="cuda")
    plan = [("squared", m, y, 1.0, 30), ("squared", m, y, 1.0, 30), ("squared", m, y, 8.0, 30),
            ("squared", m, y, 8.0, 30), ("logistic", ml, yl, 1.0, 30), ("logistic", ml, yl, 1.0, 30),
            ("logistic", ml, yl, 1.0, 21), ("squared", m, y, 1.0, 30)]
    for i, (kind, mm, yy, wt, bits) in enumerate(plan):
        say("objective tree", i, kind, wt, bits)
        ctx.set_precision(bits)
        wv = (ones * np.float32(wt)).astype(np.float32)
        ctx.begin_tree_objective(kind, torch.from_numpy(mm).cuda(), torch.from_numpy(yy).cuda(),
                                 torch.from_numpy(wv).cuda())
        ctx.copy_quantized(q)
        ctx.build_level(t)
        ctx.sync()
        g, h = oracle.objective(kind, mm, yy, wv)
        qg, kg = oracle.quantize(g, False, bits)
        qh, kh = oracle.quantize(h, True, bits)
        assert ctx.get_scales() == (kg, kh)
        got = q.cpu().numpy()
        assert np.array_equal(got[:, 0], qg) and np.array_equal(got[:, 1], qh), f"tree {i}"
        assert np.array_equal(t.cpu().numpy(), oracle.build_hist(w.bins, w.n_bins, w.has_missing, qg, qh))
    ctx.close()
