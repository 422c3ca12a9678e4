"""GPU parity of the device-resident objective (hgb_begin_tree_objective)
against the oracle: the fixed-point codes of every row and the scales must be
identical to quantizing the oracle's fp32 (g, h) of the same scores, labels and
weights."""
import numpy as np
import pytest

import oracle
from histogram_gradient_boosted_amd import synth

from test_gpu_parity import say

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


def oracle_codes(kind, m, y, w, bits):
    g, h = oracle.objective(kind, m, y, w)
    qg, kg = oracle.quantize(g, False, bits)
    qh, kh = oracle.quantize(h, True, bits)
    return np.stack([qg, qh], axis=1), kg, kh


def device_codes(hgb, torch, kind, m, y, w, bits, offset=0):
    """Run begin_tree_objective on device copies of (m, y, w).  offset > 0
    places the arrays `offset` floats into their allocations, which takes the
    kernels' unaligned (one row at a time) path."""
    n = m.shape[0]
    ctx = hgb.Context(0)
    ctx.set_precision(bits)
    ctx.upload_bins(np.zeros((1, n), dtype=np.uint8), 2, False)

    def dev(a):
        if a is None:
            return None
        t = torch.zeros(n + offset, dtype=torch.float32, device="cuda")
        t[offset:] = torch.from_numpy(a).cuda()
        return t[offset:]

    try:
        ctx.begin_tree_objective(kind, dev(m), dev(y), dev(w))
        q = ctx.copy_quantized().cpu().numpy()
        return q, ctx.get_scales()
    finally:
        ctx.close()


CASES = [
    # seed, n, kind, weighted, bits, offset
    (1, 1, "logistic", False, 30, 0), (2, 3, "squared", True, 30, 0),
    (3, 5, "poisson", False, 30, 1), (4, 1027, "logistic", True, 30, 0),
    (5, 1027, "squared", False, 19, 1), (6, 100_003, "poisson", True, 30, 0),
    (7, 300_000, "logistic", False, 30, 0), (8, 300_000, "logistic", True, 19, 2),
    (9, 262_147, "squared", True, 30, 3), (10, 262_144, "poisson", False, 19, 0),
]


@pytest.mark.parametrize("seed,n,kind,weighted,bits,offset", CASES)
def test_objective_codes_vs_oracle(hgb, torch, seed, n, kind, weighted, bits, offset):
    say("objective", seed, n, kind, weighted, bits, offset)
    m, y, w = synth.objective_inputs(seed, n, kind, weighted)
    want, kg, kh = oracle_codes(kind, m, y, w, bits)
    got, (gkg, gkh) = device_codes(hgb, torch, kind, m, y, w, bits, offset)
    assert (gkg, gkh) == (kg, kh)
    bad = np.nonzero((got != want).any(axis=1))[0]
    assert bad.size == 0, f"{bad.size} rows differ, first {bad[:5]}: m={m[bad[:5]]} y={y[bad[:5]]}"


def test_objective_extreme_scores(hgb, torch):
    """Scores where the logistic probability saturates (h = 0 exactly) or is
    tiny enough that h is an fp32 subnormal, and exp arguments past the
    clamp; at 8 bits the codes are small, at 30 they resolve the tiny values
    only when every hessian is tiny (the second half of the test)."""
    say("objective extremes")
    m = np.concatenate([np.linspace(-120, 120, 4001), [1e30, -1e30, 3e38, -3e38, 0.0, -0.0]]).astype(np.float32)
    y = (np.arange(m.size) % 2).astype(np.float32)
    for bits in (8, 30):
        want, kg, kh = oracle_codes("logistic", m, y, None, bits)
        got, scales = device_codes(hgb, torch, "logistic", m, y, None, bits)
        assert scales == (kg, kh)
        assert np.array_equal(got, want)
    # only tiny probabilities: max h is itself subnormal, so the scale and every
    # code depend on the subnormal fp32 results
    m2 = np.linspace(-103.9, -88.0, 1000).astype(np.float32)
    y2 = np.zeros_like(m2)
    want, kg, kh = oracle_codes("logistic", m2, y2, None, 30)
    got, scales = device_codes(hgb, torch, "logistic", m2, y2, None, 30)
    assert scales == (kg, kh)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("kind,m,y,w", [
    ("poisson", 100.0, 1.0, None),           # e^100 overflows fp32
    ("squared", np.nan, 0.0, None),
    ("logistic", 0.0, np.inf, None),
    ("squared", 1.0, 0.0, -1.0),             # negative weight: negative hessian
])
def test_objective_errors_match_oracle(hgb, torch, kind, m, y, w):
    say("objective error", kind, m, y, w)
    n = 1000
    mm = np.zeros(n, dtype=np.float32)
    yy = np.zeros(n, dtype=np.float32)
    ww = None if w is None else np.ones(n, dtype=np.float32)
    mm[617], yy[617] = m, y
    if ww is not None:
        ww[617] = w
    with pytest.raises(oracle.OracleError) as oe:
        oracle_codes(kind, mm, yy, ww, 30)
    assert oe.value.status == oracle.E_NONFINITE
    with pytest.raises(hgb.HGBError) as e:
        device_codes(hgb, torch, kind, mm, yy, ww, 30)
    assert e.value.status == hgb.HGB_E_NONFINITE


def test_objective_argument_errors(hgb, torch):
    say("objective arguments")
    ctx = hgb.Context(0)
    ctx.upload_bins(np.zeros((1, 8), dtype=np.uint8), 2, False)
    t = torch.zeros(8, dtype=torch.float32, device="cuda")
    with pytest.raises(hgb.HGBError) as e:
        ctx.begin_tree_objective(9, t, t)
    assert e.value.status == hgb.HGB_E_INVALID
    with pytest.raises(hgb.HGBError) as e:
        ctx.copy_quantized()
    assert e.value.status == hgb.HGB_E_STATE
    ctx.close()


@pytest.mark.parametrize("bits", [30, 19])
def test_c3_objective_full_size(hgb, torch, bits):
    """The c3 workload at full size (10M rows): logistic (g, h) derived on the
    device from the recipe's fp32 scores and labels; every row's codes, then
    the root histograms built from them, equal the oracle's."""
    say("c3 objective", bits)
    w = synth.make("c3")
    want, kg, kh = oracle_codes("logistic", w.margin, w.label, None, bits)
    ctx = hgb.Context(0)
    ctx.set_precision(bits)
    ctx.upload_bins(w.bins, w.n_bins, w.has_missing)
    ctx.begin_tree_objective("logistic", torch.from_numpy(w.margin).cuda(),
                             torch.from_numpy(w.label).cuda())
    assert ctx.get_scales() == (kg, kh)
    got = ctx.copy_quantized().cpu().numpy()
    assert np.array_equal(got, want)
    hist = torch.empty((1, w.n_features, w.n_slots, 2), dtype=torch.int64, device="cuda")
    ctx.build_level(hist)
    ctx.sync()
    # the root histogram's totals per feature are the sums of the codes
    h = hist.cpu().numpy()[0]
    assert (h[:, :, 0].sum(axis=1) == want[:, 0].astype(np.int64).sum()).all()
    assert (h[:, :, 1].sum(axis=1) == want[:, 1].astype(np.int64).sum()).all()
    sub = oracle.build_hist(w.bins[:3], w.n_bins, False, want[:, 0], want[:, 1])
    assert np.array_equal(h[:3], sub[0])
    ctx.close()


@pytest.mark.parametrize("n,grow", [(300_000, False), (300_000, True), (None, False)])
def test_c3_tree_from_objective(hgb, torch, n, grow):
    """A c3 tree started from the device objective, grown with the host
    partition (replayed plan, as the benchmark times it) or the device
    partition, equals the oracle's tree grown from the oracle's logistic
    (g, h); 300,000 rows, and the full 10,000,000."""
    import dataclasses
    from histogram_gradient_boosted_amd import tree
    from test_gpu_parity import assert_splits, oracle_tree
    say("c3 objective tree", n, grow)
    w = synth.make("c3", n_rows=n)
    g, h = oracle.objective("logistic", w.margin, w.label)
    want = oracle_tree(dataclasses.replace(w, grad=g, hess=h), w.depth)
    ctx = hgb.Context(0)
    ctx.upload_bins(w.bins, w.n_bins, w.has_missing)
    obj = tree.Objective("logistic", torch.from_numpy(w.margin).cuda(), torch.from_numpy(w.label).cuda())
    if grow:
        levels = tree.grow_tree_device(ctx, obj, None, w.depth, w.lam, w.gamma)
        got = [(lv.hist, lv.splits, lv.n_nodes) for lv in levels]
    else:
        plans = tree.plan_tree(ctx, w.bins, w.n_bins, obj, None, w.depth, w.lam, w.gamma)
        tree.replay_tree(ctx, plans, obj, None, w.lam, w.gamma)
        ctx.sync()
        got = [(lp.hist, lp.splits, lp.n_nodes) for lp in plans]
    assert len(got) == len(want)
    for d, ((hist, sp, nn), (_, _, whist, wsp)) in enumerate(zip(got, want)):
        assert np.array_equal(hist.cpu().numpy(), whist), f"level {d}"
        assert_splits(hgb.splits_to_numpy(sp)[:nn], wsp, f"level {d}")
    ctx.close()
