"""The largest sizes the boundary takes.

Features: 65,535 (the most a 16-bit feature field holds), one-byte bins whose
rows fit the row-major copy (64 KiB) and two-byte bins with a missing slot
whose rows do not (the feature-major fills), root and a level, against the
oracle.

Slots: 4,096 per feature (4,096 value bins, or 4,095 and the missing slot).

Rows: n = 2^31 - 1 (the most an int32 row count holds), through upload,
begin_tree, the root fill, the split scan, the device partition and one
grown level, about 80 GB of device memory in all.  The inputs are patterns
whose exact histograms have closed forms, so nothing here walks two billion
rows on the host:

- feature 0 holds r mod 256, feature 1 holds (r div 256) mod 256 (u8, 256 bins);
- g = +1 when bit 15 of r is clear and -1 when it is set, h = 1: given as
  fp32 arrays, or derived on the device from the squared loss with score 0
  and label -g (g = m - y, h = 1).

Both maxima are 1, so the scale exponent is k = P - 1 = 29 at P = 30 and
every code is +-2^29.  Bit 15 of r is bit 7 of feature 1's bin, so the best
root split is feature 1 at bin 127, which separates the signs; the
partition's children are then the rows with bit 15 clear and set, each in
ascending order (a stable partition).  The expected split records come from
the oracle's scan of the closed-form histograms.
"""
import numpy as np
import pytest

import oracle

from histogram_gradient_boosted_amd import synth

from test_gpu_parity import assert_splits, run_level_both, run_root_both, say

N = 2**31 - 1
Q = 2**29        # the code of +-1 at k = 29
BINS = 256


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


@pytest.mark.gpu
@pytest.mark.parametrize("seed,n,B,missing,u16", [(90, 1200, 256, False, False), (91, 800, 300, True, True)])
def test_max_features(hgb, torch, seed, n, B, missing, u16):
    """65,535 features: the root, then four children built from their
    parents (parents, built children, subtraction, splits), bit-exact."""
    say("max features", seed, n, B, missing, u16)
    torch.cuda.empty_cache()
    w = synth.random_small(seed, n, 65535, B, missing, 0, u16=u16)
    run_root_both(hgb, torch, w)
    w = synth.random_small(seed, n, 65535, B, missing, 4, u16=u16)
    run_level_both(hgb, torch, w, check_exact_gain=True)
    torch.cuda.empty_cache()


@pytest.mark.gpu
@pytest.mark.parametrize("seed,n,F,B,missing", [(92, 50_000, 5, 4096, False), (93, 30_000, 40, 4095, True)])
@pytest.mark.parametrize("bits", [30, 19])
def test_max_slots(hgb, torch, seed, n, F, B, missing, bits):
    """4,096 slots per feature: the root and six children, bit-exact, with
    wide and packed sums."""
    say("max slots", seed, n, F, B, missing, bits)
    w = synth.random_small(seed, n, F, B, missing, 0, u16=True)
    run_root_both(hgb, torch, w, bits)
    w = synth.random_small(seed, n, F, B, missing, 6, u16=True)
    run_level_both(hgb, torch, w, check_exact_gain=True, bits=bits)


def zeros_among(m):
    """How many of j = 0 .. m-1 have bit 7 clear."""
    return (m // 256) * 128 + min(m % 256, 128)


def expected_histograms(n):
    """(root, right child): [F=2][256][2] int64 sums of (qg, qh) over rows
    0 .. n-1, and over those rows with bit 15 set (the right child).

    Feature 0, bin b: rows r = b + 256 j, j < m = ceil((n - b) / 256); bit 15
    of r is bit 7 of j.  Feature 1, bin b: per full cycle of 65,536 rows, 256
    rows; in the last partial cycle of n mod 65,536 rows, the rows from 256 b
    on, at most 256.  Bit 15 of those rows is bit 7 of b."""
    root = np.zeros((2, BINS, 2), dtype=object)
    right = np.zeros((2, BINS, 2), dtype=object)
    for b in range(BINS):
        m = (n - b + 255) // 256
        z = zeros_among(m)
        root[0, b] = ((z - (m - z)) * Q, m * Q)
        right[0, b] = (-(m - z) * Q, (m - z) * Q)
        cnt = (n // 65536) * 256 + max(0, min(256, n % 65536 - 256 * b))
        sign = 1 if b < 128 else -1
        root[1, b] = (sign * cnt * Q, cnt * Q)
        if b >= 128:
            right[1, b] = (-cnt * Q, cnt * Q)
    return root.astype(np.int64), right.astype(np.int64)


def test_closed_forms_small():
    """The closed forms against a direct count on a few small n (including a
    partial last cycle), so the large case rests on checked formulas."""
    for n in (1, 255, 256, 257, 40_000, 65_536, 65_537, 200_003):
        r = np.arange(n, dtype=np.int64)
        g = np.where((r >> 15) & 1, -1, 1) * Q
        root, right = expected_histograms(n)
        for f, v in ((0, r & 255), (1, (r >> 8) & 255)):
            assert np.array_equal(root[f, :, 1], np.bincount(v, minlength=BINS) * Q), (n, f)
            sg = np.zeros(BINS, dtype=np.int64)
            np.add.at(sg, v, g)
            assert np.array_equal(root[f, :, 0], sg), (n, f)
            on = ((r >> 15) & 1) == 1
            rg = np.zeros(BINS, dtype=np.int64)
            np.add.at(rg, v[on], g[on])
            assert np.array_equal(right[f, :, 0], rg), (n, f)
            assert np.array_equal(right[f, :, 1], np.bincount(v[on], minlength=BINS) * Q), (n, f)


def assert_ascending_with_bit15(torch, x, bit, first, last, count):
    """x holds `count` strictly increasing rows in [0, N), all with bit 15 =
    `bit`: since exactly `count` such rows exist, x is their sorted list."""
    assert x.numel() == count
    assert int(x[0]) == first and int(x[-1]) == last
    step = 1 << 28   # bounded temporaries
    for a in range(0, count, step):
        s = x[a: min(count, a + step + 1)]
        assert bool((s[1:] > s[:-1]).all()), f"not ascending in [{a}, {a + step}]"
        assert bool((((s >> 15) & 1) == bit).all()), f"a row of the wrong side in [{a}, {a + step}]"
        del s


@pytest.mark.gpu
@pytest.mark.timeout(300)
@pytest.mark.parametrize("source,oblivious", [("grad", False), ("squared", True)])
def test_max_rows_root_and_level(hgb, torch, source, oblivious):
    """Root and one level; the second case grows the level as an oblivious
    tree (its records: the two children's, then the level's)."""
    torch.cuda.empty_cache()
    free, _ = torch.cuda.mem_get_info()
    if free < 100 * 2**30:
        pytest.skip(f"needs about 80 GB of device memory, {free / 2**30:.0f} GiB free")
    say("max rows: n = 2^31 - 1, two u8 features,", source)
    root_want, right_want = expected_histograms(N)
    left_want = root_want - right_want
    lam, gamma = 1.0, 0.0

    ar = torch.arange(N, dtype=torch.int32, device="cuda")
    bins = torch.empty((2, N), dtype=torch.uint8, device="cuda")
    bins[0] = (ar & 255).to(torch.uint8)
    bins[1] = ((ar >> 8) & 255).to(torch.uint8)
    g = ((ar >> 15) & 1).to(torch.float32).mul_(-2.0).add_(1.0)
    del ar
    if source == "grad":
        h = torch.ones(N, dtype=torch.float32, device="cuda")
    else:
        h = torch.zeros(N, dtype=torch.float32, device="cuda")   # the score
        g.neg_()                                                  # the label
    torch.cuda.synchronize()

    ctx = hgb.Context(0)
    try:
        ctx.upload_bins(bins, BINS, False)
        del bins
        if source == "grad":
            ctx.begin_tree(g, h)
        else:
            ctx.begin_tree_objective("squared", h, g)
        assert ctx.get_scales() == (29, 29)
        say("max rows: root fill")
        hist = torch.empty((1, 2, BINS, 2), dtype=torch.int64, device="cuda")
        ctx.build_level(hist)
        sp_root = torch.empty(hgb.SPLIT_BYTES, dtype=torch.uint8, device="cuda")
        ctx.find_splits(hist, 1, lam, gamma, sp_root)
        ctx.sync()
        assert np.array_equal(hist.cpu().numpy()[0], root_want), "root histogram"
        want_sp = oracle.find_splits(root_want[None], BINS, False, 29, 29, lam, gamma)
        got_sp = hgb.splits_to_numpy(sp_root)[:1]
        assert_splits(got_sp, want_sp, "root")
        assert (int(want_sp["feature"][0]), int(want_sp["bin"][0])) == (1, 127)

        say("max rows: partition and level 1")
        child_rows = torch.empty(N, dtype=torch.int32, device="cuda")
        child_hist = torch.empty((2, 2, BINS, 2), dtype=torch.int64, device="cuda")
        n_rec = 3 if oblivious else 2
        child_sp = torch.empty(n_rec * hgb.SPLIT_BYTES, dtype=torch.uint8, device="cuda")
        offs, bir, parents, built = ctx.grow_level(hist, sp_root, None, None, child_rows, child_hist,
                                                   child_sp, lam, gamma, oblivious=oblivious)
        ctx.sync()
        n_left = 2**30   # rows with bit 15 clear: 32,768 per 65,536, the last cycle one short of full
        assert offs.tolist() == [0, n_left, N]
        assert bir.tolist() == [1] and parents.tolist() == [0] and built == N - n_left
        # the last row, 0x7FFFFFFE, has bit 15 set; the last with it clear is 0x7FFF7FFF
        assert_ascending_with_bit15(torch, child_rows[:n_left], 0, 0, 0x7FFF7FFF, n_left)
        assert_ascending_with_bit15(torch, child_rows[n_left:], 1, 0x8000, N - 1, N - n_left)
        got = child_hist.cpu().numpy()
        assert np.array_equal(got[1], right_want), "built (right) child"
        assert np.array_equal(got[0], left_want), "derived (left) child"
        both = np.stack([left_want, right_want])
        if oblivious:
            want_csp = oracle.find_level_split(both, BINS, False, 29, 29, lam, gamma)
        else:
            want_csp = oracle.find_splits(both, BINS, False, 29, 29, lam, gamma)
        assert_splits(hgb.splits_to_numpy(child_sp)[:n_rec], want_csp, "level 1")
    finally:
        ctx.close()
        del g, h
        torch.cuda.empty_cache()
