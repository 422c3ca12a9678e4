"""hgb_find_splits_noalloc, the entry point that allocates nothing, against
hgb_find_splits (the entry point it is a variant of): identical records on
two calls in a row (the second smaller, so stale scratch from the first would
show), its size limit, and no change in the device's free memory."""
import ctypes
import sys

import numpy as np
import pytest

from histogram_gradient_boosted_amd import synth

pytestmark = pytest.mark.gpu


def say(*a):
    print("[no-alloc]", *a, flush=True)
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


def level_hist(hgb, torch, w):
    """A context on workload w (tree started) and its level's children's
    histograms, built on the device."""
    L = w.level
    ctx = hgb.Context(0)
    ctx.upload_bins(w.bins, w.n_bins, w.has_missing)
    ctx.begin_tree(torch.from_numpy(w.grad).cuda(), torch.from_numpy(w.hess).cuda())
    N = 2 * L.n_pairs
    hist = torch.empty((N, w.n_features, w.n_slots, 2), dtype=torch.int64, device="cuda")
    ctx.build_level(hist, torch.from_numpy(L.children_row_index).cuda(), L.children_offsets.astype(np.int32))
    return ctx, hist, N


def both(hgb, torch, ctx, hist, n_nodes, lam, gamma):
    """(find_splits records, find_splits_noalloc records) as raw bytes; the
    no-allocation call goes through the C ABI directly."""
    ref = torch.full((n_nodes * hgb.SPLIT_BYTES,), 0xAB, dtype=torch.uint8, device="cuda")
    got = torch.full((n_nodes * hgb.SPLIT_BYTES,), 0xCD, dtype=torch.uint8, device="cuda")
    ctx.find_splits(hist, n_nodes, lam, gamma, ref)
    st = hgb.load().hgb_find_splits_noalloc(ctx._h, ctypes.c_void_p(hist.data_ptr()), ctypes.c_int32(n_nodes),
                                            ctypes.c_double(lam), ctypes.c_double(gamma),
                                            ctypes.c_void_p(got.data_ptr()))
    assert st == hgb.HGB_OK, hgb.load().hgb_last_error(ctx._h)
    ctx.sync()
    return ref.cpu().numpy(), got.cpu().numpy()


@pytest.mark.parametrize("big,small", [
    ((1, 120_000, 28, 256, False, 8), (2, 30_000, 9, 64, False, 4)),
    ((3, 120_000, 12, 1024, True, 6), (4, 40_000, 5, 300, True, 2)),
])
def test_matches_find_splits_two_calls(hgb, torch, big, small):
    """Two calls in a row on one context, the second with fewer nodes and
    features: each equals find_splits byte for byte."""
    wb = synth.random_small(*big)
    ctx, hist, N = level_hist(hgb, torch, wb)
    say("big", big, "nodes", N)
    ref, got = both(hgb, torch, ctx, hist, N, wb.lam, wb.gamma)
    assert np.array_equal(ref, got)
    sp = hgb.splits_to_numpy(got)
    assert (sp["feature"] >= 0).any()
    ctx.close()
    ws = synth.random_small(*small)
    ctx, hist, N = level_hist(hgb, torch, ws)
    say("small", small, "nodes", N)
    ref, got = both(hgb, torch, ctx, hist, N, ws.lam, 0.25)
    assert np.array_equal(ref, got)
    # and once more on the first context's shape after the smaller call
    ref2, got2 = both(hgb, torch, ctx, hist, N, ws.lam, 0.25)
    assert np.array_equal(ref2, got2) and np.array_equal(got2, got)
    ctx.close()


def test_size_limit_and_no_allocation(hgb, torch):
    """4,096 features of 2 bins: 1,024 per-block winners of 32 bytes per node,
    so 511 nodes fit the 16 MiB scratch and 512 do not.  The call that fits
    equals find_splits and leaves the device's free memory unchanged; the one
    that does not is refused before anything is launched."""
    F, n = 4096, 64
    rng = np.random.default_rng(5)
    bins = rng.integers(0, 2, size=(F, n), dtype=np.uint8)
    ctx = hgb.Context(0)
    ctx.upload_bins(bins, 2, False)
    ctx.begin_tree(torch.from_numpy(rng.standard_normal(n).astype(np.float32)).cuda(),
                   torch.from_numpy(rng.uniform(0.1, 1, n).astype(np.float32)).cuda())
    N = 512
    hist = torch.empty((N, F, 2, 2), dtype=torch.int64, device="cuda")
    gen = torch.Generator(device="cuda").manual_seed(9)
    hist[..., 0] = torch.randint(-2**20, 2**20, (N, F, 2), device="cuda", generator=gen)
    hist[..., 1] = torch.randint(0, 2**20, (N, F, 2), device="cuda", generator=gen)
    say("511 nodes x 4096 features")
    ref, got = both(hgb, torch, ctx, hist, 511, 1.0, 0.0)   # also warms both paths up
    assert np.array_equal(ref, got)
    out = torch.empty(N * hgb.SPLIT_BYTES, dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    ctx.find_splits_noalloc(hist, 511, 1.0, 0.0, out)
    ctx.find_splits_noalloc(hist, 37, 1.0, 0.0, out)
    ctx.sync()
    free1, _ = torch.cuda.mem_get_info()
    assert free1 == free0
    with pytest.raises(hgb.HGBError) as e:
        ctx.find_splits_noalloc(hist, 512, 1.0, 0.0, out)
    assert e.value.status == hgb.HGB_E_UNSUPPORTED
    ctx.sync()
    ctx.close()
