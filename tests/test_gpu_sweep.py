"""A seeded sweep of random shapes through the GPU path against the oracle:
row counts from 1 to 200,000 (ragged against every chunk size), 1 to 300
features (ragged against every feature tile), 2 to 4,095 value bins with and
without the missing slot, one- and two-byte bins, roots and levels of up to
48 children, at precisions 30, 19 and 12.  Each case is bit-exact, gains
included.  Then whole trees grown on the device (depthwise and oblivious,
one call per level or three) on random shapes, level by level against the
oracle's trees.  The shapes are drawn once from a fixed seed, so every run
checks the same cases; the ids name them.  HGB_SWEEP_SEED=k draws both
sweeps from seeds derived from k instead, for a run over shapes not seen
before (the ids still name each case)."""
import os

import numpy as np
import pytest

from histogram_gradient_boosted_amd import synth

from test_gpu_level_split import assert_records, oracle_oblivious_tree
from test_gpu_parity import assert_splits, oracle_tree, run_level_both, run_root_both, say

pytestmark = pytest.mark.gpu

_RESEED = os.environ.get("HGB_SWEEP_SEED")


def _cases(count=200, seed=2718):
    rng = np.random.default_rng(seed)
    out = []
    for k in range(count):
        n = int(rng.choice([rng.integers(1, 600), rng.integers(600, 40_000), rng.integers(40_000, 200_001)]))
        F = int(rng.choice([rng.integers(1, 9), rng.integers(9, 64), rng.integers(64, 301)]))
        B = int(rng.choice([rng.integers(2, 33), rng.integers(33, 257), rng.integers(257, 4096)]))
        missing = bool(rng.integers(0, 2))
        S = B + (1 if missing else 0)
        u16 = S > 256 or bool(rng.integers(0, 4) == 0)
        children = int(rng.choice([0, 2 * rng.integers(1, 25)]))
        bits = int(rng.choice([30, 30, 19, 12]))
        # keep the oracle's work per case to about a second
        while n * F * (1 + (children > 0)) > 6_000_000 and n > 1:
            n //= 2
        out.append((1000 + k, n, F, B, missing, children, u16, bits))
    return out


CASES = _cases() if _RESEED is None else _cases(seed=2 * int(_RESEED) + 100_003)


@pytest.mark.parametrize("seed,n,F,B,missing,children,u16,bits", CASES,
                         ids=[f"s{c[0]}-n{c[1]}-F{c[2]}-B{c[3]}{'m' if c[4] else ''}-c{c[5]}-{'u16' if c[6] else 'u8'}-P{c[7]}"
                              for c in CASES])
def test_random_shape(hgb, torch, seed, n, F, B, missing, children, u16, bits):
    say("sweep", seed, n, F, B, missing, children, u16, bits)
    w = synth.random_small(seed, n, F, B, missing, children, u16=u16)
    if children == 0:
        run_root_both(hgb, torch, w, bits)
    else:
        run_level_both(hgb, torch, w, check_exact_gain=True, bits=bits)


def _tree_cases(count=120, seed=3141):
    rng = np.random.default_rng(seed)
    out = []
    for k in range(count):
        n = int(rng.choice([rng.integers(1, 3_000), rng.integers(3_000, 120_001)]))
        F = int(rng.integers(1, 41))
        B = int(rng.choice([rng.integers(2, 17), rng.integers(17, 257), rng.integers(257, 2049)]))
        missing = bool(rng.integers(0, 2))
        u16 = B + (1 if missing else 0) > 256 or bool(rng.integers(0, 4) == 0)
        depth = int(rng.integers(2, 8))
        oblivious = bool(rng.integers(0, 2))
        fused = bool(rng.integers(0, 3) > 0)
        bits = int(rng.choice([30, 30, 19]))
        out.append((5000 + k, n, F, B, missing, u16, depth, oblivious, fused, bits))
    return out


TREES = _tree_cases() if _RESEED is None else _tree_cases(seed=2 * int(_RESEED) + 100_004)


@pytest.mark.parametrize("seed,n,F,B,missing,u16,depth,oblivious,fused,bits", TREES,
                         ids=[f"s{c[0]}-n{c[1]}-F{c[2]}-B{c[3]}{'m' if c[4] else ''}-{'u16' if c[5] else 'u8'}-d{c[6]}"
                              f"-{'obl' if c[7] else 'dw'}-{'fused' if c[8] else 'apart'}-P{c[9]}" for c in TREES])
def test_random_tree(hgb, torch, seed, n, F, B, missing, u16, depth, oblivious, fused, bits):
    say("sweep tree", seed, n, F, B, missing, u16, depth, oblivious, fused, bits)
    from histogram_gradient_boosted_amd import tree
    w = synth.random_small(seed, n, F, B, missing, 0, u16=u16)
    ctx = hgb.Context(0)
    ctx.set_precision(bits)
    ctx.upload_bins(w.bins, w.n_bins, w.has_missing)
    g = torch.from_numpy(w.grad).cuda()
    h = torch.from_numpy(w.hess).cuda()
    if oblivious:
        levels = tree.grow_oblivious_tree_device(ctx, g, h, depth, w.lam, w.gamma, fused=fused)
        want = oracle_oblivious_tree(w, depth, bits)
    else:
        levels = tree.grow_tree_device(ctx, g, h, depth, w.lam, w.gamma, fused=fused)
        want = oracle_tree(w, depth, bits)
    assert len(levels) == len(want)
    for d, (lv, (rows, offs, hist, sp)) in enumerate(zip(levels, want)):
        if d > 0:
            assert np.array_equal(lv.offsets.astype(np.int64), offs), f"level {d} offsets"
            assert np.array_equal(lv.rows.cpu().numpy()[: int(offs[-1])], rows), f"level {d} rows"
        assert np.array_equal(lv.hist.cpu().numpy(), hist), f"level {d} histograms"
        if oblivious:
            assert_records(hgb.splits_to_numpy(lv.splits)[: lv.n_nodes + 1], sp, f"level {d}")
        else:
            assert_splits(hgb.splits_to_numpy(lv.splits)[: lv.n_nodes], sp, f"level {d}")
    ctx.close()


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
