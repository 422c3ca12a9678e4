"""A seeded sweep of random shapes through the GPU path against the oracle:
row counts from 1 to 200,000 (ragged against every chunk size), 1 to 300
features (ragged against every feature tile), 2 to 4,095 value bins with and
without the missing slot, one- and two-byte bins, roots and levels of up to
48 children, at precisions 30, 19 and 12.  Each case is bit-exact, gains
included.  The shapes are drawn once from a fixed seed, so every run checks
the same cases; the ids name them."""
import numpy as np
import pytest

from histogram_gradient_boosted_amd import synth

from test_gpu_parity import run_level_both, run_root_both, say

pytestmark = pytest.mark.gpu


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


CASES = _cases()


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
