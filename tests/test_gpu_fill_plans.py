"""GPU parity of the row-major level fill under each tile layout, forced
through the planner's developer overrides (HGB_FILL_TUNE, read when a context
is created) and confirmed from the plan it prints (HGB_DEBUG_PLAN=1).

The interleaved (slot-major) tile has every lane add its row's features in a
lane-rotated order; these cases cover tiles narrower than their load (28
features in 32 positions: the spare positions take padding bytes), several
tiles per row with a ragged last one, 2-byte bins with 1,025 slots, copies,
and the skipped slot (hot features), against the oracle's histograms and
splits."""
import re

import numpy as np
import pytest

from histogram_gradient_boosted_amd import synth

from test_gpu_parity import run_level_both, run_root_both, say, with_hot_slots

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


def level_plans(err):
    """(copies, tile, il) of each row-major fill plan printed to stderr."""
    out = []
    for line in err.splitlines():
        m = re.search(r"\[hgb\] fill kind 2 acc \d+ copies (\d+) tile (\d+) lt \d+ ra \d+ il (\d)", line)
        if m:
            out.append(tuple(int(x) for x in m.groups()))
    return out


U8_28 = ("u8, 28 features", lambda: synth.random_small(300, 60_000, 28, 256, False, 8))
U8_70 = ("u8, 70 features", lambda: synth.random_small(301, 20_000, 70, 200, True, 6))
U16_13 = ("u16, 13 features, 1,025 slots", lambda: synth.random_small(302, 30_000, 13, 1024, True, 10, u16=True))
HOT_U8 = ("u8 hot slots", lambda: with_hot_slots(synth.random_small(303, 40_000, 6, 16, True, 8), 3))
HOT_U16 = ("u16 hot slots", lambda: with_hot_slots(synth.random_small(304, 30_000, 5, 1024, True, 6, u16=True), 4))
# 201 slots: a 16-position u16 tile (32-byte chunks, lane pairs) fits in LDS
U16_201 = ("u16, 13 features, 201 slots", lambda: synth.random_small(305, 30_000, 13, 200, True, 10, u16=True))
HOT_U16_201 = ("u16 hot slots, 201 slots",
               lambda: with_hot_slots(synth.random_small(306, 30_000, 5, 200, True, 6, u16=True), 4))

CASES = [
    # workload, il (2: interleaved with two lanes per row), tile, copies
    (U8_28, 2, 32, 1), (U8_28, 1, 32, 1), (U8_28, 0, 32, 1), (U8_28, 1, 16, 2), (U8_28, 1, 8, 4),
    (U8_28, 1, 4, 8), (U8_28, 1, 2, 16), (U8_70, 2, 32, 1), (U8_70, 1, 32, 1), (U8_70, 1, 16, 2),
    (U8_70, 0, 16, 2), (U16_201, 2, 16, 2), (U16_201, 2, 16, 1), (U16_201, 1, 16, 2), (U16_13, 1, 8, 1),
    (U16_13, 1, 4, 2), (U16_13, 1, 1, 8), (U16_13, 0, 8, 1), (HOT_U8, 2, 32, 1), (HOT_U8, 1, 32, 1),
    (HOT_U8, 1, 8, 2), (HOT_U8, 0, 32, 1), (HOT_U16_201, 2, 16, 2), (HOT_U16, 1, 8, 1), (HOT_U16, 1, 2, 4),
]


@pytest.mark.parametrize("bits", [30, 12])
@pytest.mark.parametrize("case,il,tile,copies", CASES, ids=lambda v: v[0] if isinstance(v, tuple) else str(v))
def test_row_fill_layouts(hgb, torch, monkeypatch, capfd, case, il, tile, copies, bits):
    name, make = case
    say("row fill layout", name, "il", il, "tile", tile, "copies", copies, "bits", bits)
    lc = copies.bit_length() - 1
    pair = 1 if il == 2 else 0   # a 32-byte interleaved plan takes lane pairs unless pair=0
    monkeypatch.setenv("HGB_FILL_TUNE", f"il={min(il, 1)},pair={pair},level_tile={tile},level_lc={lc}")
    monkeypatch.setenv("HGB_DEBUG_PLAN", "1")
    w = make()
    run_level_both(hgb, torch, w, check_exact_gain=True, bits=bits)
    plans = level_plans(capfd.readouterr().err)
    assert plans, "no row-major fill ran"
    assert set(plans) == {(copies, tile, il)}, plans
    if il == 2 and tile == 32:
        run_root_both(hgb, torch, w, bits=bits)


def test_interleaved_tile_full_size_wide_level(hgb, torch, monkeypatch, capfd):
    """131,072 x 16,384 bytes, the level of 8 nodes: the planner's own choice
    (the interleaved 32-feature tile, two lanes per row) against the oracle on
    sampled features."""
    import oracle
    from test_gpu_parity import oracle_quantized
    say("interleaved full-size wide level")
    monkeypatch.setenv("HGB_DEBUG_PLAN", "1")
    w = synth.make("c4")
    L = w.level
    ctx = hgb.Context(0)
    ctx.upload_bins(w.bins, w.n_bins, w.has_missing)
    ctx.begin_tree(torch.from_numpy(w.grad).cuda(), torch.from_numpy(w.hess).cuda())
    dev = torch.device("cuda")
    P = L.n_pairs
    ch = torch.full((2 * P, w.n_features, w.n_slots, 2), -7, dtype=torch.int64, device=dev)
    ctx.build_level(ch, torch.from_numpy(L.built_row_index).to(dev), L.built_offsets.astype(np.int32),
                    L.built_slots)
    ctx.sync()
    plans = level_plans(capfd.readouterr().err)
    assert plans and all(p[2] == 2 for p in plans), plans
    qg, qh, _, _ = oracle_quantized(w)
    rng = np.random.default_rng(9)
    feats = np.sort(rng.choice(w.n_features, 96, replace=False))
    feats = np.unique(np.concatenate([feats, [0, 31, 32, w.n_features - 1]]))
    got = ch[:, torch.from_numpy(feats).to(dev)].cpu().numpy()
    ctx.close()
    want = oracle.build_hist(w.bins[feats], w.n_bins, w.has_missing, qg, qh,
                             L.built_row_index, L.built_offsets)
    for k in range(P):
        s = int(L.built_slots[k])
        assert np.array_equal(got[s], want[k]), f"built node {k} (slot {s}) differs"


def root_plans(err):
    """(copies, tile, il) of each root fill plan printed to stderr."""
    out = []
    for line in err.splitlines():
        m = re.search(r"\[hgb\] fill kind 0 acc \d+ copies (\d+) tile (\d+) lt \d+ ra \d+ il (\d)", line)
        if m:
            out.append(tuple(int(x) for x in m.groups()))
    return out


R_U8_28 = ("root u8, 28 features", lambda: synth.random_small(310, 60_000, 28, 256, False, 0))
R_U8_70 = ("root u8, 70 features, ragged rows", lambda: synth.random_small(311, 20_003, 70, 200, True, 0))
R_U16 = ("root u16, 300 bins", lambda: synth.random_small(312, 30_002, 13, 300, True, 0, u16=True))
R_U16_1025 = ("root u16, 1,025 slots", lambda: synth.random_small(313, 12_000, 9, 1024, True, 0, u16=True))
R_HOT_U8 = ("root u8 hot slots", lambda: with_hot_slots(synth.random_small(314, 40_000, 6, 16, True, 0), 5))
R_HOT_U16 = ("root u16 hot slots", lambda: with_hot_slots(synth.random_small(315, 30_001, 5, 1024, True, 0, u16=True), 6))

# (a handful of rows puts at least 1/16 of them in some slot: these two run
# with the skipped slot)
R_TINY3 = ("root u8, 3 rows", lambda: synth.random_small(318, 3, 20, 255, True, 0))
R_TINY7 = ("root u8, 7 rows", lambda: synth.random_small(319, 7, 33, 200, False, 0))


def distinct_rows(seed, n, F):
    """n <= 256 rows whose bins are distinct within every feature, so no slot
    holds 1/16 of the rows (n >= 17) and no slot is skipped."""
    rng = np.random.default_rng(seed)
    bins = np.stack([rng.permutation(256)[:n] for _ in range(F)]).astype(np.uint8)
    g = rng.standard_normal(n).astype(np.float32)
    h = rng.uniform(0.1, 1.0, n).astype(np.float32)
    return synth.Workload(f"distinct{n}", bins, 256, False, g, h, kind="root")


R_FEW19 = ("root u8, 19 rows", lambda: distinct_rows(320, 19, 20))
R_FEW20 = ("root u8, 20 rows", lambda: distinct_rows(321, 20, 37))

ROOT_CASES = [
    # workload, tile (feature positions), copies
    (R_U8_28, 32, 1), (R_U8_28, 16, 2), (R_U8_28, 8, 4), (R_U8_70, 32, 1), (R_U8_70, 16, 1),
    (R_U8_70, 8, 2), (R_U16, 16, 1), (R_U16, 8, 2), (R_U16_1025, 8, 1), (R_HOT_U8, 16, 2),
    (R_HOT_U8, 8, 1), (R_HOT_U16, 8, 1), (R_TINY3, 16, 2), (R_TINY7, 8, 4), (R_FEW19, 32, 1),
    (R_FEW20, 16, 1),
]


@pytest.mark.parametrize("bits", [30, 20])
@pytest.mark.parametrize("case,tile,copies", ROOT_CASES, ids=lambda v: v[0] if isinstance(v, tuple) else str(v))
def test_root_fill_interleaved(hgb, torch, monkeypatch, capfd, case, tile, copies, bits):
    """The root's interleaved tile: full and partial tiles, rows in whole
    groups of four and ragged (one row at a time), items of a few rows (3, 7,
    19, 20), copies, 2-byte bins and the skipped slot, against the oracle's
    root histogram and split."""
    name, make = case
    say("root interleaved", name, "tile", tile, "copies", copies, "bits", bits)
    lc = copies.bit_length() - 1
    monkeypatch.setenv("HGB_FILL_TUNE", f"root_il=1,root_tile={tile},root_lc={lc}")
    monkeypatch.setenv("HGB_DEBUG_PLAN", "1")
    run_root_both(hgb, torch, make(), bits=bits)
    plans = root_plans(capfd.readouterr().err)
    assert plans == [(copies, tile, 1)], plans


def root_plans_acc(err):
    """(acc, copies, tile, il) of each root fill plan printed to stderr."""
    out = []
    for line in err.splitlines():
        m = re.search(r"\[hgb\] fill kind 0 acc (\d+) copies (\d+) tile (\d+) lt \d+ ra \d+ il (\d)", line)
        if m:
            out.append(tuple(int(x) for x in m.groups()))
    return out


R_U8_256M = ("root u8, 255 bins + missing", lambda: synth.random_small(316, 50_000, 20, 255, True, 0))

PACKED_ROOT_CASES = [
    # workload, copies
    (R_U8_28, 2), (R_U8_28, 4), (R_U8_70, 2), (R_U8_70, 4), (R_U8_256M, 2), (R_U8_256M, 4),
    (R_FEW19, 2), (R_FEW20, 4),
]


@pytest.mark.parametrize("bits", [19, 12])
@pytest.mark.parametrize("case,copies", PACKED_ROOT_CASES,
                         ids=lambda v: v[0] if isinstance(v, tuple) else str(v))
def test_root_fill_interleaved_packed(hgb, torch, monkeypatch, capfd, case, copies, bits):
    """The root's interleaved tile with packed sums (one add per cell, drained
    into registers): 16 positions with 2 or 4 copies, a partial last tile,
    rows in whole groups of four and ragged (one row at a time), items of 19
    and 20 rows, and all 256 slots of one-byte bins (the missing slot
    included), against the oracle."""
    name, make = case
    say("root interleaved packed", name, "copies", copies, "bits", bits)
    lc = copies.bit_length() - 1
    monkeypatch.setenv("HGB_FILL_TUNE", f"root_il=1,root_tile=16,root_lc={lc}")
    monkeypatch.setenv("HGB_DEBUG_PLAN", "1")
    run_root_both(hgb, torch, make(), bits=bits)
    plans = root_plans_acc(capfd.readouterr().err)
    assert plans == [(1, copies, 16, 1)], plans


def saturated_root(sign):
    """3,145,728 rows x 16 features where every row's |g| and h quantize to
    exactly 2^19 at P = 19 (fp32 1 - 2^-24: e = 0, k = 19, rint rounds up),
    and the rows come in runs of 12,288 -- one root item, three steps of the
    fill -- that share one bin in every feature (18 bins, so no slot holds a
    sixteenth of the rows and no slot is skipped).  Each copy-slot then takes
    the most rows the drain period allows at the largest codes."""
    n, F, run = 3_145_728, 16, 12_288
    r = np.arange(n)
    bins = np.stack([((r // run) + f) % 18 for f in range(F)]).astype(np.uint8)
    v = np.float32(np.nextafter(np.float32(1), np.float32(0)))
    g = np.full(n, sign * v, dtype=np.float32)
    h = np.full(n, v, dtype=np.float32)
    return synth.Workload("saturated", bins, 18, False, g, h, kind="root")


@pytest.mark.parametrize("sign", [1, -1])
@pytest.mark.parametrize("copies", [2, 4])
def test_root_fill_interleaved_packed_drain_bound(hgb, torch, monkeypatch, capfd, sign, copies):
    say("root interleaved packed, drain bound", sign, copies)
    import oracle
    w = saturated_root(sign)
    qg, _ = oracle.quantize(w.grad, False, 19)
    qh, _ = oracle.quantize(w.hess, True, 19)
    assert (np.abs(qg) == 2 ** 19).all() and (qh == 2 ** 19).all()
    lc = copies.bit_length() - 1
    monkeypatch.setenv("HGB_FILL_TUNE", f"root_il=1,root_tile=16,root_lc={lc}")
    monkeypatch.setenv("HGB_DEBUG_PLAN", "1")
    run_root_both(hgb, torch, w, bits=19)
    err = capfd.readouterr().err
    assert root_plans_acc(err) == [(1, copies, 16, 1)], err[-2000:]
    chunks = re.findall(r"\[hgb\] fill kind 0 .* chunk (\d+) ", err)
    assert chunks == ["12288"], chunks


@pytest.mark.parametrize("plan_host", ["0", "1"])
def test_plan_staging_modes(hgb, torch, monkeypatch, plan_host):
    """Launch plans read in place from pinned host memory (the default) or
    from a device copy (HGB_PLAN_HOST=0): the same histograms and splits,
    through the root, level fills with partial merges, the fused tail and a
    level of 300 pairs (whose subtraction plan is staged too)."""
    say("plan staging", plan_host)
    monkeypatch.setenv("HGB_PLAN_HOST", plan_host)
    run_root_both(hgb, torch, synth.random_small(320, 50_000, 28, 256, False, 0))
    run_level_both(hgb, torch, synth.random_small(321, 60_000, 28, 256, False, 8), check_exact_gain=True)
    run_level_both(hgb, torch, synth.random_small(322, 20_000, 3, 16, True, 600), check_exact_gain=True,
                   fused=True)


@pytest.mark.parametrize("ipc", [1, 4])
def test_merge_lists_short_and_long(hgb, torch, monkeypatch, capfd, ipc):
    """Partial histograms summed by k_merge: a short merge list travels in the
    kernel's arguments, a long one (more than 128 entries: here 4 shares per
    CU over 200 built nodes, so most nodes span several shares) is read from
    its staged plan; both against the oracle."""
    say("merge lists", ipc)
    monkeypatch.setenv("HGB_FILL_TUNE", f"level_ipc={ipc}")
    monkeypatch.setenv("HGB_DEBUG_PLAN", "1")
    w = synth.random_small(330, 400_000, 28, 256, False, 400)
    run_level_both(hgb, torch, w, check_exact_gain=True)
    merges = [int(m) for m in re.findall(r"\[hgb\] fill kind 2 .* merges (\d+)", capfd.readouterr().err)]
    assert merges, "no level fill ran"
    if ipc == 4:
        assert max(merges) > 128, merges
