"""GPU parity of the oblivious level split (hgb_find_level_split) and of
oblivious trees grown on the device, against the oracle.  The level score is a
floating-point sum taken in node order on both sides, so every record --
feature, bin, direction, integer sums and gains -- must be bit-identical."""
import numpy as np
import pytest

import oracle
from histogram_gradient_boosted_amd import synth

from test_gpu_parity import assert_splits, oracle_quantized, say

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


def assert_records(got, want, where):
    assert_splits(got, want, where)
    assert np.array_equal(got["gain"].view(np.int64), want["gain"].view(np.int64)), \
        f"{where}: gains differ in bits at {np.nonzero(got['gain'] != want['gain'])[0][:8]}"


def level_both(hgb, torch, w, rows, offs, lam=1.0, gamma=0.0, offset=0):
    """The oracle's histograms of the given nodes, fed to the oracle's and the
    device's level split (the device gets a copy of the oracle's histograms:
    this compares the split step alone).  offset > 0 misaligns the device copy
    by that many int64 words."""
    qg, qh, kg, kh = oracle_quantized(w)
    if rows is None:
        hist = oracle.build_hist(w.bins, w.n_bins, w.has_missing, qg, qh)
    else:
        hist = oracle.build_hist(w.bins, w.n_bins, w.has_missing, qg, qh, rows, offs)
    want = oracle.find_level_split(hist, w.n_bins, w.has_missing, kg, kh, lam, gamma)
    N = hist.shape[0]
    ctx = hgb.Context(0)
    ctx.upload_bins(w.bins, w.n_bins, w.has_missing)
    ctx.begin_tree(torch.from_numpy(w.grad).cuda(), torch.from_numpy(w.hess).cuda())
    assert ctx.get_scales() == (kg, kh)
    flat = torch.zeros(hist.size + offset, dtype=torch.int64, device="cuda")
    flat[offset:] = torch.from_numpy(hist.reshape(-1)).cuda()
    out = torch.full(((N + 1) * hgb.SPLIT_BYTES,), 0xAB, dtype=torch.uint8, device="cuda")
    ctx.find_level_split(flat[offset:], N, lam, gamma, out)
    ctx.sync()
    got = hgb.splits_to_numpy(out)[: N + 1]
    ctx.close()
    return got, want


SMALL = [
    # seed, n, F, B, missing, children, u16, gamma, offset
    (80, 5000, 4, 16, False, 8, None, 0.0, 0), (81, 20000, 6, 64, True, 16, None, 0.5, 0),
    (82, 3000, 3, 300, True, 6, True, 0.0, 0), (83, 70000, 3, 1024, True, 4, True, 0.0, 0),
    (84, 9000, 2, 2000, False, 2, True, 0.0, 0), (85, 12000, 5, 255, True, 10, None, 0.0, 1),
    (86, 40, 3, 8, True, 12, None, 0.0, 0), (87, 800, 2, 64, False, 0, None, 0.0, 0),
]


@pytest.mark.parametrize("seed,n,F,B,missing,children,u16,gamma,offset", SMALL)
def test_level_split_vs_oracle(hgb, torch, seed, n, F, B, missing, children, u16, gamma, offset):
    say("level split", seed, n, F, B, missing, children, gamma, offset)
    w = synth.random_small(seed, n, F, B, missing, children, u16=u16)
    rows = None if children == 0 else w.level.children_row_index
    offs = None if children == 0 else w.level.children_offsets
    got, want = level_both(hgb, torch, w, rows, offs, 1.0, gamma, offset)
    assert_records(got, want, f"seed {seed}")


def test_level_split_no_candidate(hgb, torch):
    """One value bin: every candidate leaves the right side empty."""
    say("level split no candidate")
    w = synth.random_small(88, 3000, 3, 1, False, 4)
    got, want = level_both(hgb, torch, w, w.level.children_row_index, w.level.children_offsets)
    assert (want["feature"] == -1).all()
    assert_records(got, want, "no candidate")


@pytest.mark.parametrize("name,n_rows,children", [("c3", 1_000_000, 128), ("c4", 16_384, 8),
                                                  ("c5", 500_000, 128), ("c2", 200_000, 32)])
def test_level_split_workload_shapes(hgb, torch, name, n_rows, children):
    """Levels of each workload's feature and bin shape (rows reduced so that
    the oracle builds the histograms in seconds): c4 keeps all 16,384
    features, so the candidate space is the full 4.2M of its level 3."""
    say("level split shape", name, n_rows, children)
    w = synth.make(name, n_rows=n_rows)
    node_id = np.random.default_rng(5).integers(0, children, w.n_rows)
    lvl = synth.level_from_node_ids(node_id, children)
    got, want = level_both(hgb, torch, w, lvl.children_row_index, lvl.children_offsets)
    assert want[children]["feature"] >= 0
    assert_records(got, want, name)


def test_level_split_errors(hgb, torch):
    say("level split errors")
    w = synth.random_small(89, 100, 2, 8, False, 0)
    ctx = hgb.Context(0)
    ctx.upload_bins(w.bins, w.n_bins, w.has_missing)
    h = torch.zeros((1, 2, 8, 2), dtype=torch.int64, device="cuda")
    out = torch.zeros(2 * hgb.SPLIT_BYTES, dtype=torch.uint8, device="cuda")
    with pytest.raises(hgb.HGBError) as e:
        ctx.find_level_split(h, 1, 1.0, 0.0, out)
    assert e.value.status == hgb.HGB_E_STATE
    ctx.begin_tree(torch.from_numpy(w.grad).cuda(), torch.from_numpy(w.hess).cuda())
    with pytest.raises(hgb.HGBError) as e:
        ctx.find_level_split(h, 1, -1.0, 0.0, out)
    assert e.value.status == hgb.HGB_E_INVALID
    ctx.close()


def oracle_oblivious_tree(w, depth, bits):
    qg, qh, kg, kh = oracle_quantized(w, bits)
    B, M = w.n_bins, w.has_missing
    hist = oracle.build_hist(w.bins, B, M, qg, qh)
    sp = oracle.find_level_split(hist, B, M, kg, kh, w.lam, w.gamma)
    levels = [(None, None, hist, sp)]
    rows, offs = None, None
    for _ in range(1, depth):
        rows, offs = oracle.partition(w.bins, B, rows, offs, sp[:-1])
        if len(offs) == 1:
            break
        hist = oracle.build_hist(w.bins, B, M, qg, qh, rows, offs)
        sp = oracle.find_level_split(hist, B, M, kg, kh, w.lam, w.gamma)
        levels.append((rows, offs, hist, sp))
    return levels


@pytest.mark.parametrize("name,n,bits,fused", [("c3", 300_000, 30, True), ("c3", 300_000, 30, False),
                                               ("c3", 300_000, 19, True), ("c5", 200_000, 30, True)])
def test_oblivious_tree(hgb, torch, name, n, bits, fused):
    """A whole oblivious tree grown on the device (partition, build, subtract,
    level split per level) equals the oracle's, level by level."""
    say("oblivious tree", name, n, bits)
    from histogram_gradient_boosted_amd import tree
    w = synth.make(name, n_rows=n)
    depth = 8
    want = oracle_oblivious_tree(w, depth, bits)
    ctx = hgb.Context(0)
    ctx.set_precision(bits)
    ctx.upload_bins(w.bins, w.n_bins, w.has_missing)
    g = torch.from_numpy(w.grad).cuda()
    h = torch.from_numpy(w.hess).cuda()
    levels = tree.grow_oblivious_tree_device(ctx, g, h, depth, w.lam, w.gamma, fused=fused)
    assert len(levels) == len(want)
    for d, (lv, (rows, offs, hist, sp)) in enumerate(zip(levels, want)):
        say("oblivious level", d, lv.n_nodes)
        assert lv.n_nodes == hist.shape[0]
        if d > 0:
            assert np.array_equal(lv.offsets.astype(np.int64), offs)
            assert np.array_equal(lv.rows.cpu().numpy()[: int(offs[-1])], rows)
        assert np.array_equal(lv.hist.cpu().numpy(), hist), f"level {d} histograms differ"
        assert_records(hgb.splits_to_numpy(lv.splits)[: lv.n_nodes + 1], sp, f"level {d}")
    ctx.close()
