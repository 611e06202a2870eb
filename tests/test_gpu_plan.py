"""GPU split planner vs the oracle's plan: counts, offsets and the whole work list must be
bit-exact, on the configs' length vectors and on random and edge-case ones."""
import numpy as np
import pytest
import torch

import oracle
from absorbed_mla_split_amd import binding
from absorbed_mla_split_amd import workloads as wl

pytestmark = pytest.mark.gpu


def plan_both(lengths, M, mode=binding.PLAN_BALANCED, min_split_tokens=256, workers=None,
              max_splits=256, split_cost=None):
    lengths = np.asarray(lengths, dtype=np.int32)
    R = len(lengths)
    cols = max(1, int(((lengths.astype(np.int64) + 63) // 64).max()) if R else 1)
    dec = binding.FoldedDecoder(max(R, 1), M, mode=mode, min_split_tokens=min_split_tokens,
                                workers=workers, max_splits=max_splits,
                                split_cost_pages=split_cost)
    dec.work.fill_(12345)
    dec.counts.fill_(777)
    dec.offsets.fill_(777)
    dec.plan(torch.from_numpy(lengths).cuda(), cols)
    counts, offsets, work, n = dec.plan_host()
    p = dec.params
    rc, ro, rw, rn = oracle.plan(lengths, cols, M, p.mtile, p.workers, min_split_tokens,
                                 max_splits, mode, list_len=dec.work.numel(),
                                 split_cost=p.split_cost_pages)
    assert dec.device_status() == 0
    assert n == rn
    np.testing.assert_array_equal(counts, rc)
    np.testing.assert_array_equal(offsets, ro)
    np.testing.assert_array_equal(work, rw)
    return dec


@pytest.mark.parametrize("cfg", ["c1", "c2", "c3", "c4", "c5"])
@pytest.mark.parametrize("mode", [binding.PLAN_BALANCED, binding.PLAN_FIXED])
def test_plan_configs(cfg, mode):
    c = wl.CONFIGS[cfg]
    lengths = wl.draw_lengths(c.lengths, c.R, np.random.default_rng(0))
    plan_both(lengths, c.M, mode)


@pytest.mark.parametrize("seed", range(8))
def test_plan_random(seed):
    rng = np.random.default_rng(seed)
    R = int(rng.integers(1, 300))
    lengths = rng.integers(0, 40000, R).astype(np.int32)
    lengths[rng.random(R) < 0.15] = 0
    M = int(rng.choice([8, 32, 56, 128, 256, 448]))
    plan_both(lengths, M, int(rng.integers(0, 2)), int(rng.choice([0, 64, 256, 4096])),
              split_cost=int(rng.choice([0, 1, 4, 100])))


def test_plan_edges():
    plan_both([0], 32)
    plan_both([0, 0, 0], 448)
    plan_both([1], 32)
    plan_both([64], 32, min_split_tokens=0)
    plan_both([131072] + [1024] * 15, 448)
    plan_both([10 ** 6], 32, max_splits=7)
    plan_both([10 ** 6, 64, 0, 700], 32, split_cost=binding.MAX_SPLIT_COST)
    plan_both([64] * 300, 56, min_split_tokens=0, split_cost=0)
    rng = np.random.default_rng(5)
    plan_both(rng.integers(0, 3000, binding.MAX_REQS).astype(np.int32), 32)
    plan_both(rng.integers(0, 3000, binding.MAX_REQS).astype(np.int32), 256, binding.PLAN_FIXED)


def test_plan_bad_length_sets_status_and_empties_plan():
    dec = binding.FoldedDecoder(3, 32)
    lengths = torch.tensor([100, -5, 64], dtype=torch.int32, device="cuda")
    dec.plan(lengths, 4)
    counts, offsets, work, n = dec.plan_host()
    assert dec.device_status() & binding.DEV_BAD_LENGTH
    G = dec.params.workers                 # 32 rows in 32-row tiles: one worker per group
    gb = 2 * (3 + dec.params.workers)
    assert n == 0 and np.all(counts == 0) and np.all(work[:gb] == -1)
    assert np.all(work[gb:gb + G + 1] == 0) and np.all(work[gb + G + 1:] == -1)
    lengths = torch.tensor([100, 64 * 5, 64], dtype=torch.int32, device="cuda")   # > 4 columns
    dec.plan(lengths, 4)
    assert dec.device_status() & binding.DEV_BAD_LENGTH


@pytest.mark.parametrize("R", [63, 64, 65, 128, 255, 256, 257])
def test_plan_request_count_boundaries(R):
    # up to 256 requests one per plan thread, more several per thread
    rng = np.random.default_rng(R)
    lengths = rng.integers(0, 20000, R).astype(np.int32)
    lengths[rng.random(R) < 0.1] = 0
    for M, workers in ((32, None), (56, 16), (448, 96)):
        plan_both(lengths, M, binding.PLAN_BALANCED, 256, workers=workers)
        plan_both(lengths, M, binding.PLAN_FIXED, 0, workers=workers)
    plan_both(np.full(R, 8192, np.int32), 32)            # uniform: the lower bound is the chunk
    plan_both(np.full(R, 8192, np.int32), 32, max_splits=3)


@pytest.mark.parametrize("R", [100, 300, 1000])
def test_plan_balances_skewed_batches(R):
    # log-uniform lengths, bit-exact with the oracle; every group's cost (its pages and the
    # split cost per item) within two minimum splits and two split costs of the mean (from the
    # device's own list)
    rng = np.random.default_rng(R)
    lengths = np.floor(np.exp(rng.uniform(np.log(64), np.log(65536), R))).astype(np.int32)
    dec = plan_both(lengths, 56)
    counts, offsets, work, n = dec.plan_host()
    pages = (lengths.astype(np.int64) + 63) // 64
    W = dec.params.workers
    gs = work[2 * (R + W):2 * (R + W) + W + 1]
    a = dec.params.split_cost_pages
    V = int(pages.sum()) + a * R
    Gp = min(W, V // 4)
    for g in range(Gp):
        got = 0
        for i in range(gs[g], gs[g + 1]):
            r = work[2 * i]
            end = work[2 * i + 3] if i + 1 < n and work[2 * i + 2] == r else pages[r]
            got += end - work[2 * i + 1] + a
        assert abs(got - V / Gp) < 2 * 4 + 2 * a, (g, got, V / Gp)
