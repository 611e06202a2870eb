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
              max_splits=256):
    lengths = np.asarray(lengths, dtype=np.int32)
    R = len(lengths)
    cols = max(1, int(((lengths.astype(np.int64) + 63) // 64).max()) if R else 1)
    dec = binding.FoldedDecoder(max(R, 1), M, mode=mode, min_split_tokens=min_split_tokens,
                                workers=workers, max_splits=max_splits)
    dec.work.fill_(12345)
    dec.counts.fill_(777)
    dec.offsets.fill_(777)
    dec.plan(torch.from_numpy(lengths).cuda(), cols)
    counts, offsets, work, n = dec.plan_host()
    p = dec.params
    rc, ro, rw, rn = oracle.plan(lengths, cols, M, p.mtile, p.workers, min_split_tokens,
                                 max_splits, mode, list_len=dec.work.numel())
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
    plan_both(lengths, M, int(rng.integers(0, 2)), int(rng.choice([0, 64, 256, 4096])))


def test_plan_edges():
    plan_both([0], 32)
    plan_both([0, 0, 0], 448)
    plan_both([1], 32)
    plan_both([64], 32, min_split_tokens=0)
    plan_both([131072] + [1024] * 15, 448)
    plan_both([10 ** 6], 32, max_splits=7)
    rng = np.random.default_rng(5)
    plan_both(rng.integers(0, 3000, binding.MAX_REQS).astype(np.int32), 32)
    plan_both(rng.integers(0, 3000, binding.MAX_REQS).astype(np.int32), 256, binding.PLAN_FIXED)


def test_plan_bad_length_sets_status_and_empties_plan():
    dec = binding.FoldedDecoder(3, 32)
    lengths = torch.tensor([100, -5, 64], dtype=torch.int32, device="cuda")
    dec.plan(lengths, 4)
    counts, offsets, work, n = dec.plan_host()
    assert dec.device_status() & binding.DEV_BAD_LENGTH
    assert n == 0 and np.all(counts == 0) and np.all(work == -1)
    lengths = torch.tensor([100, 64 * 5, 64], dtype=torch.int32, device="cuda")   # > 4 columns
    dec.plan(lengths, 4)
    assert dec.device_status() & binding.DEV_BAD_LENGTH


@pytest.mark.parametrize("R", [63, 64, 65, 128, 255, 256, 257])
def test_plan_request_count_boundaries(R):
    # up to 256 requests take the single-pass planner, more the block-wide one
    rng = np.random.default_rng(R)
    lengths = rng.integers(0, 20000, R).astype(np.int32)
    lengths[rng.random(R) < 0.1] = 0
    for M, workers in ((32, None), (56, 16), (448, 96)):
        plan_both(lengths, M, binding.PLAN_BALANCED, 256, workers=workers)
        plan_both(lengths, M, binding.PLAN_FIXED, 0, workers=workers)
    plan_both(np.full(R, 8192, np.int32), 32)            # uniform: the lower bound is the chunk
    plan_both(np.full(R, 8192, np.int32), 32, max_splits=3)


@pytest.mark.parametrize("R", [100, 300, 1000])
def test_plan_rebalanced_skewed_batches(R):
    # log-uniform lengths: the longest split at one unit per worker exceeds 5/4 of the mean,
    # so the plan takes the finer chunk (more items than workers); both planners, bit-exact
    rng = np.random.default_rng(R)
    lengths = np.floor(np.exp(rng.uniform(np.log(64), np.log(65536), R))).astype(np.int32)
    dec = plan_both(lengths, 32)
    n = dec.plan_host()[3]
    assert n > dec.params.workers
