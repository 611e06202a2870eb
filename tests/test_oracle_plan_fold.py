"""Pins of the oracle's split plan and of the host fold rules.

The fold rules are pinned by the worked examples the pages print (tests/golden).  The
split plan is this project's reading of a rule the pages leave open; it is pinned by a
hand-worked example and by the properties that define it: the splits tile each
request's pages, split sizes of a request differ by at most one, the work list is
ordered longest first with the pages' tie rule, and no uniform chunk size could have met
the worker budget with shorter splits (checked by exhaustive search).
"""
import itertools
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "fold_examples.txt")


def golden(kind):
    rows = []
    for line in open(GOLDEN):
        line = line.strip()
        if line and not line.startswith("#") and line.split()[0] == kind:
            rows.append([int(v) for v in line.split()[1:]])
    assert rows, kind
    return rows


def test_fold_plan_pages_example():
    for k, heads, need_lse, cap, expect in golden("fold_plan"):
        assert oracle.fold_plan(k, heads, bool(need_lse), cap) == expect


def test_foldable_pages_example():
    for causal, reqs, rows, tokens, bt_rows, mql, expect in golden("foldable"):
        assert oracle.foldable(bool(causal), reqs, rows, tokens, bt_rows, mql) == expect


def test_fold_rules_other_cases():
    assert oracle.fold_plan(4, 8, True, 128) == 4
    assert oracle.fold_plan(7, 64, True, 128) == 1
    assert oracle.fold_plan(7, 8, True, 128) == 7
    assert oracle.fold_plan(6, 64, True, 128) == 2
    assert oracle.fold_plan(7, 64, False, 128) == 7      # no LSE: everything folds
    assert oracle.foldable(False, 2, 8, 8, 2, 4) == 4
    assert oracle.foldable(True, 2, 8, 8, 2, 4) == 0     # causal
    assert oracle.foldable(False, 2, 2, 2, 2, 1) == 0    # one token each
    assert oracle.foldable(False, 2, 8, 9, 2, 4) == 0    # rows are not the decode tokens
    assert oracle.foldable(False, 3, 8, 8, 3, 4) == 0    # uneven
    assert oracle.foldable(False, 2, 8, 8, 1, 4) == 0    # too few table rows


# ---------------------------------------------------------------------------- plan

def pages_of(lengths):
    return [(int(L) + 63) // 64 for L in lengths]


def check_plan(lengths, M, MT, W, min_tokens=256, max_splits=256, mode=oracle.BALANCED):
    R = len(lengths)
    counts, offsets, work, n = oracle.plan(lengths, max(pages_of(lengths) + [1]), M, MT, W,
                                           min_tokens, max_splits, mode)
    pages = pages_of(lengths)
    mt = -(-M // MT)
    assert offsets[0] == 0 and np.array_equal(np.diff(offsets), counts) and offsets[R] == n
    assert n <= R + 2 * W
    sizes = {}
    for r in range(R):
        if pages[r] == 0:
            assert counts[r] == 0
            continue
        assert 1 <= counts[r] <= min(max_splits, pages[r])
        covered = []
        for s in range(counts[r]):
            a, b = oracle.split_range(lengths[r], counts[r], s)
            assert a % 64 == 0 and a < b <= lengths[r]
            covered.append((a, b))
            sizes[(r, s)] = (-(-b // 64)) - a // 64
        assert covered[0][0] == 0 and covered[-1][1] == lengths[r]
        assert all(x[1] == y[0] for x, y in zip(covered, covered[1:]))
        szs = [sizes[(r, s)] for s in range(counts[r])]
        assert sum(szs) == pages[r] and max(szs) - min(szs) <= 1
    pairs = [(int(work[2 * i]), int(work[2 * i + 1])) for i in range(n)]
    assert sorted(pairs) == sorted(sizes)
    keys = [(-sizes[p], p[0], p[1]) for p in pairs]
    assert keys == sorted(keys)
    assert np.all(work[2 * n:] == -1)
    return counts, offsets, work, n, sizes, mt


def test_plan_worked_example_two_requests():
    # pages [4, 5]; one row tile; the 4-page minimum sets the chunk: counts [1, 2]
    counts, offsets, work, n = oracle.plan([200, 317], 5, M=32, MT=32, W=256)
    assert counts.tolist() == [1, 2] and offsets.tolist() == [0, 1, 3] and n == 3
    assert oracle.split_range(200, 1, 0) == (0, 200)
    assert oracle.split_range(317, 2, 0) == (0, 192)
    assert oracle.split_range(317, 2, 1) == (192, 317)
    assert work[:6].tolist() == [0, 0, 1, 0, 1, 1] and np.all(work[6:] == -1)


def test_plan_uniform_batch_fills_workers():
    # 64 requests x 128 pages, 256 workers: 4 splits of 32 pages each
    counts, offsets, work, n = oracle.plan([8192] * 64, 128, M=32, MT=32, W=256)
    assert np.all(counts == 4) and n == 256


def test_plan_fixed_mode():
    rng = np.random.default_rng(0)
    lengths = np.floor(np.exp(rng.uniform(np.log(512), np.log(65536), 128))).astype(np.int32)
    counts, *_ = oracle.plan(lengths, 1024, M=56, MT=64, W=256, mode=oracle.FIXED)
    assert np.all(counts == 2)                  # floor(256 / 128) splits, every request
    counts, *_ = oracle.plan([64, 10000], 200, M=32, MT=32, W=256, mode=oracle.FIXED)
    assert counts.tolist() == [1, 128]          # never more splits than pages


def best_uniform_chunk(pages, mt, W, min_pages, max_splits):
    """Exhaustive: the shortest longest-split over every uniform chunk that fits W."""
    best = None
    for c in range(1, max(pages + [1]) + 1):
        cc = max(c, min_pages)
        cnt = [0 if p == 0 else min(max_splits, -(-p // cc)) for p in pages]
        if mt * sum(cnt) <= W:
            longest = max([-(-p // k) for p, k in zip(pages, cnt) if k] + [0])
            best = longest if best is None else min(best, longest)
    return best


def expected_longest(pages, mt, W, min_pages, max_splits):
    """The plan's longest split by exhaustive search: the best uniform chunk within W
    workers, or within 2W when that longest split exceeds 5/4 of the mean per worker."""
    best = best_uniform_chunk(pages, mt, W, min_pages, max_splits)
    if best is not None and 4 * best * W > 5 * mt * sum(pages):
        best = best_uniform_chunk(pages, mt, 2 * W, min_pages, max_splits)
    return best


@pytest.mark.parametrize("seed", range(12))
def test_plan_properties_random(seed):
    rng = np.random.default_rng(seed)
    R = int(rng.integers(1, 40))
    lengths = rng.integers(0, 5000, R)
    lengths[rng.random(R) < 0.2] = 0
    M = int(rng.choice([8, 32, 56, 256, 448]))
    MT = 32 if M <= 32 else (64 if M <= 64 else 128)
    W = int(rng.choice([8, 64, 256]))
    min_tokens = int(rng.choice([0, 64, 256, 1000]))
    counts, offsets, work, n, sizes, mt = check_plan(lengths, M, MT, W, min_tokens)
    pages = pages_of(lengths)
    best = expected_longest(pages, mt, W, -(-min_tokens // 64), 256)
    longest = max(sizes.values()) if sizes else 0
    if best is not None:
        assert longest == best


def test_plan_exhaustive_small():
    # every length vector over {0, 1, 64, 65, 200, 640} for up to 3 requests
    choices = [0, 1, 64, 65, 200, 640]
    for R in (1, 2, 3):
        for lengths in itertools.product(choices, repeat=R):
            for W in (1, 3, 8):
                counts, offsets, work, n, sizes, mt = check_plan(list(lengths), 32, 32, W, 0)
                pages = pages_of(lengths)
                best = expected_longest(pages, 1, W, 0, 256)
                if best is not None and sizes:
                    assert max(sizes.values()) == best
                check_plan(list(lengths), 32, 32, W, 0, mode=oracle.FIXED)


def test_plan_rejects_bad_input():
    with pytest.raises(ValueError):
        oracle.plan([-1], 4, 32, 32, 256)
    with pytest.raises(ValueError):
        oracle.plan([64 * 5], 4, 32, 32, 256)          # more pages than table columns
    with pytest.raises(ValueError):
        oracle.plan([64] * 4, 4, 32, 32, 256, list_len=3)


def test_plan_rebalances_a_skewed_batch():
    # pages [7, 1], 4 workers: chunk(4) = 3 gives splits 3, 2, 2 and 1 page, the longest (3)
    # above 5/4 of the mean per worker (8 / 4 = 2), so the plan takes chunk(8) = 1: eight
    # one-page splits, two per worker
    counts, offsets, work, n = oracle.plan(np.array([7 * 64, 64], np.int32), 8, 32, 32, 4,
                                           min_split_tokens=0)
    assert counts.tolist() == [7, 1] and offsets.tolist() == [0, 7, 8] and n == 8
    assert work[:16].tolist() == [0, 0, 0, 1, 0, 2, 0, 3, 0, 4, 0, 5, 0, 6, 1, 0]
    assert np.all(work[16:] == -1)
    # pages [10, 1, 1, 1], 8 workers: chunk(8) = 2, longest 2 against a mean of 13/8 (not
    # above 5/4 of it): no rebalancing
    counts, _, _, n = oracle.plan(np.array([640, 64, 64, 64], np.int32), 16, 32, 32, 8,
                                  min_split_tokens=0)
    assert counts.tolist() == [5, 1, 1, 1] and n == 8
