"""Pins of the oracle's split plan and of the host fold rules.

The fold rules are pinned by the worked examples the pages print (tests/golden).  The
split plan is this project's reading of a rule the pages leave open (the lengths laid end
to end and cut into equal page ranges, one per worker group, each cut moved to the nearer
request boundary when it would leave a piece shorter than the minimum split); it is pinned
by hand-worked examples and by the properties that define it, checked exhaustively on
small batches: the items tile every request in request order, every piece is at least the
minimum split or a whole request, the group boundaries are the cuts at g * P / Gp or the
request boundary within a minimum split of one, and a cut only moves when it must.
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


def groups_of(W, M, MT):
    return max(1, W // -(-M // MT))


def pieces(work, n, lengths):
    """Items as (request, first page, end page) from the work pairs: an item ends where the
    next item of its request starts, the last one at the request's end."""
    pages = pages_of(lengths)
    out = []
    for i in range(n):
        r, f = int(work[2 * i]), int(work[2 * i + 1])
        nxt = int(work[2 * i + 3]) if i + 1 < n and int(work[2 * i + 2]) == r else pages[r]
        out.append((r, f, nxt))
    return out


def check_plan(lengths, M, MT, W, min_tokens=256, max_splits=256, mode=oracle.BALANCED,
               cost=0):
    """Every property of a plan that holds in both modes, plus the group rule of each mode;
    returns (counts, offsets, work, n, items, gstart)."""
    lengths = list(lengths)
    R = len(lengths)
    counts, offsets, work, n = oracle.plan(lengths, max(pages_of(lengths) + [1]), M, MT, W,
                                           min_tokens, max_splits, mode, split_cost=cost)
    pages = pages_of(lengths)
    P = sum(pages)
    G = groups_of(W, M, MT)
    minp = max(1, -(-min_tokens // 64))
    assert offsets[0] == 0 and np.array_equal(np.diff(offsets), counts) and offsets[R] == n
    assert n <= R + W
    assert np.all(work[2 * n:2 * (R + W)] == -1) and np.all(work[2 * (R + W) + G + 1:] == -1)
    items = pieces(work, n, lengths)
    # request order; every request with keys covered by its items, end to end
    for r in range(R):
        mine = items[offsets[r]:offsets[r + 1]]
        assert all(it[0] == r for it in mine)
        if pages[r] == 0:
            assert counts[r] == 0
            continue
        assert 1 <= counts[r] <= min(max_splits, pages[r])
        assert mine[0][1] == 0 and mine[-1][2] == pages[r]
        assert all(x[2] == y[1] and x[1] < x[2] for x, y in zip(mine, mine[1:] + [(r, pages[r], 0)]))
        for k, (_, f, e) in enumerate(mine):
            assert oracle.item_range(work, n, lengths, offsets[r] + k) == \
                (r, 64 * f, min(64 * e, lengths[r]))
    gstart = oracle.group_starts(work, R, W, M, MT).tolist()
    assert len(gstart) == G + 1 and gstart[0] == 0 and gstart[-1] == n
    assert all(x <= y for x, y in zip(gstart, gstart[1:]))
    if mode == oracle.FIXED:
        # equal splits: sizes of a request differ by at most one, the longer ones first
        for r in range(R):
            sz = [e - f for _, f, e in items[offsets[r]:offsets[r + 1]]]
            assert sz == sorted(sz, reverse=True) and (not sz or sz[0] - sz[-1] <= 1)
        assert gstart == [g * n // G for g in range(G + 1)]
        return counts, offsets, work, n, items, gstart
    # BALANCED: pieces at least the minimum split unless whole requests
    assert all(e - f >= minp or (f == 0 and e == pages[r]) for r, f, e in items)
    # each non-empty request a head of `cost` pages and its pages, end to end
    v = [p + cost if p else 0 for p in pages]
    voff = [sum(v[:r]) for r in range(R)]
    V = sum(v)
    Gp = max(1, min(G, max_splits, V // minp))
    assert all(g == n for g in gstart[Gp:])
    # group g takes [B_g, B_{g+1}): B_g is the start of its first item (V if none), a
    # request's first item starting at its head
    starts = [voff[r] + (cost + f if f else 0) for r, f, _ in items]
    bounds = [starts[i] if i < n else V for i in gstart[:Gp + 1]]
    for g, B in enumerate(bounds):
        c = g * V // Gp
        inside = [r for r in range(R) if voff[r] < c < voff[r] + v[r]]
        if not inside:
            assert B == c
        else:
            r = inside[0]
            x = c - voff[r] - cost
            if x < minp:
                assert B == voff[r]
            elif pages[r] - x < minp:
                assert B == voff[r] + v[r]
            else:
                assert B == c
    # a request's splits start at page 0 and at the group boundaries strictly inside it
    for r in range(R):
        if pages[r]:
            cuts = sorted({B - voff[r] - cost for B in bounds if voff[r] < B < voff[r] + v[r]})
            assert [f for _, f, _ in items[offsets[r]:offsets[r + 1]]] == [0] + cuts
    return counts, offsets, work, n, items, gstart


def test_plan_worked_example_two_requests():
    # pages [4, 5] (P = 9), minimum split 4 pages: Gp = min(256, 9 // 4) = 2 groups, cut at
    # 9 // 2 = 4, the boundary between the requests: one item each
    counts, offsets, work, n = oracle.plan([200, 317], 5, M=32, MT=32, W=256)
    assert counts.tolist() == [1, 1] and offsets.tolist() == [0, 1, 2] and n == 2
    assert work[:4].tolist() == [0, 0, 1, 0] and np.all(work[4:2 * (2 + 256)] == -1)
    g = oracle.group_starts(work, 2, 256, 32, 32)
    assert g[:3].tolist() == [0, 1, 2] and np.all(g[3:] == 2) and len(g) == 257
    assert oracle.item_range(work, n, [200, 317], 1) == (1, 0, 317)


def test_plan_worked_example_cuts_inside_a_request():
    # pages [7, 1], 4 groups, minimum 1 page: cuts at 0, 2, 4, 6, 8, three of them inside
    # request 0; group 3 takes the last page of request 0 and request 1
    counts, offsets, work, n = oracle.plan([7 * 64, 64], 8, M=32, MT=32, W=4, min_split_tokens=0)
    assert counts.tolist() == [4, 1] and offsets.tolist() == [0, 4, 5] and n == 5
    assert work[:10].tolist() == [0, 0, 0, 2, 0, 4, 0, 6, 1, 0]
    assert np.all(work[10:12] == -1)
    assert work[12:17].tolist() == [0, 1, 2, 3, 5] and np.all(work[17:] == -1)
    assert oracle.item_range(work, n, [7 * 64, 64], 3) == (0, 384, 448)


def test_plan_worked_example_moved_cuts():
    # pages [5, 3], 4 groups, minimum 2 pages: cuts 2, 4, 6; cut 4 leaves 1 page at the end
    # of request 0 and moves to its end (5); cut 6 leaves 1 page at the start of request 1
    # and moves to its start (5): group 2 is empty
    counts, offsets, work, n = oracle.plan([5 * 64, 3 * 64 - 10], 5, M=32, MT=32, W=4,
                                           min_split_tokens=128)
    assert counts.tolist() == [2, 1] and n == 3
    assert work[:6].tolist() == [0, 0, 0, 2, 1, 0]
    assert oracle.group_starts(work, 2, 4, 32, 32).tolist() == [0, 1, 2, 2, 3]
    assert oracle.item_range(work, n, [320, 182], 2) == (1, 0, 182)


def test_plan_worked_example_split_cost():
    # pages [4, 5] with a 2-page head each: V = 13 over 4 groups, cuts at 3, 6, 9; cut 3 is
    # page 1 of request 0, 6 the start of request 1, 9 page 1 of request 1
    counts, offsets, work, n = oracle.plan([256, 300], 5, M=32, MT=32, W=4, min_split_tokens=0,
                                           split_cost=2)
    assert counts.tolist() == [2, 2] and n == 4
    assert work[:8].tolist() == [0, 0, 0, 1, 1, 0, 1, 1]
    assert oracle.group_starts(work, 2, 4, 32, 32).tolist() == [0, 1, 2, 3, 4]
    # the same lengths without the heads: cuts at 2, 4 (the boundary) and 6
    counts, _, work, n = oracle.plan([256, 300], 5, M=32, MT=32, W=4, min_split_tokens=0)
    assert work[:8].tolist() == [0, 0, 0, 2, 1, 0, 1, 2]
    # a head of 3 pages, 2 groups, minimum 2 pages: V = 15, cut 7 is page 7 - 7 - 3 < 2 of
    # request 1 (whose head starts at 7): moved to its start
    counts, _, work, n = oracle.plan([256, 300], 5, M=32, MT=32, W=2, min_split_tokens=128,
                                     split_cost=3)
    assert counts.tolist() == [1, 1] and oracle.group_starts(work, 2, 2, 32, 32).tolist() == [0, 1, 2]


def test_plan_worked_example_row_tiles_and_max_splits():
    # 448 rows in 128-row tiles: 4 workers per group, 8 workers -> 2 groups; one request of
    # 10 pages: one cut at 5
    counts, _, work, n = oracle.plan([640], 10, M=448, MT=128, W=8, min_split_tokens=0)
    assert counts.tolist() == [2] and work[:4].tolist() == [0, 0, 0, 5]
    assert oracle.group_starts(work, 1, 8, 448, 128).tolist() == [0, 1, 2]
    # at most 3 splits: Gp = 3, cuts at 3 and 6
    counts, _, work, n = oracle.plan([640], 10, M=32, MT=32, W=8, min_split_tokens=0,
                                     max_splits=3)
    assert counts.tolist() == [3] and work[:6].tolist() == [0, 0, 0, 3, 0, 6]
    assert oracle.group_starts(work, 1, 8, 32, 32).tolist() == [0, 1, 2, 3, 3, 3, 3, 3, 3]


def test_plan_uniform_batch_fills_workers():
    # 64 requests x 128 pages, 256 groups of 32 pages: 4 equal splits per request
    counts, offsets, work, n, items, gstart = check_plan([8192] * 64, M=32, MT=32, W=256)
    assert np.all(counts == 4) and n == 256 and gstart == list(range(257))
    assert all(e - f == 32 for _, f, e in items)


def test_plan_fixed_mode():
    rng = np.random.default_rng(0)
    lengths = np.floor(np.exp(rng.uniform(np.log(512), np.log(65536), 128))).astype(np.int32)
    counts, *_ = check_plan(lengths, M=56, MT=64, W=256, mode=oracle.FIXED)
    assert np.all(counts == 2)                  # floor(256 / 128) splits, every request
    counts, *_ = check_plan([64, 10000], M=32, MT=32, W=256, mode=oracle.FIXED)
    assert counts.tolist() == [1, 128]          # never more splits than pages
    # pages [5, 2, 0], 8 workers: 2 splits each (3 + 2 pages, 1 + 1), groups floor(g * 4 / 8)
    counts, offsets, work, n = oracle.plan([300, 128, 0], 5, M=32, MT=32, W=8, mode=oracle.FIXED)
    assert counts.tolist() == [2, 2, 0] and offsets.tolist() == [0, 2, 4, 4]
    assert work[:8].tolist() == [0, 0, 0, 3, 1, 0, 1, 1]
    assert oracle.group_starts(work, 3, 8, 32, 32).tolist() == [0, 0, 1, 1, 2, 2, 3, 3, 4]


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
    max_splits = int(rng.choice([2, 16, 256]))
    for mode in (oracle.BALANCED, oracle.FIXED):
        for cost in (0, 3):
            check_plan(lengths, M, MT, W, min_tokens, max_splits, mode, cost)


@pytest.mark.parametrize("cost", [0, 4])
def test_plan_balance_bound(cost):
    # every group's cost (its pages and `cost` per item) lies within two minimum splits and
    # two heads of V / Gp
    rng = np.random.default_rng(7)
    for _ in range(20):
        R = int(rng.integers(1, 200))
        lengths = np.floor(np.exp(rng.uniform(np.log(64), np.log(65536), R))).astype(np.int64)
        minp = 4
        counts, offsets, work, n, items, gstart = check_plan(lengths, 56, 64, 256, 64 * minp,
                                                             cost=cost)
        V = sum(pages_of(lengths)) + cost * R
        Gp = min(256, V // minp)
        for g in range(Gp):
            got = sum(e - f + cost for _, f, e in items[gstart[g]:gstart[g + 1]])
            assert abs(got - V / Gp) < 2 * minp + 2 * cost


def test_plan_exhaustive_small():
    # every length vector over {0, 1, 64, 65, 200, 640} for up to 3 requests
    choices = [0, 1, 64, 65, 200, 640]
    for R in (1, 2, 3):
        for lengths in itertools.product(choices, repeat=R):
            for W in (1, 3, 8):
                for min_tokens in (0, 128, 256):
                    for cost in (0, 1, 4):
                        check_plan(list(lengths), 32, 32, W, min_tokens, cost=cost)
                check_plan(list(lengths), 32, 32, W, 0, mode=oracle.FIXED)


def test_plan_rejects_bad_input():
    with pytest.raises(ValueError):
        oracle.plan([-1], 4, 32, 32, 256)
    with pytest.raises(ValueError):
        oracle.plan([64 * 5], 4, 32, 32, 256)          # more pages than table columns
    with pytest.raises(ValueError):
        oracle.plan([64] * 4, 4, 32, 32, 256, list_len=2 * (4 + 2 * 256) - 1)
    with pytest.raises(ValueError):
        oracle.item_range(np.array([0, 0, 0, 2], np.int32), 2, [64], 0)   # first beyond end
