"""Pins of the oracle's DCP functions (the shard layout, the causal mask in global
positions, the per-rank decode and the merge over sources), each against the plain
unsharded definition or a closed form rather than against themselves."""
import numpy as np
import pytest

import oracle
from absorbed_mla_split_amd import workloads as wl


def test_owner_closed_form_example():
    # world 2, interleave 2: positions 0 1 | 2 3 | 4 5 | 6 7 -> ranks 0 0 1 1 0 0 1 1,
    # local positions 0 1 0 1 2 3 2 3
    got = [oracle.dcp_owner(p, 2, 2) for p in range(8)]
    assert got == [(0, 0), (0, 1), (1, 0), (1, 1), (0, 2), (0, 3), (1, 2), (1, 3)]
    # world 3, interleave 1: round robin
    assert [oracle.dcp_owner(p, 3, 1) for p in range(7)] == [
        (0, 0), (1, 0), (2, 0), (0, 1), (1, 1), (2, 1), (0, 2)]


@pytest.mark.parametrize("world,interleave", [(1, 1), (2, 1), (3, 2), (4, 64), (8, 16)])
def test_owner_is_a_bijection_in_global_order(world, interleave):
    n = 1000
    seen = {d: [] for d in range(world)}
    for p in range(n):
        d, loc = oracle.dcp_owner(p, world, interleave)
        seen[d].append(loc)
    for d in range(world):
        assert seen[d] == list(range(len(seen[d])))          # 0, 1, 2, ... in global order
        assert oracle.dcp_local_count(n, world, d, interleave) == len(seen[d])
    assert sum(len(v) for v in seen.values()) == n


def test_visible_keys():
    assert oracle.visible_keys(100, 4, 0, False) == 100
    assert [oracle.visible_keys(100, 4, t, True) for t in range(4)] == [97, 98, 99, 100]
    assert oracle.visible_keys(2, 4, 0, True) == 0


def _global():
    # requests whose lengths are not multiples of the interleave or the page
    return wl.small(3, 4, 2, [301, 5, 1000], seed=17)


def test_causal_last_token_equals_non_causal_and_prefix_equals_truncation():
    w = _global()
    k, H = 4, 2
    c_out, c_lse = oracle.decode_causal(w.q8, w.kv8, w.block_table, w.lengths, k, H, w.q_scale,
                                        w.k_scale, w.sm_scale, causal=True)
    n_out, n_lse = oracle.decode(w.q8, w.kv8, w.block_table, w.lengths, w.q_scale, w.k_scale,
                                 w.sm_scale)
    M = k * H
    c_out = c_out.reshape(w.R, M, 512)
    n_out = n_out.reshape(w.R, M, 512)
    last = slice((k - 1) * H, k * H)
    assert np.array_equal(c_out[:, last], n_out[:, last])
    # token t sees the first T - k + t + 1 keys: the non-causal decode of a truncated cache
    for t in range(k):
        trunc = np.maximum(w.lengths - (k - 1 - t), 0).astype(np.int32)
        o, l = oracle.decode(w.q8, w.kv8, w.block_table, trunc, w.q_scale, w.k_scale, w.sm_scale)
        o = o.reshape(w.R, M, 512)
        assert np.array_equal(c_out[:, t * H:(t + 1) * H], o[:, t * H:(t + 1) * H])


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("world,interleave", [(2, 1), (3, 2), (4, 64), (2, 256)])
def test_sharded_merge_equals_unsharded(world, interleave, causal):
    w = _global()
    k, H = 4, 2
    ref, ref_lse = oracle.decode_causal(w.q8, w.kv8, w.block_table, w.lengths, k, H, w.q_scale,
                                        w.k_scale, w.sm_scale, causal=causal)
    shards = wl.dcp_shards(w, world, interleave)
    outs, lses = [], []
    for d, s in enumerate(shards):
        o, l = oracle.decode_dcp_rank(s.q8, s.kv8, s.block_table, s.lengths, w.lengths, k, H,
                                      w.q_scale, w.k_scale, w.sm_scale, world, d, interleave,
                                      causal=causal)
        outs.append(o)
        lses.append(l)
    out, lse = oracle.merge_sources(outs, lses)
    fin = np.isfinite(ref_lse)
    assert np.array_equal(fin, np.isfinite(lse))
    assert np.max(np.abs(out - ref)) <= 1e-12 * max(1.0, np.abs(ref).max())
    assert np.max(np.abs(lse[fin] - ref_lse[fin]), initial=0) <= 1e-12 * 20


def test_sharded_causal_detects_a_wrong_local_count(monkeypatch):
    # a planted off-by-one in the rank's visible prefix must break the equality above
    w = _global()
    k, H, world, interleave = 4, 2, 2, 1
    real = oracle.dcp_local_count
    monkeypatch.setattr(oracle, "dcp_local_count",
                        lambda n, W, d, I: max(0, real(n, W, d, I) - (1 if d == 1 else 0)))
    with pytest.raises(AssertionError):
        test_sharded_merge_equals_unsharded(world, interleave, True)


def test_merge_sources_closed_forms():
    rng = np.random.default_rng(3)
    o = rng.standard_normal((2, 4, 512))
    # equal LSEs: mean of the rows, lse + 1
    out, lse = oracle.merge_sources(o, np.full((2, 4), 3.0))
    assert np.allclose(out, o.mean(axis=0), rtol=0, atol=1e-14) and np.allclose(lse, 4.0)
    # an empty source carries no weight; all-empty rows stay empty
    l = np.array([[1.0, -np.inf], [-np.inf, -np.inf]])
    out, lse = oracle.merge_sources(o[:, :2], l)
    assert np.array_equal(out[0], o[0, 0]) and lse[0] == 1.0
    assert np.all(out[1] == 0) and np.isneginf(lse[1])


def test_shards_hold_every_key_once():
    w = _global()
    for world, interleave in ((2, 1), (3, 64)):
        shards = wl.dcp_shards(w, world, interleave)
        assert sum(int(s.lengths.sum()) for s in shards) == int(w.lengths.sum())
        for d, s in enumerate(shards):
            for r in range(w.R):
                for j in range(0, int(s.lengths[r]), 7):
                    # local key j of rank d is global position p with dcp_owner(p) = (d, j)
                    blk, off = divmod(j, interleave)
                    p = (blk * world + d) * interleave + off
                    assert oracle.dcp_owner(p, world, interleave) == (d, j)
                    g = w.kv8[w.block_table[r, p // 64], p % 64]
                    assert np.array_equal(s.kv8[s.block_table[r, j // 64], j % 64], g)
