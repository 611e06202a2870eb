"""Pins of the CPU oracle against things other than itself.

- E4M3 decode: every code against torch's float8_e4m3fn cast (a library routine) and
  the format's closed values.
- Attention: an independent pure-Python brute force (math.fsum / math.exp, torch's FP8
  decode) on tiny inputs; torch's float64 softmax-attention routine on small ones; the
  uniform-key closed form; the single-key case; zero-length requests.
- Invariants the pages state: folding is the same attention (folded == unfolded rows with
  replicated tables); only split points differ (any split + LSE merge == no split);
  renaming physical pages changes nothing.
A planted mistake in the oracle (a dropped scale, a sign, a swapped index, a wrong LSE
base, a wrong value slice) fails at least one of these.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from absorbed_mla_split_amd import workloads as wl

LOG2E = 1.0 / math.log(2.0)


def torch_decode_codes(codes: np.ndarray) -> np.ndarray:
    """FP8 E4M3FN codes -> float64 through torch (independent of the oracle's decode)."""
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def gather_keys(w, r):
    """[L, 576] FP8 codes of request r's keys in order, through its block table."""
    L = int(w.lengths[r])
    rows = [w.kv8[w.block_table[r, j // 64], j % 64] for j in range(L)]
    return np.stack(rows) if rows else np.zeros((0, 576), np.uint8)


# ------------------------------------------------------------------------------ E4M3

def test_e4m3_table_matches_torch_all_codes():
    mine = oracle.e4m3_table()
    ref = torch_decode_codes(np.arange(256, dtype=np.uint8))
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan], ref[~nan])
    assert np.array_equal(np.signbit(mine[~nan]), np.signbit(ref[~nan]))


def test_e4m3_closed_values():
    # sign | 4-bit exponent (bias 7) | 3-bit mantissa; no infinities, S.1111.111 = NaN
    assert oracle.e4m3_value(0x38) == 1.0
    assert oracle.e4m3_value(0x7E) == 448.0
    assert oracle.e4m3_value(0xFE) == -448.0
    assert oracle.e4m3_value(0x01) == 2.0 ** -9      # smallest subnormal
    assert oracle.e4m3_value(0x08) == 2.0 ** -6      # smallest normal
    assert oracle.e4m3_value(0x07) == 7 * 2.0 ** -9  # largest subnormal
    assert math.isnan(oracle.e4m3_value(0x7F)) and math.isnan(oracle.e4m3_value(0xFF))
    assert oracle.e4m3_value(0x78) == 256.0


# ------------------------------------------------------------------------- attention

def brute_force_row(q_codes, k_codes, q_scale, k_scale, sm_scale):
    """Plain-Python exact softmax attention of one query row over keys (codes)."""
    q = [q_scale * v for v in torch_decode_codes(q_codes).tolist()]
    keys = torch_decode_codes(k_codes).tolist()
    if not keys:
        return [0.0] * 512, -math.inf
    s = [sm_scale * math.fsum(qd * (k_scale * kd) for qd, kd in zip(q, key)) for key in keys]
    m = max(s)
    w = [math.exp(x - m) for x in s]
    l = math.fsum(w)
    out = [math.fsum(wj * (k_scale * key[c]) for wj, key in zip(w, keys)) / l for c in range(512)]
    return out, (m + math.log(l)) * LOG2E


def test_attend_matches_python_brute_force():
    # 3 pages incl. a partial one, shuffled tables, poisoned tails and spare pages
    w = wl.small(R=2, k=2, H=2, lengths=[130, 67], seed=3)
    out, lse = oracle.decode(w.q8, w.kv8, w.block_table, w.lengths, w.q_scale, w.k_scale, w.sm_scale)
    n = 0
    for r in range(w.R):
        keys = gather_keys(w, r)
        for i in range(w.M):
            ref, ref_lse = brute_force_row(w.q8[r, i], keys, w.q_scale, w.k_scale, w.sm_scale)
            np.testing.assert_allclose(out[n], ref, rtol=1e-12, atol=1e-14)
            assert abs(lse[n] - ref_lse) <= 1e-12 * max(1.0, abs(ref_lse))
            n += 1


@pytest.mark.parametrize("lengths", [[1, 64, 65], [200, 317], [0, 127, 500]])
def test_attend_matches_torch_float64_attention(lengths):
    w = wl.small(R=len(lengths), k=3, H=4, lengths=lengths, seed=11)
    out, lse = oracle.decode(w.q8, w.kv8, w.block_table, w.lengths, w.q_scale, w.k_scale, w.sm_scale)
    out = out.reshape(w.R, w.M, 512)
    lse = lse.reshape(w.R, w.M)
    for r in range(w.R):
        q = torch.from_numpy(torch_decode_codes(w.q8[r]) * w.q_scale)                 # [M, 576]
        k = torch.from_numpy(torch_decode_codes(gather_keys(w, r)) * w.k_scale)       # [L, 576]
        if k.shape[0] == 0:
            assert np.all(out[r] == 0.0) and np.all(lse[r] == -np.inf)
            continue
        scores = (q @ k.T) * w.sm_scale
        ref = torch.softmax(scores, dim=-1) @ k[:, :512]
        ref_lse = torch.logsumexp(scores, dim=-1) * LOG2E
        np.testing.assert_allclose(out[r], ref.numpy(), rtol=1e-11, atol=1e-13)
        np.testing.assert_allclose(lse[r], ref_lse.numpy(), rtol=1e-12, atol=1e-12)


def test_uniform_keys_closed_form():
    # Query latent dims zero, every key the same rope part: all scores are equal, so the
    # output is the plain mean of the values and lse = s * log2(e) + log2(L).
    w = wl.small(R=1, k=2, H=2, lengths=[150], seed=5)
    q8 = w.q8.copy()
    q8[:, :, :512] = 0
    kv8 = w.kv8.copy()
    rope = w.kv8[w.block_table[0, 0], 0, 512:].copy()
    for j in range(150):
        kv8[w.block_table[0, j // 64], j % 64, 512:] = rope
    out, lse = oracle.decode(q8, kv8, w.block_table, w.lengths, w.q_scale, w.k_scale, w.sm_scale)
    keys = torch_decode_codes(np.stack([kv8[w.block_table[0, j // 64], j % 64] for j in range(150)]))
    mean_v = keys[:, :512].mean(axis=0) * w.k_scale
    for i in range(w.M):
        qr = torch_decode_codes(q8[0, i, 512:]) * w.q_scale
        s = w.sm_scale * float(np.dot(qr, torch_decode_codes(rope) * w.k_scale))
        np.testing.assert_allclose(out[i], mean_v, rtol=1e-13, atol=1e-15)
        assert abs(lse[i] - (s * LOG2E + math.log2(150))) < 1e-12


def test_single_key():
    w = wl.small(R=1, k=1, H=3, lengths=[1], seed=9)
    out, lse = oracle.decode(w.q8, w.kv8, w.block_table, w.lengths, w.q_scale, w.k_scale, w.sm_scale)
    key = torch_decode_codes(w.kv8[w.block_table[0, 0], 0])
    for i in range(w.M):
        q = torch_decode_codes(w.q8[0, i]) * w.q_scale
        s = w.sm_scale * float(np.dot(q, key * w.k_scale))
        np.testing.assert_array_equal(out[i], key[:512] * w.k_scale)
        assert abs(lse[i] - s * LOG2E) < 1e-12


def test_zero_length_request():
    w = wl.small(R=3, k=2, H=2, lengths=[0, 70, 0], seed=1)
    out, lse = oracle.decode(w.q8, w.kv8, w.block_table, w.lengths, w.q_scale, w.k_scale, w.sm_scale)
    out = out.reshape(3, w.M, 512)
    lse = lse.reshape(3, w.M)
    assert np.all(out[0] == 0) and np.all(out[2] == 0)
    assert np.all(np.isneginf(lse[0])) and np.all(np.isneginf(lse[2]))
    assert np.all(np.isfinite(lse[1]))


def test_out_of_range_task_rejected():
    w = wl.small(R=1, k=1, H=2, lengths=[10], seed=1)
    with pytest.raises(ValueError):
        oracle.attend(w.q8, w.kv8, w.block_table, w.lengths, [[0, 0, 0, 11]], 1, 1, 1)
    bt = w.block_table.copy()
    bt[0, 0] = w.kv8.shape[0]
    with pytest.raises(ValueError):
        oracle.attend(w.q8, w.kv8, bt, w.lengths, [[0, 0, 0, 10]], 1, 1, 1)


# ------------------------------------------------------------------------ invariants

def test_fold_equals_unfolded_rows():
    # [R*k, H, D] -> [R, k*H, D]: request r, row t*H + h is stock row (r*k + t, head h),
    # which has its own copy of the request's block table and length.
    R, k, H = 2, 3, 4
    w = wl.small(R=R, k=k, H=H, lengths=[190, 77], seed=21)
    folded, folded_lse = oracle.decode(w.q8, w.kv8, w.block_table, w.lengths,
                                       w.q_scale, w.k_scale, w.sm_scale)
    q_unf = w.q8.reshape(R * k, H, 576)
    row_req = np.arange(R * k) // k
    unf, unf_lse = oracle.decode(q_unf, w.kv8, w.block_table[row_req], w.lengths[row_req],
                                 w.q_scale, w.k_scale, w.sm_scale)
    np.testing.assert_array_equal(folded, unf)
    np.testing.assert_array_equal(folded_lse, unf_lse)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_split_merge_equals_no_split(seed):
    rng = np.random.default_rng(100 + seed)
    w = wl.small(R=1, k=2, H=2, lengths=[333], seed=seed)
    L = 333
    full, full_lse = oracle.decode(w.q8, w.kv8, w.block_table, w.lengths,
                                   w.q_scale, w.k_scale, w.sm_scale)
    for _ in range(4):
        cuts = np.sort(rng.choice(np.arange(1, L), size=rng.integers(1, 6), replace=False))
        bounds = [0, *cuts.tolist(), L]
        for i in range(w.M):
            tasks = [(0, i, a, b) for a, b in zip(bounds[:-1], bounds[1:])]
            o, l = oracle.attend(w.q8, w.kv8, w.block_table, w.lengths, tasks,
                                 w.q_scale, w.k_scale, w.sm_scale)
            mo, ml = oracle.merge(o, l)
            np.testing.assert_allclose(mo, full[i], rtol=1e-11, atol=1e-13)
            assert abs(ml - full_lse[i]) < 1e-12


def test_merge_ignores_empty_partials_and_handles_all_empty():
    o = np.random.default_rng(0).standard_normal((3, 512))
    lse = np.array([-np.inf, 2.0, -np.inf])
    mo, ml = oracle.merge(o, lse)
    np.testing.assert_array_equal(mo, o[1])
    assert ml == 2.0
    mo, ml = oracle.merge(o, np.full(3, -np.inf))
    assert np.all(mo == 0) and ml == -np.inf


def test_merge_two_equal_halves():
    # two partials with equal lse: weights 1/2 each, lse + 1
    o = np.stack([np.ones(512), 3 * np.ones(512)])
    mo, ml = oracle.merge(o, np.array([5.0, 5.0]))
    np.testing.assert_array_equal(mo, 2 * np.ones(512))
    assert ml == 6.0


def test_page_renaming_changes_nothing():
    w = wl.small(R=2, k=2, H=2, lengths=[129, 64], seed=4)
    a, la = oracle.decode(w.q8, w.kv8, w.block_table, w.lengths, w.q_scale, w.k_scale, w.sm_scale)
    perm = np.random.default_rng(7).permutation(w.kv8.shape[0]).astype(np.int32)
    kv2 = np.empty_like(w.kv8)
    kv2[perm] = w.kv8                      # physical page p moves to perm[p]
    bt2 = np.where(w.block_table >= 0, perm[np.maximum(w.block_table, 0)], -1).astype(np.int32)
    b, lb = oracle.decode(w.q8, kv2, bt2, w.lengths, w.q_scale, w.k_scale, w.sm_scale)
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(la, lb)


def test_poisoned_slots_are_never_read():
    # every slot past a request's length holds NaN codes; results must stay finite
    w = wl.small(R=2, k=2, H=2, lengths=[65, 3], seed=8)
    out, lse = oracle.decode(w.q8, w.kv8, w.block_table, w.lengths, w.q_scale, w.k_scale, w.sm_scale)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
