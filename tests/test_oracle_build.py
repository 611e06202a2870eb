"""Pins of the oracle's query build and cache write: the E4M3 encoder against torch's
cast, the rotary embedding against closed forms, the absorbed query against a
pure-Python brute force and one-hot cases that expose a transposed weight."""
import math

import numpy as np
import pytest
import torch

import oracle
from absorbed_mla_split_amd import workloads as wl


def _torch_codes(x32):
    return torch.from_numpy(np.ascontiguousarray(x32, np.float32)).to(torch.float8_e4m3fn) \
        .view(torch.uint8).numpy()


def test_e4m3_encode_matches_torch_cast():
    table = oracle.e4m3_table()
    vals = table[np.isfinite(table)].astype(np.float32)
    mids = ((np.sort(vals)[1:] + np.sort(vals)[:-1]) / 2).astype(np.float32)   # exact ties
    rng = np.random.default_rng(0)
    rnd = (rng.standard_normal(20000) * np.exp(rng.uniform(-12, 6, 20000))).astype(np.float32)
    rnd = np.clip(rnd, -448, 448)
    for x in (vals, mids, rnd, np.array([0.0, -0.0, 448.0, -448.0, 2.0 ** -10, 2.0 ** -9 * 1.5],
                                        np.float32)):
        got = oracle.e4m3_encode(x.astype(np.float64))
        ref = _torch_codes(x)
        assert np.array_equal(got, ref), x[got != ref][:5]
    # saturation of out-of-range values (clip, then cast)
    assert oracle.e4m3_encode(np.array([1e6, -500.0])).tolist() == [0x7E, 0xFE]


def test_bf16_round_matches_torch_cast():
    rng = np.random.default_rng(7)
    x = (rng.standard_normal(50000) * np.exp(rng.uniform(-20, 20, 50000))).astype(np.float32)
    # exact ties between neighbouring BF16 values, both parities
    b = oracle.bf16_values(rng.integers(0x0080, 0x7F00, 2000).astype(np.uint16))
    ties = (b * (1 + 2.0 ** -8)).astype(np.float32)
    for v in (x, ties, np.array([0.0, -0.0, 1.0, -3.0], np.float32)):
        ref = torch.from_numpy(v).to(torch.bfloat16).double().numpy()
        assert np.array_equal(oracle.bf16_round(v.astype(np.float64)), ref)


def test_rope_closed_forms():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((3, 64))
    one, zero = np.ones((3, 32)), np.zeros((3, 32))
    for neox in (False, True):
        assert np.array_equal(oracle.rope(x, one, zero, neox), x)
        r = oracle.rope(x, zero, one, neox)                     # a quarter turn
        if neox:
            assert np.array_equal(r[:, :32], -x[:, 32:]) and np.array_equal(r[:, 32:], x[:, :32])
        else:
            assert np.array_equal(r[:, 0::2], -x[:, 1::2]) and np.array_equal(r[:, 1::2], x[:, 0::2])
        a, b = rng.uniform(-3, 3, (3, 32)), rng.uniform(-3, 3, (3, 32))
        two = oracle.rope(oracle.rope(x, np.cos(a), np.sin(a), neox), np.cos(b), np.sin(b), neox)
        assert np.allclose(two, oracle.rope(x, np.cos(a + b), np.sin(a + b), neox), atol=1e-12)


def _inputs(n, H, seed=0, max_pos=4096):
    return wl.query_build_inputs(n, H, seed=seed, max_pos=max_pos)


def test_query_build_brute_force():
    inp = _inputs(3, 2, seed=4)
    q, rows = oracle.build_query_and_cache(inp.q, inp.w_uk, inp.kv_c, inp.k_pe, inp.positions,
                                           inp.cos_sin, inp.neox)
    qv = oracle.bf16_values(inp.q)
    wv = oracle.bf16_values(inp.w_uk)            # [h][l][c]
    for t in range(3):
        for h in range(2):
            for l in (0, 1, 77, 511):
                ref = math.fsum(qv[t, h, c] * wv[h, l, c] for c in range(128))
                assert abs(q[t, h, l] - ref) <= 1e-12 * (1 + abs(ref))
            cs = inp.cos_sin[inp.positions[t]]
            for i in range(32):
                c, s = float(cs[i]), float(cs[32 + i])
                j0, j1 = (i, i + 32) if inp.neox else (2 * i, 2 * i + 1)
                x0, x1 = qv[t, h, 128 + j0], qv[t, h, 128 + j1]
                assert abs(q[t, h, 512 + j0] - (x0 * c - x1 * s)) <= 1e-12
                assert abs(q[t, h, 512 + j1] - (x1 * c + x0 * s)) <= 1e-12
    assert np.array_equal(rows[:, :512], oracle.bf16_values(inp.kv_c))


def test_query_build_one_hot_picks_the_weight_column():
    # q_nope = e_c for token t: ql_nope[t, h, :] = W_UK_T[h, c, :], stored [h][:, c]
    inp = _inputs(4, 3, seed=5)
    qb = inp.q.copy()
    qb[:, :, :128] = 0
    cs = [3, 64, 127, 0]
    for t, c in enumerate(cs):
        qb[t, :, c] = 0x3F80
    q, _ = oracle.build_query_and_cache(qb, inp.w_uk, inp.kv_c, inp.k_pe, inp.positions,
                                        inp.cos_sin, inp.neox)
    wv = oracle.bf16_values(inp.w_uk)
    for t, c in enumerate(cs):
        for h in range(3):
            assert np.array_equal(q[t, h, :512], wv[h, :, c])
            assert not np.array_equal(q[t, h, :512], wv[(h + 1) % 3, :, c])


def test_valid_code_interval_contains_the_exact_cast():
    rng = np.random.default_rng(2)
    y = rng.standard_normal(5000) * 30
    lo, hi = oracle.e4m3_valid_codes(y, 2.0 ** -8)
    t = oracle.e4m3_table()
    exact = t[oracle.e4m3_encode(y)]
    a, b = np.minimum(t[lo], t[hi]), np.maximum(t[lo], t[hi])
    assert np.all((a <= exact) & (exact <= b))
    assert np.mean(lo == hi) > 0.9          # most values are far from a rounding tie


def test_pins_catch_build_mutants(monkeypatch):
    real_rope = oracle.rope
    mutants = {
        "sin_sign": lambda x, c, s, n: real_rope(x, c, -s, n),
        "pairing": lambda x, c, s, n: real_rope(x, c, s, not n),
        "cos_sin_swapped": lambda x, c, s, n: real_rope(x, s, c, n),
    }
    for name, fn in mutants.items():
        monkeypatch.setattr(oracle, "rope", fn)
        caught = False
        for pin in (test_rope_closed_forms, test_query_build_brute_force):
            try:
                pin()
            except AssertionError:
                caught = True
                break
        monkeypatch.setattr(oracle, "rope", real_rope)
        assert caught, name


def _torch_scaled_cast(x, scale):
    """The FP32-scaled E4M3 cast computed by torch alone: the FP32 value times the FP32
    reciprocal of the FP32 scale (torch's FP32 product), clipped to +-448 (torch's cast
    turns larger values into NaN), then torch's float8_e4m3fn cast."""
    xt = torch.tensor(np.asarray(x, dtype=np.float64), dtype=torch.float32)
    inv = torch.tensor(1.0, dtype=torch.float32) / torch.tensor(scale, dtype=torch.float32)
    y = torch.clamp(xt * inv, -448.0, 448.0)
    return y.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _cast_cases(scale):
    """BF16 values whose scaled quotient lands on or next to every E4M3 rounding midpoint,
    plus random BF16 values of every magnitude up to past saturation."""
    t = oracle.e4m3_table()[:0x7F]
    mids = (t[:-1] + t[1:]) / 2
    near = np.concatenate([mids, -mids, mids * (1 + 2.0 ** -9), mids * (1 - 2.0 ** -9)])
    rng = np.random.default_rng(7)
    rand = rng.standard_normal(20000) * np.exp2(rng.uniform(-12, 10, 20000))
    return oracle.bf16_round(np.concatenate([near, rand]) * scale)


@pytest.mark.parametrize("scale", [6.3 / 448, 1.0 / 64, 0.37, 2.5e-3])
def test_scaled_cast_matches_torch_fp32_route(scale):
    # pins e4m3_cast_scaled by a route that shares none of its code: every code equal to
    # torch's FP32 product and float8 cast, on tie-adjacent and random values
    x = _cast_cases(scale)
    got = oracle.e4m3_cast_scaled(x, scale)
    ref = _torch_scaled_cast(x, scale)
    assert np.array_equal(got, ref), np.count_nonzero(got != ref)


def test_scaled_cast_cases_tell_fp32_from_exact_division():
    # the case set above is sharp: with the synthetic query scale an exact division settles
    # some of its ties differently from the FP32 product (so a cast written with one would
    # fail the pin written with the other)
    scale = 6.3 / 448
    x = _cast_cases(scale)
    exact = oracle.e4m3_encode(np.asarray(x, dtype=np.float64) / scale)
    assert np.count_nonzero(exact != _torch_scaled_cast(x, scale)) > 0
    # a known tie: 50 * fp32(scale) / scale is exactly between 48 and 52; the FP32 product
    # lands just off it
    x1 = np.array([50.0 * np.float32(scale)])
    assert oracle.e4m3_cast_scaled(x1, scale)[0] == _torch_scaled_cast(x1, scale)[0]
