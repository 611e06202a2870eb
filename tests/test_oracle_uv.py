"""Pins of the oracle's value stage (the W_UV up-projection after the merge), each
against something other than the oracle itself: torch's BF16 cast, a pure-Python brute
force with its own BF16 decode, and closed forms that expose a wrong head, a transposed
weight or a wrong row order."""
import math
import struct

import numpy as np
import torch

import oracle
from absorbed_mla_split_amd import workloads as wl


def _bf16_py(bits):
    # independent decode: the BF16 pattern is the high half of a big-endian float32
    return struct.unpack(">f", struct.pack(">HH", int(bits), 0))[0]


def test_bf16_decode_all_patterns_match_torch():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = oracle.bf16_values(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert oracle.bf16_values(np.array([0x3F80, 0xC000, 0x7F80], np.uint16)).tolist() == [1.0, -2.0, math.inf]


def test_uv_project_brute_force():
    rng = np.random.default_rng(5)
    R, k, H = 2, 2, 3
    M = k * H
    lat = rng.standard_normal((R, M, 512))
    w = wl.uv_weights(H, seed=3)
    got = oracle.uv_project(lat, w, H)
    for r in range(R):
        for i in range(M):
            t, h = divmod(i, H)
            for v in range(0, 128, 9):
                ref = math.fsum(lat[r, i, c] * _bf16_py(w[h, v, c]) for c in range(512))
                assert abs(got[r, i, v] - ref) <= 1e-12 * (1 + abs(ref)), (r, i, v)


def test_uv_project_one_hot_rows_pick_their_heads_weights():
    # latent row (r, i) = e_c with c depending on the row: the output is W_UV[h(i), c, :],
    # i.e. storage [h][:, c]; distinct weights make a wrong head, a transposed weight or a
    # token-major/head-major mix-up visible
    R, k, H = 2, 3, 4
    M = k * H
    w = wl.uv_weights(H, seed=9)
    wv = oracle.bf16_values(w)
    lat = np.zeros((R, M, 512))
    cs = {}
    for r in range(R):
        for i in range(M):
            c = (37 * (r * M + i) + 11) % 512
            cs[(r, i)] = c
            lat[r, i, c] = 1.0
    got = oracle.uv_project(lat, w, H)
    for (r, i), c in cs.items():
        h = i % H
        assert np.array_equal(got[r, i], wv[h, :, c]), (r, i)
        assert not np.array_equal(got[r, i], wv[(h + 1) % H, :, c])


def test_uv_project_selection_weights_closed_form():
    # W_UV[h, c, v] = 1 when c = v + 128 * (h % 4), else 0: the output is a 128-wide slice
    # of the latent that moves with the head
    H, R, k = 4, 3, 2
    M = k * H
    bits = np.zeros((H, 128, 512), np.uint16)
    for h in range(H):
        for v in range(128):
            bits[h, v, v + 128 * (h % 4)] = 0x3F80          # BF16 1.0
    lat = np.random.default_rng(1).standard_normal((R, M, 512))
    got = oracle.uv_project(lat, bits, H)
    for i in range(M):
        h = i % H
        assert np.array_equal(got[:, i, :], lat[:, i, 128 * h:128 * h + 128])


def test_uv_project_is_linear_and_zero_on_empty_rows():
    H = 2
    w = wl.uv_weights(H, seed=4)
    rng = np.random.default_rng(2)
    a, b = rng.standard_normal((2, 1, 2 * H, 512))
    pa, pb = oracle.uv_project(a, w, H), oracle.uv_project(b, w, H)
    assert np.allclose(oracle.uv_project(2 * a - b, w, H), 2 * pa - pb, rtol=0, atol=1e-12)
    assert np.all(oracle.uv_project(np.zeros((1, 2 * H, 512)), w, H) == 0)


def test_uv_weights_layout_and_scale():
    w = wl.uv_weights(8, seed=0)
    assert w.shape == (8, 128, 512) and w.dtype == np.uint16
    v = oracle.bf16_values(w)
    assert abs(v.std() * math.sqrt(512) - 1) < 0.01
    assert np.array_equal(w, wl.uv_weights(8, seed=0))


def _mutants(real):
    def wrong_head(latent, bits, heads):          # head from the token index
        lat = np.asarray(latent, np.float64)
        w = oracle.bf16_values(bits).reshape(heads, 128, 512)
        k = lat.shape[1] // heads
        out = np.empty(lat.shape[:2] + (128,))
        for i in range(lat.shape[1]):
            out[:, i] = lat[:, i] @ w[(i // k) % heads].T
        return out

    def transposed(latent, bits, heads):          # weight read as [H][512][128]
        lat = np.asarray(latent, np.float64)
        w = oracle.bf16_values(bits).reshape(heads, 512, 128)
        out = np.empty(lat.shape[:2] + (128,))
        for h in range(heads):
            out[:, h::heads] = lat[:, h::heads] @ w[h]
        return out

    def truncated_k(latent, bits, heads):         # drops the last 64 latent dims
        lat = np.array(latent, np.float64)
        lat[..., 448:] = 0
        return real(lat, bits, heads)

    def bf16_low_bits(latent, bits, heads):       # decodes the pattern as the low half
        lat = np.asarray(latent, np.float64)
        w = np.asarray(bits, np.uint16).astype(np.uint32).view(np.float32).astype(np.float64)
        w = w.reshape(heads, 128, 512)
        out = np.empty(lat.shape[:2] + (128,))
        for h in range(heads):
            out[:, h::heads] = lat[:, h::heads] @ w[h].T
        return out

    return {"wrong_head": wrong_head, "transposed": transposed, "truncated_k": truncated_k,
            "bf16_low_bits": bf16_low_bits}


PINS = [test_uv_project_brute_force, test_uv_project_one_hot_rows_pick_their_heads_weights,
        test_uv_project_selection_weights_closed_form]


def test_pins_catch_value_stage_mutants(monkeypatch):
    real = oracle.uv_project
    for name, fn in _mutants(real).items():
        monkeypatch.setattr(oracle, "uv_project", fn)
        caught = False
        for pin in PINS:
            try:
                pin()
            except (AssertionError, ValueError, IndexError):
                caught = True
                break
        monkeypatch.setattr(oracle, "uv_project", real)
        assert caught, f"no pin caught the mutant {name}"
