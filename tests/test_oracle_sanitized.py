"""The oracle's C code built with the address and undefined-behaviour sanitizers (host
code only) and run on the inputs the pins use: a ragged decode with NaN-poisoned slots
past the lengths and in unused pages, split plans of several batches in both modes, and
LSE merges with -inf partials.  Any out-of-bounds access, use of freed memory or
undefined arithmetic aborts the run; the results must equal the regular build's bit for
bit."""
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
from absorbed_mla_split_amd import workloads as wl

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    d = tmp_path_factory.mktemp("asan")
    exe = str(d / "oracle_driver")
    cmd = ["gcc", "-std=c99", "-O1", "-g", "-fopenmp", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           os.path.join(ROOT, "oracle", "oracle.c"), os.path.join(HERE, "asan", "oracle_driver.c"),
           "-o", exe, "-lm"]
    subprocess.run(cmd, check=True, capture_output=True)
    return exe, d


def run(driver, mode, payload, n_out_bytes):
    exe, d = driver
    fin, fout = str(d / f"{mode}.in"), str(d / f"{mode}.out")
    with open(fin, "wb") as f:
        f.write(payload)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="4")
    res = subprocess.run([exe, mode, fin, fout], capture_output=True, text=True, env=env)
    assert res.returncode == 0, res.stderr[-3000:]
    data = open(fout, "rb").read()
    assert len(data) == n_out_bytes
    return data


def test_sanitized_attend_matches(driver):
    w = wl.small(3, 4, 8, [200, 0, 317], seed=5)       # ragged, an empty request, poison
    tasks = [(r, i, 0, int(w.lengths[r])) for r in range(w.R) for i in range(w.M)]
    tasks += [(2, 5, 60, 130), (0, 31, 199, 200), (2, 0, 0, 0)]
    tasks = np.array(tasks, dtype=np.int32)
    R, M = w.R, w.M
    cols, pool = w.block_table.shape[1], w.kv8.shape[0]
    payload = (np.array([R, M, cols, pool, len(tasks)], np.int32).tobytes()
               + np.array([w.q_scale, w.k_scale, w.sm_scale], np.float64).tobytes()
               + w.q8.tobytes() + w.kv8.tobytes() + w.block_table.astype(np.int32).tobytes()
               + w.lengths.astype(np.int32).tobytes() + tasks.tobytes())
    n = len(tasks)
    data = run(driver, "attend", payload, 4 + n * 512 * 8 + n * 8)
    rc = np.frombuffer(data[:4], np.int32)[0]
    out = np.frombuffer(data[4:4 + n * 4096], np.float64).reshape(n, 512)
    lse = np.frombuffer(data[4 + n * 4096:], np.float64)
    ref_out, ref_lse = oracle.attend(w.q8, w.kv8, w.block_table, w.lengths, tasks, w.q_scale,
                                     w.k_scale, w.sm_scale)
    assert rc == 0
    assert np.array_equal(out, ref_out) and np.array_equal(lse, ref_lse)


@pytest.mark.parametrize("lengths,M,MT,W,ms,mode,cost", [
    ([200, 317], 32, 32, 256, 256, 0, 0),
    ([0, 0, 5, 64 * 300, 1], 56, 64, 40, 0, 0, 3),
    ([8192] * 64, 32, 32, 256, 256, 1, 4),
    ([131072] + [1024] * 15, 448, 128, 256, 256, 0, 4),
    (list(range(0, 5000, 37)), 256, 128, 96, 64, 1, 0),
])
def test_sanitized_plan_matches(driver, lengths, M, MT, W, ms, mode, cost):
    R = len(lengths)
    list_len = 2 * (R + 2 * W)
    cols = max(1, max((l + 63) // 64 for l in lengths))
    lens = np.array(lengths, np.int32)
    payload = (np.array([R, cols, M, MT, W, ms, 256, cost, mode, list_len], np.int32).tobytes() +
               lens.tobytes())
    data = np.frombuffer(run(driver, "plan", payload, 4 * (1 + R + R + 1 + list_len)), np.int32)
    counts, offsets, work, n = oracle.plan(lens, cols, M, MT, W, min_split_tokens=ms,
                                           mode=mode, list_len=list_len, split_cost=cost)
    assert data[0] == n
    assert np.array_equal(data[1:1 + R], counts)
    assert np.array_equal(data[1 + R:2 + 2 * R], offsets)
    assert np.array_equal(data[2 + 2 * R:], work)


def test_sanitized_merge_matches(driver):
    rng = np.random.default_rng(3)
    o = rng.standard_normal((5, 512))
    lse = np.array([1.5, -np.inf, 30.0, -2.0, -np.inf])
    payload = np.array([5], np.int32).tobytes() + o.tobytes() + lse.tobytes()
    data = np.frombuffer(run(driver, "merge", payload, 513 * 8), np.float64)
    ref, ref_lse = oracle.merge(o, lse)
    assert np.array_equal(data[:512], ref) and data[512] == ref_lse
    payload = np.array([2], np.int32).tobytes() + o[:2].tobytes() + np.full(2, -np.inf).tobytes()
    data = np.frombuffer(run(driver, "merge", payload, 513 * 8), np.float64)
    assert np.all(data[:512] == 0) and np.isneginf(data[512])
