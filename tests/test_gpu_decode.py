"""GPU folded split-KV decode + combine vs the CPU oracle, element by element.

Small cases (every row) span several 64-key pages, ragged tails, empty requests, several
splits per request and every row-tile shape; the five workload configurations run at full
size in the benchmark's launch configuration and are checked on sampled rows.  Inputs
carry NaN codes in every cache slot past a request's length and in unused pages, and the
outputs, LSE and workspace start as NaN.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from absorbed_mla_split_amd import binding
from absorbed_mla_split_amd import workloads as wl
from gpu_util import compare, run_gpu, sample_rows, to_dev, ws_partials, vmax, LSE_TOL, OUT_TOL

pytestmark = pytest.mark.gpu


def test_c1_every_row():
    w = wl.generate("c1")
    out, lse, dec = run_gpu(w)
    counts, offsets, work, n = dec.plan_host()
    assert counts.tolist() == [1, 1]             # 4 + 5 pages, 4-page minimum: no cut inside
    compare(w, out, lse, tag="c1")
    assert dec.device_status() == 0


@pytest.mark.parametrize("workers", [4, 6])
def test_c1_split_partials_match_oracle_chunks(workers):
    # 4 workers, one-page minimum, no split cost: cuts at pages 2, 4 (the request boundary)
    # and 6, so both requests are cut in two; 6 workers: cuts 1, 3, 4, 6, 7
    w = wl.generate("c1")
    out, lse, dec = run_gpu(w, min_split_tokens=0, workers=workers, split_cost=0)
    counts, offsets, work, n = dec.plan_host()
    assert counts.tolist() == ([2, 2] if workers == 4 else [3, 3])
    part, plse = ws_partials(dec, w)
    vm = vmax(w)
    for i in range(n):
        r, a, b = oracle.item_range(work, n, w.lengths, i)
        tasks = [(r, j, a, b) for j in range(w.M)]
        ro, rl = oracle.attend(w.q8, w.kv8, w.block_table, w.lengths, tasks, w.q_scale,
                               w.k_scale, w.sm_scale)
        err = np.max(np.abs(part[i] - ro))      # item i's workspace slot is i
        assert err <= OUT_TOL * vm, (r, a, b, err)
        assert np.max(np.abs(plse[i] - rl)) <= 1e-3, (r, a, b)
    compare(w, out, lse, tag=f"c1-W{workers}")


SHAPES = [
    # (k, H, lengths)
    (4, 2, [1, 63, 64, 65]),
    (4, 8, [200, 317, 0, 1000]),
    (7, 8, [513, 2047, 64 * 9 + 5]),
    (2, 32, [130, 1]),
    (3, 32, [700, 0, 0, 129]),
    (4, 64, [1500, 64]),
    (3, 11, [300, 64]),          # M = 33: a 64-row tile with one row in its second block
    (5, 13, [129, 700]),         # M = 65: a 128-row tile with one row in its third block
    (3, 43, [100, 640]),         # M = 129: two 128-row tiles, the second with one row
    (16, 64, [70]),              # M = 1024, the most rows per request
    (7, 64, [1025, 3000]),
    (1, 3, [77, 500]),
]


@pytest.mark.parametrize("k,H,lengths", SHAPES)
@pytest.mark.parametrize("min_split_tokens", [0, 256])
def test_small_shapes_every_row(k, H, lengths, min_split_tokens):
    w = wl.small(len(lengths), k, H, lengths, seed=k * 100 + H)
    out, lse, dec = run_gpu(w, min_split_tokens=min_split_tokens)
    compare(w, out, lse, tag=f"k{k}H{H}L{lengths}ms{min_split_tokens}")
    assert dec.device_status() == 0


@pytest.mark.parametrize("k,H,mtile", [(4, 8, 64), (4, 8, 128), (7, 8, 32), (7, 8, 128),
                                        (4, 64, 32), (4, 64, 64), (3, 11, 128), (7, 64, 128),
                                        (5, 13, 128), (3, 43, 128)])
def test_every_tile_size_for_any_rows(k, H, mtile):
    # the row tile is a free parameter of the ABI: every kernel on shapes it is not picked
    # for by default (several tiles per split, or most of a tile idle)
    w = wl.small(3, k, H, [1000, 64 * 7 + 3, 2500], seed=k * H + mtile)
    out, lse, dec = run_gpu(w, mtile=mtile)
    assert dec.params.mtile == mtile
    compare(w, out, lse, tag=f"M{k * H} MT{mtile}")
    assert dec.device_status() == 0


@pytest.mark.parametrize("mtile,workers", [(128, 2), (128, 5), (64, 4), (32, 3)])
def test_short_units_back_to_back(mtile, workers):
    # few workers, many requests of one to five pages (ragged last pages): each worker runs
    # many short units in a row, so the page ring is refilled across unit ends over and over
    # (the 128-row kernel's spare copy of a unit's last page, and its wait before the next
    # unit's first DMA; the stream kernel's ring that runs on across units)
    lengths = [1, 63, 64, 65, 130, 200, 257, 300, 5, 128, 192, 319]
    w = wl.small(len(lengths), 4, 64 if mtile != 32 else 8, lengths, seed=mtile + workers)
    out, lse, dec = run_gpu(w, mtile=mtile, workers=workers)
    assert dec.params.mtile == mtile and dec.params.workers == workers
    compare(w, out, lse, tag=f"short units MT{mtile} W{workers}")
    assert dec.device_status() == 0


def test_many_splits_small_workers():
    # few workers and no minimum split: long requests cut into many 1-page splits
    w = wl.small(3, 4, 8, [2000, 64 * 40, 90], seed=3)
    out, lse, _ = run_gpu(w, min_split_tokens=0, workers=96)
    compare(w, out, lse, tag="many-splits")


def test_over_64_splits_per_request():
    # 271 pages over 256 groups (at most 256 splits): 190 and 66 splits of one or two
    # pages, so the reducer holds several LSEs per lane
    w = wl.small(2, 4, 8, [64 * 200 + 5, 64 * 70], seed=6)
    out, lse, dec = run_gpu(w, min_split_tokens=0, workers=300, split_cost=0)
    assert dec.plan_host()[0].tolist() == [190, 66]
    compare(w, out, lse, tag="201-splits")


def test_most_splits_per_request():
    # 300 pages, one-page minimum and 600 workers: the split count hits its cap of 256, so
    # the reducer holds four LSEs on every lane; the second request is empty
    w = wl.small(2, 4, 8, [64 * 300, 0], seed=9)
    out, lse, dec = run_gpu(w, min_split_tokens=0, workers=600, split_cost=0)
    assert dec.plan_host()[0].tolist() == [binding.MAX_SPLITS, 0]
    compare(w, out, lse, tag="256-splits")


def test_more_requests_than_plan_threads():
    # 300 requests (some plan threads own two) of mixed short lengths, some empty
    rng = np.random.default_rng(21)
    lengths = rng.integers(0, 900, 300)
    lengths[rng.random(300) < 0.1] = 0
    w = wl.small(300, 4, 8, lengths.tolist(), seed=21)
    out, lse, dec = run_gpu(w)
    assert dec.device_status() == 0
    compare(w, out, lse, rows=sample_rows(w, 2), tag="R300")


def test_most_requests():
    # the largest batch one plan takes: 4096 requests of 1..130 keys
    rng = np.random.default_rng(22)
    lengths = rng.integers(1, 131, binding.MAX_REQS)
    w = wl.small(binding.MAX_REQS, 2, 8, lengths.tolist(), seed=22)
    out, lse, dec = run_gpu(w)
    assert dec.device_status() == 0
    rows = [(r, i) for r in range(0, binding.MAX_REQS, 97) for i in (0, 15)]
    compare(w, out, lse, rows=rows, tag="R4096")


@pytest.mark.parametrize("mode", [binding.PLAN_BALANCED, binding.PLAN_FIXED])
def test_plans_agree(mode):
    w = wl.small(5, 7, 8, [3000, 100, 6000, 64, 9000], seed=2)
    out, lse, _ = run_gpu(w, mode=mode)
    compare(w, out, lse, tag=f"mode{mode}")


def test_fold_equals_unfolded_rows():
    # [R*k, H, D] folded to [R, k*H, D] vs the stock layout: R*k requests of H rows with
    # row-replicated block tables and lengths.
    R, k, H = 3, 4, 8
    w = wl.small(R, k, H, [900, 333, 1200], seed=11)
    out_f, lse_f, _ = run_gpu(w)
    row_req = np.arange(R * k) // k
    wu = wl.Workload(w.cfg, w.lengths[row_req], w.block_table[row_req],
                     w.q8.reshape(R * k, H, 576), w.kv8, w.q_scale, w.k_scale)
    out_u, lse_u, _ = run_gpu(wu)
    vm = vmax(w)
    assert np.max(np.abs(out_f.reshape(R * k, H, 512) - out_u)) <= OUT_TOL * vm
    assert np.max(np.abs(lse_f.reshape(R * k, H) - lse_u)) <= 1e-3
    compare(wu, out_u, lse_u, tag="unfolded")


@pytest.mark.parametrize("k,H", [(4, 8), (7, 8), (4, 64), (3, 43)])
@pytest.mark.parametrize("peak", [120.0, 200.0])
def test_score_outliers_move_the_reference(k, H, peak):
    # Keys far above the rest of their split: the even rows of each request equal its row 0,
    # and three keys of each request (one on its first page) equal that row, so those rows
    # score `peak` (log2 units) on them and about peak/24 elsewhere.  A split whose first
    # page holds no such key sees a later page pass its reference by more than the kernels'
    # headroom (the reference moves, the output tiles are rescaled); the split holding the
    # first-page copy sees later pages far below it (down to the -127 clamp of the scale).
    w = wl.small(2, k, H, [3000, 1500], seed=k * 7 + H)
    for r in range(w.R):
        w.q8[r, 2::2, :] = w.q8[r, 0, :]
        L = int(w.lengths[r])
        for pos in (0, L // 3, (2 * L) // 3 + 5):
            w.kv8[w.block_table[r, pos // 64], pos % 64, :] = w.q8[r, 0, :]
    qv = oracle.e4m3_table()[w.q8[0, 0, :]].astype(np.float64)
    dot = float((qv * qv).sum()) * w.q_scale * w.k_scale
    w.sm_scale = peak / (dot * math.log2(math.e))
    out, lse, dec = run_gpu(w)
    counts, _, _, _ = dec.plan_host()
    assert counts.max() >= 3, counts            # several splits per request
    # The scores come from FP8 MFMAs whose FP32 sums carry an error of order 2^-16 of the
    # dot product's magnitude: at a score of `peak` log2 units the LSE may be off by that
    # much more than the usual 1e-3.
    compare(w, out, lse, tag=f"outlier k{k}H{H}p{peak}", lse_tol=LSE_TOL + peak * 2.0**-15)
    assert dec.device_status() == 0


def test_deterministic_bitwise():
    w = wl.small(4, 4, 16, [5000, 700, 64, 2500], seed=4)
    t = to_dev(w)
    a = run_gpu(w, tensors=t)
    b = run_gpu(w, tensors=t)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_empty_batch_rows():
    w = wl.small(3, 2, 8, [0, 0, 0], seed=1)
    out, lse, dec = run_gpu(w)
    assert np.all(out == 0) and np.all(np.isneginf(lse))


def test_bad_page_id_flags_status_without_fault():
    w = wl.small(2, 4, 8, [300, 200], seed=6)
    w.block_table[1, 1] = w.kv8.shape[0] + 1000          # out of the pool
    out, lse, dec = run_gpu(w)
    assert dec.device_status() & binding.DEV_BAD_PAGE


@pytest.mark.parametrize("cfg", ["c2", "c3", "c4", "c5"])
def test_full_size_sampled(cfg):
    w = wl.generate(cfg)
    out, lse, dec = run_gpu(w)
    assert dec.device_status() == 0
    compare(w, out, lse, rows=sample_rows(w, 4 if cfg != "c3" else 2), tag=cfg)


@pytest.mark.parametrize("cfg,mtile", [("c4", 64), ("c5", 128)])
def test_full_size_other_tile_sampled(cfg, mtile):
    # the tile size the launch shape does not pick for these rows (c4: 64-row tiles; c5:
    # 128-row tiles, half of the last one idle)
    w = wl.generate(cfg)
    out, lse, dec = run_gpu(w, mtile=mtile)
    assert dec.params.mtile == mtile and dec.device_status() == 0
    compare(w, out, lse, rows=sample_rows(w, 4), tag=f"{cfg}-MT{mtile}")


def test_c5_unfolded_baseline_sampled():
    # the stock flattening of c5: 112 single-token requests of 64 heads, each with its own
    # copy of the request's table (k times the KV reads)
    w = wl.generate("c5")
    R, k, H = w.cfg.R, w.cfg.k, w.cfg.H
    row_req = np.arange(R * k) // k
    wu = wl.Workload(w.cfg, w.lengths[row_req], w.block_table[row_req],
                     w.q8.reshape(R * k, H, 576), w.kv8, w.q_scale, w.k_scale)
    out, lse, _ = run_gpu(wu)
    rows = [(rr, i) for rr in (0, 3, 6, 7, 50, 111) for i in (0, 17, 63)]
    compare(wu, out, lse, rows=rows, tag="c5-unfolded")


@pytest.mark.parametrize("k,H", [(4, 8), (7, 8), (4, 64)])
def test_graph_capture_replay(k, H):
    # one case per decode kernel (32-, 64- and 128-row tiles)
    w = wl.small(4, k, H, [3000, 1000, 64, 2200], seed=8)
    q, kv, bt, lengths = to_dev(w)
    dec = binding.FoldedDecoder(w.R, w.M)
    bmm1, bmm2 = binding.bmm_scales(w.sm_scale, w.q_scale, w.k_scale)
    out = torch.empty((w.R, w.M, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.R, w.M), dtype=torch.float32, device="cuda")
    dec.plan(lengths, bt.shape[1])
    dec.decode(q, kv, bt, lengths, bmm1, bmm2, out, lse)
    torch.cuda.synchronize()
    ref_out, ref_lse = out.clone(), lse.clone()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            dec.plan(lengths, bt.shape[1])
            dec.decode(q, kv, bt, lengths, bmm1, bmm2, out, lse)
    torch.cuda.current_stream().wait_stream(s)
    for _ in range(3):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse)
