"""GPU decode context parallelism on one GPU vs the CPU oracle.

A global workload's KV is split over `world` simulated ranks (interleaved blocks); every
rank runs plan + the DCP decode over its shard (the causal mask in global positions, or
none) + the reducer; the head owner's merge over the sources then gives the rows of the
unsharded decode.  Checks, through the C ABI:
  - every rank's rows and LSE against the oracle's decode of that rank's visible keys, at
    the attention bar (1.5e-2 max|V_hat|, 1e-3 log2, -inf exact);
  - the merge over sources against the oracle's merge of the GPU's own BF16 source rows
    (one BF16 rounding plus FP32 accumulation: 2^-8 |ref| + 2^-16 max_s |row_s|);
  - the merged rows against the oracle's unsharded (causal) decode: the sources' bar plus
    the merge's rounding (1.5e-2 max|V_hat| + 2^-9 max|V_hat|), LSE 1e-3;
  - with causal = 0, the DCP decode equals the plain decode bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
from absorbed_mla_split_amd import binding
from absorbed_mla_split_amd import workloads as wl
from gpu_util import LSE_TOL, OUT_TOL, to_dev, vmax

pytestmark = pytest.mark.gpu


def run_rank(s, totals, heads, world, rank, interleave, causal, min_split_tokens=256,
             workers=None, plain=False):
    q, kv, bt, lengths = to_dev(s)
    tot = torch.from_numpy(np.asarray(totals, np.int32)).cuda()
    dec = binding.FoldedDecoder(s.R, s.M, min_split_tokens=min_split_tokens, workers=workers)
    dec.workspace[256:].fill_(0xFF)
    out = torch.full((s.R, s.M, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((s.R, s.M), float("nan"), dtype=torch.float32, device="cuda")
    dec.plan(lengths, bt.shape[1])
    bmm1, bmm2 = binding.bmm_scales(s.sm_scale, s.q_scale, s.k_scale)
    R = s.R
    if plain:
        binding.folded_decode(q, kv, bt, lengths, dec.params, bmm1, bmm2, dec.counts[:R],
                              dec.offsets[:R + 1], dec.work, dec.workspace)
    else:
        dcp = binding.DcpParams(heads, int(causal), world, rank, interleave)
        binding.folded_decode_dcp(q, kv, bt, lengths, dec.params, bmm1, bmm2, dec.counts[:R],
                                  dec.offsets[:R + 1], dec.work, dec.workspace, dcp, tot)
    binding.combine(dec.workspace, dec.counts[:R], dec.offsets[:R + 1], R, dec.params,
                    dec.compute_units, out, lse)
    torch.cuda.synchronize()
    assert dec.device_status() == 0, binding.status_string(dec.device_status())
    return out, lse


def check_rows(got, got_lse, ref, ref_lse, bound, tag):
    empty = np.isneginf(ref_lse)
    assert np.array_equal(np.isneginf(got_lse), empty), f"{tag}: -inf LSE mismatch"
    assert np.all(np.isfinite(got)), f"{tag}: non-finite rows"
    assert np.all(got[empty] == 0), f"{tag}: empty rows not zero"
    err = float(np.max(np.abs(got - ref)))
    lerr = float(np.max(np.abs(got_lse[~empty] - ref_lse[~empty]), initial=0))
    print(f"[{tag}] err {err:.3e} (bound {bound:.3e}) lse {lerr:.2e}", flush=True)
    assert err <= bound and lerr <= LSE_TOL, tag


def run_dcp(w, k, H, world, interleave, causal, **kw):
    shards = wl.dcp_shards(w, world, interleave)
    vm = vmax(w)
    outs, lses = [], []
    for d, s in enumerate(shards):
        out, lse = run_rank(s, w.lengths, H, world, d, interleave, causal, **kw)
        o = out.float().cpu().numpy().reshape(-1, 512)
        l = lse.cpu().numpy().reshape(-1)
        ro, rl = oracle.decode_dcp_rank(s.q8, s.kv8, s.block_table, s.lengths, w.lengths, k, H,
                                        w.q_scale, w.k_scale, w.sm_scale, world, d, interleave,
                                        causal=causal)
        check_rows(o, l, ro, rl, OUT_TOL * vm, f"rank {d}/{world} I{interleave} c{int(causal)}")
        outs.append(out)
        lses.append(lse)
    rows = torch.stack(outs).contiguous()
    lse_s = torch.stack(lses).contiguous()
    n = w.R * w.M
    merged = torch.full((n, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
    mlse = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
    binding.merge_sources(rows, lse_s, merged, mlse)
    torch.cuda.synchronize()
    got = merged.float().cpu().numpy()
    got_lse = mlse.cpu().numpy()
    # the merge itself, on the GPU's own source rows
    src = rows.float().cpu().numpy().reshape(world, n, 512)
    ro, rl = oracle.merge_sources(src, lse_s.cpu().numpy().reshape(world, n))
    # one BF16 rounding of the result, plus FP32 accumulation over at most 64 sources
    bound = 2.0 ** -8 * np.abs(ro) + 2.0 ** -16 * np.abs(src).max(axis=0)
    merr = np.abs(got - ro)
    print(f"[merge {world}] max err {merr.max():.3e}, worst margin {(merr - bound).max():.3e}",
          flush=True)
    assert np.all(merr <= bound), "merge over sources"
    fin = np.isfinite(rl)
    assert np.array_equal(fin, np.isfinite(got_lse))
    assert np.max(np.abs(got_lse[fin] - rl[fin]), initial=0) <= 1e-5
    # end to end against the unsharded decode
    ref, ref_lse = oracle.decode_causal(w.q8, w.kv8, w.block_table, w.lengths, k, H, w.q_scale,
                                        w.k_scale, w.sm_scale, causal=causal)
    check_rows(got, got_lse, ref, ref_lse, (OUT_TOL + 2.0 ** -9) * vm,
               f"merged {world} I{interleave} c{int(causal)}")


CASES = [
    # (k, H, lengths, world, interleave)
    (4, 8, [300, 1000, 64 * 9 + 5, 33], 2, 1),
    (4, 8, [300, 1000, 64 * 9 + 5, 33], 8, 64),        # a request on one rank only
    (7, 8, [2047, 513, 130], 4, 16),                   # M = 56
    (2, 64, [1500, 64, 700], 3, 1),                    # M = 128
    (7, 64, [900, 2000], 2, 256),                      # M = 448
    (4, 8, [5000, 64], 1, 1),                          # one rank: the plain causal decode
]


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("k,H,lengths,world,interleave", CASES)
def test_dcp_ranks_and_merge(k, H, lengths, world, interleave, causal):
    w = wl.small(len(lengths), k, H, lengths, seed=k + H + world)
    run_dcp(w, k, H, world, interleave, causal)


def test_fully_masked_splits():
    # one-page splits: the rows of early tokens see none of the last split's keys
    k, H = 16, 2
    w = wl.small(2, k, H, [130, 64 * 3 + 10], seed=31)
    run_dcp(w, k, H, 1, 1, True, min_split_tokens=0)


def test_non_causal_dcp_equals_plain_decode():
    k, H = 4, 8
    w = wl.small(3, k, H, [700, 2500, 64], seed=12)
    s = wl.dcp_shards(w, 2, 64)[1]
    a = run_rank(s, w.lengths, H, 2, 1, 64, False)
    b = run_rank(s, w.lengths, H, 2, 1, 64, False, plain=True)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_totals_that_disagree_with_the_shard_are_flagged():
    k, H = 4, 8
    w = wl.small(2, k, H, [700, 300], seed=5)
    s = wl.dcp_shards(w, 2, 1)[0]
    q, kv, bt, lengths = to_dev(s)
    bad_totals = torch.from_numpy(w.lengths + np.int32(64)).cuda()
    dec = binding.FoldedDecoder(s.R, s.M)
    dec.plan(lengths, bt.shape[1])
    b1, b2 = binding.bmm_scales(s.sm_scale, s.q_scale, s.k_scale)
    binding.folded_decode_dcp(q, kv, bt, lengths, dec.params, b1, b2, dec.counts[:s.R],
                              dec.offsets[:s.R + 1], dec.work, dec.workspace,
                              binding.DcpParams(H, 1, 2, 0, 1), bad_totals)
    torch.cuda.synchronize()
    assert dec.device_status() & binding.DEV_BAD_LENGTH


@pytest.mark.parametrize("rank", [0, 7])
def test_c4_rank_of_eight_sampled(rank):
    # c4's requests as the global cache of an 8-way interleaved DCP, one rank's causal decode
    w = wl.generate("c4")
    k, H, world = w.cfg.k, w.cfg.H, 8
    s = wl.dcp_shards(w, world, 1)[rank]
    out, lse = run_rank(s, w.lengths, H, world, rank, 1, True)
    rows = [(r, i) for r in (0, 13, 31) for i in (0, 63, 64, 191, 255)]
    o = out.float().cpu().numpy()
    l = lse.cpu().numpy()
    got = np.stack([o[r, i] for r, i in rows])
    gl = np.array([l[r, i] for r, i in rows])
    ro, rl = oracle.decode_dcp_rank(s.q8, s.kv8, s.block_table, s.lengths, w.lengths, k, H,
                                    w.q_scale, w.k_scale, w.sm_scale, world, rank, 1,
                                    causal=True, rows=rows)
    check_rows(got, gl, ro, rl, OUT_TOL * vmax(s), f"c4 rank {rank}/8")
