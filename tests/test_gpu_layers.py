"""One decode step as a model runs it: one split plan, reused by the decode and the
reducer of several layers, captured into one HIP graph and replayed; every layer's output
is compared with the CPU oracle's decode of that layer's query and cache.

Page "...runtime.providers", class Attention: only the first MLA layer of a step plans, the
later ones reuse its plan.  Page "...cutedsl.mla.balanced", BalancedMla.plan: the plan is
made once per step from the lengths.  Each layer here has its own query rows and its own
cache pool behind the same block tables (the lengths, and so the plan, are the step's).
Also here: the fixed-split comparator plan on the log-uniform workload at full size.
"""
import numpy as np
import pytest
import torch

from absorbed_mla_split_amd import binding
from absorbed_mla_split_amd import workloads as wl
from gpu_util import compare, run_gpu, sample_rows

pytestmark = pytest.mark.gpu

LAYERS = 4


@pytest.mark.parametrize("k,H,lengths", [
    (4, 8, [3000, 100, 0, 1500, 6000]),        # 32 rows: decode32
    (7, 8, [2500, 64, 9000, 700]),             # 56 rows: decode64
    (4, 64, [1800, 0, 130, 3000]),             # 256 rows: decode128, two row tiles
])
def test_one_plan_many_layers_in_a_graph(k, H, lengths):
    w0 = wl.small(len(lengths), k, H, lengths, seed=31 + k * H)
    ws = wl.layers(w0, LAYERS, seed=7)
    dev = torch.device("cuda")
    bt = torch.from_numpy(w0.block_table).to(dev)
    lens = torch.from_numpy(w0.lengths).to(dev)
    qs = [torch.from_numpy(w.q8).to(dev) for w in ws]
    kvs = [torch.from_numpy(w.kv8).to(dev) for w in ws]
    R, M = w0.R, w0.M
    outs = [torch.empty((R, M, 512), dtype=torch.bfloat16, device=dev) for _ in ws]
    lses = [torch.empty((R, M), dtype=torch.float32, device=dev) for _ in ws]
    scales = [binding.bmm_scales(w.sm_scale, w.q_scale, w.k_scale) for w in ws]
    dec = binding.FoldedDecoder(R, M)
    dec.workspace[256:].fill_(0xFF)               # FP32 NaN pattern in every partial

    def step():
        dec.plan(lens, bt.shape[1])
        for li in range(LAYERS):
            dec.decode(qs[li], kvs[li], bt, lens, scales[li][0], scales[li][1], outs[li],
                       lses[li])

    # warm up eagerly (the library allocates nothing, so capture may follow directly)
    step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()

    first = None
    for rep in range(3):
        for o, l in zip(outs, lses):
            o.fill_(float("nan"))
            l.fill_(float("nan"))
        dec.workspace[256:].fill_(0xFF)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert dec.device_status() == 0
        got = [(o.float().cpu().numpy(), l.cpu().numpy()) for o, l in zip(outs, lses)]
        if first is None:
            first = got
            for li, (w, (o, l)) in enumerate(zip(ws, got)):
                compare(w, o, l, tag=f"layer{li} M{M}")
        else:   # every replay gives the first replay's results, bit for bit
            for (a, b), (c, d) in zip(first, got):
                assert np.array_equal(a, c, equal_nan=False) and np.array_equal(b, d)
    # the layers really differ (each read its own cache)
    assert not np.array_equal(first[0][0], first[1][0])


def test_c3_fixed_plan_full_size_sampled():
    # the comparator of page "...cutedsl.mla.balanced" (equal split counts for every
    # request) on the log-uniform batch, at full size, in the benchmark's launch shape
    w = wl.generate("c3")
    out, lse, dec = run_gpu(w, mode=binding.PLAN_FIXED)
    assert dec.device_status() == 0
    counts = dec.plan_host()[0]
    assert len(set(counts.tolist())) == 1          # one split count for every request
    compare(w, out, lse, rows=sample_rows(w, 2), tag="c3-fixed")
