"""The allocation-free entry point (plan, decode and merge in one call, with the plan and the
split partials in the library's static device scratch) against the entry points that take
a caller workspace, on the same inputs: two calls in a row, the second with a smaller
batch, each compared with the workspace path bit for bit (the same kernels on the same
plan) and with the CPU oracle at the parity bar.  Outputs start as NaN."""
import numpy as np
import pytest
import torch

from absorbed_mla_split_amd import binding
from absorbed_mla_split_amd import workloads as wl
from gpu_util import compare, run_gpu, to_dev

pytestmark = pytest.mark.gpu


def params_for(w, workers=None):
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    W, mt = binding.decode_config(cus, w.M)
    return binding.make_params(w.M, mt, workers or W), cus


def noalloc(w, t, workers=None):
    q, kv, bt, lengths = t
    p, cus = params_for(w, workers)
    out = torch.full((w.R, w.M, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((w.R, w.M), float("nan"), dtype=torch.float32, device="cuda")
    status = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    bmm1, bmm2 = binding.bmm_scales(w.sm_scale, w.q_scale, w.k_scale)
    binding.folded_decode_noalloc(q, kv, bt, lengths, p, bmm1, bmm2, cus, out, lse, status)
    return out, lse, status


@pytest.mark.parametrize("shapes", [
    # (R, k, H, lengths, workers) of the first call, then of the smaller second call
    ((5, 4, 8, [3000, 100, 0, 1500, 6000], None), (2, 4, 8, [700, 64], None)),
    ((5, 7, 8, [2500, 64, 9000, 700, 1], None), (3, 7, 8, [200, 0, 130], None)),
    ((3, 4, 64, [1800, 130, 3000], 32), (1, 2, 64, [500], 32)),
])
def test_noalloc_matches_workspace_path(shapes):
    ws = [wl.small(R, k, H, L, seed=50 + i) for i, (R, k, H, L, _) in enumerate(shapes)]
    ts = [to_dev(w) for w in ws]
    # two calls in a row on the one scratch, the second with fewer requests and keys
    got = [noalloc(w, t, workers=s[4]) for w, t, s in zip(ws, ts, shapes)]
    torch.cuda.synchronize()
    for w, t, s, (out, lse, status) in zip(ws, ts, shapes, got):
        assert int(status.item()) == 0
        o, l = out.float().cpu().numpy(), lse.cpu().numpy()
        ref_o, ref_l, _ = run_gpu(w, tensors=t, workers=s[4])
        assert np.array_equal(o, ref_o) and np.array_equal(l, ref_l)
        compare(w, o, l, tag=f"noalloc R{w.R} M{w.M}")


def test_noalloc_reports_device_status():
    w = wl.small(2, 4, 8, [300, 200], seed=6)
    w.block_table[1, 1] = w.kv8.shape[0] + 1000          # out of the pool
    out, lse, status = noalloc(w, to_dev(w))
    torch.cuda.synchronize()
    assert int(status.item()) & binding.DEV_BAD_PAGE
    # the next call on the same scratch starts clean
    w2 = wl.small(2, 4, 8, [300, 200], seed=7)
    _, _, status2 = noalloc(w2, to_dev(w2))
    torch.cuda.synchronize()
    assert int(status2.item()) == 0


def test_noalloc_rejects_past_the_scratch():
    w = wl.small(4, 4, 64, [100, 100, 100, 100], seed=8)   # 256 rows, 256 workers: too big
    with pytest.raises(binding.AmlaError):
        noalloc(w, to_dev(w))
