"""Helpers for the GPU parity tests: run the HIP path through the C ABI on a seeded
workload, and compare it with the CPU oracle at the stated tolerances.

Tolerances: max |out_gpu - out_oracle| <= 1.5e-2 * max|V_hat| (max over the dequantised
value dims of every key any request reads), |lse_gpu - lse_oracle| <= 1e-3 in log2 units,
and -inf LSE (empty requests) must match exactly.
"""
import numpy as np
import torch

import oracle
from absorbed_mla_split_amd import binding
from absorbed_mla_split_amd import workloads as wl

OUT_TOL = 1.5e-2
LSE_TOL = 1e-3


def to_dev(w):
    dev = torch.device("cuda")
    return (torch.from_numpy(w.q8).to(dev), torch.from_numpy(w.kv8).to(dev),
            torch.from_numpy(w.block_table).to(dev), torch.from_numpy(w.lengths).to(dev))


def run_gpu(w, mode=binding.PLAN_BALANCED, min_split_tokens=256, workers=None, mtile=None,
            decoder=None, tensors=None, split_cost=None):
    """Plan + decode + combine on cuda:0.  Output, LSE and workspace start as NaN, so any
    value the kernels fail to write shows up."""
    q, kv, bt, lengths = tensors if tensors is not None else to_dev(w)
    dec = decoder or binding.FoldedDecoder(w.R, w.M, mode=mode, min_split_tokens=min_split_tokens,
                                           workers=workers, mtile=mtile,
                                           split_cost_pages=split_cost)
    dec.workspace[256:].fill_(0xFF)                      # FP32 NaN pattern
    out = torch.full((w.R, w.M, 512), float("nan"), dtype=torch.bfloat16, device=q.device)
    lse = torch.full((w.R, w.M), float("nan"), dtype=torch.float32, device=q.device)
    dec.plan(lengths, bt.shape[1])
    bmm1, bmm2 = binding.bmm_scales(w.sm_scale, w.q_scale, w.k_scale)
    dec.decode(q, kv, bt, lengths, bmm1, bmm2, out, lse)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), lse.cpu().numpy(), dec


def vmax(w):
    """max |V_hat| over every key any request reads."""
    table = oracle.e4m3_table()
    m = 0.0
    for r in range(w.R):
        L = int(w.lengths[r])
        for p in range((L + 63) // 64):
            n = min(64, L - 64 * p)
            vals = np.abs(table[w.kv8[w.block_table[r, p], :n, :512]])
            m = max(m, float(vals.max()))
    return m * w.k_scale


def sample_rows(w, per_req):
    rows = []
    for r in range(w.R):
        picks = {0, w.M - 1}
        rng = np.random.default_rng(1000 + r)
        picks.update(int(x) for x in rng.integers(0, w.M, max(0, per_req - 2)))
        rows.extend((r, i) for i in sorted(picks))
    return rows


def compare(w, out, lse, rows=None, tag="", lse_tol=LSE_TOL):
    """Oracle on ``rows`` (default: all) vs GPU out [R, M, 512], lse [R, M]."""
    if rows is None:
        rows = [(r, i) for r in range(w.R) for i in range(w.M)]
    ref, ref_lse = oracle.decode(w.q8, w.kv8, w.block_table, w.lengths, w.q_scale, w.k_scale,
                                 w.sm_scale, rows=rows)
    got = np.stack([out[r, i] for r, i in rows])
    got_lse = np.array([lse[r, i] for r, i in rows])
    vm = vmax(w)
    empty = np.isneginf(ref_lse)
    assert np.array_equal(np.isneginf(got_lse), empty), f"{tag}: -inf LSE mismatch"
    assert np.all(got[empty] == 0), f"{tag}: empty rows not zero"
    assert np.all(np.isfinite(got)), f"{tag}: non-finite output"
    err = float(np.max(np.abs(got - ref))) if len(rows) else 0.0
    lerr = float(np.max(np.abs(got_lse[~empty] - ref_lse[~empty]))) if (~empty).any() else 0.0
    print(f"[{tag}] rows={len(rows)} max|V|={vm:.4g} out_err={err:.3e} "
          f"(rel {err / max(vm, 1e-30):.3e}) lse_err={lerr:.3e}", flush=True)
    assert err <= OUT_TOL * vm, f"{tag}: out error {err} > {OUT_TOL} * {vm}"
    assert lerr <= lse_tol, f"{tag}: lse error {lerr} > {lse_tol}"
    return err / max(vm, 1e-30), lerr


def ws_partials(dec, w):
    """FP32 partials [slots, M, 512] and LSE [slots, M] from the decoder's workspace."""
    W = dec.params.workers
    slots = dec.max_reqs + binding.PLAN_SLACK * W
    ws = dec.workspace.cpu().numpy()
    part = ws[256:256 + slots * w.M * 512 * 4].view(np.float32).reshape(slots, w.M, 512)
    off = 256 + slots * w.M * 512 * 4
    lse = ws[off:off + slots * w.M * 4].view(np.float32).reshape(slots, w.M)
    return part, lse
