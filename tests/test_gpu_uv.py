"""GPU merge fused with the W_UV up-projection (the value stage) vs the CPU oracle.

Per case, through the C ABI (plan, decode, then the fused merge + W_UV):
  1. the merged BF16 latent and LSE the fused kernel writes (its optional outputs) meet the
     attention bar against the oracle's exact attention, and agree with the plain
     reducer's to one BF16 rounding;
  2. the projection: attn_out against the oracle's uv_project of the kernel's own BF16
     latent, within one BF16 rounding of the result plus FP32 accumulation error
     (|err| <= 2^-8 |ref| + 2^-13 sum_c |latent_c W_cv|);
  3. end to end: attn_out against uv_project of the oracle's exact attention, within the
     attention bar carried through W_UV (|sum_c e_c W_cv| <= max|e| sum_c |W_cv|) plus
     the output rounding.
Outputs start as NaN; W_UV is synthetic BF16 N(0, 1/512).
"""
import numpy as np
import pytest
import torch

import oracle
from absorbed_mla_split_amd import binding
from absorbed_mla_split_amd import workloads as wl
from gpu_util import OUT_TOL, compare, sample_rows, to_dev, vmax

pytestmark = pytest.mark.gpu


def run_uv(w, heads, seed=0, workers=None, min_split_tokens=256, with_latent=True, tensors=None,
           w_uv=None, split_cost=None):
    q, kv, bt, lengths = tensors if tensors is not None else to_dev(w)
    dev = q.device
    wbits = w_uv if w_uv is not None else wl.uv_weights(heads, seed=seed)
    wdev = torch.from_numpy(wbits.view(np.int16)).to(dev)
    dec = binding.FoldedDecoder(w.R, w.M, workers=workers, min_split_tokens=min_split_tokens,
                                split_cost_pages=split_cost)
    dec.workspace[256:].fill_(0xFF)
    k = w.M // heads
    attn = torch.full((w.R * k, heads * 128), float("nan"), dtype=torch.bfloat16, device=dev)
    lat = lse = None
    if with_latent:
        lat = torch.full((w.R, w.M, 512), float("nan"), dtype=torch.bfloat16, device=dev)
        lse = torch.full((w.R, w.M), float("nan"), dtype=torch.float32, device=dev)
    dec.plan(lengths, bt.shape[1])
    bmm1, bmm2 = binding.bmm_scales(w.sm_scale, w.q_scale, w.k_scale)
    dec.decode_uv(q, kv, bt, lengths, bmm1, bmm2, heads, wdev, attn, lat, lse)
    torch.cuda.synchronize()
    assert dec.device_status() == 0
    res = dict(attn=attn.float().cpu().numpy().reshape(w.R, w.M, 128), wbits=wbits, dec=dec)
    if with_latent:
        res["lat"] = lat.float().cpu().numpy()
        res["lse"] = lse.cpu().numpy()
        # the plain reducer on the same partials
        out2 = torch.empty_like(lat)
        lse2 = torch.empty_like(lse)
        binding.combine(dec.workspace, dec.counts[:w.R], dec.offsets[:w.R + 1], w.R, dec.params,
                        dec.compute_units, out2, lse2)
        torch.cuda.synchronize()
        res["lat_plain"] = out2.float().cpu().numpy()
        res["lse_plain"] = lse2.cpu().numpy()
    return res


def check_projection(w, heads, res, rows=None, tag=""):
    attn, wbits = res["attn"], res["wbits"]
    wv = oracle.bf16_values(wbits).reshape(heads, 128, 512)
    if rows is None:
        rows = [(r, i) for r in range(w.R) for i in range(w.M)]
    idx_r = np.array([r for r, _ in rows])
    idx_i = np.array([i for _, i in rows])
    got = attn[idx_r, idx_i]
    assert np.all(np.isfinite(got)), f"{tag}: non-finite attention output"

    # 2. the projection of the kernel's own BF16 latent
    lat = res["lat"][idx_r, idx_i]
    ref = np.empty_like(got)
    mag = np.empty_like(got)
    for n, i in enumerate(idx_i):
        h = i % heads
        ref[n] = oracle.uv_project(lat[n][None, None], wbits[h:h + 1], 1)[0, 0]
        mag[n] = np.abs(lat[n]) @ np.abs(wv[h]).T
    err2 = np.abs(got - ref)
    bound2 = 2.0 ** -8 * np.abs(ref) + 2.0 ** -13 * mag
    worst = float(np.max(err2 - bound2))
    print(f"[{tag}] projection: max err {err2.max():.3e}, worst margin {worst:.3e}", flush=True)
    assert np.all(err2 <= bound2), f"{tag}: projection error beyond one BF16 rounding"

    # 3. end to end against the oracle's exact attention
    ref_lat, _ = oracle.decode(w.q8, w.kv8, w.block_table, w.lengths, w.q_scale, w.k_scale,
                               w.sm_scale, rows=rows)
    ref3 = np.empty_like(got)
    s = np.abs(wv).sum(axis=2)                       # [h][v]: sum_c |W_UV[h, c, v]|
    bound3 = np.empty_like(got)
    vm = vmax(w)
    for n, i in enumerate(idx_i):
        h = i % heads
        ref3[n] = oracle.uv_project(ref_lat[n][None, None], wbits[h:h + 1], 1)[0, 0]
        bound3[n] = OUT_TOL * vm * s[h] * 1.01 + 2.0 ** -7 * np.abs(ref3[n]) + 1e-6
    err3 = np.abs(got - ref3)
    print(f"[{tag}] end to end: max err {err3.max():.3e} (bound min {bound3.min():.3e})", flush=True)
    assert np.all(err3 <= bound3), f"{tag}: end-to-end error beyond the attention bar"


def check_latent(w, res, rows=None, tag=""):
    compare(w, res["lat"], res["lse"], rows=rows, tag=tag + " latent")
    a, b = res["lat"], res["lat_plain"]
    assert np.all(np.abs(a - b) <= 2.0 ** -7 * np.abs(b)), f"{tag}: latent differs from combine"
    fin = np.isfinite(res["lse_plain"])
    assert np.array_equal(fin, np.isfinite(res["lse"]))
    assert np.max(np.abs(res["lse"][fin] - res["lse_plain"][fin]), initial=0) <= 1e-5


SHAPES = [
    # (k, H, lengths)
    (4, 8, [200, 317, 0, 1000]),     # an empty request
    (7, 8, [513, 2047, 64 * 9 + 5]),
    (2, 32, [130, 1]),
    (4, 64, [1500, 64]),
    (3, 11, [300, 64]),              # 6 rows per head: one partial 16-row tile
    (16, 64, [70]),                  # M = 1024 (8-row tiles)
    (16, 64, [70, 130, 64, 1]),      # 4 x 16-row tiles per head, 256 workgroups: 16-row tiles
    (5, 4, [900, 64, 2000, 7, 333]),  # 25 rows per head: a full and a partial tile
    # 8 x 16 rows per head, 4 x 32-row tiles per head x 64 heads: 32-row tiles
    (16, 64, [70, 130, 64, 1, 300, 2, 65, 900]),
    # 100 rows per head: three full 32-row tiles and one of 4 rows
    (4, 64, [1 + 37 * i for i in range(25)]),
]


@pytest.mark.parametrize("k,H,lengths", SHAPES)
def test_small_shapes_every_row(k, H, lengths):
    w = wl.small(len(lengths), k, H, lengths, seed=k * 100 + H)
    res = run_uv(w, H, seed=k + H)
    tag = f"k{k}H{H}L{lengths}"
    check_latent(w, res, tag=tag)
    check_projection(w, H, res, tag=tag)
    empty = w.lengths == 0
    assert np.all(res["attn"][empty] == 0)


def test_many_splits_per_request():
    w = wl.small(2, 4, 8, [64 * 200 + 5, 64 * 70], seed=6)
    res = run_uv(w, 8, workers=300, min_split_tokens=0, split_cost=0)
    assert res["dec"].plan_host()[0].tolist() == [190, 66]
    check_latent(w, res, tag="201-splits")
    check_projection(w, 8, res, tag="201-splits")


def test_optional_outputs_do_not_change_the_projection():
    w = wl.small(3, 4, 16, [700, 2500, 64], seed=12)
    t = to_dev(w)
    a = run_uv(w, 16, tensors=t)
    b = run_uv(w, 16, tensors=t, with_latent=False)
    assert np.array_equal(a["attn"], b["attn"])


def test_selection_weights_copy_latent_slices():
    # W_UV[h, c, v] = [c == v + 128 (h % 4)]: attn_out rows are exact slices of the BF16
    # latent (each output is one latent value times 1.0, accumulated with zeros)
    H = 8
    bits = np.zeros((H, 128, 512), np.uint16)
    for h in range(H):
        bits[h, np.arange(128), np.arange(128) + 128 * (h % 4)] = 0x3F80
    w = wl.small(2, 4, H, [1000, 64 * 5 + 3], seed=21)
    res = run_uv(w, H, w_uv=bits)
    for i in range(w.M):
        h = i % H
        assert np.array_equal(res["attn"][:, i], res["lat"][:, i, 128 * (h % 4):128 * (h % 4) + 128])


@pytest.mark.parametrize("cfg", ["c2", "c4"])
def test_full_size_sampled(cfg):
    w = wl.generate(cfg)
    H = w.cfg.H
    res = run_uv(w, H)
    rows = sample_rows(w, 3)
    check_latent(w, res, rows=rows, tag=cfg)
    check_projection(w, H, res, rows=rows, tag=cfg)


def test_graph_capture_replay():
    w = wl.small(4, 4, 8, [3000, 1000, 64, 2200], seed=8)
    q, kv, bt, lengths = to_dev(w)
    H = 8
    wdev = torch.from_numpy(wl.uv_weights(H).view(np.int16)).cuda()
    dec = binding.FoldedDecoder(w.R, w.M)
    bmm1, bmm2 = binding.bmm_scales(w.sm_scale, w.q_scale, w.k_scale)
    attn = torch.empty((w.R * 4, H * 128), dtype=torch.bfloat16, device="cuda")
    dec.plan(lengths, bt.shape[1])
    dec.decode_uv(q, kv, bt, lengths, bmm1, bmm2, H, wdev, attn)
    torch.cuda.synchronize()
    ref = attn.clone()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            dec.plan(lengths, bt.shape[1])
            dec.decode_uv(q, kv, bt, lengths, bmm1, bmm2, H, wdev, attn)
    torch.cuda.current_stream().wait_stream(s)
    for _ in range(3):
        attn.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(attn, ref)
