"""GPU query build and cache write (the step before the decode) vs the CPU oracle.

Each E4M3 code the kernel writes must be a valid cast of the oracle's exact value: inside
[y - d, y + d] with y = exact / scale and d covering the kernel's roundings before the cast
(one BF16 rounding, 2^-8 |y|; FP32 accumulation and scaling, 2^-16 of the summed
magnitudes).  That interval does not depend on how the kernel rounds, and every code of
every test must lie in it.  As a second check, at least 99.9 % of the codes must equal the
oracle's FP32-scaled cast of the exact value rounded to BF16 (pinned against torch's FP32
product and float8 cast; only a BF16 tie flipped by the FP32 accumulation may differ).
Cache bytes outside the tokens' slots must be untouched.
"""
import numpy as np
import pytest
import torch

import oracle
from absorbed_mla_split_amd import binding
from absorbed_mla_split_amd import workloads as wl

pytestmark = pytest.mark.gpu

SENTINEL = 0x5A


def to_dev(inp, n, pool_pages, seed):
    dev = torch.device("cuda")
    rng = np.random.default_rng(seed)
    slots = rng.permutation(pool_pages * 64)[:n].astype(np.int64)
    slots[rng.random(n) < 0.1] = -1                       # padding tokens
    t = dict(
        q=torch.from_numpy(inp.q.view(np.int16)).to(dev),
        w_uk=torch.from_numpy(inp.w_uk.view(np.int16)).to(dev),
        kv_c=torch.from_numpy(inp.kv_c.view(np.int16)).to(dev),
        k_pe=torch.from_numpy(inp.k_pe.view(np.int16)).to(dev),
        positions=torch.from_numpy(inp.positions).to(dev),
        cos_sin=torch.from_numpy(inp.cos_sin).to(dev),
        slots=torch.from_numpy(slots).to(dev),
    )
    return t, slots


def run(inp, n, H, pool_pages, seed=0, slots_override=None):
    t, slots = to_dev(inp, n, pool_pages, seed)
    if slots_override is not None:
        slots = slots_override
        t["slots"] = torch.from_numpy(slots).cuda()
    q_out = torch.full((n, H, 576), 0xEE, dtype=torch.uint8, device="cuda")
    cache = torch.full((pool_pages, 64, 576), SENTINEL, dtype=torch.uint8, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    binding.build_query_cache(t["q"], t["w_uk"], t["kv_c"], t["k_pe"], t["positions"],
                              t["cos_sin"], t["slots"], inp.neox, inp.q_scale, inp.k_scale, q_out,
                              cache, status)
    torch.cuda.synchronize()
    return q_out.cpu().numpy(), cache.cpu().numpy(), int(status.item()), slots


def check_codes(codes, exact, mag, scale, tag):
    table = oracle.e4m3_table()
    y = exact / scale
    d = 2.0 ** -8 * np.abs(y) + 2.0 ** -16 * mag / scale + 1e-12
    lo, hi = table[oracle.e4m3_encode(y - d)], table[oracle.e4m3_encode(y + d)]
    got = table[codes]
    ok = (got >= lo) & (got <= hi)
    assert np.all(ok), f"{tag}: {np.count_nonzero(~ok)} codes outside the valid interval"
    same = np.mean(codes == oracle.e4m3_cast_scaled(oracle.bf16_round(exact), scale))
    print(f"[{tag}] codes {codes.size}, equal to the oracle's cast {same:.6f}", flush=True)
    assert same >= 0.999, tag


def check_build(inp, n, H, q_out, cache, slots, tag):
    """Every query code and every cache code at a live slot inside its valid-cast interval
    (and mostly equal to the oracle's cast); every other cache byte untouched."""
    query, rows = oracle.build_query_and_cache(inp.q, inp.w_uk, inp.kv_c, inp.k_pe,
                                               inp.positions, inp.cos_sin, inp.neox)
    qv = oracle.bf16_values(inp.q)
    wv = oracle.bf16_values(inp.w_uk)
    mag = np.empty_like(query)
    for h in range(H):
        mag[:, h, :512] = np.abs(qv[:, h, :128]) @ np.abs(wv[h]).T
    mag[:, :, 512:] = np.abs(qv[:, :, 128:]).max(axis=2, keepdims=True) * 2   # |x0 c| + |x1 s|
    check_codes(q_out, query, mag, inp.q_scale, f"query {tag}")
    flat = cache.reshape(-1, 576)
    live = slots >= 0
    kmag = np.abs(oracle.bf16_values(inp.k_pe)).max(axis=1, keepdims=True) * 2
    rmag = np.concatenate([np.abs(rows[:, :512]), np.broadcast_to(kmag, (n, 64))], axis=1)
    check_codes(flat[slots[live]], rows[live], rmag[live], inp.k_scale, f"cache {tag}")
    untouched = np.ones(flat.shape[0], bool)
    untouched[slots[live]] = False
    assert np.all(flat[untouched] == SENTINEL), f"{tag}: bytes outside the slots written"


@pytest.mark.parametrize("n,H,neox", [(37, 8, False), (37, 8, True), (256, 64, False),
                                      (5, 1, True), (100, 32, False), (100, 64, True)])
def test_query_and_cache_rows(n, H, neox):
    inp = wl.query_build_inputs(n, H, seed=n + H, max_pos=4096, neox=neox)
    pool = (n + 63) // 64 + 3
    q_out, cache, status, slots = run(inp, n, H, pool, seed=n)
    assert status == 0
    check_build(inp, n, H, q_out, cache, slots, f"n{n} H{H} neox{neox}")


def test_bad_slot_and_position_are_flagged():
    n, H = 8, 4
    inp = wl.query_build_inputs(n, H, seed=3, max_pos=64)
    inp.positions[2] = 10 ** 6                            # outside the table
    pool = 2
    slots = np.arange(n, dtype=np.int64)
    slots[5] = pool * 64 + 7                              # past the pool
    _, cache, status, _ = run(inp, n, H, pool, slots_override=slots)
    assert status & binding.DEV_BAD_PAGE and status & binding.DEV_BAD_POSITION
    flat = cache.reshape(-1, 576)
    assert np.all(flat[n:] == SENTINEL)


def test_c2_shape_every_row():
    # c2's step: 64 requests x 4 draft tokens, 8 heads (TP8 rank), cache rows into a big pool
    n, H = 256, 8
    inp = wl.query_build_inputs(n, H, seed=11)
    q_out, cache, status, slots = run(inp, n, H, 4096, seed=2)
    assert status == 0
    check_build(inp, n, H, q_out, cache, slots, "c2 shape")
