#!/usr/bin/env python3
"""Benchmark of the folded split-KV absorbed-MLA decode on one MI355X.

One step = one pass of the whole hot path over one batch: the split plan, the persistent
split-KV decode and the reducer, all on one stream, inputs resident in HBM.  The workload
is the R=64, k=4, H=8 (32 folded rows), L=8192 draft step (``--config c2``, default);
``--config`` selects another of the seeded workloads for exploration.  Three copies of the
KV pool are rotated over the steps so the 256 MB last-level cache does not serve the pages.

Prints ONE JSON line (rank 0): KV-cache GB/s (sum_r L_r * 576 B per step time) as
``value``, folded rows/s alongside, the dominant kernel's roofline (live HIP-event timing
of the decode kernel on its stream), and the CPU oracle's rate on a bounded sample of the
same workload.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense FP8 MFMA, TFLOP/s
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_traffic.json")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="c2", choices=["c1", "c2", "c3", "c4", "c5"])
    ap.add_argument("--mode", default="balanced", choices=["balanced", "fixed"])
    ap.add_argument("--unfolded", action="store_true",
                    help="stock flattening: R*k single-token requests with replicated tables")
    ap.add_argument("--pools", type=int, default=3, help="KV pool copies rotated over steps")
    ap.add_argument("--mtile", type=int, default=None, choices=[32, 64, 128],
                    help="rows per decode work unit (default: the library's choice)")
    ap.add_argument("--workers", type=int, default=None,
                    help="persistent decode workgroups and plan budget (default: one per CU)")
    ap.add_argument("--eager", action="store_true",
                    help="launch the three kernels per step directly instead of replaying "
                         "captured HIP graphs of consecutive steps")
    ap.add_argument("--graph-steps", type=int, default=12,
                    help="steps per captured HIP graph (rounded to a multiple of --pools)")
    ap.add_argument("--layers", type=int, default=61,
                    help="also time a decode step of this many layers as the model runs it: "
                         "one plan, then decode + combine per layer, in one HIP graph "
                         "(0: skip)")
    ap.add_argument("--uv", action="store_true",
                    help="end each step with the merge fused with the W_UV up-projection "
                         "(attention output [R*k, H*128]) instead of the plain merge")
    ap.add_argument("--dcp", type=int, default=0,
                    help="decode the workload as rank 0's KV shard of this many interleaved "
                         "DCP ranks (interleave 1) with the causal mask in global positions, "
                         "and time the merge of as many source rows")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=20.0,
                    help="target CPU time of the oracle sample")
    return ap.parse_args()


def source_digest():
    h = hashlib.sha256()
    with open(os.path.join(ROOT, "absorbed_mla_split_amd", "csrc", "amla.hip"), "rb") as f:
        h.update(f.read())
    return h.hexdigest()[:16]


def traffic_for(config, mode, unfolded):
    """HBM bytes per decode launch measured by rocprofv3 counters, if recorded for the
    current kernel source (null once the kernel has changed)."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    key = f"{config}/{mode}/{'unfolded' if unfolded else 'folded'}"
    ent = rec.get(key)
    if not ent or ent.get("source") != source_digest():
        return None
    return ent.get("bytes_per_launch")


def cpu_baseline(w, target_s):
    """The oracle (as it stands) on a bounded sample of rows of this workload, on the host
    cores; scaled to KV-cache GB/s of the whole workload."""
    import oracle

    threads = oracle.threads()
    R, M = w.R, w.M
    keys_total = float(w.lengths.astype(np.int64).sum()) * M          # (row, key) pairs
    # calibrate on a few rows of the longest request
    r0 = int(np.argmax(w.lengths))
    cal = [(r0, i) for i in range(min(M, max(1, threads)))]
    t = time.perf_counter()
    oracle.decode(w.q8, w.kv8, w.block_table, w.lengths, w.q_scale, w.k_scale, w.sm_scale, rows=cal)
    dt = time.perf_counter() - t
    per_pair = dt / max(1.0, len(cal) * float(w.lengths[r0]))
    want_pairs = target_s / max(per_pair, 1e-12)
    passes = 1
    if want_pairs >= keys_total:
        rows = [(r, i) for r in range(R) for i in range(M)]
        passes = max(1, min(100, int(want_pairs / keys_total)))
        sample = f"all {R * M} rows, {passes} passes"
    else:
        stride = max(1, int(np.ceil(keys_total / want_pairs)))
        rows = [(r, i) for r in range(R) for i in range(M) if (r * M + i) % stride == 0]
        sample = f"{len(rows)} of {R * M} rows (every {stride}th, request-major), full key sets"
    pairs = float(sum(int(w.lengths[r]) for r, _ in rows)) * passes
    t = time.perf_counter()
    for _ in range(passes):
        oracle.decode(w.q8, w.kv8, w.block_table, w.lengths, w.q_scale, w.k_scale, w.sm_scale,
                      rows=rows)
    dt = time.perf_counter() - t
    full_s = dt * keys_total / max(pairs, 1.0)
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    return {"value": round(w.kv_bytes / full_s / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle", "sample": f"{sample}; {dt:.1f} s measured, scaled to the workload",
            "rows_per_s": round(R * M / full_s, 2), "cpu_model": cpu_model,
            "affinity_cpus": len(os.sched_getaffinity(0))}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU; --gpus {args.gpus} is not supported (the per-GPU "
              "path is the single-GPU kernel; sharding across GPUs is not part of it)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from absorbed_mla_split_amd import binding
    from absorbed_mla_split_amd import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    binding.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    t0 = time.perf_counter()
    w = wl.generate(args.config)
    if args.unfolded:
        R, k, H = w.cfg.R, w.cfg.k, w.cfg.H
        row_req = np.arange(R * k) // k
        w = wl.Workload(w.cfg, w.lengths[row_req], w.block_table[row_req],
                        w.q8.reshape(R * k, H, 576), w.kv8, w.q_scale, w.k_scale)
    gen_s = time.perf_counter() - t0
    R, M = w.R, w.M
    q = torch.from_numpy(w.q8).to(dev)
    bt = torch.from_numpy(w.block_table).to(dev)
    lengths = torch.from_numpy(w.lengths).to(dev)
    kv0 = torch.from_numpy(w.kv8).to(dev)
    pools = [kv0] + [kv0.clone() for _ in range(max(0, args.pools - 1))]
    mode = binding.PLAN_FIXED if args.mode == "fixed" else binding.PLAN_BALANCED
    dec = binding.FoldedDecoder(R, M, device=dev, mode=mode, mtile=args.mtile,
                                workers=args.workers)
    bmm1, bmm2 = binding.bmm_scales(w.sm_scale, w.q_scale, w.k_scale)
    out = torch.empty((R, M, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((R, M), dtype=torch.float32, device=dev)
    H = w.M // w.cfg.k if not args.unfolded else w.M
    w_uv = torch.from_numpy(wl.uv_weights(H).view(np.int16)).to(dev)
    attn_out = torch.empty((R * (M // H), H * 128), dtype=torch.bfloat16, device=dev)
    k_tok = M // H
    dcp = None
    if args.dcp > 1:
        # the lengths are rank 0's shard of global lengths N * L (interleave 1: rank 0
        # holds positions 0, N, 2N, ...: ceil(N L / N) = L of them)
        dcp = binding.DcpParams(H, 1, args.dcp, 0, 1)
        totals = torch.from_numpy(w.lengths.astype(np.int64) * args.dcp).to(torch.int32).to(dev)

    def decode(pool, stream):
        if dcp is None:
            binding.folded_decode(q, pool, bt, lengths, dec.params, bmm1, bmm2, dec.counts[:R],
                                  dec.offsets[:R + 1], dec.work, dec.workspace, stream)
        else:
            binding.folded_decode_dcp(q, pool, bt, lengths, dec.params, bmm1, bmm2,
                                      dec.counts[:R], dec.offsets[:R + 1], dec.work,
                                      dec.workspace, dcp, totals, stream)

    def merge(stream):
        if args.uv:
            binding.combine_uv(dec.workspace, dec.counts[:R], dec.offsets[:R + 1], R, dec.params,
                               H, w_uv, attn_out, None, None, stream)
        else:
            binding.combine(dec.workspace, dec.counts[:R], dec.offsets[:R + 1], R, dec.params,
                            dec.compute_units, out, lse, stream)

    def step(i):
        stream = torch.cuda.current_stream()
        dec.plan(lengths, bt.shape[1], stream)
        decode(pools[i % len(pools)], stream)
        merge(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    status = dec.device_status()
    if status != 0:
        print(f"device status {status}: {binding.status_string(status)}", file=sys.stderr)
        sys.exit(1)

    # Consecutive steps captured into HIP graphs, as a serving loop replays a decode step's
    # layers: `chain` steps per graph (a multiple of the pool count, so the pool rotation
    # runs on across replays) and one graph for the remainder of --steps.
    plan_graphs = []          # (graph, steps it holds) in timed order
    if not args.eager:
        P = len(pools)
        chain = max(P, (max(1, args.graph_steps) + P - 1) // P * P)
        chain = min(chain, max(P, (args.steps + P - 1) // P * P))
        full, rest = divmod(args.steps, chain)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())

        def capture(n):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.stream(side):
                with torch.cuda.graph(g, stream=side):
                    for i in range(n):
                        step(i)
            return g

        g_full = capture(chain) if full else None
        g_rest = capture(rest) if rest else None
        torch.cuda.current_stream().wait_stream(side)
        plan_graphs = [(g_full, chain)] * full + ([(g_rest, rest)] if rest else [])
        for g, _ in plan_graphs[:max(1, args.warmup // chain)]:
            g.replay()
        torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    # events between graph replays (or eager steps) give the per-step spread; the value
    # itself is the total over exactly `steps` steps between `start` and `end`
    marks = []
    start.record(stream)
    if plan_graphs:
        for g, n in plan_graphs:
            g.replay()
            e = torch.cuda.Event(enable_timing=True)
            e.record(stream)
            marks.append((e, n))
    else:
        for i in range(args.steps):
            step(i)
            e = torch.cuda.Event(enable_timing=True)
            e.record(stream)
            marks.append((e, 1))
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    status = dec.device_status()
    if status != 0:
        print(f"device status {status} after the timed steps: {binding.status_string(status)}",
              file=sys.stderr)
        sys.exit(1)
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / args.steps
    per_step_us, prev = [], start
    for e, n in marks:
        per_step_us.append(prev.elapsed_time(e) * 1e3 / n)
        prev = e
    spread = {f"p{q}": round(float(np.percentile(per_step_us, q)), 2) for q in (10, 50, 90)}
    spread["samples"] = len(per_step_us)

    # Each kernel's own average duration, measured live with HIP events on the stream its
    # launches run on: after one plan, `steps` launches of the kernel back to back between
    # two events (the decode rotating over the KV pool copies like the timed steps), so the
    # figure is the kernel's duration plus the dispatch gap between consecutive launches.
    stream = torch.cuda.current_stream()
    dec.plan(lengths, bt.shape[1], stream)

    def timed(launch):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        launch(0)
        e0.record(stream)
        for i in range(args.steps):
            launch(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    dec_avg = timed(lambda i: decode(pools[i % len(pools)], stream))
    comb_avg = timed(lambda i: binding.combine(
        dec.workspace, dec.counts[:R], dec.offsets[:R + 1], R, dec.params, dec.compute_units,
        out, lse, stream))
    uv_avg = timed(lambda i: binding.combine_uv(
        dec.workspace, dec.counts[:R], dec.offsets[:R + 1], R, dec.params, H, w_uv, attn_out,
        None, None, stream))
    p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    p0.record(stream)
    for _ in range(args.steps):
        dec.plan(lengths, bt.shape[1], stream)
    p1.record(stream)
    torch.cuda.synchronize()
    plan_us = p0.elapsed_time(p1) / args.steps * 1e3

    # A decode step as the model runs it: one plan, reused by every layer's decode and
    # combine (each layer reads its own cache; the pool copies rotate), in one HIP graph.
    amortized = None
    if args.layers > 0 and not args.eager:
        def layered(s):
            dec.plan(lengths, bt.shape[1], s)
            for li in range(args.layers):
                decode(pools[li % len(pools)], s)
                merge(s)
        gl = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            with torch.cuda.graph(gl, stream=side):
                layered(side)
        stream.wait_stream(side)
        gl.replay()
        torch.cuda.synchronize()
        l0, l1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        l0.record(stream)
        for _ in range(2):
            gl.replay()
        l1.record(stream)
        torch.cuda.synchronize()
        lstep_ms = l0.elapsed_time(l1) / 2
        amortized = {"layers": args.layers, "step_us": round(lstep_ms * 1e3, 1),
                     "per_layer_us": round(lstep_ms * 1e3 / args.layers, 2),
                     "kv_gbs": round(w.kv_bytes * args.layers / (lstep_ms / 1e3) / 1e9, 1),
                     "note": "one plan per step, decode + combine per layer, one HIP graph"}
        status = dec.device_status()
        if status != 0:
            print(f"device status {status} after the layered step: {binding.status_string(status)}",
                  file=sys.stderr)
            sys.exit(1)

    kv_bytes = w.kv_bytes
    pages = int(((w.lengths.astype(np.int64) + 63) // 64).sum())
    dec_alg_bytes = kv_bytes + R * M * 576 + pages * 4
    flops = 2.0 * M * float(w.lengths.astype(np.int64).sum()) * (576 + 512)
    step_s = ms_per_step / 1e3
    value = kv_bytes / step_s / 1e9
    rows_per_s = R * M / step_s

    mfma_bound = M >= 256
    if mfma_bound:
        achieved = flops / (dec_avg / 1e3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": FP8_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / FP8_PEAK_TFLOPS, 4)}
    else:
        achieved = dec_alg_bytes / (dec_avg / 1e3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4)}
    roof["kernel"] = {32: "decode32_kernel", 64: "decode64_kernel"}.get(dec.params.mtile,
                                                                       "decode128_kernel")
    roof["traffic"] = traffic_for(args.config, args.mode, args.unfolded)
    roof["algorithmic_bytes_per_launch"] = int(dec_alg_bytes)
    roof["flops_per_launch"] = flops

    # the merge fused with the W_UV up-projection: split partials read, W_UV read once,
    # BF16 attention output written; 2 * 512 * 128 BF16 MMA flop per row
    n_items = int(dec.offsets[R].item())
    uv_bytes = n_items * M * 513 * 4 + H * 128 * 512 * 2 + R * M * 128 * 2
    value_stage = {"kernel": "combine_uv_kernel", "us": round(uv_avg * 1e3, 2),
                   "bytes": int(uv_bytes), "gbs": round(uv_bytes / (uv_avg / 1e3) / 1e9, 1),
                   "hbm_frac": round(uv_bytes / (uv_avg / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                   "flop": 2 * R * M * 512 * 128,
                   "in_step": bool(args.uv)}

    # the step before the decode: the absorbed query of the step's R*k tokens (H heads) and
    # their cache rows, from synthetic projections (the new rows go to the pool's last page
    # slots of a scratch pool so the workload's cache stays as generated)
    n_tok = R * k_tok
    qb = wl.query_build_inputs(n_tok, H, seed=1, max_pos=1 << 16)
    qb_t = dict(
        q=torch.from_numpy(qb.q.view(np.int16)).to(dev),
        w_uk=torch.from_numpy(qb.w_uk.view(np.int16)).to(dev),
        kv_c=torch.from_numpy(qb.kv_c.view(np.int16)).to(dev),
        k_pe=torch.from_numpy(qb.k_pe.view(np.int16)).to(dev),
        positions=torch.from_numpy(qb.positions % (1 << 16)).to(dev),
        cos_sin=torch.from_numpy(qb.cos_sin).to(dev))
    scratch_pages = (n_tok + 63) // 64
    scratch = torch.zeros((scratch_pages, 64, 576), dtype=torch.uint8, device=dev)
    qb_slots = torch.from_numpy(np.random.default_rng(5).permutation(scratch_pages * 64)[:n_tok]
                                .astype(np.int64)).to(dev)
    qb_out = torch.empty((n_tok, H, 576), dtype=torch.uint8, device=dev)
    b_avg = timed(lambda i: binding.build_query_cache(
        qb_t["q"], qb_t["w_uk"], qb_t["kv_c"], qb_t["k_pe"], qb_t["positions"], qb_t["cos_sin"],
        qb_slots, qb.neox, qb.q_scale, qb.k_scale, qb_out, scratch, None, stream))
    b_bytes = (n_tok * H * 192 * 2 + H * 512 * 128 * 2 + n_tok * (512 + 64) * 2
               + n_tok * 64 * 4 + n_tok * H * 576 + n_tok * 576)
    query_build = {"kernel": "build_query_cache_kernel", "tokens": n_tok, "heads": H,
                   "us": round(b_avg * 1e3, 2), "bytes": int(b_bytes),
                   "gbs": round(b_bytes / (b_avg / 1e3) / 1e9, 1),
                   "flop": 2 * n_tok * H * 128 * 512}

    # the head owner's merge over the DCP sources: N BF16 source rows per folded row
    dcp_res = None
    if dcp is not None:
        n = R * M
        src_rows = torch.randn((args.dcp, n, 512), device=dev).to(torch.bfloat16)
        src_lse = torch.randn((args.dcp, n), device=dev)
        m_out = torch.empty((n, 512), dtype=torch.bfloat16, device=dev)
        m_lse = torch.empty((n,), dtype=torch.float32, device=dev)
        m_avg = timed(lambda i: binding.merge_sources(src_rows, src_lse, m_out, m_lse, stream))
        m_bytes = args.dcp * n * (512 * 2 + 4) + n * (512 * 2 + 4)
        dcp_res = {"world": args.dcp, "interleave": 1, "rank": 0, "causal": True,
                   "merge_kernel": "merge_sources_kernel", "merge_us": round(m_avg * 1e3, 2),
                   "merge_bytes": int(m_bytes),
                   "merge_gbs": round(m_bytes / (m_avg / 1e3) / 1e9, 1)}

    cfg = w.cfg
    workload = (f"{args.config}: R={cfg.R} k={cfg.k} H={cfg.H} (M={cfg.M}), {cfg.description}"
                + (" [unfolded R*k rows]" if args.unfolded else "")
                + (f" [rank 0 of {args.dcp} DCP ranks, causal]" if args.dcp > 1 else ""))
    res = {
        "metric": "KV-cache HBM GB/s and folded query rows/s (R*k*H per s) per MI355X",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8",
        "data": "synthetic",
        "config": {"workload": workload, "requests": R, "rows_per_req": M,
                   "kv_tokens": int(w.lengths.astype(np.int64).sum()), "page": 64,
                   "plan": args.mode, "kv_pools_rotated": len(pools),
                   "mtile": dec.params.mtile, "workers": dec.params.workers,
                   "launch": "eager" if args.eager else
                   f"hip_graph x{plan_graphs[0][1]} steps" if plan_graphs else "hip_graph"},
        "rows_per_s": round(rows_per_s, 1),
        "step_us": round(ms_per_step * 1e3, 2),
        "step_us_spread": spread,
        "decode_us": round(dec_avg * 1e3, 2),
        "combine_us": round(comb_avg * 1e3, 2),
        "value_stage": value_stage,
        "dcp": dcp_res,
        "query_build": query_build,
        "plan_us": round(plan_us, 2),
        "layer_kv_gbs": round(kv_bytes / ((dec_avg + (uv_avg if args.uv else comb_avg)) / 1e3) / 1e9, 1),
        "layered_step": amortized,
        "roofline": roof,
        "wall_s": round(wall, 3),
        "gen_s": round(gen_s, 1),
        "source": source_digest(),
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
