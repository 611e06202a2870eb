#!/usr/bin/env python3
"""Benchmark of the folded split-KV absorbed-MLA decode on one MI355X.

One step = one pass of the whole hot path over one batch: the split plan, the persistent
split-KV decode and the reducer, all on one stream, inputs resident in HBM.  The headline
workload is the largest single-GPU one, R=128 requests of k=7 draft tokens and H=8 heads
(56 folded rows) with KV lengths log-uniform in [512, 65536] (``--config c3``, default),
the mixed batch the length-balanced plan is for.  Three copies of the KV pool are rotated
over the steps so the 256 MB last-level cache does not serve the pages.

In the same process (unless ``--no-extra``) it also measures the method's two
comparisons, the same workload with the fixed equal-split plan and the R=16, k=7, H=64
skewed batch folded vs unfolded (R*k single-token rows reading the KV k times), and the
other workloads (uniform 8192 at M=32, uniform 32768 at M=256), each with its step time,
in-step decode time and roofline fraction.

Prints ONE JSON line: KV-cache GB/s (sum_r L_r * 576 B per step time) as ``value``, folded
rows/s alongside, the decode kernel's roofline from its live in-step duration (HIP events
on its stream around each decode of an eager pass), and the CPU oracle's rate on a bounded
sample of the same workload.
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
KERNELS = {32: "decode_stream_kernel<32>", 64: "decode_stream_kernel<64>",
           128: "decode128_kernel"}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="c3", choices=["c1", "c2", "c3", "c4", "c5"])
    ap.add_argument("--mode", default="balanced", choices=["balanced", "fixed"])
    ap.add_argument("--unfolded", action="store_true",
                    help="stock flattening: R*k single-token requests with replicated tables")
    ap.add_argument("--pools", type=int, default=3, help="KV pool copies rotated over steps")
    ap.add_argument("--mtile", type=int, default=None, choices=[32, 64, 128],
                    help="rows per decode work unit (default: the library's choice)")
    ap.add_argument("--split-cost", type=int, default=None,
                    help="plan's split cost in pages (default: the library's)")
    ap.add_argument("--workers", type=int, default=None,
                    help="persistent decode workgroups and plan budget (default: one per CU)")
    ap.add_argument("--graph-steps", type=int, default=12,
                    help="steps per captured HIP graph of the timed region (rounded to a "
                         "multiple of --pools)")
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
    ap.add_argument("--no-extra", action="store_true",
                    help="headline workload only: skip the comparisons and other workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=20.0,
                    help="target CPU time of the oracle sample")
    return ap.parse_args()


def source_digest():
    """Digest of every device source (the recorded traffic is valid for this digest only)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "absorbed_mla_split_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".h")):
            h.update(name.encode())
            with open(os.path.join(csrc, name), "rb") as f:
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


def oracle_rate(w, rows, passes=1):
    """Seconds the oracle takes for `passes` passes over `rows` (full key sets)."""
    import oracle

    t = time.perf_counter()
    for _ in range(passes):
        oracle.decode(w.q8, w.kv8, w.block_table, w.lengths, w.q_scale, w.k_scale, w.sm_scale,
                      rows=rows)
    return time.perf_counter() - t


def cpu_baseline(w, target_s, single_thread):
    """The oracle (as it stands) on a bounded sample of rows of this workload, on the host
    cores; scaled to KV-cache GB/s of the whole workload.  ``single_thread``: workloads
    also timed on one thread (bounded samples, a few seconds each)."""
    import oracle

    threads = oracle.threads()
    R, M = w.R, w.M
    keys_total = float(w.lengths.astype(np.int64).sum()) * M          # (row, key) pairs
    # calibrate on a few rows of the longest request
    r0 = int(np.argmax(w.lengths))
    cal = [(r0, i) for i in range(min(M, max(1, threads)))]
    dt = oracle_rate(w, cal)
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
    dt = oracle_rate(w, rows, passes)
    full_s = dt * keys_total / max(pairs, 1.0)
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    res = {"value": round(w.kv_bytes / full_s / 1e9, 4), "unit": "GB/s", "cores": threads,
           "kind": "oracle", "sample": f"{sample}; {dt:.1f} s measured, scaled to the workload",
           "rows_per_s": round(R * M / full_s, 2), "cpu_model": cpu_model,
           "affinity_cpus": len(os.sched_getaffinity(0))}
    # one thread (the oracle's parallel loops on a single core)
    one = {}
    prev = oracle.set_threads(1)
    try:
        for name, ws in single_thread:
            keys = float(ws.lengths.astype(np.int64).sum()) * ws.M
            rows = [(r, i) for r in range(ws.R) for i in range(ws.M)]
            stride = 1
            if keys * per_pair * threads > 4.0:        # bound the sample to ~4 s
                stride = int(np.ceil(keys * per_pair * threads / 4.0))
                rows = rows[::stride]
            dt1 = oracle_rate(ws, rows)
            pairs1 = float(sum(int(ws.lengths[r]) for r, _ in rows))
            full1 = dt1 * keys / max(pairs1, 1.0)
            one[name] = {"s": round(full1, 3), "gbs": round(ws.kv_bytes / full1 / 1e9, 5),
                         "rows_per_s": round(ws.R * ws.M / full1, 2),
                         "sample": f"{len(rows)} of {ws.R * ws.M} rows (every {stride}th); "
                                   f"{dt1:.2f} s measured"}
    finally:
        oracle.set_threads(prev)
    res["single_thread"] = one
    return res


class Runner:
    """Device copies of one workload plus the decoder, and the three ways of timing it."""

    def __init__(self, w, dev, mode, mtile=None, workers=None, pools=3, uv=False, dcp=0,
                 split_cost=None):
        import torch

        from absorbed_mla_split_amd import binding
        from absorbed_mla_split_amd import workloads as wl

        self.torch, self.binding, self.w, self.dev = torch, binding, w, dev
        self.uv = uv
        R, M = w.R, w.M
        self.q = torch.from_numpy(w.q8).to(dev)
        self.bt = torch.from_numpy(w.block_table).to(dev)
        self.lengths = torch.from_numpy(w.lengths).to(dev)
        kv0 = torch.from_numpy(w.kv8).to(dev)
        self.pools = [kv0] + [kv0.clone() for _ in range(max(0, pools - 1))]
        self.dec = binding.FoldedDecoder(
            R, M, device=dev, mode=mode, mtile=mtile, workers=workers,
            split_cost_pages=split_cost)
        self.bmm1, self.bmm2 = binding.bmm_scales(w.sm_scale, w.q_scale, w.k_scale)
        self.out = torch.empty((R, M, 512), dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty((R, M), dtype=torch.float32, device=dev)
        self.H = w.cfg.H if M % w.cfg.H == 0 else M
        self.w_uv = torch.from_numpy(wl.uv_weights(self.H).view(np.int16)).to(dev)
        self.attn_out = torch.empty((R * (M // self.H), self.H * 128), dtype=torch.bfloat16,
                                    device=dev)
        self.dcp = None
        if dcp > 1:
            # the lengths are rank 0's shard of global lengths N * L (interleave 1: rank 0
            # holds positions 0, N, 2N, ...: ceil(N L / N) = L of them)
            self.dcp = binding.DcpParams(self.H, 1, dcp, 0, 1)
            self.totals = torch.from_numpy(w.lengths.astype(np.int64) * dcp).to(torch.int32).to(dev)

    @property
    def R(self):
        return self.w.R

    def plan(self, stream):
        self.dec.plan(self.lengths, self.bt.shape[1], stream)

    def decode(self, pool, stream):
        b, d, R = self.binding, self.dec, self.R
        if self.dcp is None:
            b.folded_decode(self.q, pool, self.bt, self.lengths, d.params, self.bmm1, self.bmm2,
                            d.counts[:R], d.offsets[:R + 1], d.work, d.workspace, stream)
        else:
            b.folded_decode_dcp(self.q, pool, self.bt, self.lengths, d.params, self.bmm1,
                                self.bmm2, d.counts[:R], d.offsets[:R + 1], d.work, d.workspace,
                                self.dcp, self.totals, stream)

    def merge(self, stream, uv=None):
        b, d, R = self.binding, self.dec, self.R
        if self.uv if uv is None else uv:
            b.combine_uv(d.workspace, d.counts[:R], d.offsets[:R + 1], R, d.params, self.H,
                         self.w_uv, self.attn_out, None, None, stream)
        else:
            b.combine(d.workspace, d.counts[:R], d.offsets[:R + 1], R, d.params,
                      d.compute_units, self.out, self.lse, stream)

    def step(self, i, stream):
        self.plan(stream)
        self.decode(self.pools[i % len(self.pools)], stream)
        self.merge(stream)

    def check_status(self, where):
        status = self.dec.device_status()
        if status != 0:
            print(f"device status {status} {where}: {self.binding.status_string(status)}",
                  file=sys.stderr)
            sys.exit(1)

    def warm(self, n):
        stream = self.torch.cuda.current_stream()
        for i in range(n):
            self.step(i, stream)
        self.torch.cuda.synchronize()
        self.check_status("after the warm-up")

    def eager_pass(self, steps):
        """`steps` eager steps with a HIP event on the stream before the plan, around the
        decode and after the merge of each: per-step times, the decode's in-step
        durations (it runs right after the plan, as in every step), the plan's and the
        merge's."""
        torch = self.torch
        stream = torch.cuda.current_stream()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
        torch.cuda.synchronize()
        for i in range(steps):
            e = ev[i]
            e[0].record(stream)
            self.plan(stream)
            e[1].record(stream)
            self.decode(self.pools[i % len(self.pools)], stream)
            e[2].record(stream)
            self.merge(stream)
            e[3].record(stream)
        torch.cuda.synchronize()
        self.check_status("after the eager steps")
        step = [ev[i][0].elapsed_time(ev[i][3]) * 1e3 for i in range(steps)]
        plan = [ev[i][0].elapsed_time(ev[i][1]) * 1e3 for i in range(steps)]
        dec = [ev[i][1].elapsed_time(ev[i][2]) * 1e3 for i in range(steps)]
        mrg = [ev[i][2].elapsed_time(ev[i][3]) * 1e3 for i in range(steps)]
        return {"step": step, "plan": plan, "decode": dec, "merge": mrg}

    def graph_pass(self, steps, chain_steps, warm_replays=1):
        """`steps` steps replayed from HIP graphs of `chain` consecutive steps (a multiple
        of the pool count, so the rotation runs on across replays) plus one graph for the
        remainder, between two HIP events: total milliseconds."""
        torch = self.torch
        P = len(self.pools)
        chain = max(P, (max(1, chain_steps) + P - 1) // P * P)
        chain = min(chain, max(P, (steps + P - 1) // P * P))
        full, rest = divmod(steps, chain)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())

        def capture(n):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.stream(side):
                with torch.cuda.graph(g, stream=side):
                    for i in range(n):
                        self.step(i, side)
            return g

        g_full = capture(chain) if full else None
        g_rest = capture(rest) if rest else None
        torch.cuda.current_stream().wait_stream(side)
        seq = [(g_full, chain)] * full + ([(g_rest, rest)] if rest else [])
        for g, _ in seq[:max(1, warm_replays)]:
            g.replay()
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        wall0 = time.perf_counter()
        start.record(stream)
        for g, _ in seq:
            g.replay()
        end.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
        self.check_status("after the timed steps")
        return start.elapsed_time(end), chain, wall

    def back_to_back(self, steps, launch):
        """Average milliseconds of `steps` launches of one kernel back to back between two
        HIP events on the current stream (after one untimed launch)."""
        torch = self.torch
        stream = torch.cuda.current_stream()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        launch(0, stream)
        e0.record(stream)
        for i in range(steps):
            launch(i, stream)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    def layered(self, layers):
        """A decode step of `layers` layers as the model runs it: one plan, reused by every
        layer's decode and merge (each layer reads its own cache; the pool copies rotate),
        captured as one HIP graph and replayed."""
        torch = self.torch
        stream = torch.cuda.current_stream()
        gl = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            with torch.cuda.graph(gl, stream=side):
                self.plan(side)
                for li in range(layers):
                    self.decode(self.pools[li % len(self.pools)], side)
                    self.merge(side)
        stream.wait_stream(side)
        gl.replay()
        torch.cuda.synchronize()
        l0, l1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        l0.record(stream)
        gl.replay()
        l1.record(stream)
        torch.cuda.synchronize()
        self.check_status("after the layered step")
        ms = l0.elapsed_time(l1)
        return {"layers": layers, "step_us": round(ms * 1e3, 1),
                "per_layer_us": round(ms * 1e3 / layers, 2),
                "kv_gbs": round(self.w.kv_bytes * layers / (ms / 1e3) / 1e9, 1),
                "note": "one plan per step, decode + combine per layer, one HIP graph"}

    def free(self):
        for name in ("q", "bt", "lengths", "pools", "dec", "out", "lse", "w_uv", "attn_out"):
            setattr(self, name, None)
        self.torch.cuda.empty_cache()


def spread(xs):
    d = {f"p{q}": round(float(np.percentile(xs, q)), 2) for q in (10, 50, 90)}
    d["mean"] = round(float(np.mean(xs)), 2)
    d["samples"] = len(xs)
    return d


def roofline(w, mtile, dec_us, config, mode, unfolded):
    """The decode kernel's roofline: algorithmic bytes (KV once per request, Q rows, block
    table) or FP8 MMA flop per launch over its in-step duration."""
    R, M = w.R, w.M
    pages = int(((w.lengths.astype(np.int64) + 63) // 64).sum())
    alg_bytes = w.kv_bytes + R * M * 576 + pages * 4
    flops = 2.0 * M * float(w.lengths.astype(np.int64).sum()) * (576 + 512)
    if M >= 256:
        achieved = flops / (dec_us / 1e6) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": FP8_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / FP8_PEAK_TFLOPS, 4)}
    else:
        achieved = alg_bytes / (dec_us / 1e6) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4)}
    roof["traffic"] = traffic_for(config, mode, unfolded)
    roof["kernel"] = KERNELS[mtile]
    roof["decode_us"] = round(dec_us, 2)
    roof["algorithmic_bytes_per_launch"] = int(alg_bytes)
    roof["flops_per_launch"] = flops
    return roof


def measure(w, dev, args, mode_name, config, unfolded=False, layers=0, uv=False, dcp=0):
    """Warm-up, eager in-step pass, graph-timed pass of one workload: a summary dict."""
    from absorbed_mla_split_amd import binding

    mode = binding.PLAN_FIXED if mode_name == "fixed" else binding.PLAN_BALANCED
    run = Runner(w, dev, mode, mtile=args.mtile, workers=args.workers, split_cost=args.split_cost,
                 pools=args.pools,
                 uv=uv, dcp=dcp)
    run.warm(args.warmup)
    eager = run.eager_pass(args.steps)
    total_ms, chain, wall = run.graph_pass(args.steps, args.graph_steps,
                                           warm_replays=max(1, args.warmup // args.graph_steps))
    ms_per_step = total_ms / args.steps
    dec_us = float(np.mean(eager["decode"]))
    res = {
        "run": run, "ms_per_step": ms_per_step, "chain": chain, "wall": wall,
        "step_us": round(ms_per_step * 1e3, 2),
        "value": round(w.kv_bytes / (ms_per_step / 1e3) / 1e9, 2),
        "rows_per_s": round(w.R * w.M / (ms_per_step / 1e3), 1),
        "step_us_spread": spread(eager["step"]),
        "decode_us": round(dec_us, 2),
        "decode_us_spread": spread(eager["decode"]),
        "combine_us": round(float(np.mean(eager["merge"])), 2),
        "plan_us": round(float(np.mean(eager["plan"])), 2),
        "kv_bytes": int(w.kv_bytes),
        "mtile": run.dec.params.mtile, "workers": run.dec.params.workers,
        "split_cost_pages": run.dec.params.split_cost_pages,
        "splits": int(run.dec.offsets[w.R].item()),
        "roofline": roofline(w, run.dec.params.mtile, dec_us, config, mode_name, unfolded),
    }
    if layers > 0:
        res["layered_step"] = run.layered(layers)
    return res


def summary(name, m, w):
    """The figures of a secondary workload for the JSON line."""
    r = m["roofline"]
    return {"workload": name, "requests": w.R, "rows_per_req": w.M, "kv_bytes": m["kv_bytes"],
            "step_us": m["step_us"], "value_gbs": m["value"], "rows_per_s": m["rows_per_s"],
            "decode_us": m["decode_us"], "combine_us": m["combine_us"], "plan_us": m["plan_us"],
            "splits": m["splits"], "mtile": m["mtile"],
            "roofline": {k: r[k] for k in ("bound", "achieved", "unit", "frac", "kernel",
                                           "traffic")}}


def unfold(w):
    """The stock flattening of a workload: R*k requests of H rows, each with its own copy
    of its request's block-table row and length (each reads the whole cache)."""
    from absorbed_mla_split_amd import workloads as wl

    R, k, H = w.cfg.R, w.cfg.k, w.cfg.H
    row_req = np.arange(R * k) // k
    return wl.Workload(w.cfg, w.lengths[row_req], w.block_table[row_req],
                       w.q8.reshape(R * k, H, 576), w.kv8, w.q_scale, w.k_scale)


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
        w = unfold(w)
    gen_s = time.perf_counter() - t0
    print(f"[bench] {args.config} generated in {gen_s:.1f} s", file=sys.stderr, flush=True)
    R, M = w.R, w.M

    # headline: warm-up, then the eager in-step pass (the decode launches right after the
    # warm-up ones: launches warmup .. warmup+steps-1 of its kernel in this process), then
    # the graph-timed steps that give `value`
    head = measure(w, dev, args, args.mode, args.config, unfolded=args.unfolded,
                   layers=args.layers, uv=args.uv, dcp=args.dcp)
    run = head["run"]
    stream = torch.cuda.current_stream()
    print(f"[bench] {args.config} step {head['step_us']} us, decode {head['decode_us']} us",
          file=sys.stderr, flush=True)

    # kernels next to the path, each timed back to back
    d = run.dec
    run.plan(stream)
    H = run.H
    uv_avg = run.back_to_back(args.steps, lambda i, s: run.merge(s, uv=True))
    n_items = int(d.offsets[R].item())
    uv_bytes = n_items * M * 513 * 4 + H * 128 * 512 * 2 + R * M * 128 * 2
    value_stage = {"kernel": "combine_uv_kernel", "us": round(uv_avg * 1e3, 2),
                   "bytes": int(uv_bytes), "gbs": round(uv_bytes / (uv_avg / 1e3) / 1e9, 1),
                   "hbm_frac": round(uv_bytes / (uv_avg / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                   "flop": 2 * R * M * 512 * 128, "in_step": bool(args.uv)}

    # the step before the decode: the absorbed query of the step's R*k tokens (H heads) and
    # their cache rows, from synthetic projections (into a scratch pool)
    k_tok = M // H
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
    b_avg = run.back_to_back(args.steps, lambda i, s: binding.build_query_cache(
        qb_t["q"], qb_t["w_uk"], qb_t["kv_c"], qb_t["k_pe"], qb_t["positions"], qb_t["cos_sin"],
        qb_slots, qb.neox, qb.q_scale, qb.k_scale, qb_out, scratch, None, s))
    b_bytes = (n_tok * H * 192 * 2 + H * 512 * 128 * 2 + n_tok * (512 + 64) * 2
               + n_tok * 64 * 4 + n_tok * H * 576 + n_tok * 576)
    query_build = {"kernel": "build_query_cache_kernel", "tokens": n_tok, "heads": H,
                   "us": round(b_avg * 1e3, 2), "bytes": int(b_bytes),
                   "gbs": round(b_bytes / (b_avg / 1e3) / 1e9, 1),
                   "flop": 2 * n_tok * H * 128 * 512}

    dcp_res = None
    if run.dcp is not None:
        n = R * M
        src_rows = torch.randn((args.dcp, n, 512), device=dev).to(torch.bfloat16)
        src_lse = torch.randn((args.dcp, n), device=dev)
        m_out = torch.empty((n, 512), dtype=torch.bfloat16, device=dev)
        m_lse = torch.empty((n,), dtype=torch.float32, device=dev)
        m_avg = run.back_to_back(args.steps, lambda i, s: binding.merge_sources(
            src_rows, src_lse, m_out, m_lse, s))
        m_bytes = args.dcp * n * (512 * 2 + 4) + n * (512 * 2 + 4)
        dcp_res = {"world": args.dcp, "interleave": 1, "rank": 0, "causal": True,
                   "merge_kernel": "merge_sources_kernel", "merge_us": round(m_avg * 1e3, 2),
                   "merge_bytes": int(m_bytes),
                   "merge_gbs": round(m_bytes / (m_avg / 1e3) / 1e9, 1)}
    del qb_t, scratch, qb_out
    layered = head.get("layered_step")
    run.free()

    # the method's comparisons and the other workloads, one at a time on the device
    comparisons, others = None, None
    if not args.no_extra:
        comparisons, others = {}, {}
        if args.config == "c3" and not args.unfolded:
            w3 = w
        else:
            w3 = wl.generate("c3")
        if args.config == "c3" and args.mode == "balanced" and not args.unfolded:
            bal = head
        else:
            bal = measure(w3, dev, args, "balanced", "c3")
            bal["run"].free()
        fix = measure(w3, dev, args, "fixed", "c3")
        fix["run"].free()
        comparisons["plan"] = {
            "workload": "c3: R=128 k=7 H=8 (M=56), lengths log-uniform in [512, 65536]",
            "balanced": summary("c3 balanced", bal, w3),
            "fixed": summary("c3 fixed", fix, w3),
            "fixed_over_balanced_step": round(fix["step_us"] / bal["step_us"], 3)}
        print(f"[bench] c3 fixed step {fix['step_us']} us", file=sys.stderr, flush=True)
        del w3

        w5 = wl.generate("c5")
        f5 = measure(w5, dev, args, "balanced", "c5")
        f5["run"].free()
        w5u = unfold(w5)
        u5 = measure(w5u, dev, args, "balanced", "c5", unfolded=True)
        u5["run"].free()
        comparisons["fold"] = {
            "workload": "c5: R=16 k=7 H=64 (M=448), one length 131072 and fifteen 1024",
            "folded": summary("c5 folded (16 requests x 448 rows)", f5, w5),
            "unfolded": summary("c5 unfolded (112 requests x 64 rows)", u5, w5u),
            "kv_bytes_read": {"folded": int(w5.kv_bytes), "unfolded": int(w5u.kv_bytes)},
            "unfolded_over_folded_step": round(u5["step_us"] / f5["step_us"], 3)}
        others["c5"] = comparisons["fold"]["folded"]
        print(f"[bench] c5 folded {f5['step_us']} us, unfolded {u5['step_us']} us",
              file=sys.stderr, flush=True)
        del w5, w5u
        for c in ("c2", "c4"):
            if c == args.config:
                continue
            wc = wl.generate(c)
            mc = measure(wc, dev, args, "balanced", c)
            mc["run"].free()
            others[c] = summary(wl.CONFIGS[c].description, mc, wc)
            print(f"[bench] {c} step {mc['step_us']} us", file=sys.stderr, flush=True)
            del wc

    cfg = w.cfg
    workload = (f"{args.config}: R={cfg.R} k={cfg.k} H={cfg.H} (M={cfg.M}), {cfg.description}"
                + (" [unfolded R*k rows]" if args.unfolded else "")
                + (f" [rank 0 of {args.dcp} DCP ranks, causal]" if args.dcp > 1 else ""))
    roof = head["roofline"]
    roof["measured"] = (f"mean in-step duration of the {args.steps} decode launches of the "
                        f"eager pass (launches {args.warmup}..{args.warmup + args.steps - 1} of "
                        f"{roof['kernel']} in this process), HIP events on the decode's stream")
    res = {
        "metric": "KV-cache HBM GB/s and folded query rows/s (R*k*H per s) per MI355X",
        "value": head["value"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8",
        "data": "synthetic",
        "config": {"workload": workload, "requests": R, "rows_per_req": M,
                   "kv_tokens": int(w.lengths.astype(np.int64).sum()), "page": 64,
                   "plan": args.mode, "kv_pools_rotated": args.pools,
                   "mtile": head["mtile"], "workers": head["workers"],
                   "split_cost_pages": head["split_cost_pages"],
                   "launch": f"hip_graph x{head['chain']} steps"},
        "rows_per_s": head["rows_per_s"],
        "step_us": head["step_us"],
        "step_us_spread": head["step_us_spread"],
        "decode_us": head["decode_us"],
        "decode_us_spread": head["decode_us_spread"],
        "combine_us": head["combine_us"],
        "plan_us": head["plan_us"],
        "splits": head["splits"],
        "value_stage": value_stage,
        "dcp": dcp_res,
        "query_build": query_build,
        "layer_kv_gbs": round(w.kv_bytes / ((head["decode_us"] + head["combine_us"]) / 1e6) / 1e9, 1),
        "layered_step": layered,
        "roofline": roof,
        "comparisons": comparisons,
        "other_workloads": others,
        "timing": ("value: total over exactly `steps` steps replayed from HIP graphs, two "
                   "events; spreads, decode/combine/plan: an eager pass of `steps` steps with "
                   "events around each kernel"),
        "wall_s": round(head["wall"], 3),
        "gen_s": round(gen_s, 1),
        "source": source_digest(),
    }
    if not args.no_cpu_baseline:
        singles = [("c1", wl.generate("c1"))]
        singles.append(("c2", w if args.config == "c2" and not args.unfolded else wl.generate("c2")))
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds, singles)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
