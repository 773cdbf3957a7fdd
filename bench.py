"""Benchmark of the FSDP2 mixed-dtype hot path on one MI355X.

One step = the fused reduce-scatter pack of every bucket + the all-gather
copy-in of rank 0 + the all-gather copy-out of the gathered buffer, on the
chosen workload (default: the 50.3M-element mixed bf16/fp32 transformer
layout, W=8, the layout of the pages' isolated packing test).  Inputs are
seeded synthetic tensors already resident in HBM; R independent buffer sets
are rotated so that no step finds its data in the 256 MB last-level cache.

Prints ONE JSON line (rank 0):
  value        whole-step algorithmic bytes / step time  (GB/s)
  ms_per_step  wall time per step over the K timed steps (launched as a
               caller would, nothing between the kernels)
  roofline     the pack kernel: algorithmic bytes per launch / mean launch
               time vs 8 TB/s HBM peak.  Launch times come from K further
               steps in which HIP events are stamped by each kernel's own
               dispatch at its start and end (hipExtLaunchKernelGGL on the
               launch stream);
               traffic from the committed rocprofv3 counter summary when it
               was taken on the current kernel source, else null
  cpu_baseline the CPU oracle's pack, single thread, on a bounded sample
plus, measured in the same run: per-kernel times, the pack's p10/p50/p90
cold and warm, the pre-cast-then-pack comparator, a plain-copy ceiling, the
reduce-scatter write-back of rank 0 (with the oracle's rate beside it) and
the pack beside a stream of bf16 GEMMs.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--flat]
(--flat: the workload's tensors as one FSDP1 flat parameter.)
"""
from __future__ import annotations

import argparse
import gc
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "ms per fused mixed-dtype pack + achieved HBM GB/s (% of MI355X peak)"
HBM_PEAK_GBPS = 8000.0
PAGES_H100_FUSED_MS = 0.1888      # isolated H100 test, 50.3M-element layout (context only)
PAGES_H100_PRECAST_MS = 0.3582
# the sources that decide what a pack launch reads and writes
KERNEL_SOURCES = [os.path.join(ROOT, "fsdp2_mixed_dtype_amd", "csrc", f)
                  for f in ("fsdppack_kernels.hip", "fsdppack_internal.h", "fsdppack_plan.cpp")]
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "pack_traffic.json")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="mixed50m")
    ap.add_argument("--rotate-bytes", type=float, default=2.0, help="GiB of buffers rotated across steps")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="bound on the CPU-oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--pack-only", action="store_true",
                    help="run only pack launches (for counter collection under rocprofv3)")
    ap.add_argument("--flat", action="store_true",
                    help="FSDP1 flat-parameter layout of the workload (reduce in fp32, compute in bf16)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run plain 256 MiB device copies (known size) to calibrate byte counters")
    return ap.parse_args()


def _code_only(text):
    """C/C++ source without comments and with whitespace runs collapsed, so
    that editing a comment does not count as changing the kernel."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash():
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        with open(path, encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build measures one GPU only (W is a layout parameter, no collectives); "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import fsdp2_mixed_dtype_amd as fp
    import workloads as wl

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = wl.get(args.workload)
    if args.flat:
        # one flat parameter per unit: one reduction and one param dtype
        ts = w.tensors
        w = wl.custom([t.shape for t in ts], [t.grad_dtype for t in ts], [fp.FP32] * len(ts), w.world, w.seed,
                      storage_dtypes=[t.storage_dtype for t in ts], param_dtypes=[fp.BF16] * len(ts),
                      grad_sigma=w.grad_sigma, param_sigma=w.param_sigma)
    W = w.world
    # planning is init work: the fastest of five builds, with Python's garbage
    # collector paused so that a collection of the interpreter's heap is not
    # counted as planning
    plan_fn = fp.plan_buckets_flat if args.flat else fp.plan_buckets
    descs = w.descs()
    gc_on = gc.isenabled()
    gc.disable()
    plan_times = []
    for i in range(5):
        t_plan = time.perf_counter()
        plan = plan_fn(descs, W)
        plan_times.append(time.perf_counter() - t_plan)
        if i < 4:
            plan.destroy()
    if gc_on:
        gc.enable()
    plan_us = min(plan_times) * 1e6

    # ---- algorithmic bytes (read + write) per launch
    def esz(dt):
        return fp.ELEM_SIZE[dt]
    pack_bytes = []
    for b in plan.buckets:
        rd = sum(plan.numel[i] * esz(w.tensors[i].grad_dtype) for i in b.members)
        pack_bytes.append(rd + W * b.S * esz(b.dtype))
    if args.flat:   # rank 0's pieces read, its whole row (padding included) written
        copy_in_bytes = sum(fp.valid_in_chunk(plan, i, 0) * esz(t.storage_dtype) for i, t in enumerate(w.tensors)) \
            + plan.B
    else:
        copy_in_bytes = sum(P * (esz(t.storage_dtype) + esz(t.param_dtype)) for P, t in zip(plan.P, w.tensors))
    copy_out_bytes = sum(2 * t.numel * esz(t.param_dtype) for t in w.tensors)
    step_bytes = sum(pack_bytes) + copy_in_bytes + copy_out_bytes

    # ---- inputs: seeded host draws, uploaded once per rotation set
    grads_h = wl.make_grads(w)

    def to_dev(a, dt):
        t = torch.from_numpy(np.ascontiguousarray(a))
        if dt == fp.BF16:
            t = t.view(torch.bfloat16)
        return t.to(dev)

    set_bytes = step_bytes
    # enough sets that a step never finds its data in the last-level cache,
    # capped for tiny layouts where the whole working set is a few KB
    R = min(16, max(2, math.ceil(args.rotate_bytes * 2**30 / set_bytes)))
    sets = []
    for r in range(R):
        g = [to_dev(a, t.grad_dtype) for a, t in zip(grads_h, w.tensors)]
        outs = [torch.empty(W * b.S, dtype=fp.TORCH_DTYPE[b.dtype], device=dev) for b in plan.buckets]
        shard_len = [fp.valid_in_chunk(plan, i, 0) if args.flat else plan.P[i] for i in range(len(w.tensors))]
        shards = [torch.randn(P, device=dev).to(fp.TORCH_DTYPE[t.storage_dtype]) for P, t in zip(shard_len, w.tensors)]
        ag = torch.randint(0, 255, (W * plan.B,), dtype=torch.uint8, device=dev)
        params = [torch.empty(t.numel, dtype=fp.TORCH_DTYPE[t.param_dtype], device=dev) for t in w.tensors]
        # pointer arrays validated once, reused every step (as a training loop
        # reuses its buffers)
        sets.append((fp.prepare_grads(plan, g), outs, fp.prepare_shards(plan, shards, 0), ag,
                     fp.prepare_params(plan, params), g))
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    nb = len(plan.buckets)

    def timed(pair):
        # the library stamps these events at the kernel's own start and end
        if pair is not None:
            fp.time_next_launch(*pair)

    def step(s, ev=None):
        g, outs, shards, ag, params, _ = s
        for bi in range(nb):
            timed(None if ev is None else ev[bi])
            fp.pack_reduce_scatter_input(plan, bi, g, outs[bi], stream)
        if args.pack_only:
            return
        timed(None if ev is None else ev[nb])
        fp.all_gather_copy_in(plan, 0, shards, ag, stream)
        timed(None if ev is None else ev[nb + 1])
        fp.all_gather_copy_out(plan, ag, params, stream)

    def new_event():
        e = torch.cuda.Event(enable_timing=True)
        e.record(stream)          # creates the underlying HIP event
        return e

    # prime: one pass over every buffer set (each set's first call uploads its
    # pointer tables), then the W warm-up steps
    for s_ in sets:
        step(s_)
    for i in range(args.warmup):
        step(sets[i % R])
    torch.cuda.synchronize()

    K = args.steps
    # timed region: K steps exactly as a caller would issue them (no timing
    # events between kernels), bracketed by synchronisations
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        step(sets[i % R])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / K

    # kernel timing: K more steps in which every launch is stamped by its own
    # dispatch (start and end of that kernel only)
    evs = [[(new_event(), new_event()) for _ in range(nb + 2)] for _ in range(K)]
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for i in range(K):
        step(sets[i % R], evs[i])
    torch.cuda.synchronize()
    ms_per_step_instrumented = (time.perf_counter() - t1) * 1e3 / K

    def mean_ms(j):
        return sum(e[j][0].elapsed_time(e[j][1]) for e in evs) / K

    pack_ms = [mean_ms(bi) for bi in range(nb)]
    # spread of the per-step pack time (all buckets), and the same packs with
    # their data warm: one buffer set repeated, so much of it stays in the
    # 256 MB Infinity Cache between steps
    per_step = sorted(sum(e[bi][0].elapsed_time(e[bi][1]) for bi in range(nb)) for e in evs)

    def pct(v, q):
        return v[min(len(v) - 1, int(round(q * (len(v) - 1))))]

    e_warm = [[(new_event(), new_event()) for _ in range(nb)] for _ in range(K)]
    for i in range(args.warmup + K):
        g, outs = sets[0][0], sets[0][1]
        for bi in range(nb):
            timed(e_warm[i - args.warmup][bi] if i >= args.warmup else None)
            fp.pack_reduce_scatter_input(plan, bi, g, outs[bi], stream)
    torch.cuda.synchronize()
    warm = sorted(sum(a.elapsed_time(b) for a, b in e) for e in e_warm)
    copy_in_ms = None if args.pack_only else mean_ms(nb)
    copy_out_ms = None if args.pack_only else mean_ms(nb + 1)
    pack_total_ms = sum(pack_ms)
    pack_gbps = sum(pack_bytes) / (pack_total_ms * 1e-3) / 1e9
    step_gbps = (sum(pack_bytes) if args.pack_only else step_bytes) / (ms_per_step * 1e-3) / 1e9

    extra = {}
    if not args.pack_only:
        # ---- pre-cast then homogeneous pack (the pages' comparator), our kernels, 2 launches
        bf_idx = [i for i, t in enumerate(w.tensors) if t.grad_dtype == fp.BF16]
        if bf_idx and nb == 1 and plan.buckets[0].dtype == fp.FP32 and not args.flat:
            cast_plan = fp.plan_buckets([(w.tensors[i].numel, 1, fp.BF16, fp.FP32, fp.FP32, fp.FP32)
                                         for i in bf_idx], 1)
            homo = fp.plan_buckets([(t.dim0, t.inner, fp.FP32, fp.FP32, fp.FP32, fp.FP32) for t in w.tensors], W)
            temp_elems = cast_plan.buckets[0].S
            cast_offsets = cast_plan.buckets[0].O
            csets = []
            for r in range(R):
                tmp = torch.empty(temp_elems, dtype=torch.float32, device=dev)
                views = list(sets[r][5])
                for k, i in enumerate(bf_idx):
                    views[i] = tmp[cast_offsets[k]: cast_offsets[k] + w.tensors[i].numel]
                csets.append((tmp, fp.prepare_grads(homo, views), sets[r][1][0],
                              fp.prepare_grads(cast_plan, [sets[r][5][j] for j in bf_idx])))
            e_c = [(new_event(), new_event(), new_event(), new_event()) for _ in range(K)]
            for i in range(args.warmup + K):
                tmp, views, out, bf = csets[i % R]
                e = e_c[i - args.warmup] if i >= args.warmup else None
                timed(None if e is None else e[0:2])
                fp.pack_reduce_scatter_input(cast_plan, 0, bf, tmp, stream)
                timed(None if e is None else e[2:4])
                fp.pack_reduce_scatter_input(homo, 0, views, out, stream)
            torch.cuda.synchronize()
            precast_ms = sum(a.elapsed_time(b) + c.elapsed_time(d) for a, b, c, d in e_c) / K
            extra.update(precast_then_pack_ms=round(precast_ms, 5), precast_vs_fused=round(precast_ms / pack_total_ms, 3),
                         precast_temporaries_MiB=round(temp_elems * 4 / 2**20, 2))
            cast_plan.destroy()
            homo.destroy()

        # ---- plain-copy ceiling: device-to-device copy moving the pack's byte count
        nbytes = sum(pack_bytes) // 2
        src = [torch.empty(nbytes // 4, dtype=torch.float32, device=dev) for _ in range(R)]
        dst = [torch.empty_like(x) for x in src]
        for i in range(args.warmup):
            dst[i % R].copy_(src[i % R])
        c0, c1 = new_event(), new_event()
        torch.cuda.synchronize()
        c0.record(stream)
        for i in range(K):
            dst[i % R].copy_(src[i % R])
        c1.record(stream)
        torch.cuda.synchronize()
        copy_ms = c0.elapsed_time(c1) / K      # back-to-back copies, events around the batch
        extra["copy_ceiling_GBps"] = round(2 * (nbytes // 4) * 4 / (copy_ms * 1e-3) / 1e9, 1)
        extra["pack_frac_of_copy_ceiling"] = round(pack_gbps / extra["copy_ceiling_GBps"], 4)
        del src, dst

        # ---- reduce-scatter write-back of rank 0 (the step after the
        # reduce-scatter): row 0 of each bucket's packed buffer stands in for
        # the rank's reduced row, divided by W and cast to the storage dtypes
        wb_bytes = 0
        for bi, b in enumerate(plan.buckets):
            for i in b.members:
                wb_bytes += fp.valid_in_chunk(plan, i, 0) * (esz(b.dtype) + esz(w.tensors[i].storage_dtype))
        wsets = []
        for r in range(R):
            per_bucket = []
            for bi, b in enumerate(plan.buckets):
                dsts = [torch.empty(fp.valid_in_chunk(plan, i, 0), dtype=fp.TORCH_DTYPE[t.storage_dtype], device=dev)
                        if i in b.members else None for i, t in enumerate(w.tensors)]
                per_bucket.append((sets[r][1][bi][:b.S], fp.prepare_shard_grads(plan, bi, 0, dsts)))
            wsets.append(per_bucket)
        e_w = [[(new_event(), new_event()) for _ in range(nb)] for _ in range(K)]
        for i in range(args.warmup + K):
            for bi in range(nb):
                row, dsts = wsets[i % R][bi]
                timed(e_w[i - args.warmup][bi] if i >= args.warmup else None)
                fp.reduce_scatter_copy_out(plan, bi, 0, row, dsts, float(W), stream)
        torch.cuda.synchronize()
        wb_ms = sum(a.elapsed_time(b) for e in e_w for a, b in e) / K
        extra["rs_copy_out"] = {"ms": round(wb_ms, 5), "bytes": wb_bytes,
                                "GBps": round(wb_bytes / (wb_ms * 1e-3) / 1e9, 1),
                                "frac_of_peak": round(wb_bytes / (wb_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                                "rank": 0, "divide_factor": W, "buckets": nb}
        del wsets

        # ---- pack under concurrent load: packs on a side stream (default
        # priority) while a stream of bf16 GEMMs keeps the GPU busy, as FSDP
        # overlaps its gradient staging with the backward's compute
        n_mm = 4096
        ma = torch.randn(n_mm, n_mm, device=dev).to(torch.bfloat16)
        mb = torch.randn(n_mm, n_mm, device=dev).to(torch.bfloat16)
        mc = torch.empty(n_mm, n_mm, dtype=torch.bfloat16, device=dev)
        side = torch.cuda.Stream(device=dev)

        def gemms(k):
            for _ in range(k):
                torch.mm(ma, mb, out=mc)

        gemms(5)
        g0, g1 = new_event(), new_event()
        torch.cuda.synchronize()
        G = 100
        g0.record(stream)
        gemms(G)
        g1.record(stream)
        torch.cuda.synchronize()
        gemm_ms = g0.elapsed_time(g1) / G
        n_packs = max(K, math.ceil(G * gemm_ms / pack_total_ms))
        e_p = [[(new_event(), new_event()) for _ in range(nb)] for _ in range(n_packs)]
        c0, c1, m0, m1 = new_event(), new_event(), new_event(), new_event()
        torch.cuda.synchronize()
        c0.record(stream)
        side.wait_event(c0)
        for i in range(n_packs):
            g, outs, _, _, _, _ = sets[i % R]
            for bi in range(nb):
                timed(e_p[i][bi])
                fp.pack_reduce_scatter_input(plan, bi, g, outs[bi], side)
        m0.record(stream)
        gemms(G)
        m1.record(stream)
        side_done = torch.cuda.Event()
        side_done.record(side)
        stream.wait_event(side_done)
        c1.record(stream)
        torch.cuda.synchronize()
        both_ms = c0.elapsed_time(c1)
        pack_load_ms = sum(a.elapsed_time(b) for e in e_p for a, b in e) / n_packs
        extra["pack_under_load"] = {
            "gemm": f"bf16 mm {n_mm}x{n_mm}x{n_mm}, {G} back to back on the current stream",
            "gemm_ms_alone": round(gemm_ms, 5),
            "gemm_TFLOPs_alone": round(2 * n_mm ** 3 / (gemm_ms * 1e-3) / 1e12, 1),
            "gemm_ms_beside_packs": round(m0.elapsed_time(m1) / G, 5),
            "packs": n_packs,
            "pack_ms_alone": round(pack_total_ms, 5),
            "pack_ms_under_load": round(pack_load_ms, 5),
            "pack_slowdown": round(pack_load_ms / pack_total_ms, 3),
            "sequential_ms": round(G * gemm_ms + n_packs * pack_total_ms, 3),
            "concurrent_ms": round(both_ms, 3),
            "overlap_saving": round(1 - both_ms / (G * gemm_ms + n_packs * pack_total_ms), 4),
        }
        del ma, mb, mc

    if args.calib_copy:
        # plain device-to-device copies of a known size: what a byte counter
        # reads for them calibrates the counter against real traffic
        n = 256 * 2**20 // 4
        a = torch.ones(n, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        extra["calib_copy_bytes_each_way"] = n * 4
        del a, b

    # ---- roofline of the dominant kernel (the pack of the largest bucket)
    dom = max(range(nb), key=lambda i: pack_bytes[i])
    achieved = pack_bytes[dom] / (pack_ms[dom] * 1e-3) / 1e9
    traffic = None
    try:
        with open(TRAFFIC_SUMMARY) as f:
            summ = json.load(f).get(args.workload)
        # counter figures only stand while the kernel they were taken on does;
        # a layout with several buckets has them per bucket
        if summ and summ.get("kernel_source_sha256_16") == kernel_source_hash():
            rec = summ if nb == 1 else summ.get("buckets", {}).get(str(dom))
            if rec:
                traffic = rec.get("traffic_bytes_per_launch")
    except (OSError, ValueError):
        pass
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                "kernel": "window_kernel<pack>", "bytes_per_launch": pack_bytes[dom]}

    # ---- CPU baseline: the oracle, as it stands, on a bounded sample of the same pack
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        ref = oracle.plan(w.descs(), W)
        reps, t_cpu = 0, 0.0
        t_start = time.perf_counter()
        packed_h = [None] * nb
        while reps == 0 or (time.perf_counter() - t_start) < args.cpu_seconds:
            ta = time.perf_counter()
            for bi in range(nb):
                packed_h[bi] = oracle.pack(ref, bi, grads_h)
            t_cpu += time.perf_counter() - ta
            reps += 1
        cpu_gbps = reps * sum(pack_bytes) / t_cpu / 1e9
        cpu_model = None
        try:
            with open("/proc/cpuinfo") as f:
                cpu_model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), None)
        except OSError:
            pass
        cpu = {"value": round(cpu_gbps, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
               "host_cores_available": len(os.sched_getaffinity(0)), "cpu_model": cpu_model,
               "sample": f"oracle pack of every bucket of {args.workload}, full size, repeated {reps}x "
                         f"({t_cpu:.1f} s, single thread); GB/s under the same byte model",
               "ms_per_pack": round(t_cpu / reps * 1e3, 2)}
        if "rs_copy_out" in extra:
            # the oracle's write-back of rank 0 beside the kernel's, same byte model
            reps_w, t_w = 0, 0.0
            while reps_w == 0 or t_w < min(args.cpu_seconds, 3.0):
                ta = time.perf_counter()
                for bi in range(nb):
                    oracle.rs_copy_out(ref, bi, 0, packed_h[bi][0], float(W))
                t_w += time.perf_counter() - ta
                reps_w += 1
            extra["rs_copy_out"]["cpu_oracle_GBps"] = round(reps_w * extra["rs_copy_out"]["bytes"] / t_w / 1e9, 3)

    out = {
        "metric": METRIC,
        "value": round(step_gbps, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "ms_per_step_with_kernel_events": round(ms_per_step_instrumented, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16,fp32",
        "data": "synthetic",
        "config": {"workload": args.workload + (" (FSDP1 flat layout)" if args.flat else ""), "world": W,
                   "tensors": len(w.tensors),
                   "elements": sum(t.numel for t in w.tensors), "buckets": nb,
                   "step": "pack(all buckets)" + ("" if args.pack_only else " + copy_in(rank 0) + copy_out"),
                   "rotated_sets": R},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "pack_ms": round(pack_total_ms, 5),
        "pack_GBps": round(pack_gbps, 1),
        "pack_frac_of_peak": round(pack_gbps / HBM_PEAK_GBPS, 4),
        "pack_bytes": sum(pack_bytes),
        "pack_ms_p10_p50_p90": [round(pct(per_step, q), 5) for q in (0.1, 0.5, 0.9)],
        "pack_ms_warm_p10_p50_p90": [round(pct(warm, q), 5) for q in (0.1, 0.5, 0.9)],
        "copy_in_ms": None if copy_in_ms is None else round(copy_in_ms, 5),
        "copy_in_GBps": None if copy_in_ms is None else round(copy_in_bytes / (copy_in_ms * 1e-3) / 1e9, 1),
        "copy_out_ms": None if copy_out_ms is None else round(copy_out_ms, 5),
        "copy_out_GBps": None if copy_out_ms is None else round(copy_out_bytes / (copy_out_ms * 1e-3) / 1e9, 1),
        "step_bytes": step_bytes,
        "plan_us": round(plan_us, 1),
        "pages_h100_fused_pack_ms": PAGES_H100_FUSED_MS if args.workload == "mixed50m" else None,
        "pages_h100_precast_ms": PAGES_H100_PRECAST_MS if args.workload == "mixed50m" else None,
        "kernel_source_sha256_16": kernel_source_hash(),
    }
    out.update(extra)
    print(json.dumps(out), flush=True)
    plan.destroy()


if __name__ == "__main__":
    main()
