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
  ms_per_pack  the metric's quantity: mean time of the fused pack (all
               buckets), from HIP events stamped by each pack kernel's own
               dispatch at its start and end (hipExtLaunchKernelGGL on the
               launch stream), over K further steps
  roofline     the pack kernel of the largest bucket: algorithmic bytes per
               launch / mean launch time vs 8 TB/s HBM peak; traffic from the
               committed rocprofv3 counter summary when it was taken on the
               current kernel source, else null
  targets      the pack of both target layouts (the 50.3M-element layout and
               one block of the 1.75B KDA-style model), measured in this run
  cpu_baseline the CPU oracle's pack, unchanged, on all host cores (one task
               per member and block of ranks) with the single-thread figure
               beside it; median of 5 after one warm-up, repeated for a few
               seconds of CPU work
plus, measured in the same run: per-kernel times, the pack's p10/p50/p90 cold
and warm, the pre-cast-then-pack comparator (its output checked equal to the
fused pack's), a plain-copy ceiling, the reduce-scatter write-back of rank 0
(with the oracle's rate beside it), the launch floor of every launch of the
step (an empty kernel of the same grid), a pointer-churn leg (new gradient
pointers on every call) and the pack beside a stream of bf16 GEMMs.

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
TARGET_WORKLOADS = ("mixed50m", "kda_block")     # the layouts the >= 80 % target names
WINDOW_BYTES = 2048                               # destination bytes per workgroup of the library's kernels
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
    ap.add_argument("--cpu-seconds", type=float, default=4.0,
                    help="minimum seconds of each CPU-oracle timing (single thread, all cores)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-targets", action="store_true", help="skip the other target layout's pack")
    ap.add_argument("--pack-only", action="store_true",
                    help="run only pack launches (for counter collection under rocprofv3)")
    ap.add_argument("--flat", action="store_true",
                    help="FSDP1 flat-parameter layout of the workload (reduce in fp32, compute in bf16)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run plain 256 MiB device copies (known size) to calibrate byte counters")
    ap.add_argument("--mark-legs", action="store_true",
                    help="launch an empty kernel of LEG workgroups (1, 2, ...) at the start of each leg, so that a "
                         "profiler's kernel trace can be split by leg (LEGS lists them)")
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


def pct(v, q):
    v = sorted(v)
    return v[min(len(v) - 1, int(round(q * (len(v) - 1))))]


def median(v):
    return pct(v, 0.5)


class Bench:
    """Device-side helpers shared by the legs (torch only for memory, streams
    and events; every step of the work runs in the library's kernels)."""

    def __init__(self, args):
        import numpy as np
        import torch

        import fsdp2_mixed_dtype_amd as fp
        import workloads as wl
        self.np, self.torch, self.fp, self.wl = np, torch, fp, wl
        self.args = args
        self.dev = torch.device("cuda:0")
        torch.cuda.set_device(self.dev)
        self.stream = torch.cuda.current_stream()

    def new_event(self):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record(self.stream)          # creates the underlying HIP event
        return e

    def to_dev(self, a, dt):
        t = self.torch.from_numpy(self.np.ascontiguousarray(a))
        if dt == self.fp.BF16:
            t = t.view(self.torch.bfloat16)
        return t.to(self.dev)

    def esz(self, dt):
        return self.fp.ELEM_SIZE[dt]

    def pack_bytes(self, w, plan):
        W = w.world
        out = []
        for b in plan.buckets:
            rd = sum(plan.numel[i] * self.esz(w.tensors[i].grad_dtype) for i in b.members)
            out.append(rd + W * b.S * self.esz(b.dtype))
        return out

    def grad_sets(self, w, plan, grads_h, R):
        """R independent sets of device gradients and packed outputs."""
        sets = []
        for _ in range(R):
            g = [self.to_dev(a, t.grad_dtype) for a, t in zip(grads_h, w.tensors)]
            outs = [self.torch.empty(w.world * b.S, dtype=self.fp.TORCH_DTYPE[b.dtype], device=self.dev)
                    for b in plan.buckets]
            sets.append((self.fp.prepare_grads(plan, g), outs, g))
        return sets

    def time_packs(self, plan, sets, K, warmup):
        """Per-bucket kernel times (ms) of K packs over the rotated sets, each
        stamped by its own dispatch; returns [K][nb]."""
        fp = self.fp
        nb = len(plan.buckets)
        ev = [[(self.new_event(), self.new_event()) for _ in range(nb)] for _ in range(K)]
        self.torch.cuda.synchronize()
        # warm-up launches run straight into the stamped ones, with no host
        # synchronisation between them: the first launch after an idle GPU
        # takes several microseconds longer (54.6 against 47.5 us for the
        # 50.3M-element pack on MI355X), a cost of the idle gap, not of the kernel
        for i in range(len(sets) + warmup):
            g, outs, _ = sets[i % len(sets)]
            for bi in range(nb):
                fp.pack_reduce_scatter_input(plan, bi, g, outs[bi], self.stream)
        for i in range(K):
            g, outs, _ = sets[i % len(sets)]
            for bi in range(nb):
                fp.time_next_launch(*ev[i][bi])
                fp.pack_reduce_scatter_input(plan, bi, g, outs[bi], self.stream)
        self.torch.cuda.synchronize()
        return [[a.elapsed_time(b) for a, b in e] for e in ev]

    def time_empty(self, workgroups, K):
        """Mean time (ms) of an empty kernel of `workgroups` 64-thread workgroups."""
        fp = self.fp
        ev = [(self.new_event(), self.new_event()) for _ in range(K)]
        self.torch.cuda.synchronize()
        for _ in range(3):      # straight into the stamped launches (time_packs)
            fp.empty_launch(workgroups, 64, self.stream)
        for e in ev:
            fp.time_next_launch(*e)
            fp.empty_launch(workgroups, 64, self.stream)
        self.torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in ev) / K


# The bench's legs, in launch order; with --mark-legs each starts with an
# empty kernel of (its index + 1) workgroups
LEGS = ["prime and warm-up", "timed steps", "stamped steps", "warm repeats", "isolated pack", "comparator",
        "copy ceiling", "write-back", "launch floors", "pointer churn", "under load", "other target",
        "calibration copy"]

# Fewest stamped launches behind an isolated pack figure (each one of the
# 50.3M-element layout is ~0.05 ms, so 100 cost a few milliseconds)
PACK_LAUNCHES_MIN = 100


def pack_target(B, name, K, warmup, rotate_bytes):
    """The pack of workload `name` alone (the per-parameter layout), as the
    pages' isolated packing test: max(K, PACK_LAUNCHES_MIN) packs back to back
    over rotated buffer sets, each stamped by its own dispatch."""
    w = B.wl.get(name)
    plan = B.fp.plan_buckets(w.descs(), w.world)
    pb = B.pack_bytes(w, plan)
    R = min(16, max(2, math.ceil(rotate_bytes * 2**30 / sum(pb))))
    sets = B.grad_sets(w, plan, B.wl.make_grads(w), R)
    Kp = max(K, PACK_LAUNCHES_MIN)
    per = B.time_packs(plan, sets, Kp, warmup)
    dom = max(range(len(pb)), key=lambda i: pb[i])
    ms = [sum(x) for x in per]
    bucket_ms = [sum(x[bi] for x in per) / Kp for bi in range(len(pb))]
    res = {"ms_per_pack": round(sum(ms) / Kp, 5), "pack_bytes": sum(pb),
           "GBps": round(sum(pb) / (sum(ms) / Kp * 1e-3) / 1e9, 1),
           "frac_of_peak": round(pb[dom] / (bucket_ms[dom] * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
           "ms_p10_p50_p90": [round(pct(ms, q), 5) for q in (0.1, 0.5, 0.9)],
           "bucket_ms": [round(x, 5) for x in bucket_ms],
           "launches": Kp, "buckets": len(pb), "rotated_sets": R}
    del sets
    plan.destroy()
    return res


def cpu_oracle_pack(ref, grads_h, threads, seconds):
    """Time the oracle's pack of every bucket (the unchanged C routine) on
    `threads` host threads: each task packs one member's rows [r0, r1) (the
    routine called on that sub-layout: W = r1 - r0 rows, the gradient from
    element r0*P, the output from row r0).  Tasks write disjoint bytes, and the
    routine releases the interpreter lock while it runs.  Returns the per-pack
    times (s) after one warm-up, at least 5 and at least `seconds` in all."""
    import ctypes
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    import oracle
    lib = oracle._load()
    outs = [np.empty((ref.W, b.S), dtype=oracle.NP_DTYPE[b.dtype]) for b in ref.buckets]
    gs = [np.ascontiguousarray(g).reshape(-1) for g in grads_h]
    total = sum(ref.W * P for b in ref.buckets for P in b.P)
    chunk = max(1, total // (threads * 8))          # elements per task, roughly
    tasks = []
    for bi, b in enumerate(ref.buckets):
        osz = oracle.ELEM_SIZE[b.dtype]
        for k, i in enumerate(b.members):
            P, O = b.P[k], b.O[k]
            if P == 0:
                continue
            d = ref.params[i]
            gsz = oracle.ELEM_SIZE[d.grad_dtype]
            rows = max(1, min(ref.W, chunk // P))
            for r0 in range(0, ref.W, rows):
                r1 = min(ref.W, r0 + rows)
                valid = max(0, d.numel - r0 * P)
                src = gs[i].ctypes.data + (r0 * P * gsz if valid else 0)
                tasks.append((r1 - r0, src, d.grad_dtype, valid, P, O, b.S, b.dtype,
                              outs[bi].ctypes.data + r0 * b.S * osz, (r1 - r0) * P))
    tasks.sort(key=lambda t: -t[-1])
    args = [(W_, (ctypes.c_void_p * 1)(src), np.array([gdt], np.int32), np.array([valid], np.int64),
             np.array([P], np.int64), np.array([O], np.int64), S, dt, dst)
            for W_, src, gdt, valid, P, O, S, dt, dst, _ in tasks]

    def run(a):
        W_, src, gdt, valid, P, O, S, dt, dst = a
        rc = lib.oracle_pack(W_, 1, src, gdt.ctypes.data, valid.ctypes.data, P.ctypes.data, O.ctypes.data, S, dt, dst)
        if rc:
            raise RuntimeError("oracle_pack: bad layout")

    times = []
    with ThreadPoolExecutor(max_workers=threads) as ex:
        t_all = time.perf_counter()
        while len(times) < 6 or (time.perf_counter() - t_all < seconds and len(times) < 200):
            t0 = time.perf_counter()
            if threads == 1:
                for a in args:
                    run(a)
            else:
                list(ex.map(run, args))
            times.append(time.perf_counter() - t0)
    return times[1:], outs


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build measures one GPU only (W is a layout parameter, no collectives); "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    B = Bench(args)
    np, torch, fp, wl = B.np, B.torch, B.fp, B.wl
    dev = B.dev
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
    esz = B.esz
    pack_bytes = B.pack_bytes(w, plan)
    if args.flat:   # rank 0's pieces read, its whole row (padding included) written
        copy_in_bytes = sum(fp.valid_in_chunk(plan, i, 0) * esz(t.storage_dtype) for i, t in enumerate(w.tensors)) \
            + plan.B
    else:
        copy_in_bytes = sum(P * (esz(t.storage_dtype) + esz(t.param_dtype)) for P, t in zip(plan.P, w.tensors))
    copy_out_bytes = sum(2 * t.numel * esz(t.param_dtype) for t in w.tensors)
    step_bytes = sum(pack_bytes) + copy_in_bytes + copy_out_bytes

    # ---- inputs: seeded host draws, uploaded once per rotation set
    grads_h = wl.make_grads(w)
    set_bytes = step_bytes
    # enough sets that a step never finds its data in the last-level cache,
    # capped for tiny layouts where the whole working set is a few KB
    R = min(16, max(2, math.ceil(args.rotate_bytes * 2**30 / set_bytes)))
    sets = []
    for gset in B.grad_sets(w, plan, grads_h, R):
        g_prep, outs, g = gset
        shard_len = [fp.valid_in_chunk(plan, i, 0) if args.flat else plan.P[i] for i in range(len(w.tensors))]
        shards = [torch.randn(P, device=dev).to(fp.TORCH_DTYPE[t.storage_dtype]) for P, t in zip(shard_len, w.tensors)]
        ag = torch.randint(0, 255, (W * plan.B,), dtype=torch.uint8, device=dev)
        params = [torch.empty(t.numel, dtype=fp.TORCH_DTYPE[t.param_dtype], device=dev) for t in w.tensors]
        # pointer arrays validated once, reused every step (as a training loop
        # reuses its buffers)
        sets.append((g_prep, outs, fp.prepare_shards(plan, shards, 0), ag, fp.prepare_params(plan, params), g))
    torch.cuda.synchronize()

    stream = B.stream
    nb = len(plan.buckets)
    new_event = B.new_event

    def mark(leg):
        if args.mark_legs:
            fp.empty_launch(LEGS.index(leg) + 1, 64, stream)

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

    # prime: one pass over every buffer set (each set's first call uploads its
    # pointer tables), then the W warm-up steps
    mark("prime and warm-up")
    for s_ in sets:
        step(s_)
    for i in range(args.warmup):
        step(sets[i % R])
    torch.cuda.synchronize()

    K = args.steps
    # timed region: K steps exactly as a caller would issue them (no timing
    # events between kernels), bracketed by synchronisations
    mark("timed steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        step(sets[i % R])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / K

    # kernel timing: K more steps in which every launch is stamped by its own
    # dispatch (start and end of that kernel only).  One untimed step runs
    # first, so that the first stamped kernel does not start on an idle GPU
    # (the first launch after a host synchronisation runs several
    # microseconds long); the loop's own GPU time is taken by two events.
    evs = [[(new_event(), new_event()) for _ in range(nb + 2)] for _ in range(K)]
    loop0, loop1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    mark("stamped steps")
    step(sets[(K + R - 1) % R])
    loop0.record(stream)
    for i in range(K):
        step(sets[i % R], evs[i])
    loop1.record(stream)
    torch.cuda.synchronize()
    ms_per_step_instrumented = loop0.elapsed_time(loop1) / K

    def mean_ms(j):
        return sum(e[j][0].elapsed_time(e[j][1]) for e in evs) / K

    pack_ms = [mean_ms(bi) for bi in range(nb)]
    # spread of the per-step pack time (all buckets), and the same packs with
    # their data warm: one buffer set repeated, so much of it stays in the
    # 256 MB Infinity Cache between steps
    per_step = [sum(e[bi][0].elapsed_time(e[bi][1]) for bi in range(nb)) for e in evs]
    pack_in_step_ms = sum(pack_ms)
    mark("warm repeats")
    warm = [sum(x) for x in B.time_packs(plan, [sets[0][:2] + (None,)], K, args.warmup)]
    copy_in_ms = None if args.pack_only else mean_ms(nb)
    copy_out_ms = None if args.pack_only else mean_ms(nb + 1)
    # the metric's quantity: the workload's pack alone (the pages' isolated
    # packing test), over at least PACK_LAUNCHES_MIN stamped launches; the
    # in-step figure above (a pack that follows the previous step's copy-out)
    # is reported beside it
    isolated = None
    if not args.flat and not args.pack_only:
        mark("isolated pack")
        isolated = pack_target(B, args.workload, K, args.warmup, args.rotate_bytes)
        pack_ms = isolated["bucket_ms"]
    pack_total_ms = sum(pack_ms)
    pack_gbps = sum(pack_bytes) / (pack_total_ms * 1e-3) / 1e9
    step_gbps = (sum(pack_bytes) if args.pack_only else step_bytes) / (ms_per_step * 1e-3) / 1e9

    extra = {}
    if not args.pack_only:
        mark("comparator")
        # ---- pre-cast then homogeneous pack (the pages' comparator), our kernels, 2 launches;
        # its output must equal the fused pack's, byte for byte
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
                cmp_out = torch.empty_like(sets[r][1][0])
                csets.append((tmp, fp.prepare_grads(homo, views), cmp_out,
                              fp.prepare_grads(cast_plan, [sets[r][5][j] for j in bf_idx])))
            e_c = [(new_event(), new_event(), new_event(), new_event()) for _ in range(K)]
            for i in range(args.warmup + K):
                tmp, views, out, bf = csets[i % R]
                e = e_c[i - args.warmup] if i >= args.warmup else None
                timed(None if e is None else e[0:2])
                fp.pack_reduce_scatter_input(cast_plan, 0, bf, tmp, stream)
                timed(None if e is None else e[2:4])
                fp.pack_reduce_scatter_input(homo, 0, views, out, stream)
            # the comparator computes the same result: check it on every set
            for r in range(R):
                fp.pack_reduce_scatter_input(plan, 0, sets[r][0], sets[r][1][0], stream)
            torch.cuda.synchronize()
            for r in range(R):
                if not torch.equal(csets[r][2].view(torch.int32), sets[r][1][0].view(torch.int32)):
                    raise SystemExit("bench.py: the pre-cast-then-pack comparator's output differs from the "
                                     f"fused pack's (set {r})")
            precast_ms = sum(a.elapsed_time(b) + c.elapsed_time(d) for a, b, c, d in e_c) / K
            extra.update(precast_then_pack_ms=round(precast_ms, 5), precast_vs_fused=round(precast_ms / pack_total_ms, 3),
                         precast_temporaries_MiB=round(temp_elems * 4 / 2**20, 2),
                         precast_output_equals_fused=True)
            cast_plan.destroy()
            homo.destroy()
            del csets

        # ---- plain-copy ceiling: device-to-device copy moving the pack's byte count
        mark("copy ceiling")
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

        mark("write-back")
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
        wb_ms_b = [sum(e[bi][0].elapsed_time(e[bi][1]) for e in e_w) / K for bi in range(nb)]
        wb_ms = sum(wb_ms_b)
        extra["rs_copy_out"] = {"ms": round(wb_ms, 5), "bytes": wb_bytes,
                                "GBps": round(wb_bytes / (wb_ms * 1e-3) / 1e9, 1),
                                "frac_of_peak": round(wb_bytes / (wb_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                                "rank": 0, "divide_factor": W, "buckets": nb}
        if nb > 1:
            # the same write-back, every bucket in one launch
            asets = []
            for r in range(R):
                dsts = [None] * len(w.tensors)
                for per in wsets[r]:
                    for i, t in enumerate(per[1].tensors):
                        if t is not None:
                            dsts[i] = t
                asets.append(([per[0] for per in wsets[r]], fp.prepare_shard_grads(plan, None, 0, dsts)))
            e_a = [(new_event(), new_event()) for _ in range(K)]
            for i in range(args.warmup + K):
                rows_i, dsts = asets[i % R]
                timed(e_a[i - args.warmup] if i >= args.warmup else None)
                fp.reduce_scatter_copy_out_all(plan, 0, rows_i, dsts, float(W), stream)
            torch.cuda.synchronize()
            wb_all_ms = sum(a.elapsed_time(b) for a, b in e_a) / K
            extra["rs_copy_out"]["all_buckets_one_launch"] = {
                "ms": round(wb_all_ms, 5), "GBps": round(wb_bytes / (wb_all_ms * 1e-3) / 1e9, 1),
                "frac_of_peak": round(wb_bytes / (wb_all_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}
            del asets
        del wsets

        mark("launch floors")
        # ---- launch floor: each launch of the step against an empty kernel
        # of the same number of 64-thread workgroups (the dispatch of its
        # workgroups and the launch's fixed cost)
        def ceil_div(a, b):
            return -(-a // b)
        shift = sets[0][3].data_ptr() % 128
        wg = {}
        for bi, b in enumerate(plan.buckets):
            rows = 1 if args.flat else W
            row_bytes = (W * b.S if args.flat else b.S) * esz(b.dtype)
            wg[f"pack[{bi}]"] = (ceil_div(row_bytes, WINDOW_BYTES) + 1) * rows
        if args.flat:
            wg["copy_in"] = ceil_div(shift + plan.B, WINDOW_BYTES)
        else:
            # each parameter's segment [A_t, A_t+1) of the row gets the windows
            # its worst line alignment needs (a segment starts <= 124 bytes past a line)
            ends = list(plan.A[1:]) + [plan.B]
            wg["copy_in"] = sum(ceil_div(e - a + 124, WINDOW_BYTES) for a, e in zip(plan.A, ends) if e > a)
        wg["copy_out"] = sum(ceil_div(t.numel * esz(t.param_dtype), WINDOW_BYTES) for t in w.tensors if t.numel)
        for bi, b in enumerate(plan.buckets):
            if args.flat:
                wg[f"write_back[{bi}]"] = ceil_div(plan.c * esz(b.dtype), WINDOW_BYTES)
            else:
                wg[f"write_back[{bi}]"] = sum(ceil_div(P * esz(w.tensors[i].storage_dtype), WINDOW_BYTES)
                                              for i, P in zip(b.members, b.P) if P)
        kernel_ms = {f"pack[{bi}]": pack_ms[bi] for bi in range(nb)}
        kernel_ms.update(copy_in=copy_in_ms, copy_out=copy_out_ms)
        kernel_ms.update({f"write_back[{bi}]": wb_ms_b[bi] for bi in range(nb)})
        if nb > 1:
            wg["write_back_all"] = sum(wg[f"write_back[{bi}]"] for bi in range(nb))
            kernel_ms["write_back_all"] = wb_all_ms
        floors = {}
        for name, n in wg.items():
            f_ms = B.time_empty(n, K)
            floors[name] = {"workgroups": n, "kernel_us": round(kernel_ms[name] * 1e3, 2),
                            "floor_us": round(f_ms * 1e3, 2),
                            "above_floor_us": round((kernel_ms[name] - f_ms) * 1e3, 2)}
        extra["launch_floor"] = floors

        mark("pointer churn")
        # ---- pointer churn: every call brings a new set of gradient pointers
        # (as when gradients are allocated afresh each backward), cycling
        # through more sets than the library's 16-entry table cache (which
        # only units of more than 960 parameters use: smaller pointer sets
        # travel in the launch arguments)
        n_churn = 20
        churn = [fp.prepare_grads(plan, [B.to_dev(a, t.grad_dtype) for a, t in zip(grads_h, w.tensors)])
                 for _ in range(n_churn)]
        outs0 = sets[0][1]
        for i in range(2 * n_churn):                # warm: every slot holds one of these sets
            for bi in range(nb):
                fp.pack_reduce_scatter_input(plan, bi, churn[i % n_churn], outs0[bi], stream)
        torch.cuda.synchronize()
        cnt0 = fp.counters()
        e_ch = [[(new_event(), new_event()) for _ in range(nb)] for _ in range(K)]
        host = []
        torch.cuda.synchronize()
        t_ch = time.perf_counter()
        for i in range(K):
            for bi in range(nb):
                fp.time_next_launch(*e_ch[i][bi])
                h0 = time.perf_counter()
                fp.pack_reduce_scatter_input(plan, bi, churn[(i + 2 * n_churn) % n_churn], outs0[bi], stream)
                host.append(time.perf_counter() - h0)
        torch.cuda.synchronize()
        churn_wall = (time.perf_counter() - t_ch) * 1e3 / K
        cnt1 = fp.counters()
        # the same packs with tensor lists, validated on every call: the host
        # time per step of a caller whose gradients are new tensors each step
        host_lists = []
        for i in range(K):
            gl = churn[(i + 2 * n_churn) % n_churn].tensors
            h0 = time.perf_counter()
            for bi in range(nb):
                fp.pack_reduce_scatter_input(plan, bi, gl, outs0[bi], stream)
            host_lists.append(time.perf_counter() - h0)
        torch.cuda.synchronize()
        churn_pack = sum(a.elapsed_time(b) for e in e_ch for a, b in e) / K
        # the same loop without kernel-stamped events (whose dispatch adds a
        # few microseconds per launch): the wall time per pack a caller sees
        t_pl = time.perf_counter()
        for i in range(K):
            for bi in range(nb):
                fp.pack_reduce_scatter_input(plan, bi, churn[(i + 2 * n_churn) % n_churn], outs0[bi], stream)
        torch.cuda.synchronize()
        churn_plain = (time.perf_counter() - t_pl) * 1e3 / K
        # the same calls queued behind ~2 ms of GPU work: a replacement never
        # waits for the device, so 16 calls return long before that work ends
        a_mm = torch.randn(4096, 4096, device=dev, dtype=torch.bfloat16)
        b_mm = torch.randn(4096, 4096, device=dev, dtype=torch.bfloat16)
        torch.mm(a_mm, b_mm)                        # (loads the GEMM's code before the timed part)
        for i in range(n_churn):                    # slots refilled before the busy work
            for bi in range(nb):
                fp.pack_reduce_scatter_input(plan, bi, churn[i], outs0[bi], stream)
        torch.cuda.synchronize()
        busy0, busy1 = new_event(), new_event()
        busy0.record(stream)
        for _ in range(16):
            torch.mm(a_mm, b_mm)
        busy1.record(stream)
        h0 = time.perf_counter()
        for i in range(16):
            for bi in range(nb):
                fp.pack_reduce_scatter_input(plan, bi, churn[i], outs0[bi], stream)
        host_behind_busy = (time.perf_counter() - h0) * 1e3
        torch.cuda.synchronize()
        extra["pointer_churn"] = {
            "sets": n_churn, "table_slots": 16,
            "pack_kernel_ms": round(churn_pack, 5),
            "wall_ms_per_pack": round(churn_plain, 5),
            "wall_ms_per_pack_stamped": round(churn_wall, 5),
            "host_us_per_call_p50": round(median(host) * 1e6, 1),
            "host_us_per_step_tensor_lists_p50": round(median(host_lists) * 1e6, 1),
            "inline_pointer_launches": cnt1[6] - cnt0[6],
            "table_uploads": cnt1[1] - cnt0[1], "table_replacements": cnt1[4] - cnt0[4],
            "cross_stream_waits": cnt1[5] - cnt0[5],
            "host_ms_for_16_calls_behind_busy_gpu": round(host_behind_busy, 3),
            "busy_gpu_ms": round(busy0.elapsed_time(busy1), 3),
            "host_waits": cnt1[7] - cnt0[7],
        }
        del churn, a_mm, b_mm

        mark("under load")
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

        def packs(n, st, stamps=None):
            for i in range(n):
                g, outs, _, _, _, _ = sets[i % R]
                for bi in range(nb):
                    timed(None if stamps is None else stamps[i][bi])
                    fp.pack_reduce_scatter_input(plan, bi, g, outs[bi], st)

        def side_by_side(n, stamps=None):
            """n packs on the side stream beside G GEMMs on the current one;
            returns (both streams' span, the GEMMs' span) in ms."""
            c0, c1, m0, m1 = new_event(), new_event(), new_event(), new_event()
            torch.cuda.synchronize()
            c0.record(stream)
            side.wait_event(c0)
            packs(n, side, stamps)
            m0.record(stream)
            gemms(G)
            m1.record(stream)
            side_done = torch.cuda.Event()
            side_done.record(side)
            stream.wait_event(side_done)
            c1.record(stream)
            torch.cuda.synchronize()
            return c0.elapsed_time(c1), m0.elapsed_time(m1)

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
        # the packs alone, back to back and unstamped, as they run beside the GEMMs
        p0, p1 = new_event(), new_event()
        packs(R, stream)
        torch.cuda.synchronize()
        p0.record(stream)
        packs(n_packs, stream)
        p1.record(stream)
        torch.cuda.synchronize()
        pack_wall_ms = p0.elapsed_time(p1) / n_packs
        # side by side: one untimed pass first (the first pass of packs and
        # GEMMs on the two streams ran 15-20 % longer than the ones after it,
        # a cost of the first concurrent use, not of the steady state), then
        # the median of three passes of unstamped packs for the wall times (a
        # stamped dispatch adds a few microseconds of gap to its stream), then
        # stamped packs for the pack's own kernel time under the load
        side_by_side(n_packs)
        passes = sorted(side_by_side(n_packs) for _ in range(3))
        both_ms, gemm_beside_ms = passes[1]
        e_p = [[(new_event(), new_event()) for _ in range(nb)] for _ in range(n_packs)]
        side_by_side(n_packs, e_p)
        pack_load_ms = sum(a.elapsed_time(b) for e in e_p for a, b in e) / n_packs
        seq_ms = G * gemm_ms + n_packs * pack_wall_ms
        extra["pack_under_load"] = {
            "gemm": f"bf16 mm {n_mm}x{n_mm}x{n_mm}, {G} back to back on the current stream",
            "gemm_ms_alone": round(gemm_ms, 5),
            "gemm_TFLOPs_alone": round(2 * n_mm ** 3 / (gemm_ms * 1e-3) / 1e12, 1),
            "gemm_ms_beside_packs": round(gemm_beside_ms / G, 5),
            "packs": n_packs,
            "pack_ms_alone": round(pack_total_ms, 5),
            "pack_wall_ms_alone": round(pack_wall_ms, 5),
            "pack_ms_under_load": round(pack_load_ms, 5),
            "pack_slowdown": round(pack_load_ms / pack_total_ms, 3),
            "sequential_ms": round(seq_ms, 3),
            "concurrent_ms": round(both_ms, 3),
            "concurrent_ms_passes": [round(x[0], 3) for x in passes],
            "overlap_saving": round(1 - both_ms / seq_ms, 4),
        }
        del ma, mb, mc

    if args.calib_copy:
        mark("calibration copy")
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
            summ = json.load(f).get(args.workload + ("_flat" if args.flat else ""))
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
                "kernel": "pack_kernel", "bytes_per_launch": pack_bytes[dom]}

    # ---- the pack of both target layouts, measured in this run
    targets = None
    if not args.flat and not args.pack_only and not args.no_targets:
        targets = {}
        for name in TARGET_WORKLOADS:
            if name == args.workload and isolated is not None:
                targets[name] = isolated
            else:
                mark("other target")
                targets[name] = pack_target(B, name, K, args.warmup, args.rotate_bytes)
            targets[name]["meets_80pct"] = targets[name]["frac_of_peak"] >= 0.80

    # ---- CPU baseline: the oracle, as it stands, on the same pack
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        ref = oracle.plan(w.descs(), W) if not args.flat else None
        if ref is not None:
            cores = len(os.sched_getaffinity(0))
            single, packed_h = cpu_oracle_pack(ref, grads_h, 1, args.cpu_seconds)
            multi, packed_m = cpu_oracle_pack(ref, grads_h, cores, args.cpu_seconds)
            # the parallel run computes the same bytes as the single-thread run
            for a_, b_ in zip(packed_h, packed_m):
                if a_.tobytes() != b_.tobytes():
                    raise SystemExit("bench.py: the oracle's pack on several threads differs from one thread")
            cpu_model = None
            try:
                with open("/proc/cpuinfo") as f:
                    cpu_model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), None)
            except OSError:
                pass
            ms_1, ms_n = median(single) * 1e3, median(multi) * 1e3
            cpu = {"value": round(sum(pack_bytes) / (ms_n * 1e-3) / 1e9, 3), "unit": "GB/s", "cores": cores,
                   "kind": "oracle", "cpu_model": cpu_model, "ms_per_pack": round(ms_n, 3),
                   "single_thread": {"value": round(sum(pack_bytes) / (ms_1 * 1e-3) / 1e9, 3), "unit": "GB/s",
                                     "ms_per_pack": round(ms_1, 3), "samples": len(single)},
                   "sample": f"the oracle's pack of every bucket of {args.workload}, full size; median of "
                             f"{len(multi)} packs on {cores} threads (one task per member and block of ranks) and of "
                             f"{len(single)} on one thread, each after one warm-up; GB/s under the same byte model"}
            if "rs_copy_out" in extra:
                # the oracle's write-back of rank 0 beside the kernel's, same byte model (one thread)
                reps_w, t_w = 0, 0.0
                while reps_w == 0 or t_w < 1.0:
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
        "ms_per_pack": round(pack_total_ms, 5),
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
        "targets": targets,
        "pack_ms": round(pack_total_ms, 5),
        "pack_GBps": round(pack_gbps, 1),
        "pack_frac_of_peak": round(pack_gbps / HBM_PEAK_GBPS, 4),
        "pack_bytes": sum(pack_bytes),
        "pack_ms_p10_p50_p90": (isolated["ms_p10_p50_p90"] if isolated is not None
                                else [round(pct(per_step, q), 5) for q in (0.1, 0.5, 0.9)]),
        "pack_launches_timed": isolated["launches"] if isolated is not None else K,
        "pack_in_step_ms": round(pack_in_step_ms, 5),
        "pack_in_step_ms_p10_p50_p90": [round(pct(per_step, q), 5) for q in (0.1, 0.5, 0.9)],
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
