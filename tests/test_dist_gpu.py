"""The library's kernels in the multi-rank data flow: 2 ranks (2 processes on
the one GPU), collectives over gloo on host copies.

Each rank packs its gradients with libfsdppack, the packed buffer goes
through a reduce-scatter (gloo, on a host copy), the rank's reduced row comes
back to the GPU and the library writes back its sharded gradients divided by
W; each rank copies its shards into its all-gather row with the library, the
rows are all-gathered (gloo, host copies), and the library copies the full
parameters out.  Checked against the plain definitions (the rank's slice of
the averaged gradient, the cast parameters), for both layouts.  Gradients
are small integers, so the sums and the division by W = 2 are exact.
"""
import os
import socket

import numpy as np
import pytest

import oracle
import workloads as wl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)
dist = pytest.importorskip("torch.distributed")
mp = pytest.importorskip("torch.multiprocessing")
BF16, FP32 = oracle.BF16, oracle.FP32
TDT = {BF16: torch.bfloat16, FP32: torch.float32}


def _free_port():
    with socket.socket() as s:
        s.bind(("127.0.0.1", 0))
        return s.getsockname()[1]


def _layout(W, flat):
    shapes = [(3 * W + 1, 5), (W, 4), (7,), (1,), (2 * W, 3), (513, 129)]
    gdt = [BF16, FP32, FP32, BF16, BF16, BF16]
    if flat:
        return wl.custom(shapes, gdt, [FP32] * 6, W, seed=W, storage_dtypes=[FP32, BF16, FP32, FP32, BF16, FP32],
                         param_dtypes=[BF16] * 6)
    return wl.custom(shapes, gdt, [FP32, FP32, BF16, 0, FP32, FP32], W, seed=W,
                     storage_dtypes=[FP32, BF16, FP32, FP32, BF16, FP32])


def _int_grads(w, rank):
    rng = np.random.default_rng(100 + rank)
    out = []
    for t in w.tensors:
        v = rng.integers(-64, 65, size=t.numel).astype(np.float32)
        out.append(oracle.convert(v, FP32, BF16) if t.grad_dtype == BF16 else v)
    return out


def _dev(a, dt):
    t = torch.from_numpy(np.ascontiguousarray(a).copy())
    if dt == BF16:
        t = t.view(torch.bfloat16)
    return t.to("cuda:0")


def _host_bytes(t):
    return t.detach().contiguous().view(torch.uint8).cpu().numpy()


def _worker(rank, W, port, flat, errors):
    try:
        import fsdp2_mixed_dtype_amd as fp
        os.environ["MASTER_ADDR"] = "127.0.0.1"
        os.environ["MASTER_PORT"] = str(port)
        torch.cuda.set_device(0)
        dist.init_process_group("gloo", rank=rank, world_size=W)
        w = _layout(W, flat)
        plan = (fp.plan_buckets_flat if flat else fp.plan_buckets)(w.descs(), W)
        ref = oracle.plan_flat(w.descs(), W) if flat else oracle.plan(w.descs(), W)
        everyone = [_int_grads(w, q) for q in range(W)]
        g_dev = [_dev(g, t.grad_dtype) for g, t in zip(everyone[rank], w.tensors)]

        # gradient path
        for bi, b in enumerate(plan.buckets):
            out = torch.empty(W * b.S, dtype=TDT[b.dtype], device="cuda:0")
            fp.pack_reduce_scatter_input(plan, bi, g_dev, out)
            torch.cuda.synchronize()
            row = torch.empty(b.S, dtype=TDT[b.dtype])                       # host, for gloo
            dist.reduce_scatter_tensor(row, out.cpu())
            row_dev = row.to("cuda:0")
            dst = [torch.empty(fp.valid_in_chunk(plan, i, rank), dtype=TDT[t.storage_dtype], device="cuda:0")
                   if i in b.members else None for i, t in enumerate(w.tensors)]
            fp.reduce_scatter_copy_out(plan, bi, rank, row_dev, dst, float(W))
            torch.cuda.synchronize()
            for k, i in enumerate(b.members):
                t = w.tensors[i]
                mean = sum(oracle.convert(g[i], t.grad_dtype, FP32).astype(np.float64) for g in everyone) / W
                if flat:
                    lo, hi = oracle.flat_piece(ref, i, rank)
                    part = mean[max(0, lo - ref.F[i]): max(0, hi - ref.F[i])]
                else:
                    P = b.P[k]
                    part = mean[rank * P: rank * P + oracle.valid_in_chunk(t.numel, P, rank)]
                want = oracle.convert(oracle.convert(part.astype(np.float32), FP32, b.dtype), b.dtype,
                                      t.storage_dtype)
                assert np.array_equal(_host_bytes(dst[i]), want.view(np.uint8)), ("grad", bi, i)

        # parameter path
        params = wl.make_params(w)
        if flat:
            shards = []
            for i, (x, t) in enumerate(zip(params, w.tensors)):
                lo, hi = oracle.flat_piece(ref, i, rank)
                shards.append(_dev(x[lo - ref.F[i]: hi - ref.F[i]], t.storage_dtype) if hi > lo else None)
        else:
            shards = [_dev(oracle.shard(ref, i, x, rank), t.storage_dtype) for i, (x, t) in enumerate(zip(params, w.tensors))]
        ag = torch.zeros(W * plan.B, dtype=torch.uint8, device="cuda:0")
        fp.all_gather_copy_in(plan, rank, shards, ag)
        torch.cuda.synchronize()
        full = torch.empty(W * plan.B, dtype=torch.uint8)
        dist.all_gather_into_tensor(full, ag[rank * plan.B:(rank + 1) * plan.B].cpu())
        full_dev = full.to("cuda:0")
        outs = [torch.empty(t.numel, dtype=TDT[t.param_dtype], device="cuda:0") for t in w.tensors]
        fp.all_gather_copy_out(plan, full_dev, outs)
        torch.cuda.synchronize()
        for i, (x, t) in enumerate(zip(params, w.tensors)):
            want = oracle.convert(x, t.storage_dtype, t.param_dtype)
            assert np.array_equal(_host_bytes(outs[i]), want.view(np.uint8)), ("param", i)
        plan.destroy()
        dist.destroy_process_group()
    except BaseException as e:
        errors.put(f"rank {rank}: {type(e).__name__}: {e}")
        raise


@pytest.mark.parametrize("flat", [False, True])
def test_two_ranks_on_one_gpu_through_gloo(flat):
    print(f"[dist gpu] W=2 flat={flat}", flush=True)
    W = 2
    ctx = mp.get_context("spawn")
    errors = ctx.SimpleQueue()
    port = _free_port()
    procs = [ctx.Process(target=_worker, args=(r, W, port, flat, errors)) for r in range(W)]
    for p in procs:
        p.start()
    for p in procs:
        p.join(timeout=150)
    msgs = []
    while not errors.empty():
        msgs.append(errors.get())
    alive = [p for p in procs if p.is_alive()]
    for p in alive:
        p.kill()
    assert not alive, "a rank did not finish"
    assert not msgs and all(p.exitcode == 0 for p in procs), msgs
