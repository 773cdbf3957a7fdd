"""The layouts against real collectives: W processes over gloo on the CPU.

How the path shards across GPUs: every rank packs its own gradients into
the bucket's [W, S] reduce-scatter input, a reduce-scatter leaves rank r the
sum of everyone's row r, and the write-back turns that row into the rank's
sharded gradients; on the way in, every rank copies its shards into its row
of the [W, B] all-gather buffer, an all-gather fills the other rows, and the
copy-out rebuilds the full parameters ("The unit you wrapped", the
paragraphs on the collectives FSDP issues).  These tests run that data flow
with torch.distributed (gloo, CPU tensors, 127.0.0.1) and the oracle's
element loops, for both layouts, and check the results against the plain
definitions: the rank's slice of the averaged gradient, and the cast
parameters.  Gradients are small integers, so every sum and every division
by a power-of-two W is exact.
"""
import os
import socket

import numpy as np
import pytest

import oracle
import workloads as wl

torch = pytest.importorskip("torch")
dist = pytest.importorskip("torch.distributed")
mp = pytest.importorskip("torch.multiprocessing")
BF16, FP32 = oracle.BF16, oracle.FP32
TDT = {BF16: torch.bfloat16, FP32: torch.float32}


def _free_port():
    with socket.socket() as s:
        s.bind(("127.0.0.1", 0))
        return s.getsockname()[1]


def _layout(W, flat):
    shapes = [(3 * W + 1, 5), (W, 4), (7,), (1,), (2 * W, 3)]
    gdt = [BF16, FP32, FP32, BF16, BF16]
    if flat:
        return wl.custom(shapes, gdt, [FP32] * 5, W, seed=W, storage_dtypes=[FP32, BF16, FP32, FP32, BF16],
                         param_dtypes=[BF16] * 5)
    return wl.custom(shapes, gdt, [FP32, FP32, BF16, 0, FP32], W, seed=W,
                     storage_dtypes=[FP32, BF16, FP32, FP32, BF16])


def _int_grads(w, rank):
    """Rank-dependent small-integer gradients, exact in bf16 and in fp32 sums."""
    rng = np.random.default_rng(100 + rank)
    out = []
    for t in w.tensors:
        v = rng.integers(-64, 65, size=t.numel).astype(np.float32)
        out.append(oracle.convert(v, FP32, BF16) if t.grad_dtype == BF16 else v)
    return out


def _to_torch(a, dt):
    t = torch.from_numpy(np.ascontiguousarray(a).copy())
    return t.view(torch.bfloat16) if dt == BF16 else t


def _from_torch(t, dt):
    t = t.contiguous()
    return t.view(torch.int16).numpy().view(np.uint16) if dt == BF16 else t.numpy()


def _worker(rank, W, port, flat, errors):
    try:
        os.environ["MASTER_ADDR"] = "127.0.0.1"
        os.environ["MASTER_PORT"] = str(port)
        dist.init_process_group("gloo", rank=rank, world_size=W)
        w = _layout(W, flat)
        grads = _int_grads(w, rank)
        everyone = [_int_grads(w, q) for q in range(W)]
        params = wl.make_params(w)

        # ---- gradient path: pack -> reduce-scatter (sum) -> write-back with 1/W
        if flat:
            fpl = oracle.plan_flat(w.descs(), W)
            packed = oracle.pack_flat(fpl, grads)
            row = torch.empty(fpl.c, dtype=TDT[fpl.dtype])
            dist.reduce_scatter_tensor(row, _to_torch(packed, fpl.dtype).reshape(-1))
            shards = oracle.rs_copy_out_flat(fpl, rank, _from_torch(row, fpl.dtype), float(W))
            for i, t in enumerate(w.tensors):
                mean = sum(oracle.convert(g[i], t.grad_dtype, FP32).astype(np.float64) for g in everyone) / W
                lo, hi = oracle.flat_piece(fpl, i, rank)
                part = mean[max(0, lo - fpl.F[i]): max(0, hi - fpl.F[i])].astype(np.float32)
                want = oracle.convert(oracle.convert(part, FP32, fpl.dtype), fpl.dtype, t.storage_dtype)
                assert np.array_equal(shards[i].view(np.uint8), want.view(np.uint8)), ("flat grad", i)
        else:
            pl = oracle.plan(w.descs(), W)
            for bi, b in enumerate(pl.buckets):
                packed = oracle.pack(pl, bi, grads)
                row = torch.empty(b.S, dtype=TDT[b.dtype])
                dist.reduce_scatter_tensor(row, _to_torch(packed, b.dtype).reshape(-1))
                shards = oracle.rs_copy_out(pl, bi, rank, _from_torch(row, b.dtype), float(W))
                for k, i in enumerate(b.members):
                    t = w.tensors[i]
                    mean = sum(oracle.convert(g[i], t.grad_dtype, FP32).astype(np.float64) for g in everyone) / W
                    P = b.P[k]
                    v = oracle.valid_in_chunk(t.numel, P, rank)
                    part = mean[rank * P: rank * P + v].astype(np.float32)
                    want = oracle.convert(oracle.convert(part, FP32, b.dtype), b.dtype, t.storage_dtype)
                    assert np.array_equal(shards[k].view(np.uint8), want.view(np.uint8)), ("grad", bi, i)

        # ---- parameter path: copy-in of this rank's row -> all-gather -> copy-out
        if flat:
            pieces = []
            for i, x in enumerate(params):
                lo, hi = oracle.flat_piece(fpl, i, rank)
                pieces.append(x[max(0, lo - fpl.F[i]): max(0, hi - fpl.F[i])].copy() if hi > lo
                              else np.zeros(0, x.dtype))
            mine = oracle.copy_in_flat(fpl, rank, pieces)
            full = torch.empty(W * fpl.c, dtype=TDT[fpl.param_dtype])
            dist.all_gather_into_tensor(full, _to_torch(mine, fpl.param_dtype))
            back = oracle.copy_out_flat(fpl, _from_torch(full, fpl.param_dtype))
        else:
            ag = np.zeros((W, pl.B), np.uint8)
            shards_in = [oracle.shard(pl, i, x, rank) for i, x in enumerate(params)]
            oracle.copy_in(pl, rank, shards_in, ag)
            full = torch.empty(W * pl.B, dtype=torch.uint8)
            dist.all_gather_into_tensor(full, torch.from_numpy(ag[rank].copy()))
            back = oracle.copy_out(pl, full.numpy())
        for i, (x, t) in enumerate(zip(params, w.tensors)):
            want = oracle.convert(x, t.storage_dtype, t.param_dtype)
            assert np.array_equal(back[i].view(np.uint8), want.view(np.uint8)), ("param", i)
        dist.destroy_process_group()
    except BaseException as e:     # report to the parent, which fails the test
        errors.put(f"rank {rank}: {type(e).__name__}: {e}")
        raise


@pytest.mark.parametrize("flat", [False, True])
@pytest.mark.parametrize("W", [2, 4])
def test_layouts_through_gloo_collectives(W, flat):
    ctx = mp.get_context("spawn")
    errors = ctx.SimpleQueue()
    port = _free_port()
    procs = [ctx.Process(target=_worker, args=(r, W, port, flat, errors)) for r in range(W)]
    for p in procs:
        p.start()
    for p in procs:
        p.join(timeout=240)
    msgs = []
    while not errors.empty():
        msgs.append(errors.get())
    alive = [p for p in procs if p.is_alive()]
    for p in alive:
        p.kill()
    assert not alive, "a rank did not finish"
    assert not msgs and all(p.exitcode == 0 for p in procs), msgs
