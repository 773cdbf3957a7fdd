"""GPU parity: libfsdppack's HIP kernels (through the C ABI) against the CPU
oracle, byte for byte (0 ULP), on the same seeded inputs.

Covered: the reduce-scatter pack of every bucket of the five workloads at
full size (the launch configuration the benchmark times), the same with
special values injected, random layouts with misaligned sources and outputs,
the all-gather copy-in and copy-out, the copy-in -> all-gather -> copy-out
round trip, every float32 bit pattern through the fp32 -> bf16 cast, edge
cases (empty, W = 1, dim0 < W, zero-size tensors), determinism, one launch per
call, and pointer-table reuse / eviction.  Destination buffers are poisoned
with 0xAB and surrounded by guard bytes that must stay untouched.
"""
import random

import numpy as np
import pytest

import oracle
import workloads as wl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)
import fsdp2_mixed_dtype_amd as fp  # noqa: E402

BF16, FP32 = 1, 2
DEV = torch.device("cuda:0")
GUARD = 256          # guard bytes on each side of every destination
POISON = 0xAB


def to_dev(a, dt, elem_offset=0):
    """Copy a host array (bf16 as uint16 bits, or float32) to the GPU,
    optionally as a view starting `elem_offset` elements into a larger
    allocation (to test misaligned sources)."""
    a = np.ascontiguousarray(a).reshape(-1)
    base = torch.empty(a.size + elem_offset, dtype=fp.TORCH_DTYPE[dt], device=DEV)
    t = base[elem_offset:]
    host = torch.from_numpy(a.copy())
    if dt == BF16:
        host = host.view(torch.bfloat16)
    t.copy_(host)
    return t


def host_bytes(t):
    return t.detach().contiguous().view(torch.uint8).cpu().numpy()


class Guarded:
    """A poisoned destination of `numel` elements at `elem_offset` elements
    past a 256-byte aligned start, with guard bytes on both sides."""

    def __init__(self, numel, dt, elem_offset=0):
        # dt: BF16 / FP32, or None for a plain byte buffer
        esz = fp.ELEM_SIZE[dt] if dt else 1
        self.front = GUARD + elem_offset * esz
        self.nbytes = numel * esz
        self.raw = torch.full((self.front + self.nbytes + GUARD,), POISON, dtype=torch.uint8, device=DEV)
        self.t = self.raw[self.front:self.front + self.nbytes]
        if dt:
            self.t = self.t.view(fp.TORCH_DTYPE[dt])

    def result(self):
        h = host_bytes(self.raw)
        assert np.all(h[:self.front] == POISON), "write before the destination"
        assert np.all(h[self.front + self.nbytes:] == POISON), "write past the destination"
        return h[self.front:self.front + self.nbytes]


def gpu_pack(plan, bucket, g_dev, out_offset=0):
    b = plan.buckets[bucket]
    out = Guarded(plan.world * b.S, b.dtype, out_offset)
    fp.pack_reduce_scatter_input(plan, bucket, g_dev, out.t)
    torch.cuda.synchronize()
    return out.result()


def check_pack(w, grads, src_offsets=None, out_offset=0):
    ref = oracle.plan(w.descs(), w.world)
    plan = fp.plan_buckets(w.descs(), w.world)
    src_offsets = src_offsets or [0] * len(grads)
    g_dev = [to_dev(g, t.grad_dtype, o) for g, t, o in zip(grads, w.tensors, src_offsets)]
    for bi in range(len(ref.buckets)):
        got = gpu_pack(plan, bi, g_dev, out_offset)
        want = oracle.pack(ref, bi, grads).view(np.uint8).reshape(-1)
        if not np.array_equal(got, want):
            bad = np.flatnonzero(got != want)
            pytest.fail(f"{w.name} bucket {bi}: {bad.size} bytes differ, first at byte {bad[0]}")
    plan.destroy()


_grad_cache = {}


def grads_of(name):
    if name not in _grad_cache:
        _grad_cache.clear()
        _grad_cache[name] = wl.make_grads(wl.get(name))
    return _grad_cache[name]


# --------------------------------------------------------------------------- pack

@pytest.mark.parametrize("name", ["tiny", "mixed50m", "layout500", "kda_block", "hetero500"])
def test_pack_full_size_matches_oracle(name):
    print(f"[pack parity] workload={name}", flush=True)
    w = wl.get(name)
    check_pack(w, grads_of(name))


def test_pack_special_values_heterogeneous():
    print("[pack parity] hetero500 + specials", flush=True)
    w = wl.hetero500()
    grads = [g.copy() for g in grads_of("hetero500")]
    wl.inject_specials(grads, [t.grad_dtype for t in w.tensors], seed=5)
    check_pack(w, grads)


def test_pack_direct_windows_every_dtype_pair_and_shift():
    """Windows inside one rank chunk take the kernel's direct copy: all four
    dtype pairs, bf16 chunks at odd elements, two members per map stretch,
    sources shifted by an element and outputs off a 16-byte boundary."""
    from conftest import direct_window_layout
    shapes, gdt, rdt, W = direct_window_layout()
    w = wl.custom(shapes, gdt, rdt, W, seed=11)
    grads = wl.make_grads(w)
    wl.inject_specials(grads, gdt, seed=11)
    for src_shift, out_off in ((0, 0), (1, 0), (0, 6), (1, 2)):
        print(f"[pack direct] src_shift={src_shift} out_off={out_off}", flush=True)
        check_pack(w, grads, [src_shift] * len(grads), out_off)


def test_pack_direct_windows_single_pair_buckets():
    """One bucket per dtype pair, every gradient of one dtype: the direct
    copy of each pair on its own, with bf16 chunks at odd elements, shifted
    sources and outputs off a 16-byte boundary."""
    from conftest import single_pair_layouts
    for shapes, gdt, rdt, W, pair in single_pair_layouts():
        w = wl.custom(shapes, gdt, rdt, W, seed=13)
        grads = wl.make_grads(w)
        wl.inject_specials(grads, gdt, seed=13)
        for src_shift, out_off in ((0, 0), (1, 0), (0, 6), (1, 2)):
            print(f"[pack pair] pair={pair} src_shift={src_shift} out_off={out_off}", flush=True)
            check_pack(w, grads, [src_shift] * len(grads), out_off)


def _random_workload(rng, seed):
    W = rng.choice([1, 2, 3, 4, 5, 8, 16, 33, 128])
    n = rng.randint(1, 9)
    shapes, gdt, rdt = [], [], []
    for _ in range(n):
        dim0 = rng.choice([0, 1, 2, W - 1, W, W + 1, rng.randint(1, 9 * W + 5), rng.randint(1, 3000)])
        inner = rng.choice([1, 2, 3, 7, 8, 64, 33, 129])
        shapes.append((max(dim0, 0), inner))
        gdt.append(rng.choice([BF16, FP32]))
        rdt.append(rng.choice([0, BF16, FP32]))
    return wl.custom(shapes, gdt, rdt, W, seed, storage_dtypes=[rng.choice([BF16, FP32]) for _ in range(n)])


def test_pack_random_layouts_misaligned():
    rng = random.Random(2024)
    for case in range(60):
        w = _random_workload(rng, case)
        grads = wl.make_grads(w)
        wl.inject_specials(grads, [t.grad_dtype for t in w.tensors], seed=case)
        offsets = [rng.choice([0, 0, 1, 2, 3, 5, 7]) for _ in grads]
        # small offsets, and ones that put the output start just short of a
        # 2 KiB boundary (the buffer itself starts 256 bytes past a 512-byte one)
        out_off = rng.choice([0, 0, 1, 2, 3, 6, 443, 447, 893, 895])
        print(f"[pack random] case={case} W={w.world} n={len(w.tensors)} src_off={offsets} out_off={out_off}",
              flush=True)
        check_pack(w, grads, offsets, out_off)


def test_pack_every_f32_pattern_to_bf16():
    """All 2**32 float32 bit patterns through the fp32 -> bf16 pack (W=1)."""
    chunk = 1 << 28
    plan = fp.plan_buckets([(chunk, 1, FP32, BF16, FP32, FP32)], 1)
    out = torch.empty(chunk, dtype=torch.bfloat16, device=DEV)
    for start in range(0, 1 << 32, chunk):
        print(f"[exhaustive fp32->bf16] chunk start={start:#x}", flush=True)
        x = torch.arange(start, start + chunk, dtype=torch.int64, device=DEV)
        x = torch.where(x >= 2**31, x - 2**32, x).to(torch.int32).view(torch.float32)
        fp.pack_reduce_scatter_input(plan, 0, [x], out)
        got = out.view(torch.int16).cpu().numpy().view(np.uint16)
        del x
        u = np.arange(start, start + chunk, dtype=np.uint64).astype(np.uint32)
        want = oracle.convert(u.view(np.float32), FP32, BF16)
        assert np.array_equal(got, want), f"mismatch in chunk {start:#x}"
    plan.destroy()


def test_pack_every_bf16_pattern_to_fp32():
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    w = wl.custom([(1 << 16,)], [BF16], [FP32], 1)
    check_pack(w, [h])
    w4 = wl.custom([(1 << 16,)], [BF16], [FP32], 3)       # ragged, W=3
    check_pack(w4, [h], [1])


def test_pack_edge_cases():
    cases = [
        wl.custom([(0, 4), (0, 1)], [FP32, BF16], [FP32, FP32], 4),          # nothing to do
        wl.custom([(1,)], [BF16], [FP32], 8),                                  # one element, W > dim0
        wl.custom([(5, 3)], [FP32], [BF16], 1),                                # W = 1
        wl.custom([(3, 1), (2, 5), (7, 2)], [BF16, FP32, BF16], [FP32, FP32, FP32], 1000),  # large W
        wl.custom([(0, 3), (4, 4), (0, 9)], [FP32, FP32, BF16], [0, 0, 0], 3),  # empty members
        wl.custom([(8, 0), (2, 2)], [BF16, BF16], [0, 0], 2),                  # inner 0
    ]
    for i, w in enumerate(cases):
        print(f"[pack edge] case={i}", flush=True)
        check_pack(w, wl.make_grads(w))


def test_pack_non_members_may_be_none():
    w = wl.custom([(6, 6), (5, 1), (9, 2)], [BF16, FP32, BF16], [BF16, FP32, 0], 4)
    grads = wl.make_grads(w)
    ref = oracle.plan(w.descs(), w.world)
    plan = fp.plan_buckets(w.descs(), w.world)
    g_dev = [to_dev(g, t.grad_dtype) for g, t in zip(grads, w.tensors)]
    for bi, b in enumerate(plan.buckets):
        only = [g if i in b.members else None for i, g in enumerate(g_dev)]
        got = gpu_pack(plan, bi, only)
        assert np.array_equal(got, oracle.pack(ref, bi, grads).view(np.uint8).reshape(-1))


def test_deterministic_one_launch_and_table_reuse():
    w = wl.mixed50m()
    grads = grads_of("mixed50m")
    plan = fp.plan_buckets(w.descs(), w.world)
    g_dev = [to_dev(g, t.grad_dtype) for g, t in zip(grads, w.tensors)]
    out1 = torch.empty(w.world * plan.buckets[0].S, dtype=torch.float32, device=DEV)
    out2 = torch.full_like(out1, 7.0)
    c0 = fp.counters()
    fp.pack_reduce_scatter_input(plan, 0, g_dev, out1)
    c1 = fp.counters()
    fp.pack_reduce_scatter_input(plan, 0, g_dev, out2)
    c2 = fp.counters()
    torch.cuda.synchronize()
    assert torch.equal(out1.view(torch.int32), out2.view(torch.int32))
    assert c1[0] - c0[0] == 1 and c2[0] - c1[0] == 1          # one launch per call
    assert c2[1] - c0[1] == 0                                  # 32 pointers: no table upload ...
    assert c1[6] - c0[6] == 1 and c2[6] - c1[6] == 1          # ... they travel in the launch arguments
    plan.destroy()


def test_new_pointers_every_call_inline():
    """Gradients at new addresses on every call (a fresh autograd allocation each
    backward): the pointers travel in the launch arguments, so nothing is
    uploaded or cached, and every result is exact."""
    w = wl.custom([(4 * 1025, 3), (5,), (64, 2), (4 * 700, 8)], [BF16, FP32, BF16, BF16], [FP32, FP32, FP32, BF16], 4)
    ref = oracle.plan(w.descs(), w.world)
    plan = fp.plan_buckets(w.descs(), w.world)
    c0 = fp.counters()
    outs, wants = [], []
    for k in range(24):
        grads = wl.make_grads(w, seed=500 + k)
        g_dev = [to_dev(g, t.grad_dtype, k % 3) for g, t in zip(grads, w.tensors)]
        for bi, b in enumerate(plan.buckets):
            out = torch.empty(w.world * b.S, dtype=fp.TORCH_DTYPE[b.dtype], device=DEV)
            fp.pack_reduce_scatter_input(plan, bi, g_dev, out)
            outs.append((out, g_dev))
            wants.append(oracle.pack(ref, bi, grads))
    torch.cuda.synchronize()
    c1 = fp.counters()
    for (out, _), want in zip(outs, wants):
        assert np.array_equal(host_bytes(out), want.view(np.uint8).reshape(-1))
    assert c1[1] - c0[1] == 0 and c1[4] - c0[4] == 0
    assert c1[6] - c0[6] == len(outs)
    plan.destroy()


def test_mid_size_pointer_sets_inline_then_cached():
    """A bucket of 200 members (more than the small argument table holds): a
    pointer set seen for the first time travels in the launch arguments and
    is uploaded behind the launch; the same set next time uses its cached
    device table (also from another stream, which waits for the upload);
    every result is exact."""
    w = _many_params(200, W=4, seed=3)
    ref = oracle.plan(w.descs(), w.world)
    plan = fp.plan_buckets(w.descs(), w.world)
    assert any(len(b.members) > 64 for b in plan.buckets)
    side = torch.cuda.Stream(device=DEV)
    sets = []
    for k in range(2):
        grads = wl.make_grads(w, seed=700 + k)
        sets.append((grads, [to_dev(g, t.grad_dtype, k % 3) for g, t in zip(grads, w.tensors)]))
    big = [bi for bi, b in enumerate(plan.buckets) if len(b.members) > 64]

    def pack(k, stream=None):
        grads, g_dev = sets[k]
        outs = []
        for bi in big:
            b = plan.buckets[bi]
            out = torch.empty(w.world * b.S, dtype=fp.TORCH_DTYPE[b.dtype], device=DEV)
            if stream is None:
                fp.pack_reduce_scatter_input(plan, bi, g_dev, out)
            else:
                with torch.cuda.stream(stream):
                    fp.pack_reduce_scatter_input(plan, bi, g_dev, out)
            outs.append((bi, out))
        return grads, outs

    def check(grads, outs, stream=None):
        (stream or torch.cuda.current_stream()).synchronize()
        for bi, out in outs:
            assert np.array_equal(host_bytes(out), oracle.pack(ref, bi, grads).view(np.uint8).reshape(-1))

    nb = len(big)
    c0 = fp.counters()
    check(*pack(0))                                       # new set: inline, then uploaded
    c1 = fp.counters()
    assert c1[6] - c0[6] == nb and c1[1] - c0[1] == nb and c1[2] - c0[2] == 0
    check(*pack(0))                                       # same set: its cached table
    c2 = fp.counters()
    assert c2[6] - c1[6] == 0 and c2[1] - c1[1] == 0 and c2[2] - c1[2] == nb
    check(*pack(1))                                       # another new set
    c3 = fp.counters()
    assert c3[6] - c2[6] == nb and c3[1] - c2[1] == nb
    check(*pack(1, side), side)                           # the cached table from another stream
    c4 = fp.counters()
    assert c4[6] - c3[6] == 0 and c4[2] - c3[2] == nb
    plan.destroy()


def test_mid_size_pointer_churn_on_two_streams():
    """20 pointer sets of a 200-member bucket, more than the 16 cached tables,
    passed twice in turn on two streams: every call either finds its set
    cached or passes it in the launch arguments (uploading it behind the
    launch when that needs no host wait, possibly replacing an older table
    that a kernel on the other stream read); every result is exact."""
    w = _many_params(200, W=4, seed=5)
    ref = oracle.plan(w.descs(), w.world)
    plan = fp.plan_buckets(w.descs(), w.world)
    side = torch.cuda.Stream(device=DEV)
    main = torch.cuda.current_stream()
    n_sets = 20
    sets = []
    for k in range(n_sets):
        grads = wl.make_grads(w, seed=900 + k)
        sets.append((grads, [to_dev(g, t.grad_dtype, k % 3) for g, t in zip(grads, w.tensors)]))
    b = plan.buckets[0]
    c0 = fp.counters()
    results = []
    for rnd in range(2):
        for k in range(n_sets):
            stream = side if (k // 3 + rnd) % 2 else main
            grads, g_dev = sets[k]
            out = torch.empty(w.world * b.S, dtype=fp.TORCH_DTYPE[b.dtype], device=DEV)
            stream.wait_stream(main)
            with torch.cuda.stream(stream):
                fp.pack_reduce_scatter_input(plan, 0, g_dev, out)
            out.record_stream(stream)
            results.append((k, out))
        k = n_sets - 1                                    # the last set again: now cached
        out = torch.empty(w.world * b.S, dtype=fp.TORCH_DTYPE[b.dtype], device=DEV)
        fp.pack_reduce_scatter_input(plan, 0, sets[k][1], out)
        results.append((k, out))
    torch.cuda.synchronize()
    c1 = fp.counters()
    for k, out in results:
        assert np.array_equal(host_bytes(out), oracle.pack(ref, 0, sets[k][0]).view(np.uint8).reshape(-1)), k
    assert c1[0] - c0[0] == len(results)
    assert c1[1] - c0[1] >= 16                            # the first sets filled the free tables
    assert c1[7] - c0[7] == 0                             # an upload behind a launch never waits on the host
    plan.destroy()


def test_one_plan_shared_by_threads_on_their_own_streams():
    """One plan used by four host threads at once (the library's calls run
    without the GIL), each on a stream of its own with its own rotation of
    six gradient buffer sets, five rounds.  A 200-member bucket exercises
    pointer sets passed in the launch arguments and uploaded behind the
    launch, cached tables, and tables replaced while other streams read
    them (24 sets, 16 tables); a 1000-member bucket, device tables staged
    before the launch.  Every pack equals the oracle's."""
    import threading
    n_threads, n_sets, rounds = 4, 6, 5
    for w in (_many_params(200, W=4, seed=6), _many_params(1000, W=4, seed=7)):
        print(f"[threads] {len(w.tensors)} members", flush=True)
        ref = oracle.plan(w.descs(), w.world)
        plan = fp.plan_buckets(w.descs(), w.world)
        b = plan.buckets[0]
        sets = []
        for th in range(n_threads):
            mine = []
            for k in range(n_sets):
                grads = wl.make_grads(w, seed=1000 * (th + 1) + k)
                g_dev = [to_dev(g, t.grad_dtype, k % 3) for g, t in zip(grads, w.tensors)]
                mine.append((grads, fp.prepare_grads(plan, g_dev)))
            sets.append(mine)
        outs = [[torch.empty(w.world * b.S, dtype=fp.TORCH_DTYPE[b.dtype], device=DEV)
                 for _ in range(rounds * n_sets)] for _ in range(n_threads)]
        torch.cuda.synchronize()
        errors = []

        def work(th):
            try:
                stream = torch.cuda.Stream(device=DEV)
                with torch.cuda.stream(stream):
                    for i in range(rounds * n_sets):
                        fp.pack_reduce_scatter_input(plan, 0, sets[th][i % n_sets][1], outs[th][i])
                stream.synchronize()
            except Exception as e:          # reported below, on the test's thread
                errors.append((th, e))

        threads = [threading.Thread(target=work, args=(th,)) for th in range(n_threads)]
        for t in threads:
            t.start()
        for t in threads:
            t.join()
        assert not errors, errors
        torch.cuda.synchronize()
        for th in range(n_threads):
            expect = [oracle.pack(ref, 0, sets[th][k][0]).view(np.uint8).reshape(-1) for k in range(n_sets)]
            for i in range(rounds * n_sets):
                assert np.array_equal(host_bytes(outs[th][i]), expect[i % n_sets]), (len(w.tensors), th, i)
        plan.destroy()


def _many_params(k=1000, W=4, seed=0):
    """A unit of more parameters than a launch's arguments carry (the pointer
    table goes through the device-table cache)."""
    shapes = [(1 + (i * 7) % 13, 1 + (i * 3) % 5) for i in range(k)]
    gdt = [BF16 if i % 3 else FP32 for i in range(k)]
    return wl.custom(shapes, gdt, [FP32] * k, W, seed=seed)


def test_prepared_pointer_arrays_match_tensor_lists():
    w = wl.hetero500()
    grads = grads_of("hetero500")
    ref = oracle.plan(w.descs(), w.world)
    plan = fp.plan_buckets(w.descs(), w.world)
    g_dev = [to_dev(g, t.grad_dtype) for g, t in zip(grads, w.tensors)]
    prepared = fp.prepare_grads(plan, g_dev)
    for bi, b in enumerate(plan.buckets):
        out = Guarded(w.world * b.S, b.dtype)
        fp.pack_reduce_scatter_input(plan, bi, prepared, out.t)
        torch.cuda.synchronize()
        assert np.array_equal(out.result(), oracle.pack(ref, bi, grads).view(np.uint8).reshape(-1))
    other = fp.plan_buckets(w.descs(), w.world)
    with pytest.raises(ValueError):
        fp.pack_reduce_scatter_input(other, 0, prepared, out.t)      # prepared for another plan
    other.destroy()
    plan.destroy()


def test_pointer_table_eviction_keeps_results_correct():
    w = _many_params()
    ref = oracle.plan(w.descs(), w.world)
    plan = fp.plan_buckets(w.descs(), w.world)
    outs, wants = [], []
    for k in range(40):     # more distinct pointer sets than the cache holds
        grads = wl.make_grads(w, seed=100 + k)
        g_dev = [to_dev(g, t.grad_dtype, k % 3) for g, t in zip(grads, w.tensors)]
        out = torch.empty(w.world * plan.buckets[0].S, dtype=torch.float32, device=DEV)
        fp.pack_reduce_scatter_input(plan, 0, g_dev, out)
        outs.append((out, g_dev))
        wants.append(oracle.pack(ref, 0, grads))
    torch.cuda.synchronize()
    for (out, _), want in zip(outs, wants):
        assert np.array_equal(host_bytes(out), want.view(np.uint8).reshape(-1))
    plan.destroy()


def test_pointer_churn_on_two_streams():
    """More distinct pointer sets than the table cache holds, on two streams
    in turns of 16 calls: every call after the first 16 replaces a table that
    the other stream may still be reading; results stay exact and the library
    orders the replacement with the other stream's work (cross-stream waits,
    no device-wide synchronisation)."""
    w = _many_params(seed=3)
    ref = oracle.plan(w.descs(), w.world)
    plan = fp.plan_buckets(w.descs(), w.world)
    side = torch.cuda.Stream(device=DEV)
    main = torch.cuda.current_stream()
    c0 = fp.counters()
    outs, wants = [], []
    for k in range(40):
        grads = wl.make_grads(w, seed=300 + k)
        g_dev = [to_dev(g, t.grad_dtype, k % 2) for g, t in zip(grads, w.tensors)]
        out = torch.empty(w.world * plan.buckets[0].S, dtype=torch.float32, device=DEV)
        st = side if (k // 16) % 2 else main        # the table a call replaces was filled 16 calls before
        st.wait_stream(main)              # the inputs were written on the main stream
        with torch.cuda.stream(st):
            fp.pack_reduce_scatter_input(plan, 0, g_dev, out, stream=st)
        outs.append((out, g_dev, st))
        wants.append(oracle.pack(ref, 0, grads))
    torch.cuda.synchronize()
    c1 = fp.counters()
    for (out, _, _), want in zip(outs, wants):
        assert np.array_equal(host_bytes(out), want.view(np.uint8).reshape(-1))
    assert c1[1] - c0[1] == 40                       # every set uploaded once
    assert c1[4] - c0[4] == 40 - 16                  # the rest replaced older tables
    assert c1[5] - c0[5] > 0                         # ... some of them used by the other stream
    assert c1[7] - c0[7] == c1[4] - c0[4]            # one host wait (for an old upload) per replacement
    plan.destroy()


def test_armed_timing_events_are_taken_by_a_call_that_launches_nothing():
    """Events armed with time_next_launch belong to the next compute call even
    when it has nothing to write or is rejected for its arguments: a later,
    unrelated kernel must not stamp them."""
    a = torch.randn(2048, 2048, device=DEV)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(20):
        a = a @ a.T / 2048.0
    e1.record()
    torch.cuda.synchronize()
    before = e0.elapsed_time(e1)
    assert before > 0.05
    empty = fp.plan_buckets([(0, 8, BF16, FP32, FP32, FP32)], 4)        # one bucket, S = 0: no launch
    fp.time_next_launch(e0, e1)
    c0 = fp.counters()
    fp.pack_reduce_scatter_input(empty, 0, [None], torch.empty(0, dtype=torch.float32, device=DEV))
    assert fp.counters()[0] == c0[0]
    w = wl.tiny()
    plan = fp.plan_buckets(w.descs(), w.world)
    g_dev = [to_dev(g, t.grad_dtype) for g, t in zip(wl.make_grads(w), w.tensors)]
    gpu_pack(plan, 0, g_dev)                          # a real launch, after the empty call
    assert e0.elapsed_time(e1) == before               # not stamped by it
    # a call rejected for its arguments takes them too (every compute entry point)
    L = fp.lib()
    rejected = [lambda: L.fsdppack_pack_reduce_scatter_input(plan.handle, 99, None, None, None),
                lambda: L.fsdppack_pack_reduce_scatter_input_noalloc(plan.handle, 99, None, None, None),
                lambda: L.fsdppack_all_gather_copy_in(plan.handle, -1, None, None, None),
                lambda: L.fsdppack_all_gather_copy_out(plan.handle, None, None, None),
                lambda: L.fsdppack_reduce_scatter_copy_out(plan.handle, 99, 0, None, 1.0, None, None),
                lambda: L.fsdppack_reduce_scatter_copy_out_all(plan.handle, -1, None, 1.0, None, None)]
    for call in rejected:
        fp.time_next_launch(e0, e1)
        assert call() == -1
        gpu_pack(plan, 0, g_dev)
        assert e0.elapsed_time(e1) == before
    fp.time_next_launch(e0, e1)
    gpu_pack(plan, 0, g_dev)
    assert e0.elapsed_time(e1) < before                # stamped when armed right before
    plan.destroy()
    empty.destroy()


def test_empty_launch_floor():
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    e1.record()
    c0 = fp.counters()
    for wg in (1, 4096, 100000):
        fp.time_next_launch(e0, e1)
        fp.empty_launch(wg, 64)
        torch.cuda.synchronize()
        assert 0 <= e0.elapsed_time(e1) < 5.0
    assert fp.counters()[0] == c0[0]                  # not a compute launch


def test_precast_then_pack_equals_fused_pack():
    """The pages' comparator (bf16 gradients cast into fp32 temporaries, then a
    homogeneous fp32 pack), run with the library's own kernels as the benchmark
    runs it, gives the fused pack's bytes on the 50.3M-element layout."""
    w = wl.mixed50m()
    grads = grads_of("mixed50m")
    plan = fp.plan_buckets(w.descs(), w.world)
    g_dev = [to_dev(g, t.grad_dtype) for g, t in zip(grads, w.tensors)]
    fused = gpu_pack(plan, 0, g_dev)
    bf = [i for i, t in enumerate(w.tensors) if t.grad_dtype == BF16]
    cast_plan = fp.plan_buckets([(w.tensors[i].numel, 1, BF16, FP32, FP32, FP32) for i in bf], 1)
    homo = fp.plan_buckets([(t.dim0, t.inner, FP32, FP32, FP32, FP32) for t in w.tensors], w.world)
    tmp = torch.empty(cast_plan.buckets[0].S, dtype=torch.float32, device=DEV)
    fp.pack_reduce_scatter_input(cast_plan, 0, [g_dev[i] for i in bf], tmp)
    views = list(g_dev)
    for k, i in enumerate(bf):
        o = cast_plan.buckets[0].O[k]
        views[i] = tmp[o:o + w.tensors[i].numel]
    out = torch.empty(w.world * homo.buckets[0].S, dtype=torch.float32, device=DEV)
    fp.pack_reduce_scatter_input(homo, 0, views, out)
    torch.cuda.synchronize()
    assert np.array_equal(host_bytes(out), fused)
    cast_plan.destroy()
    homo.destroy()
    plan.destroy()


def test_pack_on_side_stream():
    w = wl.tiny()
    grads = wl.make_grads(w)
    ref = oracle.plan(w.descs(), w.world)
    plan = fp.plan_buckets(w.descs(), w.world)
    g_dev = [to_dev(g, t.grad_dtype) for g, t in zip(grads, w.tensors)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    out = torch.empty(w.world * plan.buckets[0].S, dtype=torch.float32, device=DEV)
    # the binding launches on the stream torch reports as current
    assert fp._stream(None) == torch.cuda.current_stream().cuda_stream
    with torch.cuda.stream(s):
        assert fp._stream(None) == s.cuda_stream
        fp.pack_reduce_scatter_input(plan, 0, g_dev, out)
    fp.pack_reduce_scatter_input(plan, 0, g_dev, out, stream=s)      # same table, explicit stream
    s.synchronize()
    assert np.array_equal(host_bytes(out), oracle.pack(ref, 0, grads).view(np.uint8).reshape(-1))
    plan.destroy()


def test_pack_concurrent_with_gemm_and_write_back():
    """Packs on one stream while a bf16 GEMM runs on the current stream and
    write-backs run on a third (FSDP overlaps its staging with compute):
    every result still matches the oracle."""
    print("[concurrent] mixed50m pack + write-back beside a GEMM", flush=True)
    w = wl.get("mixed50m")
    W = w.world
    grads = wl.make_grads(w)
    ref = oracle.plan(w.descs(), W)
    plan = fp.plan_buckets(w.descs(), W)
    g_dev = fp.prepare_grads(plan, [to_dev(g, t.grad_dtype) for g, t in zip(grads, w.tensors)])
    b = plan.buckets[0]
    want = oracle.pack(ref, 0, grads)
    a = torch.randn(4096, 4096, device=DEV).to(torch.bfloat16)
    m = torch.randn(4096, 4096, device=DEV).to(torch.bfloat16)
    main = torch.cuda.current_stream()
    s_pack, s_wb = torch.cuda.Stream(), torch.cuda.Stream()
    outs = [torch.empty(W * b.S, dtype=torch.float32, device=DEV) for _ in range(3)]
    dsts = [[torch.empty(fp.valid_in_chunk(plan, i, r), dtype=fp.TORCH_DTYPE[t.storage_dtype], device=DEV)
             for i, t in enumerate(w.tensors)] for r in range(3)]
    s_pack.wait_stream(main)
    s_wb.wait_stream(main)
    for k in range(3):
        c = a
        for _ in range(4):
            c = torch.mm(c, m)                     # keeps the current stream busy
        fp.pack_reduce_scatter_input(plan, 0, g_dev, outs[k], stream=s_pack)
        done = torch.cuda.Event()
        done.record(s_pack)
        s_wb.wait_event(done)
        fp.reduce_scatter_copy_out(plan, 0, k, outs[k][k * b.S:(k + 1) * b.S], dsts[k], float(W), stream=s_wb)
    torch.cuda.synchronize()
    for k in range(3):
        assert np.array_equal(host_bytes(outs[k]), want.view(np.uint8).reshape(-1)), k
        wb = oracle.rs_copy_out(ref, 0, k, want[k], float(W))
        for i, wv in zip(b.members, wb):
            assert np.array_equal(host_bytes(dsts[k][i]), wv.view(np.uint8)), (k, i)
    plan.destroy()


# --------------------------------------------------------------------------- all-gather staging

def _shards_random(w, ref, rank):
    return [wl.random_array(P, t.storage_dtype, seed=1000 * rank + i) for i, (t, P) in
            enumerate(zip(w.tensors, ref.P))]


@pytest.mark.parametrize("name", ["tiny", "layout500", "mixed50m", "kda_block", "hetero500"])
def test_copy_in_matches_oracle(name):
    print(f"[copy-in parity] workload={name}", flush=True)
    w = wl.get(name)
    ref = oracle.plan(w.descs(), w.world)
    plan = fp.plan_buckets(w.descs(), w.world)
    ranks = range(w.world) if w.world <= 4 else [0, 1, w.world - 1]
    ag = Guarded(w.world * plan.B, None)
    ag_u8 = ag.t
    ag_ref = np.full((w.world, ref.B), POISON, np.uint8)
    for r in ranks:
        shards = _shards_random(w, ref, r)
        offs = [(i + r) % 3 for i in range(len(shards))]
        fp.all_gather_copy_in(plan, r, [to_dev(s, t.storage_dtype, o) for s, t, o in
                                        zip(shards, w.tensors, offs)], ag_u8)
        oracle.copy_in(ref, r, shards, ag_ref)
    torch.cuda.synchronize()
    got = ag.result().reshape(w.world, -1)
    assert np.array_equal(got, ag_ref), "copy-in rows differ (untouched rows must keep the poison)"
    plan.destroy()


@pytest.mark.parametrize("name", ["tiny", "layout500", "mixed50m", "kda_block", "hetero500"])
def test_copy_out_matches_oracle(name):
    print(f"[copy-out parity] workload={name}", flush=True)
    w = wl.get(name)
    ref = oracle.plan(w.descs(), w.world)
    plan = fp.plan_buckets(w.descs(), w.world)
    gathered = np.random.default_rng(7).integers(0, 256, size=w.world * ref.B, dtype=np.uint8)
    ag = torch.from_numpy(gathered.copy()).to(DEV)
    outs = [Guarded(t.numel, t.param_dtype, i % 3) for i, t in enumerate(w.tensors)]
    fp.all_gather_copy_out(plan, ag, [o.t for o in outs])
    torch.cuda.synchronize()
    wants = oracle.copy_out(ref, gathered)
    for i, (o, want) in enumerate(zip(outs, wants)):
        assert np.array_equal(o.result(), want.view(np.uint8)), f"param {i} differs"
    plan.destroy()


def test_copy_out_gathered_windows():
    """Copy-out windows over many small rank chunks (gathered element by
    element by the kernel), bf16 and fp32, outputs at element offsets 0-2."""
    from conftest import gathered_copy_out_layout
    for k, (shapes, pdt, W) in enumerate(gathered_copy_out_layout()):
        print(f"[copy-out gathered] layout {k} W={W}", flush=True)
        n = len(shapes)
        w = wl.custom(shapes, [FP32] * n, [0] * n, W, storage_dtypes=[FP32] * n, param_dtypes=pdt)
        ref = oracle.plan(w.descs(), W)
        plan = fp.plan_buckets(w.descs(), W)
        gathered = np.random.default_rng(k).integers(0, 256, size=W * ref.B, dtype=np.uint8)
        ag = torch.from_numpy(gathered.copy()).to(DEV)
        for shift in range(3):
            outs = [Guarded(t.numel, t.param_dtype, (i + shift) % 3) for i, t in enumerate(w.tensors)]
            fp.all_gather_copy_out(plan, ag, [o.t for o in outs])
            torch.cuda.synchronize()
            wants = oracle.copy_out(ref, gathered)
            for i, (o, want) in enumerate(zip(outs, wants)):
                assert np.array_equal(o.result(), want.view(np.uint8)), f"layout {k} shift {shift}: param {i} differs"
        plan.destroy()


def test_copy_in_small_segments_every_dtype_pair():
    """Copy-in windows of many small segments in all four storage -> param
    dtype pairs, with the all-gather buffer 0, 4, 8 or 12 bytes past a
    16-byte boundary (segment ends off the line and vector boundaries of
    memory); shards at element offsets 0-2."""
    from conftest import small_segment_copy_in_layout
    shapes, sdt, pdt, W = small_segment_copy_in_layout()
    n = len(shapes)
    w = wl.custom(shapes, [FP32] * n, [0] * n, W, storage_dtypes=sdt, param_dtypes=pdt)
    ref = oracle.plan(w.descs(), W)
    plan = fp.plan_buckets(w.descs(), W)
    for row_off in (0, 4, 8, 12):
        print(f"[copy-in small segments] all-gather buffer at +{row_off} bytes", flush=True)
        ag = Guarded(W * plan.B, None, row_off)
        ag_ref = np.full((W, ref.B), POISON, np.uint8)
        for r in range(W):
            shards = _shards_random(w, ref, r)
            wl.inject_specials(shards, sdt, seed=r)
            offs = [(i + r) % 3 for i in range(n)]
            fp.all_gather_copy_in(plan, r, [to_dev(s_, t.storage_dtype, o) for s_, t, o in
                                            zip(shards, w.tensors, offs)], ag.t)
            oracle.copy_in(ref, r, shards, ag_ref)
        torch.cuda.synchronize()
        got = ag.result().reshape(W, -1)
        assert np.array_equal(got, ag_ref), f"copy-in rows differ (buffer at +{row_off} bytes)"
    plan.destroy()


def _edge_layouts():
    """The pack's edge layouts plus a crowded one: tiny parameters with
    zero-size ones between them, so that copy-in windows meet empty
    segments and gathered copy-out windows empty rank chunks."""
    return [
        wl.custom([(0, 4), (0, 1)], [FP32, BF16], [FP32, FP32], 4),
        wl.custom([(1,)], [BF16], [FP32], 8, param_dtypes=[FP32]),
        wl.custom([(5, 3)], [FP32], [BF16], 1),
        wl.custom([(3, 1), (2, 5), (7, 2)], [BF16, FP32, BF16], [FP32, FP32, FP32], 1000),
        wl.custom([(0, 3), (4, 4), (0, 9)], [FP32, FP32, BF16], [0, 0, 0], 3),
        wl.custom([(8, 0), (2, 2)], [BF16, BF16], [0, 0], 2),
        wl.custom([(3, 1), (0, 4), (2, 1), (0, 1), (5, 1), (1, 3), (0, 2), (7, 1), (900, 1), (13, 7)],
                  [BF16, FP32] * 5, [0] * 10, 4, storage_dtypes=[BF16, FP32, FP32, BF16, FP32] * 2,
                  param_dtypes=[BF16, BF16, FP32, FP32, BF16] * 2),
    ]


def test_copy_paths_edge_cases():
    """Copy-in (every rank, or a sample for large W), copy-out and the
    divided write-back on the edge layouts, against the oracle."""
    for ci, w in enumerate(_edge_layouts()):
        print(f"[copy edge] case={ci} W={w.world}", flush=True)
        W = w.world
        ref = oracle.plan(w.descs(), W)
        plan = fp.plan_buckets(w.descs(), W)
        ranks = range(W) if W <= 8 else [0, 1, W - 1]
        if ref.B:
            ag = Guarded(W * plan.B, None)
            ag_ref = np.full((W, ref.B), POISON, np.uint8)
            for r in ranks:
                shards = _shards_random(w, ref, r)
                fp.all_gather_copy_in(plan, r, [to_dev(s_, t.storage_dtype, (i + r) % 3) if s_.size else None
                                                for i, (s_, t) in enumerate(zip(shards, w.tensors))], ag.t)
                oracle.copy_in(ref, r, shards, ag_ref)
            torch.cuda.synchronize()
            assert np.array_equal(ag.result().reshape(W, -1), ag_ref), f"case {ci}: copy-in rows differ"
        gathered = np.random.default_rng(ci).integers(0, 256, size=W * ref.B, dtype=np.uint8)
        outs = [Guarded(t.numel, t.param_dtype, i % 3) if t.numel else None for i, t in enumerate(w.tensors)]
        fp.all_gather_copy_out(plan, torch.from_numpy(gathered.copy()).to(DEV), [o.t if o else None for o in outs])
        torch.cuda.synchronize()
        for i, (o, want) in enumerate(zip(outs, oracle.copy_out(ref, gathered))):
            if o is not None:
                assert np.array_equal(o.result(), want.view(np.uint8)), f"case {ci}: copy-out param {i} differs"
        for bi, b in enumerate(ref.buckets):
            for r in sorted({0, W - 1}):
                row = wl.random_array(b.S, b.dtype, seed=ci * 10 + bi)
                check_rs_copy_out(w, ref, plan, bi, r, row, float(W))
        plan.destroy()


@pytest.mark.parametrize("name", ["tiny", "mixed50m", "hetero500"])
def test_copy_in_all_gather_copy_out_round_trip(name):
    """copy-out(all-gather(copy-in(shards of X))) == cast(X), storage -> param dtype."""
    print(f"[round trip] workload={name}", flush=True)
    w = wl.get(name)
    ref = oracle.plan(w.descs(), w.world)
    plan = fp.plan_buckets(w.descs(), w.world)
    params = wl.make_params(w)
    ag = torch.empty(w.world * plan.B, dtype=torch.uint8, device=DEV)
    x_dev = [to_dev(x, t.storage_dtype) for x, t in zip(params, w.tensors)]
    for r in range(w.world):
        shards = []
        for i, (x, t) in enumerate(zip(x_dev, w.tensors)):
            P = ref.P[i]
            s = torch.zeros(P, dtype=x.dtype, device=DEV)
            v = max(0, min(P, t.numel - r * P))
            s[:v] = x[r * P: r * P + v]
            shards.append(s)
        fp.all_gather_copy_in(plan, r, shards, ag)
    outs = [torch.empty(t.numel, dtype=fp.TORCH_DTYPE[t.param_dtype], device=DEV) for t in w.tensors]
    fp.all_gather_copy_out(plan, ag, outs)
    torch.cuda.synchronize()
    for i, (o, x, t) in enumerate(zip(outs, params, w.tensors)):
        want = oracle.convert(x, t.storage_dtype, t.param_dtype)
        assert np.array_equal(host_bytes(o), want.view(np.uint8)), f"param {i} differs after the round trip"
    plan.destroy()


# --------------------------------------------------------------------------- reduce-scatter write-back

def check_rs_copy_out(w, ref, plan, bucket, rank, row, factor, row_offset=0, dst_offsets=None):
    """HIP write-back of rank `rank`'s reduced row of `bucket` vs the oracle,
    byte for byte, into guarded destinations (nothing written outside them)."""
    b = ref.buckets[bucket]
    rs = to_dev(row, b.dtype, row_offset)
    outs = [None] * len(w.tensors)
    for k, i in enumerate(b.members):
        v = oracle.valid_in_chunk(w.tensors[i].numel, b.P[k], rank)
        if v:
            off = dst_offsets[i] if dst_offsets else i % 3
            outs[i] = Guarded(v, w.tensors[i].storage_dtype, off)
    fp.reduce_scatter_copy_out(plan, bucket, rank, rs, [o.t if o is not None else None for o in outs], factor)
    torch.cuda.synchronize()
    wants = oracle.rs_copy_out(ref, bucket, rank, row, factor)
    for k, i in enumerate(b.members):
        if outs[i] is None:
            assert wants[k].size == 0
            continue
        got = outs[i].result()
        want = wants[k].view(np.uint8)
        if not np.array_equal(got, want):
            bad = np.flatnonzero(got != want)
            pytest.fail(f"{w.name} bucket {bucket} rank {rank} factor {factor}: param {i}: {bad.size} bytes differ, "
                        f"first at byte {bad[0]}")


def check_rs_copy_out_all(w, ref, plan, rank, rows, factor, row_offsets=None, dst_offsets=None, prepared=False):
    """HIP write-back of every bucket in one launch vs the oracle's write-back
    of each bucket, byte for byte, into guarded destinations."""
    rs = [to_dev(row, b.dtype, row_offsets[bi] if row_offsets else 0) for bi, (row, b) in enumerate(zip(rows, ref.buckets))]
    outs = [None] * len(w.tensors)
    for b in ref.buckets:
        for k, i in enumerate(b.members):
            v = oracle.valid_in_chunk(w.tensors[i].numel, b.P[k], rank)
            if v:
                outs[i] = Guarded(v, w.tensors[i].storage_dtype, dst_offsets[i] if dst_offsets else i % 3)
    dst = [o.t if o is not None else None for o in outs]
    if prepared:
        dst = fp.prepare_shard_grads(plan, None, rank, dst)
    c0 = fp.counters()[0]
    fp.reduce_scatter_copy_out_all(plan, rank, rs, dst, factor)
    torch.cuda.synchronize()
    assert fp.counters()[0] - c0 <= 1, "more than one launch"
    for bi, b in enumerate(ref.buckets):
        wants = oracle.rs_copy_out(ref, bi, rank, rows[bi], factor)
        for k, i in enumerate(b.members):
            if outs[i] is None:
                assert wants[k].size == 0
                continue
            got, want = outs[i].result(), wants[k].view(np.uint8)
            if not np.array_equal(got, want):
                bad = np.flatnonzero(got != want)
                pytest.fail(f"{w.name} all buckets rank {rank} factor {factor}: bucket {bi} param {i}: "
                            f"{bad.size} bytes differ, first at byte {bad[0]}")


@pytest.mark.parametrize("name", ["tiny", "mixed50m", "hetero500"])
def test_rs_copy_out_all_buckets_matches_oracle(name):
    """The write-back of every bucket in one launch (one bucket: the per-bucket call)."""
    print(f"[write-back all] workload={name}", flush=True)
    w = wl.get(name)
    ref = oracle.plan(w.descs(), w.world)
    plan = fp.plan_buckets(w.descs(), w.world)
    W = w.world
    rows = []
    for bi, b in enumerate(ref.buckets):
        row = wl.random_array(b.S, b.dtype, seed=31 + bi)
        wl.inject_specials([row], [b.dtype], seed=7 + bi)
        rows.append(row)
    ranks = range(W) if W <= 4 else [0, 1, W // 2, W - 1]
    for rank in ranks:
        for factor in (1.0, float(W), 3.0):
            print(f"[write-back all] {name} buckets={len(rows)} rank={rank} factor={factor}", flush=True)
            check_rs_copy_out_all(w, ref, plan, rank, rows, factor, prepared=(rank % 2 == 1))
    plan.destroy()


def test_rs_copy_out_all_buckets_random_layouts_misaligned():
    rng = random.Random(5151)
    done = 0
    for case in range(400):
        w = _random_workload(rng, case)
        ref = oracle.plan(w.descs(), w.world)
        if len(ref.buckets) < 2:
            continue
        plan = fp.plan_buckets(w.descs(), w.world)
        rows = []
        for bi, b in enumerate(ref.buckets):
            row = wl.random_array(b.S, b.dtype, seed=case * 7 + bi)
            wl.inject_specials([row], [b.dtype], seed=case + bi)
            rows.append(row)
        rank = rng.randrange(w.world)
        factor = rng.choice([1.0, 2.0, 3.0, 0.5, 6.0, float(np.float32(1e-3)), 1e30])
        row_offs = [rng.choice([0, 0, 1, 3]) for _ in rows]
        offs = {i: rng.choice([0, 0, 1, 2, 3, 5, 7]) for i in range(len(w.tensors))}
        print(f"[write-back all random] case={case} W={w.world} buckets={len(rows)} rank={rank} factor={factor} "
              f"row_off={row_offs} dst_off={offs}", flush=True)
        check_rs_copy_out_all(w, ref, plan, rank, rows, factor, row_offs, offs)
        plan.destroy()
        done += 1
        if done == 40:
            break
    assert done >= 20


@pytest.mark.parametrize("name", ["tiny", "mixed50m", "layout500", "kda_block", "hetero500"])
def test_rs_copy_out_matches_oracle(name):
    print(f"[write-back parity] workload={name}", flush=True)
    w = wl.get(name)
    ref = oracle.plan(w.descs(), w.world)
    plan = fp.plan_buckets(w.descs(), w.world)
    W = w.world
    ranks = range(W) if W <= 4 else [0, 1, W // 2, W - 1]
    factors = [1.0, float(W), 3.0]
    for bi, b in enumerate(ref.buckets):
        row = wl.random_array(b.S, b.dtype, seed=17 + bi)
        wl.inject_specials([row], [b.dtype], seed=bi)
        for rank in ranks:
            for factor in factors:
                print(f"[write-back parity] {name} bucket={bi} rank={rank} factor={factor}", flush=True)
                check_rs_copy_out(w, ref, plan, bi, rank, row, factor)
    plan.destroy()


def test_rs_copy_out_random_layouts_misaligned():
    rng = random.Random(4242)
    for case in range(50):
        w = _random_workload(rng, case)
        ref = oracle.plan(w.descs(), w.world)
        plan = fp.plan_buckets(w.descs(), w.world)
        for bi, b in enumerate(ref.buckets):
            row = wl.random_array(b.S, b.dtype, seed=case * 7 + bi)
            wl.inject_specials([row], [b.dtype], seed=case)
            rank = rng.randrange(w.world)
            factor = rng.choice([1.0, 2.0, 3.0, 0.5, 6.0, 7.5, float(np.float32(1e-3)), 1e30])
            row_off = rng.choice([0, 0, 1, 2, 3])
            offs = {i: rng.choice([0, 0, 1, 2, 3, 5, 7]) for i in range(len(w.tensors))}
            print(f"[write-back random] case={case} W={w.world} bucket={bi} rank={rank} factor={factor} "
                  f"row_off={row_off} dst_off={offs}", flush=True)
            check_rs_copy_out(w, ref, plan, bi, rank, row, factor, row_off, offs)
        plan.destroy()


def test_rs_copy_out_pack_round_trip_with_divide():
    """pack -> W identical ranks summed (W * row, exact for power-of-two W) ->
    write-back with divide W == the rank chunk of cast(cast(g)), on the GPU."""
    print("[write-back round trip] mixed50m", flush=True)
    w = wl.get("mixed50m")
    ref = oracle.plan(w.descs(), w.world)
    plan = fp.plan_buckets(w.descs(), w.world)
    W = w.world
    grads = wl.make_grads(w)
    g_dev = [to_dev(g, t.grad_dtype) for g, t in zip(grads, w.tensors)]
    b = plan.buckets[0]
    out = torch.empty(W * b.S, dtype=fp.TORCH_DTYPE[b.dtype], device=DEV)
    fp.pack_reduce_scatter_input(plan, 0, g_dev, out)
    summed = (out.view(W, b.S).float() * W).to(fp.TORCH_DTYPE[b.dtype])   # exact: power-of-two scale
    for rank in (0, W - 1):
        dst = [torch.empty(fp.valid_in_chunk(plan, i, rank), dtype=fp.TORCH_DTYPE[t.storage_dtype], device=DEV)
               for i, t in enumerate(w.tensors)]
        fp.reduce_scatter_copy_out(plan, 0, rank, summed[rank].contiguous(), dst, float(W))
        torch.cuda.synchronize()
        for i, t in enumerate(w.tensors):
            P = ref.P[i]
            v = oracle.valid_in_chunk(t.numel, P, rank)
            want = oracle.convert(oracle.convert(grads[i], t.grad_dtype, b.dtype), b.dtype, t.storage_dtype)
            assert np.array_equal(host_bytes(dst[i]), want[rank * P: rank * P + v].view(np.uint8)), i
    plan.destroy()


# --------------------------------------------------------------------------- FSDP1 flat layout

def _flat_of(w, reduce_dt=FP32, param_dt=BF16, W=None):
    ts = w.tensors
    return wl.custom([t.shape for t in ts], [t.grad_dtype for t in ts], [reduce_dt] * len(ts), W or w.world, w.seed,
                     storage_dtypes=[t.storage_dtype for t in ts], param_dtypes=[param_dt] * len(ts))


def check_flat(w, ranks, factors, seed=0, offsets=None):
    """Pack, write-back, copy-in and copy-out of a flat plan vs the oracle."""
    W = w.world
    ref = oracle.plan_flat(w.descs(), W)
    plan = fp.plan_buckets_flat(w.descs(), W)
    assert plan.c == ref.c
    rng = random.Random(seed)
    off = (lambda i: rng.choice([0, 0, 1, 2, 3])) if offsets else (lambda i: 0)
    # pack
    grads = wl.make_grads(w)
    wl.inject_specials(grads, [t.grad_dtype for t in w.tensors], seed=seed)
    g_dev = [to_dev(g, t.grad_dtype, off(i)) for i, (g, t) in enumerate(zip(grads, w.tensors))]
    packed = oracle.pack_flat(ref, grads)
    if plan.buckets:
        got = gpu_pack(plan, 0, g_dev, off(-1))
        if not np.array_equal(got, packed.view(np.uint8).reshape(-1)):
            bad = np.flatnonzero(got != packed.view(np.uint8).reshape(-1))
            pytest.fail(f"{w.name}: flat pack differs in {bad.size} bytes, first at {bad[0]}")
    print(f"[flat parity] {w.name}: pack checked", flush=True)
    # write-back of each rank's row (the packed row standing in for the reduced one)
    for r in ranks:
        for d in factors:
            rs = to_dev(packed[r].copy(), ref.dtype, off(-2))
            outs = [Guarded(oracle.piece_len(ref, i, r), t.storage_dtype, off(i)) if oracle.piece_len(ref, i, r)
                    else None for i, t in enumerate(w.tensors)]
            if plan.buckets:
                fp.reduce_scatter_copy_out(plan, 0, r, rs, [o.t if o is not None else None for o in outs], d)
                torch.cuda.synchronize()
            wants = oracle.rs_copy_out_flat(ref, r, packed[r].copy(), d)
            for i, (o, want) in enumerate(zip(outs, wants)):
                if o is None:
                    assert want.size == 0
                elif not np.array_equal(o.result(), want.view(np.uint8)):
                    pytest.fail(f"{w.name}: flat write-back rank {r} factor {d} param {i} differs")
    print(f"[flat parity] {w.name}: write-back checked", flush=True)
    # copy-in of every rank, then copy-out of the gathered flat parameter
    params = wl.make_params(w)
    ag = Guarded(W * ref.c, ref.param_dtype, off(-3))
    rows = []
    for r in range(W):
        pieces = []
        for i, (x, t) in enumerate(zip(params, w.tensors)):
            lo, hi = oracle.flat_piece(ref, i, r)
            pieces.append(x[max(0, lo - ref.F[i]): max(0, hi - ref.F[i])].copy() if hi > lo else np.zeros(0, x.dtype))
        if plan.n:
            fp.all_gather_copy_in(plan, r, [to_dev(p_, t.storage_dtype, off(i)) if p_.size else None
                                            for i, (p_, t) in enumerate(zip(pieces, w.tensors))], ag.t)
        rows.append(oracle.copy_in_flat(ref, r, pieces))
    torch.cuda.synchronize()
    flat = np.concatenate(rows) if rows else np.zeros(0, oracle.NP_DTYPE[ref.param_dtype])
    if ref.c:
        assert np.array_equal(ag.result(), flat.view(np.uint8)), f"{w.name}: flat copy-in rows differ"
    outs = [Guarded(t.numel, ref.param_dtype, off(i)) for i, t in enumerate(w.tensors)]
    if plan.n:
        fp.all_gather_copy_out(plan, ag.t, [o.t for o in outs])
        torch.cuda.synchronize()
    for i, (o, want) in enumerate(zip(outs, oracle.copy_out_flat(ref, flat))):
        assert np.array_equal(o.result(), want.view(np.uint8)), f"{w.name}: flat copy-out param {i} differs"
    plan.destroy()


@pytest.mark.parametrize("name", ["tiny", "mixed50m", "layout500", "kda_block", "hetero500"])
def test_flat_layout_matches_oracle(name):
    print(f"[flat parity] workload={name}", flush=True)
    w = _flat_of(wl.get(name))
    W = w.world
    check_flat(w, ranks=range(W) if W <= 4 else [0, 1, W - 1], factors=[1.0, float(W)])


def test_flat_layout_printed_units_and_random_misaligned():
    # the page's units: two blocks of two Linear(6,6) on 4 (36 / 18 / 9 per rank), Linear(3,3) on 4
    for k in (4, 2, 1):
        print(f"[flat parity] {k} x Linear(6,6), W=4", flush=True)
        check_flat(wl.custom([(6, 6)] * k, [FP32] * k, [FP32] * k, 4, seed=k), range(4), [1.0, 4.0])
    check_flat(wl.custom([(3, 3)], [FP32], [FP32], 4, seed=9), range(4), [1.0, 2.0])
    rng = random.Random(77)
    for case in range(40):
        base = _random_workload(rng, case)
        w = _flat_of(base, rng.choice([BF16, FP32]), rng.choice([BF16, FP32]))
        print(f"[flat random] case={case} W={w.world} n={len(w.tensors)}", flush=True)
        check_flat(w, sorted({0, w.world - 1, rng.randrange(w.world)}), [1.0, rng.choice([2.0, 3.0, 0.5])],
                   seed=case, offsets=True)


# --------------------------------------------------------------------------- beyond 2^31 elements

def _pattern_bits(idx):
    """bf16 bit pattern of element idx (int64 array or tensor): a hash of the
    index, finite (|exponent| bits below 0x80), with a hashed sign."""
    h = (idx * 2654435761) & 0xFFFFFFFF
    return ((h >> 16) & 0x3FFF) | ((h >> 1) & 0x8000)


def _oracle_sampled_pack(bits: np.ndarray) -> np.ndarray:
    """The oracle's fp32 pack of bf16 gradient elements given by their bits,
    element by element: a one-row layout of just these elements."""
    m = int(bits.size)
    ref = oracle.plan([(m, 1, BF16, FP32, FP32, BF16)], 1)
    return oracle.pack(ref, 0, [bits.astype(np.uint16).view(np.uint16)])[0].view(np.uint32)


def test_pack_and_write_back_beyond_2_31_elements():
    """One bf16 gradient of 2^31 + 2^20 + 3 elements (4.3 GB) and a small fp32
    one, W=2: the [2, S] fp32 pack (8.6 GB) and rank 1's write-back divided by 2,
    checked on sampled positions against the oracle, which computes each
    sampled output from the same seeded input (element offsets past 2^31
    exercise every 64-bit index path)."""
    numel = (1 << 31) + (1 << 20) + 3
    print(f"[beyond 2^31] numel={numel}", flush=True)
    descs = [(numel, 1, BF16, FP32, FP32, BF16), (5, 3, FP32, FP32, FP32, BF16)]
    plan = fp.plan_buckets(descs, 2)
    b = plan.buckets[0]
    P0, P1, S = b.P[0], b.P[1], b.S
    ref = oracle.plan(descs, 2)
    assert (b.O[0], b.O[1]) == (ref.buckets[0].O[0], ref.buckets[0].O[1]) == (0, P0) and P0 == ref.P[0]
    g0 = torch.empty(numel, dtype=torch.bfloat16, device=DEV)
    bits0 = g0.view(torch.int16)
    chunk = 1 << 28
    for s in range(0, numel, chunk):
        idx = torch.arange(s, min(numel, s + chunk), dtype=torch.int64, device=DEV)
        bits0[s:s + idx.numel()] = _pattern_bits(idx).to(torch.int16)
        del idx
    g1_h = wl.random_array(15, FP32, seed=3)
    g1 = to_dev(g1_h, FP32)
    out = torch.empty(2 * S, dtype=torch.float32, device=DEV)
    fp.pack_reduce_scatter_input(plan, 0, [g0, g1], out)
    torch.cuda.synchronize()

    rng = np.random.default_rng(31)
    j = np.unique(np.concatenate([
        rng.integers(0, P0, 20000),
        np.arange(max(0, (1 << 31) - P0 - 4), min(P0, (1 << 31) - P0 + 4)),   # flat source index 2^31 on rank 1
        np.arange(0, 4), np.arange(P0 - 4, P0)]))
    # the small tensor's part of the rows, from the oracle's pack of the whole
    # layout with the large tensor replaced by a 2-element stand-in (its own
    # columns are not compared here)
    small_ref = oracle.plan([(2, 1, BF16, FP32, FP32, BF16), descs[1]], 2)
    small_rows = oracle.pack(small_ref, 0, [np.zeros(2, np.uint16), g1_h])
    pad_ref = oracle.plan([(1, 1, BF16, FP32, FP32, BF16)], 2)      # rank 1's chunk is all padding
    pad_bits = oracle.pack(pad_ref, 0, [np.zeros(1, np.uint16)])[1].view(np.uint32)[0]
    rows_want = {}
    for r in (0, 1):
        src = r * P0 + j
        real = src < numel
        want = np.zeros(j.size, np.uint32)
        want[real] = _oracle_sampled_pack((_pattern_bits(src[real]).astype(np.int64) & 0xFFFF).astype(np.uint16))
        want[~real] = pad_bits                 # past the tensor's end: the oracle's padding
        rows_want[r] = want
        got = out.view(torch.int32)[torch.from_numpy(r * S + j).to(DEV)].cpu().numpy().view(np.uint32)
        assert np.array_equal(got, want), f"rank {r}: pack of the large tensor differs"
        small = out[r * S + P0: r * S + P0 + P1].cpu().numpy()
        assert np.array_equal(small.view(np.uint32), small_rows[r, small_ref.buckets[0].O[1]:].view(np.uint32))

    # write-back of rank 1 (its row of the pack standing in for the reduced row), divided by 2
    v0 = numel - P0
    dst0 = torch.empty(v0, dtype=torch.float32, device=DEV)
    dst1 = torch.empty(max(0, min(P1, 15 - P1)), dtype=torch.float32, device=DEV)
    fp.reduce_scatter_copy_out(plan, 0, 1, out[S:2 * S], [dst0, dst1], 2.0)
    torch.cuda.synchronize()
    keep = j < v0
    jj = j[keep]
    # the oracle's write-back of the sampled elements of the oracle's row 1
    wb_ref = oracle.plan([(int(jj.size), 1, FP32, FP32, FP32, BF16)], 1)
    want = oracle.rs_copy_out(wb_ref, 0, 0, rows_want[1][keep].view(np.float32), 2.0)[0].view(np.uint32)
    got = dst0.view(torch.int32)[torch.from_numpy(jj).to(DEV)].cpu().numpy().view(np.uint32)
    assert np.array_equal(got, want), "write-back of the large tensor differs"
    del g0, out, dst0
    torch.cuda.empty_cache()
    plan.destroy()
