"""Host checks of the library's planner and work lists (no GPU needed).

* The planner behind the C ABI (fsdppack_plan.cpp) agrees with the oracle's
  planner on every layout: buckets, members, P, O, S, A and B.
* A sanitizer build of the same planner (tests/native/worklist_check.cpp)
  runs every window of every launch through the kernels' own window -> range
  mapping and verifies the bounds invariants the HIP kernels rely on --
  every range reads and writes inside its buffers and the windows cover every
  destination byte exactly once -- for the five workloads and for random
  layouts.
* Argument errors are reported synchronously with the documented codes.
"""
import os
import random
import subprocess

import pytest

import oracle
import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
fp = pytest.importorskip("fsdp2_mixed_dtype_amd")
BF16, FP32 = 1, 2


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("wlc") / "worklist_check")
    subprocess.check_call(["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
                           "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "include"),
                           os.path.join(ROOT, "tests", "native", "worklist_check.cpp"),
                           os.path.join(ROOT, "fsdp2_mixed_dtype_amd", "csrc", "fsdppack_plan.cpp"),
                           "-o", exe])
    return exe


def _run(exe, descs, W, flat=False):
    text = f"{W} {len(descs)}\n" + "".join(" ".join(str(int(x)) for x in d) + "\n" for d in descs)
    res = subprocess.run([exe] + (["flat"] if flat else []), input=text, capture_output=True, text=True, timeout=600)
    assert res.returncode == 0 and res.stdout.startswith("OK"), res.stdout + res.stderr[-3000:]


def _random_layout(rng):
    W = rng.choice([1, 2, 3, 4, 7, 8, 16, 128, 300])
    n = rng.randint(0, 12)
    descs = []
    for _ in range(n):
        dim0 = rng.choice([0, 1, 2, 3, W - 1, W, W + 1, rng.randint(1, 5 * W + 3)])
        inner = rng.choice([0, 1, 2, 3, 5, 8, 64, 33]) if dim0 else rng.randint(0, 4)
        descs.append((max(dim0, 0), inner, rng.choice([BF16, FP32]), rng.choice([0, BF16, FP32]),
                      rng.choice([BF16, FP32]), rng.choice([BF16, FP32])))
    return descs, W


@pytest.mark.parametrize("name", list(wl.WORKLOADS))
def test_worklists_in_bounds_workloads(checker, name):
    w = wl.get(name)
    _run(checker, w.descs(), w.world)


def test_direct_windows_are_exercised(checker):
    """The direct-copy layout of the GPU tests really produces direct pack
    windows (and the checker finds each equal to its general range)."""
    from conftest import direct_window_layout
    shapes, gdt, rdt, W = direct_window_layout()
    w = wl.custom(shapes, gdt, rdt, W)
    text = f"{W} {len(w.descs())}\n" + "".join(" ".join(str(int(x)) for x in d) + "\n" for d in w.descs())
    res = subprocess.run([checker], input=text, capture_output=True, text=True, timeout=600)
    assert res.returncode == 0 and res.stdout.startswith("OK"), res.stdout + res.stderr[-3000:]
    direct = int(res.stdout.rsplit("direct pack windows", 1)[1].split()[0].rstrip(","))
    assert direct > 100, res.stdout


def test_gathered_copy_out_windows_are_exercised(checker):
    """The gathered copy-out layouts of the GPU tests really produce copy-out
    windows that the kernel gathers element by element (and the checker finds
    each element read from the byte the chunk walk reads)."""
    from conftest import gathered_copy_out_layout
    for shapes, pdt, W in gathered_copy_out_layout():
        w = wl.custom(shapes, [FP32] * len(shapes), [0] * len(shapes), W, storage_dtypes=[FP32] * len(shapes),
                      param_dtypes=pdt)
        text = f"{W} {len(w.descs())}\n" + "".join(" ".join(str(int(x)) for x in d) + "\n" for d in w.descs())
        res = subprocess.run([checker], input=text, capture_output=True, text=True, timeout=600)
        assert res.returncode == 0 and res.stdout.startswith("OK"), res.stdout + res.stderr[-3000:]
        gathered = int(res.stdout.rsplit("gathered copy-out windows", 1)[1].split()[0].rstrip(","))
        assert gathered >= 2, res.stdout


def test_small_segment_copy_in_windows(checker):
    """The small-segment layout of the GPU tests: every segment gets windows
    of its own (at least one each), each one range, which the checker walks
    at every row offset."""
    from conftest import small_segment_copy_in_layout
    shapes, sdt, pdt, W = small_segment_copy_in_layout()
    n = len(shapes)
    w = wl.custom(shapes, [FP32] * n, [0] * n, W, storage_dtypes=sdt, param_dtypes=pdt)
    text = f"{W} {n}\n" + "".join(" ".join(str(int(x)) for x in d) + "\n" for d in w.descs())
    res = subprocess.run([checker], input=text, capture_output=True, text=True, timeout=600)
    assert res.returncode == 0 and res.stdout.startswith("OK"), res.stdout + res.stderr[-3000:]
    windows = int(res.stdout.split(" copy_in ", 1)[1].split()[0])
    assert windows >= n, res.stdout


def test_worklists_in_bounds_random(checker):
    rng = random.Random(1234)
    for _ in range(150):
        descs, W = _random_layout(rng)
        _run(checker, descs, W)


def _oracle_matches(descs, W):
    p = fp.plan_buckets(descs, W)
    o = oracle.plan(descs, W)
    assert [(b.dtype, list(b.members), list(b.P), list(b.O), b.S) for b in p.buckets] == \
           [(b.dtype, b.members, b.P, b.O, b.S) for b in o.buckets]
    assert (p.B, list(p.A), list(p.P)) == (o.B, o.A, o.P)
    p.destroy()


@pytest.mark.parametrize("name", list(wl.WORKLOADS))
def test_abi_planner_matches_oracle_workloads(name):
    w = wl.get(name)
    _oracle_matches(w.descs(), w.world)


def test_abi_planner_matches_oracle_random():
    rng = random.Random(99)
    for _ in range(300):
        descs, W = _random_layout(rng)
        _oracle_matches(descs, W)


def test_planner_errors():
    with pytest.raises(fp.FsdpPackError) as e:
        fp.plan_buckets([(4, 4, FP32, 0, FP32, FP32)], 0)
    assert e.value.code == -1
    with pytest.raises(fp.FsdpPackError) as e:
        fp.plan_buckets([(4, 4, 3, 0, FP32, FP32)], 2)
    assert e.value.code == -2
    with pytest.raises(fp.FsdpPackError) as e:
        fp.plan_buckets([(4, 4, FP32, 7, FP32, FP32)], 2)
    assert e.value.code == -2
    with pytest.raises(fp.FsdpPackError) as e:
        fp.plan_buckets([(-1, 4, FP32, 0, FP32, FP32)], 2)
    assert e.value.code == -1
    with pytest.raises(fp.FsdpPackError) as e:
        fp.plan_buckets([(1 << 40, 1 << 30, FP32, 0, FP32, FP32)], 2)
    assert e.value.code == -1
    empty = fp.plan_buckets([], 3)
    assert empty.buckets == () and empty.B == 0
    empty.destroy()


def test_planner_rejects_unlaunchable_grids():
    """A launch counts its grid in 32-bit work-items: a unit whose pack, copy-in,
    copy-out or write-back would need 2^26 or more 64-thread workgroups in one
    dimension is rejected when planned, not at launch."""
    big = 1 << 35                       # fp32 elements: 2^26 windows of 2 KiB for the copy-out
    for W in (1, 8):
        for flat in (False, True):
            fn = fp.plan_buckets_flat if flat else fp.plan_buckets
            with pytest.raises(fp.FsdpPackError) as e:
                fn([(big, 1, FP32, 0, FP32, FP32)], W)
            assert e.value.code == -1 and "too many" in str(e.value)
    # a pack row of 2^26 windows with every other launch small enough
    with pytest.raises(fp.FsdpPackError) as e:
        fp.plan_buckets([(1 << 14, 1 << 21, BF16, FP32, BF16, BF16)], 1)
    assert e.value.code == -1 and "reduce-scatter buffer" in str(e.value)
    ok = fp.plan_buckets([(1 << 13, 1 << 20, BF16, 0, BF16, BF16)], 1)      # 2^34 bytes per launch: 2^23 windows
    ok.destroy()


def test_no_alloc_pack_argument_errors_before_any_gpu_work():
    import ctypes
    L = fp.lib()
    p = fp.plan_buckets([(4, 4, FP32, 0, FP32, BF16), (3, 1, BF16, 0, FP32, BF16)], 2)
    ptrs = (ctypes.c_void_p * 2)(0x1000, 0x2002)
    na = L.fsdppack_pack_reduce_scatter_input_noalloc
    assert na(p.handle, 5, ptrs, 0x4000, None) == -1                     # bucket out of range
    assert na(p.handle, 0, None, 0x4000, None) == -1                     # NULL array
    assert na(p.handle, 0, ptrs, 0x4002, None) == -1                     # misaligned out
    bad = (ctypes.c_void_p * 2)(0x1001, 0x2002)
    assert na(p.handle, 0, bad, 0x4000, None) == -1                      # misaligned gradient
    assert "grads[0]" in L.fsdppack_last_error().decode()
    assert na(None, 0, ptrs, 0x4000, None) == -5
    p.destroy()
    k = 961                                                               # one more than the arguments carry
    big = fp.plan_buckets([(2, 1, FP32, 0, FP32, FP32)] * k, 2)
    many = (ctypes.c_void_p * k)(*([0x1000] * k))
    assert na(big.handle, 0, many, 0x4000, None) == -1
    assert "members" in L.fsdppack_last_error().decode()
    big.destroy()
    assert fp.counters()[0] == 0


def test_write_back_all_argument_errors_before_any_gpu_work():
    import ctypes
    L = fp.lib()
    f = L.fsdppack_reduce_scatter_copy_out_all
    # two buckets (fp32 and bf16 reduction)
    p = fp.plan_buckets([(4, 4, FP32, FP32, FP32, BF16), (3, 1, BF16, BF16, FP32, BF16)], 2)
    assert len(p.buckets) == 2
    grads = (ctypes.c_void_p * 2)(0x1000, 0x2000)
    rows = (ctypes.c_void_p * 2)(0x4000, 0x5000)
    assert f(p.handle, 0, None, 1.0, grads, None) == -1                   # NULL rows
    assert f(p.handle, 2, rows, 1.0, grads, None) == -1                   # rank out of range
    assert f(p.handle, 0, rows, 0.0, grads, None) == -1                   # bad factor
    assert f(p.handle, 0, rows, float("inf"), grads, None) == -1
    assert f(p.handle, 0, rows, 1.0, None, None) == -1                    # NULL shard_grads
    bad_row = (ctypes.c_void_p * 2)(0x4000, 0x5001)
    assert f(p.handle, 0, bad_row, 1.0, grads, None) == -1                # misaligned bf16 row
    assert "rs_outs[1]" in L.fsdppack_last_error().decode()
    bad_grad = (ctypes.c_void_p * 2)(0x1002, 0x2000)
    assert f(p.handle, 0, rows, 1.0, bad_grad, None) == -1                # misaligned fp32 shard
    assert "shard_grads[0]" in L.fsdppack_last_error().decode()
    assert f(None, 0, rows, 1.0, grads, None) == -5
    p.destroy()
    # one bucket: the per-bucket call's checks
    q = fp.plan_buckets([(4, 4, FP32, 0, FP32, BF16)], 2)
    assert f(q.handle, 0, (ctypes.c_void_p * 1)(0x4001), 1.0, grads, None) == -1
    assert "rs_out" in L.fsdppack_last_error().decode()
    q.destroy()
    # no parameters: nothing to launch, arguments still checked
    e = fp.plan_buckets([], 2)
    assert f(e.handle, 0, rows, 1.0, grads, None) == 0
    assert f(e.handle, 3, rows, 1.0, grads, None) == -1
    e.destroy()
    assert fp.counters()[0] == 0


def test_empty_launch_argument_errors():
    L = fp.lib()
    for wg, th in ((0, 64), (-1, 64), (1, 0), (1, 63), (1, 2048), (1 << 30, 1024), ((1 << 31) - 1, 64)):
        assert L.fsdppack_empty_launch(wg, th, None) == -1, (wg, th)
    assert "empty_launch" in L.fsdppack_last_error().decode()
    assert fp.counters()[0] == 0


def test_compute_call_argument_errors_before_any_gpu_work():
    # all of these are rejected on the host, so they run without a GPU
    import ctypes
    L = fp.lib()
    p = fp.plan_buckets([(4, 4, FP32, 0, FP32, BF16), (3, 1, BF16, 0, FP32, BF16)], 2)
    ptrs = (ctypes.c_void_p * 2)(0x1000, 0x2002)
    assert L.fsdppack_pack_reduce_scatter_input(p.handle, 5, ptrs, 0x4000, None) == -1
    assert L.fsdppack_pack_reduce_scatter_input(p.handle, 0, None, 0x4000, None) == -1
    assert "grads is NULL" in L.fsdppack_last_error().decode()
    assert L.fsdppack_pack_reduce_scatter_input(p.handle, 0, ptrs, 0x4002, None) == -1       # misaligned out
    bad = (ctypes.c_void_p * 2)(0x1001, 0x2002)
    assert L.fsdppack_pack_reduce_scatter_input(p.handle, 0, bad, 0x4000, None) == -1         # misaligned grad
    assert "grads[0]" in L.fsdppack_last_error().decode()
    nul = (ctypes.c_void_p * 2)(0, 0x2002)
    assert L.fsdppack_pack_reduce_scatter_input(p.handle, 0, nul, 0x4000, None) == -1         # NULL member
    assert L.fsdppack_all_gather_copy_in(p.handle, 2, ptrs, 0x4000, None) == -1               # rank out of range
    assert L.fsdppack_all_gather_copy_in(p.handle, -1, ptrs, 0x4000, None) == -1
    assert L.fsdppack_all_gather_copy_in(p.handle, 0, ptrs, 0x4002, None) == -1               # misaligned row
    assert L.fsdppack_all_gather_copy_out(p.handle, 0x4000, None, None) == -1
    assert L.fsdppack_plan_bucket(p.handle, 3, None, None, None, None, None, None) == -1
    assert L.fsdppack_plan_bucket(None, 0, None, None, None, None, None, None) == -5
    assert L.fsdppack_pack_reduce_scatter_input(None, 0, ptrs, 0x4000, None) == -5
    # reduce-scatter write-back (one fp32 bucket; parameter 1 holds 2 then 1 real elements)
    wb = L.fsdppack_reduce_scatter_copy_out
    assert wb(p.handle, 1, 0, 0x4000, 1.0, ptrs, None) == -1                                 # bucket out of range
    assert wb(p.handle, 0, 2, 0x4000, 1.0, ptrs, None) == -1                                 # rank out of range
    assert "rank out of range" in L.fsdppack_last_error().decode()
    for factor in (0.0, -2.0, float("inf"), float("nan")):
        assert wb(p.handle, 0, 0, 0x4000, factor, ptrs, None) == -1
        assert "divide_factor" in L.fsdppack_last_error().decode()
    assert wb(p.handle, 0, 0, 0x4000, 2.0, None, None) == -1                                 # NULL array
    assert wb(p.handle, 0, 0, 0x4002, 2.0, ptrs, None) == -1                                 # misaligned row
    assert wb(p.handle, 0, 0, 0x4000, 2.0, bad, None) == -1                                  # misaligned grad
    assert "shard_grads[0]" in L.fsdppack_last_error().decode()
    assert wb(p.handle, 0, 1, 0x4000, 2.0, nul, None) == -1                                  # NULL member with data
    assert wb(None, 0, 0, 0x4000, 1.0, ptrs, None) == -5
    p.destroy()
    assert fp.counters()[0] == 0           # nothing was launched


# --------------------------------------------------------------------------- FSDP1 flat layout

def _flat_descs(descs, reduce_dt, param_dt):
    """The same shapes as one flat parameter: one reduction and one param dtype."""
    return [(d0, inner, g, reduce_dt, s_, param_dt) for d0, inner, g, _, s_, _ in descs]


@pytest.mark.parametrize("name", list(wl.WORKLOADS))
def test_flat_worklists_in_bounds_workloads(checker, name):
    w = wl.get(name)
    _run(checker, _flat_descs(w.descs(), FP32, BF16), w.world, flat=True)


def test_flat_worklists_padding_past_a_map_stretch(checker):
    # N a whole number of 2 KiB map stretches and padding that runs past the
    # last one: the last rank's row must not look up a stretch beyond N
    for n_el, W, dt in ((1536, 5, FP32), (2048, 3, BF16), (512, 3, FP32), (4096, 7, BF16)):
        _run(checker, [(n_el, 1, dt, dt, dt, dt)], W, flat=True)
        _run(checker, [(n_el - 8, 1, dt, dt, dt, dt), (8, 1, FP32, dt, BF16, dt)], W, flat=True)


def test_flat_worklists_in_bounds_random(checker):
    rng = random.Random(4321)
    for _ in range(120):
        descs, W = _random_layout(rng)
        _run(checker, _flat_descs(descs, rng.choice([BF16, FP32]), rng.choice([BF16, FP32])), W, flat=True)


def _flat_oracle_matches(descs, W):
    p = fp.plan_buckets_flat(descs, W)
    o = oracle.plan_flat(descs, W)
    if not descs:
        assert p.buckets == () and p.B == 0
    else:
        (b,) = p.buckets
        assert (b.dtype, b.S, list(b.members), list(b.O), list(b.P)) == \
               (o.dtype, o.c, list(range(len(descs))), o.F, [d.numel for d in o.params])
        esz = oracle.ELEM_SIZE[o.param_dtype]
        assert (p.B, list(p.A), list(p.P)) == (o.c * esz, [f * esz for f in o.F], [d.numel for d in o.params])
        for r in range(W):
            for i in range(len(descs)):
                assert fp.valid_in_chunk(p, i, r) == oracle.piece_len(o, i, r)
    p.destroy()


def test_abi_flat_planner_matches_oracle():
    rng = random.Random(7)
    for _ in range(200):
        descs, W = _random_layout(rng)
        _flat_oracle_matches(_flat_descs(descs, rng.choice([BF16, FP32]), rng.choice([BF16, FP32])), W)
    # the printed FSDP1 sizes: 36 / 18 / 9 per rank, and Linear(3,3) on 4
    lin = (6, 6, FP32, 0, FP32, FP32)
    for k, c in ((4, 36), (2, 18), (1, 9)):
        p = fp.plan_buckets_flat([lin] * k, 4)
        assert p.c == c
        p.destroy()
    p = fp.plan_buckets_flat([(3, 3, FP32, 0, FP32, FP32)], 4)
    assert p.c == 3 and [fp.valid_in_chunk(p, 0, r) for r in range(4)] == [3, 3, 3, 0]
    p.destroy()


def test_flat_planner_errors():
    with pytest.raises(fp.FsdpPackError) as e:       # two reduction dtypes
        fp.plan_buckets_flat([(2, 2, FP32, 0, FP32, BF16), (2, 2, BF16, 0, FP32, BF16)], 2)
    assert e.value.code == -2
    with pytest.raises(fp.FsdpPackError) as e:       # two param dtypes
        fp.plan_buckets_flat([(2, 2, FP32, 0, FP32, BF16), (2, 2, FP32, 0, FP32, FP32)], 2)
    assert e.value.code == -2
    empty = fp.plan_buckets_flat([], 3)
    assert empty.buckets == () and empty.B == 0
    empty.destroy()
