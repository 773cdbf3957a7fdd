"""The allocation-free pack (fsdppack_pack_reduce_scatter_input_noalloc) against
the ordinary pack, byte for byte, through the C ABI: two calls in a row on
the library's shared device scratch, the second with a smaller layout (so
any table left from the first call must not leak into it), plus a bucket of
fp32 gradients into bf16 and a plan that is never used by an allocating call
(its device tables are never created), the scratch's reuse of the
tables it already holds, flat plans, and calls captured into a graph."""
import numpy as np
import pytest

import workloads as wl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)
import fsdp2_mixed_dtype_amd as fp  # noqa: E402

DEV = torch.device("cuda:0")
BF16, FP32 = 1, 2


def _dev(a, dt, elem_offset=0):
    a = np.ascontiguousarray(a).reshape(-1)
    base = torch.empty(a.size + elem_offset, dtype=fp.TORCH_DTYPE[dt], device=DEV)
    t = base[elem_offset:]
    host = torch.from_numpy(a.copy())
    t.copy_(host.view(torch.bfloat16) if dt == BF16 else host)
    return t


def _both(w, out_offset=0):
    """Every bucket of layout w packed by the ordinary entry point (on one
    plan) and by the allocation-free one (on a second plan of the same
    layout); returns the byte arrays and the second plan's counter deltas."""
    grads = wl.make_grads(w)
    g_dev = [_dev(g, t.grad_dtype, i % 2) for i, (g, t) in enumerate(zip(grads, w.tensors))]
    ref_plan = fp.plan_buckets(w.descs(), w.world)
    na_plan = fp.plan_buckets(w.descs(), w.world)
    pairs = []
    for bi, b in enumerate(ref_plan.buckets):
        n = w.world * b.S
        a = torch.full((n + out_offset,), 7, dtype=fp.TORCH_DTYPE[b.dtype], device=DEV)[out_offset:]
        fp.pack_reduce_scatter_input(ref_plan, bi, g_dev, a)
        torch.cuda.synchronize()
        c0 = fp.counters()
        z = torch.full((n + out_offset,), 9, dtype=fp.TORCH_DTYPE[b.dtype], device=DEV)[out_offset:]
        fp.pack_reduce_scatter_input_noalloc(na_plan, bi, g_dev, z)
        torch.cuda.synchronize()
        c1 = fp.counters()
        pairs.append((a.view(torch.uint8).cpu().numpy(), z.view(torch.uint8).cpu().numpy(),
                      [y - x for x, y in zip(c0, c1)]))
    ref_plan.destroy()
    na_plan.destroy()
    return pairs


def test_no_alloc_pack_matches_the_pack_twice_then_smaller():
    layouts = [
        ("mixed50m", wl.mixed50m(), 0),
        # smaller: two buckets (bf16 and fp32 reduction), gradients of both dtypes, an odd output offset
        ("small two-bucket", wl.custom([(4 * 1025, 3), (5,), (64, 2), (4 * 700, 8), (33, 7)],
                                       [BF16, FP32, BF16, FP32, BF16], [FP32, BF16, FP32, BF16, 0], 4, seed=11), 1),
        ("tiny", wl.tiny(), 0),
    ]
    for name, w, off in layouts:
        print(f"[no-alloc] {name}", flush=True)
        for bi, (a, z, dc) in enumerate(_both(w, off)):
            assert np.array_equal(a, z), f"{name}: bucket {bi} differs from the ordinary pack"
            assert dc[0] == 1                     # one launch ...
            assert dc[1] == 0 and dc[3] == 0      # ... no pointer table and no plan table created


class _Layout:
    """A layout's gradients on the GPU, the ordinary pack of each bucket, and
    a second plan for the allocation-free calls."""

    def __init__(self, w):
        self.w = w
        self.g = [_dev(g, t.grad_dtype) for g, t in zip(wl.make_grads(w), w.tensors)]
        ref = fp.plan_buckets(w.descs(), w.world)
        self.ref = []
        for bi, b in enumerate(ref.buckets):
            a = torch.empty(w.world * b.S, dtype=fp.TORCH_DTYPE[b.dtype], device=DEV)
            fp.pack_reduce_scatter_input(ref, bi, self.g, a)
            self.ref.append(a)
        torch.cuda.synchronize()
        ref.destroy()
        self.plan = fp.plan_buckets(w.descs(), w.world)
        self.outs = []

    def call(self, bi):
        b = self.plan.buckets[bi]
        z = torch.full((self.w.world * b.S,), 9, dtype=fp.TORCH_DTYPE[b.dtype], device=DEV)
        c0 = fp.counters()[8]
        fp.pack_reduce_scatter_input_noalloc(self.plan, bi, self.g, z)
        self.outs.append((bi, z))
        return fp.counters()[8] - c0

    def check(self, name):
        for bi, z in self.outs:
            assert torch.equal(z.view(torch.uint8), self.ref[bi].view(torch.uint8)), \
                f"{name}: bucket {bi} differs from the ordinary pack"
        self.plan.destroy()


def test_no_alloc_pack_copies_its_tables_only_when_the_scratch_lacks_them():
    """The scratch keeps the last image copied into it.  A plan whose buckets
    fit it together copies once for all of them, and again only after another
    plan's image has replaced it; a plan whose buckets fit only one at a time
    copies at every change of bucket.  A call on a second stream, ordered
    after the first but issued while the copy may still be running, reuses
    the image (its stream waits for the copy).  Every result equals the
    ordinary pack's."""
    a = _Layout(wl.custom([(4 * 1025, 3), (5,), (64, 2), (4 * 700, 8), (33, 7)],
                          [BF16, FP32, BF16, FP32, BF16], [FP32, BF16, FP32, BF16, 0], 4, seed=12))
    b = _Layout(wl.tiny())
    # two buckets of about 620 KB of tables each (one large member and 900
    # one-element members: a column-map entry per window of the 16 MB rows)
    big = [(2 * 4 * 1024 * 1024,)] + [(1,)] * 900 + [(2 * 8 * 1024 * 1024,)] + [(1,)] * 900
    c = _Layout(wl.custom(big, [FP32] * 901 + [BF16] * 901, [FP32] * 901 + [BF16] * 901, 2, seed=13))
    assert len(a.plan.buckets) == 2 and len(c.plan.buckets) == 2
    print("[no-alloc] residency: one plan, both buckets", flush=True)
    assert a.call(0) == 1
    assert a.call(1) == 0 and a.call(0) == 0
    s2 = torch.cuda.Stream()
    s2.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s2):
        assert a.call(1) == 0
    torch.cuda.current_stream().wait_stream(s2)
    torch.cuda.synchronize()
    assert a.call(0) == 0
    print("[no-alloc] residency: another plan in between", flush=True)
    assert b.call(0) == 1 and b.call(0) == 0
    assert a.call(1) == 1
    print("[no-alloc] residency: buckets that fit one at a time", flush=True)
    assert c.call(0) == 1 and c.call(0) == 0
    assert c.call(1) == 1 and c.call(0) == 1 and c.call(1) == 1
    torch.cuda.synchronize()
    for name, lay in (("two-bucket", a), ("tiny", b), ("one bucket at a time", c)):
        lay.check(name)


def test_no_alloc_pack_of_flat_plans_matches_the_pack():
    """FSDP1 flat plans (one row of W*c elements, +0 past the flat length N)
    through the allocation-free pack, against the ordinary flat pack: a full
    size layout of mixed gradient dtypes, and a small one whose output and
    gradients sit at odd element offsets."""
    def flat(w):
        ts = w.tensors
        return wl.custom([t.shape for t in ts], [t.grad_dtype for t in ts], [FP32] * len(ts), w.world, w.seed,
                         storage_dtypes=[t.storage_dtype for t in ts], param_dtypes=[BF16] * len(ts))

    cases = [("mixed50m", flat(wl.mixed50m()), 0),
             ("small", wl.custom([(37, 3), (5,), (64, 2), (700, 8), (33, 7)], [BF16, FP32, BF16, FP32, BF16],
                                 [FP32] * 5, 4, seed=14, param_dtypes=[BF16] * 5), 1)]
    for name, w, off in cases:
        print(f"[no-alloc] flat {name}", flush=True)
        g = [_dev(x, t.grad_dtype, off * (i % 2)) for i, (x, t) in enumerate(zip(wl.make_grads(w), w.tensors))]
        ref = fp.plan_buckets_flat(w.descs(), w.world)
        na = fp.plan_buckets_flat(w.descs(), w.world)
        assert len(ref.buckets) == 1
        n = w.world * ref.c
        a = torch.full((n + off,), 7, dtype=torch.float32, device=DEV)[off:]
        z = torch.full((n + off,), 9, dtype=torch.float32, device=DEV)[off:]
        fp.pack_reduce_scatter_input(ref, 0, g, a)
        fp.pack_reduce_scatter_input_noalloc(na, 0, g, z)
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.uint8), z.view(torch.uint8)), f"flat {name} differs from the ordinary pack"
        ref.destroy()
        na.destroy()


def test_no_alloc_pack_rejects_what_it_cannot_hold():
    k = 1000                                    # more members than the launch arguments carry
    w = wl.custom([(3, 1)] * k, [FP32] * k, [FP32] * k, 2)
    plan = fp.plan_buckets(w.descs(), w.world)
    g = torch.zeros(3, device=DEV)
    with pytest.raises(fp.FsdpPackError) as e:
        fp.pack_reduce_scatter_input_noalloc(plan, 0, [g] * k, torch.empty(2 * plan.buckets[0].S, device=DEV))
    assert e.value.code == -1 and "members" in str(e.value)
    plan.destroy()


# Last in this file: once a call has been captured on the device, every later
# allocation-free call there copies its tables (the residency test above
# expects reuse).
def test_no_alloc_pack_captured_in_a_graph_and_replayed():
    """Both buckets of plan X packed by the allocation-free entry point under
    stream capture (torch.cuda.graph) and replayed three times, with eager
    calls of another plan A around each replay.  A replay copies X's tables
    into the scratch ahead of its kernels; the eager call of A after it must
    copy A's tables again rather than trust that the scratch still holds them
    (once a graph holds such a copy, every eager call copies).  Every replay
    and every eager result equals the ordinary pack's."""
    x = _Layout(wl.custom([(4 * 1025, 3), (5,), (64, 2), (4 * 700, 8), (33, 7)],
                          [BF16, FP32, BF16, FP32, BF16], [FP32, BF16, FP32, BF16, 0], 4, seed=15))
    a = _Layout(wl.tiny())
    nb = len(x.plan.buckets)
    outs = [torch.full_like(r, 9) for r in x.ref]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):                # set-up outside the capture, as torch advises
        for bi in range(nb):
            fp.pack_reduce_scatter_input_noalloc(x.plan, bi, x.g, outs[bi])
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    print("[no-alloc] capture", flush=True)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for bi in range(nb):
            fp.pack_reduce_scatter_input_noalloc(x.plan, bi, x.g, outs[bi])
    torch.cuda.synchronize()
    for rep in range(3):
        print(f"[no-alloc] replay {rep}", flush=True)
        for o in outs:
            o.fill_(9)
        assert a.call(0) == 1
        graph.replay()
        assert a.call(0) == 1                    # the replay replaced the tables: copied again
        assert x.call(rep % nb) == 1
        torch.cuda.synchronize()
        for bi in range(nb):
            assert torch.equal(outs[bi].view(torch.uint8), x.ref[bi].view(torch.uint8)), \
                f"replay {rep}: bucket {bi} differs from the ordinary pack"
    graph.reset()
    for name, lay in (("captured plan, eager calls", x), ("tiny", a)):
        lay.check(name)
