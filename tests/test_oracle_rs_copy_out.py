"""Pins of the oracle's reduce-scatter output write-back (oracle_rs_copy_out).

The step after the reduce-scatter: each rank keeps the gradient slice of the
parameters it owns ("The unit you wrapped", the paragraphs on the collectives
FSDP issues), divided by a factor when one is set, in the resident
parameter's dtype ("Mixed-Precision Training": reduce_dtype only sets how
gradients are summed).  Pinned from outside the oracle by:

* torch's CPU ops that FSDP2 itself applies to a reduce-scatter output --
  a division of the reduced tensor (in its dtype) and a cast to the storage
  dtype -- on random layouts with special values (non-NaN elements bit for
  bit; NaN stays NaN);
* with no divide, the already pinned pack: a rank's row written back is the
  gradient cast to the reduction dtype and then to the storage dtype, sliced
  to the rank's chunk;
* the divide of W identical summed rows by a power-of-two W, which is exact,
  gives the undivided write-back back bit for bit.
"""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
import workloads as wl

torch = pytest.importorskip("torch")
BF16, FP32 = oracle.BF16, oracle.FP32
TDT = {BF16: torch.bfloat16, FP32: torch.float32}
BITS = {BF16: np.uint16, FP32: np.uint32}


def _to_torch(a, dtype):
    t = torch.from_numpy(np.ascontiguousarray(a).copy())
    return t.view(torch.bfloat16) if dtype == BF16 else t


def _bits(t, dtype):
    t = t.contiguous()
    if dtype == BF16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy().view(np.uint32)


def _is_nan_bits(b, dtype):
    if dtype == BF16:
        return ((b & 0x7F80) == 0x7F80) & ((b & 0x007F) != 0)
    return ((b & 0x7F800000) == 0x7F800000) & ((b & 0x007FFFFF) != 0)


layouts = st.integers(min_value=1, max_value=9).flatmap(lambda W: st.tuples(
    st.just(W),
    st.lists(st.tuples(st.integers(0, 3 * W + 2),              # dim0 (0: empty parameter)
                       st.sampled_from([(), (1,), (3,), (2, 2), (5,)]),
                       st.sampled_from([BF16, FP32]),           # grad dtype
                       st.sampled_from([0, BF16, FP32]),        # reduce dtype (0: unset)
                       st.sampled_from([BF16, FP32])),          # storage dtype
             min_size=1, max_size=7),
    st.integers(0, 2**31 - 1),
    # divide factors exact in bf16 (so a bf16 tensor of the factor is the factor)
    st.sampled_from([1.0, 2.0, 3.0, 6.0, 8.0, 0.375, 1.5, 5.0, 1024.0])))


def _workload(W, tensors, seed):
    shapes = [(d0,) + rest for d0, rest, _, _, _ in tensors]
    return wl.custom(shapes, [g for _, _, g, _, _ in tensors], [r for _, _, _, r, _ in tensors], W, seed,
                     storage_dtypes=[s for _, _, _, _, s in tensors])


@settings(max_examples=150, deadline=None)
@given(layouts)
def test_matches_torch_divide_then_cast(layout):
    """grad_t = (row / d)[O_t : O_t + valid].to(storage) with torch's CPU ops,
    the division taken in the row's dtype between two tensors."""
    W, tensors, seed, d = layout
    w = _workload(W, tensors, seed)
    pl = oracle.plan(w.descs(), W)
    rng = np.random.default_rng(seed)
    for bi, b in enumerate(pl.buckets):
        # a reduced row with special values mixed in
        row = wl.random_array(b.S, b.dtype, seed=seed + bi)
        if b.S:
            wl.inject_specials([row], [b.dtype], seed=seed)
        for rank in sorted({0, W - 1, int(rng.integers(0, W))}):
            got = oracle.rs_copy_out(pl, bi, rank, row, d)
            t = _to_torch(row, b.dtype)
            if d != 1.0:
                t = t / torch.full_like(t, d)
            for k, i in enumerate(b.members):
                sdt = w.tensors[i].storage_dtype
                v = oracle.valid_in_chunk(w.tensors[i].numel, b.P[k], rank)
                want = _bits(t[b.O[k]: b.O[k] + v].to(TDT[sdt]), sdt)
                gb = got[k].view(BITS[sdt])
                assert gb.shape == want.shape
                nan = _is_nan_bits(want, sdt)
                assert np.array_equal(_is_nan_bits(gb, sdt), nan), (bi, rank, k)
                assert np.array_equal(gb[~nan], want[~nan]), (bi, rank, k, d)


@settings(max_examples=100, deadline=None)
@given(layouts)
def test_undivided_write_back_of_the_pack_is_the_cast_shard(layout):
    """Writing back row r of the pack (no reduction across ranks, no divide)
    gives rank r's chunk of cast(cast(g, reduce), storage)."""
    W, tensors, seed, _ = layout
    w = _workload(W, tensors, seed)
    pl = oracle.plan(w.descs(), W)
    grads = wl.make_grads(w)
    for bi, b in enumerate(pl.buckets):
        packed = oracle.pack(pl, bi, grads)
        for rank in range(W):
            got = oracle.rs_copy_out(pl, bi, rank, packed[rank], 1.0)
            for k, i in enumerate(b.members):
                sdt = w.tensors[i].storage_dtype
                full = _to_torch(grads[i], w.tensors[i].grad_dtype).to(TDT[b.dtype]).to(TDT[sdt])
                P = b.P[k]
                v = oracle.valid_in_chunk(w.tensors[i].numel, P, rank)
                want = _bits(full[rank * P: rank * P + v], sdt)
                assert np.array_equal(got[k].view(BITS[sdt]), want)


@pytest.mark.parametrize("W", [2, 4, 8, 128])
@pytest.mark.parametrize("reduce_dt", [BF16, FP32])
def test_dividing_w_summed_rows_by_power_of_two_w_is_exact(W, reduce_dt):
    """A reduce-scatter of W identical rows sums to W * row exactly (power of
    two W, no overflow); dividing by W gives the row back, bit for bit."""
    shapes = [(W * 3 + 1, 5), (7,), (W,), (1,)]
    w = wl.custom(shapes, [BF16, FP32, BF16, FP32], [reduce_dt] * 4, W, seed=W,
                  storage_dtypes=[FP32, BF16, FP32, BF16])
    pl = oracle.plan(w.descs(), W)
    b = pl.buckets[0]
    row = wl.random_array(b.S, reduce_dt, seed=11)           # finite, far from overflow
    wide = oracle.convert(row, reduce_dt, FP32)
    summed = oracle.convert(wide * np.float32(W), FP32, reduce_dt)   # exact: a power-of-two scale
    for rank in (0, W - 1):
        plain = oracle.rs_copy_out(pl, 0, rank, row, 1.0)
        back = oracle.rs_copy_out(pl, 0, rank, summed, float(W))
        for a, c in zip(plain, back):
            assert np.array_equal(a.view(np.uint8), c.view(np.uint8))
        # and the divide is not a no-op
        undivided = oracle.rs_copy_out(pl, 0, rank, summed, 1.0)
        assert any(not np.array_equal(a.view(np.uint8), u.view(np.uint8)) for a, u in zip(plain, undivided)
                   if a.size)


def test_nan_rule_and_edge_rows():
    """NaNs are not divided (quiet bit set, sign and payload kept); ranks past
    a short parameter's end get nothing."""
    w = wl.custom([(3, 2), (9,)], [FP32, FP32], [FP32, FP32], 4, seed=3, storage_dtypes=[FP32, BF16])
    pl = oracle.plan(w.descs(), 4)
    b = pl.buckets[0]
    assert b.P == [2, 3] and b.S == 5
    row = np.array([1.0, -2.0, 3.0, 4.0, 5.0], np.float32)
    row.view(np.uint32)[1] = 0xFF800001          # signalling NaN, negative
    g = oracle.rs_copy_out(pl, 0, 0, row, 2.0)
    assert g[0].view(np.uint32)[0] == np.float32(0.5).view(np.uint32)
    assert g[0].view(np.uint32)[1] == 0xFFC00001                     # quieted, payload kept
    assert g[1].view(np.uint16).tolist() == [0x3FC0, 0x4000, 0x4020]  # 1.5, 2.0, 2.5 in bf16
    # rank 1: parameter 0 holds rows [2, 3) -> 1 row of 2; parameter 1 holds [3, 6)
    g = oracle.rs_copy_out(pl, 0, 1, row, 1.0)
    assert g[0].size == 2 and g[1].size == 3
    # rank 2 and 3: parameter 0 is exhausted (3 rows of 2 over chunks of 1 row)
    g = oracle.rs_copy_out(pl, 0, 3, row, 1.0)
    assert g[0].size == 0 and g[1].size == 0
