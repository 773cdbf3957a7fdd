"""Pins of the oracle's FSDP1 flat-parameter layout (plan_flat and the *_flat
element loops).

"The unit you wrapped" (kernels.rudrite.com) prints FSDP1 numbers: each
unit's parameters are flattened and concatenated into one 1-D flat
parameter, padded so it splits evenly over the world, one contiguous piece
per rank.  Pinned by the page's printed sizes (36/18/9 for two blocks of two
Linear(6,6) on a world of 4; 3 per rank and 3 padding slots for Linear(3,3)
on 4), by torch's concatenate-pad-split of the cast gradients, by the
per-parameter pieces putting the rank's shard back together, and by the
gather round trip.
"""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
import workloads as wl
from conftest import golden

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


def _is_nan(b, dtype):
    if dtype == BF16:
        return ((b & 0x7F80) == 0x7F80) & ((b & 0x007F) != 0)
    return ((b & 0x7F800000) == 0x7F800000) & ((b & 0x007FFFFF) != 0)


@pytest.mark.parametrize("policy", ["no_policy", "per_block", "per_linear"])
def test_printed_flat_shard_sizes(policy):
    """Two blocks of two Linear(6,6,bias=False), world 4: 36 / 18 / 9 per rank."""
    g = golden("flat_sizes_144.txt")
    units, per_rank = int(g[policy][0]), int(g[policy][1])
    lin = (6, 6, FP32, 0, FP32, FP32)
    layers = {"no_policy": [4], "per_block": [2, 2], "per_linear": [1, 1, 1, 1]}[policy]
    assert len(layers) == units
    for k in layers:
        fp = oracle.plan_flat([lin] * k, 4)
        assert fp.N == 36 * k and fp.c == per_rank


def test_linear3x3_world4_padding():
    """9 parameters on a world of 4: a shard of 3 per rank, 12 slots, 3 of
    them padding (all of rank 3's)."""
    fp = oracle.plan_flat([(3, 3, FP32, 0, FP32, FP32)], 4)
    assert fp.c == 3 and fp.W * fp.c == 12 and fp.W * fp.c - fp.N == 3
    g = np.arange(1, 10, dtype=np.float32)
    packed = oracle.pack_flat(fp, [g])
    assert packed.shape == (4, 3)
    assert np.array_equal(packed[:3].reshape(-1), g)
    assert np.array_equal(packed[3].view(np.uint32), np.zeros(3, np.uint32))
    assert [oracle.piece_len(fp, 0, r) for r in range(4)] == [3, 3, 3, 0]


layouts = st.integers(min_value=1, max_value=9).flatmap(lambda W: st.tuples(
    st.just(W),
    st.lists(st.tuples(st.integers(0, 3 * W + 2),
                       st.sampled_from([(), (1,), (3,), (2, 2), (5,)]),
                       st.sampled_from([BF16, FP32]),            # grad dtype
                       st.sampled_from([BF16, FP32])),           # storage dtype
             min_size=1, max_size=7),
    st.sampled_from([BF16, FP32]),                               # the unit's reduction dtype
    st.sampled_from([BF16, FP32]),                               # the unit's param dtype
    st.integers(0, 2**31 - 1)))


def _flat_workload(layout):
    W, tensors, rdt, pdt, seed = layout
    shapes = [(d0,) + rest for d0, rest, _, _ in tensors]
    w = wl.custom(shapes, [g for _, _, g, _ in tensors], [rdt] * len(shapes), W, seed,
                  storage_dtypes=[s for _, _, _, s in tensors], param_dtypes=[pdt] * len(shapes))
    return w, oracle.plan_flat(w.descs(), W)


@settings(max_examples=150, deadline=None)
@given(layouts)
def test_pack_flat_is_torch_concat_pad_split(layout):
    w, fp = _flat_workload(layout)
    grads = wl.make_grads(w)
    wl.inject_specials(grads, [t.grad_dtype for t in w.tensors], seed=3)
    cat = torch.cat([_to_torch(g, t.grad_dtype).reshape(-1).to(TDT[fp.dtype]) for g, t in zip(grads, w.tensors)])
    ref = torch.nn.functional.pad(cat, (0, fp.W * fp.c - cat.numel())).view(fp.W, fp.c)
    got = oracle.pack_flat(fp, grads).view(BITS[fp.dtype]).reshape(-1)
    want = _bits(ref, fp.dtype).reshape(-1)
    # torch's CPU cast turns every NaN into 0xFFFF; the oracle keeps sign and payload (reading R7)
    nan = _is_nan(want, fp.dtype)
    assert np.array_equal(_is_nan(got, fp.dtype), nan)
    assert np.array_equal(got[~nan], want[~nan])


@settings(max_examples=120, deadline=None)
@given(layouts, st.sampled_from([1.0, 2.0, 3.0, 6.0, 0.375]))
def test_rs_copy_out_flat_pieces(layout, d):
    """Each parameter's piece is torch's divide-then-cast of its slice of the
    rank's row; with no divide and storage = reduction dtype, the pieces put
    together in unit order are the row's real part."""
    w, fp = _flat_workload(layout)
    row_all = wl.random_array(fp.W * fp.c, fp.dtype, seed=fp.N + 1)
    wl.inject_specials([row_all], [fp.dtype], seed=2)
    rows = row_all.reshape(fp.W, fp.c) if fp.c else row_all.reshape(fp.W, 0)
    for r in range(fp.W):
        got = oracle.rs_copy_out_flat(fp, r, rows[r].copy(), d)
        t_row = _to_torch(rows[r], fp.dtype)
        if d != 1.0:
            t_row = t_row / torch.full_like(t_row, d)
        for i, p in enumerate(fp.params):
            lo, hi = oracle.flat_piece(fp, i, r)
            n = max(0, hi - lo)
            want = _bits(t_row[lo - r * fp.c: lo - r * fp.c + n].to(TDT[p.storage_dtype]), p.storage_dtype)
            gb = got[i].view(BITS[p.storage_dtype])
            assert gb.size == n
            nan = _is_nan(want, p.storage_dtype)
            assert np.array_equal(_is_nan(gb, p.storage_dtype), nan)
            assert np.array_equal(gb[~nan], want[~nan])
        if d == 1.0 and all(p.storage_dtype == fp.dtype for p in fp.params):
            joined = np.concatenate([x.view(BITS[fp.dtype]) for x in got]) if got else np.zeros(0, BITS[fp.dtype])
            real = max(0, min(fp.c, fp.N - r * fp.c))
            assert np.array_equal(joined, rows[r].view(BITS[fp.dtype])[:real])


@settings(max_examples=120, deadline=None)
@given(layouts)
def test_flat_gather_round_trip(layout):
    """copy-out(concat over ranks of copy-in(pieces of X)) == cast(X, storage -> param)."""
    w, fp = _flat_workload(layout)
    params = wl.make_params(w)
    rows = []
    for r in range(fp.W):
        pieces = []
        for i, (p, x) in enumerate(zip(fp.params, params)):
            lo, hi = oracle.flat_piece(fp, i, r)
            pieces.append(x[max(0, lo - fp.F[i]): max(0, hi - fp.F[i])].copy() if hi > lo
                          else np.zeros(0, x.dtype))
        row = oracle.copy_in_flat(fp, r, pieces)
        real = max(0, min(fp.c, fp.N - r * fp.c))
        assert not np.any(row.view(BITS[fp.param_dtype])[real:])          # padding is +0
        rows.append(row)
    flat = np.concatenate(rows) if rows else np.zeros(0, oracle.NP_DTYPE[fp.param_dtype])
    back = oracle.copy_out_flat(fp, flat)
    for x, p, b in zip(params, fp.params, back):
        assert np.array_equal(b.view(np.uint8), oracle.convert(x, p.storage_dtype, fp.param_dtype).view(np.uint8))


def test_plan_flat_rejects_mixed_unit_dtypes():
    with pytest.raises(ValueError):
        oracle.plan_flat([(2, 2, BF16, 0, FP32, BF16), (2, 2, FP32, 0, FP32, BF16)], 2)   # two reduction dtypes
    with pytest.raises(ValueError):
        oracle.plan_flat([(2, 2, FP32, 0, FP32, BF16), (2, 2, FP32, 0, FP32, FP32)], 2)   # two param dtypes
