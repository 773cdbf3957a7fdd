"""Property pins of the oracle: a library routine that computes the same
layout (torch._chunk_cat on pre-cast inputs), special cases that reduce to a
concatenation or a reshape, and the size / round-trip identities."""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
import workloads as wl

torch = pytest.importorskip("torch")
BF16, FP32 = oracle.BF16, oracle.FP32


def _to_torch(a, dtype):
    t = torch.from_numpy(a.copy())
    return t.view(torch.bfloat16) if dtype == BF16 else t


def _from_torch(t, dtype):
    if dtype == BF16:
        return t.contiguous().view(torch.int16).numpy().view(np.uint16)
    return t.contiguous().numpy()


layouts = st.integers(min_value=1, max_value=9).flatmap(lambda W: st.tuples(
    st.just(W),
    st.lists(st.tuples(st.integers(1, 3 * W + 2),             # dim0 (>= 1: _chunk_cat rejects empty)
                       st.sampled_from([(), (1,), (3,), (2, 2), (5,)]),  # trailing dims
                       st.sampled_from([BF16, FP32]),           # grad dtype
                       st.sampled_from([0, BF16, FP32])),       # reduce dtype (0: unset)
             min_size=1, max_size=7),
    st.integers(0, 2**31 - 1)))


@settings(max_examples=150, deadline=None)
@given(layouts)
def test_pack_equals_chunk_cat_of_precast(layout):
    W, tensors, seed = layout
    shapes = [(d0,) + rest for d0, rest, _, _ in tensors]
    w = wl.custom(shapes, [g for _, _, g, _ in tensors], [r for _, _, _, r in tensors], W, seed)
    grads = wl.make_grads(w)
    pl = oracle.plan(w.descs(), W)
    for bi, b in enumerate(pl.buckets):
        pre = []
        for i in b.members:
            t = _to_torch(grads[i], w.tensors[i].grad_dtype).reshape(shapes[i])
            pre.append(t.to(torch.bfloat16 if b.dtype == BF16 else torch.float32))
        ref = _from_torch(torch._chunk_cat(pre, dim=0, num_chunks=W), b.dtype)
        got = oracle.pack(pl, bi, grads)
        assert got.shape == ref.shape == (W, b.S)
        assert np.array_equal(got.view(np.uint16 if b.dtype == BF16 else np.uint32),
                              ref.view(np.uint16 if b.dtype == BF16 else np.uint32))


@settings(max_examples=100, deadline=None)
@given(layouts)
def test_size_and_roundtrip_identities(layout):
    W, tensors, seed = layout
    shapes = [(d0,) + rest for d0, rest, _, _ in tensors]
    grad_dts = [g for _, _, g, _ in tensors]
    w = wl.custom(shapes, grad_dts, [r for _, _, _, r in tensors], W, seed,
                  storage_dtypes=[FP32 if (i % 3) else BF16 for i in range(len(shapes))])
    grads = wl.make_grads(w)
    pl = oracle.plan(w.descs(), W)
    assert sorted(i for b in pl.buckets for i in b.members) == list(range(len(shapes)))
    for bi, b in enumerate(pl.buckets):
        packed = oracle.pack(pl, bi, grads)
        numel = sum(w.tensors[i].numel for i in b.members)
        assert packed.size == W * b.S == W * sum(b.P)
        # padding count: everything past each tensor's numel is +0 bits
        flatbits = packed.view(np.uint16 if b.dtype == BF16 else np.uint32)
        assert W * b.S - numel >= 0
        assert np.count_nonzero(flatbits) <= numel
        # unpack(pack(g)) == cast(g)
        back = oracle.unpack(pl, bi, packed)
        for i, g in zip(b.members, back):
            want = oracle.convert(grads[i], w.tensors[i].grad_dtype, b.dtype)
            assert np.array_equal(g.view(np.uint8), want.view(np.uint8))
    # copy-out(all-gather(copy-in(shards))) == cast(full params), storage -> param dtype
    params = wl.make_params(w)
    ag = np.full((W, pl.B), 0xAB, np.uint8)        # poisoned: copy-in must write every byte
    for r in range(W):
        oracle.copy_in(pl, r, [oracle.shard(pl, i, params[i], r) for i in range(len(params))], ag)
    full = oracle.copy_out(pl, ag)
    for i, t in enumerate(w.tensors):
        want = oracle.convert(params[i], t.storage_dtype, t.param_dtype)
        assert np.array_equal(full[i].view(np.uint8), want.view(np.uint8))
    # gap bytes between segments are zero
    used = np.zeros(pl.B, bool)
    for i, t in enumerate(w.tensors):
        used[pl.A[i]: pl.A[i] + pl.P[i] * oracle.ELEM_SIZE[t.param_dtype]] = True
    assert np.all(ag[:, ~used] == 0)
    assert all(a % 16 == 0 for a in pl.A) and pl.B % 16 == 0


@settings(max_examples=60, deadline=None)
@given(st.lists(st.tuples(st.integers(0, 40), st.integers(1, 4)), min_size=1, max_size=6),
       st.integers(0, 1000))
def test_world1_is_concatenation(shapes, seed):
    w = wl.custom(shapes, [FP32 if s[0] % 2 else BF16 for s in shapes], [FP32] * len(shapes), 1, seed)
    grads = wl.make_grads(w)
    pl = oracle.plan(w.descs(), 1)
    packed = oracle.pack(pl, 0, grads)
    cat = np.concatenate([oracle.convert(g, t.grad_dtype, FP32) for g, t in zip(grads, w.tensors)])
    assert np.array_equal(packed.reshape(-1).view(np.uint32), cat.view(np.uint32))


@settings(max_examples=60, deadline=None)
@given(st.integers(1, 8), st.integers(1, 5), st.integers(1, 6), st.integers(0, 1000))
def test_divisible_dim0_is_reshape(W, rows_per_rank, inner, seed):
    dim0 = W * rows_per_rank
    w = wl.custom([(dim0, inner)], [FP32], [BF16], W, seed)
    g = wl.make_grads(w)[0]
    pl = oracle.plan(w.descs(), W)
    packed = oracle.pack(pl, 0, [g])
    want = torch.from_numpy(g.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(packed, want.reshape(W, -1))
