"""The Python binding's argument checks, on the host (no GPU needed).

The binding only marshals tensors into pointers; these checks run before
any GPU call, so a wrong tensor fails loudly instead of reaching a kernel.
"""
import pytest

torch = pytest.importorskip("torch")
fp = pytest.importorskip("fsdp2_mixed_dtype_amd")
BF16, FP32 = fp.BF16, fp.FP32

TINY = [(6, 6, FP32, FP32, FP32, BF16), (6, 6, BF16, FP32, BF16, BF16), (6, 1, FP32, FP32, FP32, BF16)]


@pytest.fixture
def plan():
    p = fp.plan_buckets(TINY, 4)
    yield p
    p.destroy()


def test_host_tensors_are_rejected(plan):
    grads = [torch.zeros(36), torch.zeros(36, dtype=torch.bfloat16), torch.zeros(6)]
    with pytest.raises(ValueError, match="GPU"):
        fp.pack_reduce_scatter_input(plan, 0, grads, torch.zeros(4 * plan.buckets[0].S))
    with pytest.raises(ValueError, match="GPU"):
        fp.prepare_grads(plan, grads)


def test_list_lengths_are_checked(plan):
    with pytest.raises(ValueError, match="expected 3 entries"):
        fp.pack_reduce_scatter_input(plan, 0, [None, None], None)
    with pytest.raises(ValueError, match="expected 3 entries"):
        fp.prepare_shards(plan, [None])
    with pytest.raises(ValueError, match="expected 3 entries"):
        fp.prepare_shard_grads(plan, 0, 1, [None] * 4)


def test_flat_plans_need_the_rank_for_shards():
    p = fp.plan_buckets_flat([(6, 6, FP32, FP32, FP32, BF16), (6, 1, FP32, FP32, FP32, BF16)], 4)
    assert p.flat and p.c == 11
    with pytest.raises(ValueError, match="rank"):
        fp.prepare_shards(p, [None, None])
    # N = 42, c = 11: rank 3 holds flat positions [33, 44), i.e. the last 3
    # elements of the first parameter and all 6 of the second (2 padding slots)
    assert [fp.valid_in_chunk(p, i, 3) for i in range(2)] == [3, 6]
    assert [fp.valid_in_chunk(p, 0, r) for r in range(4)] == [11, 11, 11, 3]
    p.destroy()


def test_prepared_arrays_are_tied_to_plan_bucket_and_rank(plan):
    empty = fp.prepare_shard_grads(plan, 0, 3, [None, None, None])     # rank 3 holds no real element
    with pytest.raises(ValueError, match="another plan, bucket or rank"):
        fp.reduce_scatter_copy_out(plan, 0, 2, None, empty)
    other = fp.plan_buckets(TINY, 4)
    with pytest.raises(ValueError, match="another plan"):
        fp.reduce_scatter_copy_out(other, 0, 3, None, empty)
    other.destroy()


def test_destroyed_plan_raises(plan):
    p = fp.plan_buckets(TINY, 2)
    p.destroy()
    with pytest.raises(fp.FsdpPackError):
        _ = p.handle
