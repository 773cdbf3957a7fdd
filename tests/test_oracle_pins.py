"""Pins of the CPU oracle to values the pages print and to closed forms.

Every check here compares the oracle with something other than itself: the
pages' printed worked examples (tests/golden, each with its citation), the
sizes they quote, or closed-form layouts worked out by hand.
"""
import math

import numpy as np
import pytest

import oracle
import workloads as wl
from conftest import golden

BF16, FP32 = oracle.BF16, oracle.FP32


def _linear4x4_model():
    torch = pytest.importorskip("torch")
    torch.manual_seed(0)
    nn = torch.nn
    return torch, nn.Sequential(nn.Linear(4, 4, bias=False), nn.ReLU(), nn.Linear(4, 4, bias=False))


def test_linear4x4_rank0_shard_is_first_eight_row_major():
    # "The unit you wrapped": Linear(4,4), W=2 -> rank 0 holds rows 0-1.
    g = golden("linear4x4_w2.txt")
    torch, model = _linear4x4_model()
    w = model[0].weight.detach().numpy().astype(np.float32)
    printed0 = np.array([float(v) for v in g["rank0_shard"]])
    # the seeded weights are the printed ones (printed to 10 decimals)
    assert np.allclose(w.reshape(-1)[:8], printed0, rtol=0, atol=5.1e-11)
    assert np.allclose(w[0], [float(v) for v in g["full_row0"]], rtol=0, atol=5.1e-11)
    pl = oracle.plan([(4, 4, FP32, 0, FP32, FP32)], int(g["world"][0]))
    assert pl.P == [8] and pl.buckets[0].S == 8
    packed = oracle.pack(pl, 0, [w.reshape(-1)])
    assert packed.shape == (2, 8)
    assert np.allclose(packed[0], printed0, rtol=0, atol=5.1e-11)
    # rank 1 holds the second 8 values, rows 2-3
    assert np.array_equal(packed[1], w.reshape(-1)[8:])


def test_linear4x4_grad_shard_printout():
    # the printed per-rank gradient shards after one backward
    g = golden("linear4x4_w2.txt")
    torch, model = _linear4x4_model()
    model(torch.full((2, 4), 1.0)).sum().backward()
    grad = model[0].weight.grad.detach().numpy().astype(np.float32)
    pl = oracle.plan([(4, 4, FP32, FP32, FP32, FP32)], 2)
    packed = oracle.pack(pl, 0, [grad.reshape(-1)])
    assert np.allclose(packed[0], [float(v) for v in g["rank0_grad_shard"]], rtol=0, atol=5.1e-11)
    assert np.array_equal(packed[1], np.array([float(v) for v in g["rank1_grad_shard"]], np.float32))


def _six_by_six_units(policy):
    lin = (6, 6)
    names = ["b0.a", "b0.b", "b1.a", "b1.b"]
    if policy == "no_policy":
        return [names]
    if policy == "per_block":
        return [names[:2], names[2:]]
    return [[n] for n in names]


@pytest.mark.parametrize("policy", ["no_policy", "per_block", "per_linear"])
def test_flat_sizes_144_params_world4(policy):
    # FSDP1 reading: each unit is one flat 1-D parameter -> the page's 36/18/9.
    g = golden("flat_sizes_144.txt")
    units_expected, shard_expected = int(g[policy][0]), int(g[policy][1])
    units = _six_by_six_units(policy)
    assert len(units) == units_expected
    for unit in units:
        flat_numel = 36 * len(unit)
        pl = oracle.plan([(flat_numel, 1, FP32, 0, FP32, FP32)], 4)
        assert pl.buckets[0].S == shard_expected
    # FSDP2 reading (per-parameter dim-0 sharding): Linear(6,6) on W=4 gives
    # ceil(6/4)=2 rows of 6 -> 12 per parameter per rank.
    for unit in units:
        pl = oracle.plan([(6, 6, FP32, 0, FP32, FP32)] * len(unit), 4)
        assert pl.buckets[0].S == 12 * len(unit)
        assert pl.buckets[0].S == {"no_policy": 48, "per_block": 24, "per_linear": 12}[policy]


@pytest.mark.parametrize("flat", [True, False])
def test_linear3x3_world4_padding(flat):
    g = golden("linear3x3_w4.txt")
    W, numel = int(g["world"][0]), int(g["numel"][0])
    desc = (numel, 1, FP32, 0, FP32, FP32) if flat else (3, 3, FP32, 0, FP32, FP32)
    pl = oracle.plan([desc], W)
    assert pl.buckets[0].S == int(g["shard"][0])
    x = np.arange(1, numel + 1, dtype=np.float32)
    packed = oracle.pack(pl, 0, [x])
    assert packed.size == W * int(g["shard"][0])
    assert packed.size - numel == int(g["padding"][0])
    assert np.array_equal(packed.reshape(-1)[:numel], x)
    assert np.all(packed[3] == 0)          # the last rank holds only padding


def test_tiny_layout_closed_form():
    w = wl.tiny()
    pl = oracle.plan(w.descs(), w.world)
    assert len(pl.buckets) == 1 and pl.buckets[0].dtype == FP32
    b = pl.buckets[0]
    assert b.P == [12, 12, 12, 12, 2] and b.O == [0, 12, 24, 36, 48] and b.S == 50
    grads = wl.make_grads(w)
    packed = oracle.pack(pl, 0, grads)
    assert packed.shape == (4, 50)
    assert np.count_nonzero(packed) == 150          # every draw is nonzero
    assert np.all(packed[3] == 0)                   # ceil(6/4)=2 rows -> rank 3 empty
    assert np.array_equal(packed[2, 48:50], grads[4][4:6])
    # bf16 block1.lin0 widens exactly: bits << 16
    bf = grads[2].reshape(6, 6)
    assert np.array_equal(packed[1, 24:36].view(np.uint32), (bf[2:4].reshape(-1).astype(np.uint32) << 16))
    # copy-in to bf16: 12,12,12,12,2 bf16 -> 24-byte segments at 16-byte aligned offsets
    assert pl.A == [0, 32, 64, 96, 128] and pl.B == 144


def test_pack_zero_and_scalar_tensors():
    # dim0 = 0 contributes nothing; a 0-d tensor is one element held by rank 0
    pl = oracle.plan([(0, 5, FP32, 0, FP32, FP32), (1, 1, FP32, 0, FP32, FP32),
                      (5, 1, FP32, 0, FP32, FP32)], 3)
    b = pl.buckets[0]
    assert b.P == [0, 1, 2] and b.S == 3
    packed = oracle.pack(pl, 0, [np.zeros(0, np.float32), np.array([7.0], np.float32),
                                  np.array([1, 2, 3, 4, 5], np.float32)])
    assert packed.tolist() == [[7, 1, 2], [0, 3, 4], [0, 5, 0]]


def test_isolated_test_sizes():
    g = golden("workload_counts.txt")
    w = wl.mixed50m()
    total = sum(t.numel for t in w.tensors)
    bf16 = sum(t.numel for t in w.tensors if t.grad_dtype == BF16)
    assert total == 50_339_840
    assert round(total / 1e6, 1) == float(g["isolated_elements_millions"][0])
    # the pre-cast path materialises every bf16 grad as fp32: 4 bytes each
    assert bf16 * 4 / 2**20 == pytest.approx(float(g["avoided_fp32_mib"][0]), abs=0.5)
    assert bf16 * 4 == 192 * 2**20
    k = wl.kda_block()
    blocks = int(g["kda_blocks"][0])
    per_block = sum(t.numel for t in k.tensors)
    assert per_block == 218_132_512
    assert round(blocks * per_block / 1e9, 2) == float(g["kda_params_billions"][0])
    l5 = wl.layout500()
    assert abs(len(l5.tensors) - int(g["layout_params_roughly"][0])) <= 60


def test_bucket_per_effective_reduce_dtype():
    # one bucket per effective reduction dtype; unset reduce dtype -> grad dtype
    descs = [(4, 2, BF16, 0, FP32, BF16), (3, 1, FP32, 0, FP32, FP32),
             (2, 2, BF16, FP32, FP32, BF16), (5, 1, FP32, BF16, FP32, FP32)]
    pl = oracle.plan(descs, 2)
    assert [b.dtype for b in pl.buckets] == [BF16, FP32]
    assert pl.buckets[0].members == [0, 3] and pl.buckets[1].members == [1, 2]
    same = oracle.plan([(4, 2, BF16, FP32, FP32, BF16), (3, 1, FP32, 0, FP32, FP32)], 2)
    assert len(same.buckets) == 1


def test_conversion_spot_values():
    # hand-worked RNE cases (binary32 -> bfloat16)
    cases = {
        0x3F800000: 0x3F80,   # 1.0 exact
        0x3F808000: 0x3F80,   # tie, kept part even -> stays
        0x3F818000: 0x3F82,   # tie, kept part odd -> rounds up to even
        0x3F808001: 0x3F81,   # just above the tie -> up
        0x3F807FFF: 0x3F80,   # just below -> down
        0x7F7FFFFF: 0x7F80,   # largest finite rounds to +inf
        0xFF7FFFFF: 0xFF80,   # ... and to -inf
        0x7F800000: 0x7F80,   # +inf stays
        0x00000001: 0x0000,   # smallest subnormal rounds to +0 (no flush, just small)
        0x00008000: 0x0000,   # subnormal tie, even -> down
        0x00018000: 0x0002,   # subnormal tie, odd -> up
        0x007FFFFF: 0x0080,   # largest subnormal rounds up into the normal range
        0x80000000: 0x8000,   # -0 keeps its sign
    }
    for u, h in cases.items():
        assert oracle.f32_to_bf16_bits(u) == h, hex(u)
    for u in (0x7FC00000, 0xFFC00000, 0x7F800001, 0xFF800001, 0x7FA5A5A5):
        h = oracle.f32_to_bf16_bits(u)
        assert (h & 0x7F80) == 0x7F80 and (h & 0x7F) != 0      # still NaN
        assert (h >> 15) == (u >> 31)                           # same sign
        assert h & 0x40                                        # quiet
    assert oracle.bf16_to_f32_bits(0x3F80) == 0x3F800000
    assert math.isinf(np.array([oracle.bf16_to_f32_bits(0xFF80)], np.uint32).view(np.float32)[0])
