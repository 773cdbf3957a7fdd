"""Seeded synthetic workloads for the mixed-dtype pack: layouts and values.

This module only describes shapes and draws random inputs.  It holds none of
the method's arithmetic (no chunking, padding, offsets or dtype rounding), so
both the CPU oracle's tests and the GPU path can use the very same inputs.

The five layouts are the ones the FSDP2 mixed-precision pages measure or
imply: a tiny two-block model, a roughly 500-parameter transformer layout, the
50.3M-element transformer-like layout of the isolated packing test, one block
of an eight-block 1.75B-parameter KDA-style model, and a heterogeneous
500-tensor layout with two reduction dtypes.  Gradients are drawn as float32
N(0, sigma) per tensor in unit order from ``numpy.random.default_rng(seed)``;
a bf16 tensor keeps the upper 16 bits of each float32 draw (a bit slice, not a
rounding).  No dataset or trained weight is involved.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

BF16 = 1
FP32 = 2
NONE = 0
NP_DTYPE = {BF16: np.uint16, FP32: np.float32}


@dataclass(frozen=True)
class Tensor:
    name: str
    shape: tuple
    grad_dtype: int       # dtype the gradient arrives in (the compute dtype)
    reduce_dtype: int     # policy reduce dtype, NONE when unset
    storage_dtype: int    # resident sharded parameter dtype
    param_dtype: int      # compute dtype delivered by the all-gather

    @property
    def dim0(self) -> int:
        return self.shape[0] if len(self.shape) else 1

    @property
    def inner(self) -> int:
        return int(np.prod(self.shape[1:], dtype=np.int64)) if len(self.shape) > 1 else 1

    @property
    def numel(self) -> int:
        return self.dim0 * self.inner


@dataclass(frozen=True)
class Workload:
    name: str
    tensors: tuple
    world: int
    seed: int
    grad_sigma: float
    param_sigma: float

    def descs(self):
        """(dim0, inner, grad, reduce, storage, param) per tensor, unit order."""
        return [(t.dim0, t.inner, t.grad_dtype, t.reduce_dtype, t.storage_dtype, t.param_dtype)
                for t in self.tensors]


# --------------------------------------------------------------------------- layouts

def tiny() -> Workload:
    """Two blocks of two Linear(6, 6) weights (block1.lin0 in bf16, the rest
    fp32) and one fp32 [6] norm; W=4; reduce dtype fp32; copy-in to bf16."""
    ts = []
    for b in range(2):
        for l in range(2):
            dt = BF16 if (b, l) == (1, 0) else FP32
            ts.append(Tensor(f"block{b}.lin{l}", (6, 6), dt, FP32, dt, BF16))
    ts.append(Tensor("norm", (6,), FP32, FP32, FP32, BF16))
    return Workload("tiny", tuple(ts), world=4, seed=1, grad_sigma=0.02, param_sigma=0.02)


def _block(prefix, d, ffn, with_gate, with_bias, bf16_store=FP32):
    mats = [("q", (d, d)), ("k", (d, d)), ("v", (d, d)), ("o", (d, d)), ("up", (ffn, d))]
    if with_gate:
        mats.append(("gate", (ffn, d)))
    mats.append(("down", (d, ffn)))
    ts = [Tensor(f"{prefix}.{n}", s, BF16, FP32, bf16_store, BF16) for n, s in mats]
    vecs = ["norm1", "norm2"] + (["bias1", "bias2"] if with_bias else [])
    ts += [Tensor(f"{prefix}.{n}", (d,), FP32, FP32, FP32, FP32) for n in vecs]
    return ts


def layout500() -> Workload:
    """40 transformer blocks (d=512, ffn=2048): q,k,v,o [512,512], up, gate
    [2048,512], down [512,2048] in bf16; two fp32 RMSNorm and two fp32 bias
    vectors [512] per block; five more model-level fp32 [512] vectors.
    445 tensors, W=8, fp32 reduce."""
    ts = []
    for b in range(40):
        ts += _block(f"layers.{b}", 512, 2048, with_gate=True, with_bias=True)
    ts += [Tensor(f"extra{i}", (512,), FP32, FP32, FP32, FP32) for i in range(5)]
    return Workload("layout500", tuple(ts), world=8, seed=2, grad_sigma=1e-3, param_sigma=0.02)


def mixed50m() -> Workload:
    """4 blocks (d=1024, ffn=4096): q,k,v,o [1024,1024], up [4096,1024], down
    [1024,4096] in bf16, two fp32 RMSNorm [1024] per block: 50,339,840
    elements, W=8, fp32 reduce (the isolated packing test's layout)."""
    ts = []
    for b in range(4):
        ts += _block(f"layers.{b}", 1024, 4096, with_gate=False, with_bias=False)
    return Workload("mixed50m", tuple(ts), world=8, seed=3, grad_sigma=1e-3, param_sigma=0.02)


def kda_block() -> Workload:
    """One block of an 8-block 1.75B KDA-style model: q,k,v,o [4096,4096],
    gate, up [12288,4096], down [4096,12288] in bf16; fp32 A_log [32],
    dt_bias [4096], conv [4096,4] and two RMSNorm [4096]; W=8, fp32 reduce;
    fp32 resident storage, bf16 compute for the matrices."""
    d, ffn = 4096, 12288
    mats = [("q", (d, d)), ("k", (d, d)), ("v", (d, d)), ("o", (d, d)),
            ("gate", (ffn, d)), ("up", (ffn, d)), ("down", (d, ffn))]
    ts = [Tensor(n, s, BF16, FP32, FP32, BF16) for n, s in mats]
    ts += [Tensor(n, s, FP32, FP32, FP32, FP32) for n, s in
           [("A_log", (32,)), ("dt_bias", (d,)), ("conv", (d, 4)), ("norm1", (d,)), ("norm2", (d,))]]
    return Workload("kda_block", tuple(ts), world=8, seed=4, grad_sigma=1e-3, param_sigma=0.02)


MASK64 = (1 << 64) - 1


def splitmix64(state: int):
    """SplitMix64 (Steele, Lea and Flood, 2014): yields 64-bit outputs."""
    while True:
        state = (state + 0x9E3779B97F4A7C15) & MASK64
        z = state
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
        yield z ^ (z >> 31)


def hetero500() -> Workload:
    """500 tensors [dim0, dim1]: dim0 uniform in [1, 5000], dim1 in
    {1, 64, 768}, gradient dtype bf16 or fp32 with equal odds, and exactly 350
    bf16-reduce / 150 fp32-reduce parameters in shuffled order; W=128, so many
    dim0 are not divisible by W and many rank chunks are pure padding."""
    rng = splitmix64(5)
    shapes, grads = [], []
    for _ in range(500):
        dim0 = 1 + next(rng) % 5000
        dim1 = (1, 64, 768)[next(rng) % 3]
        grads.append(BF16 if next(rng) % 2 == 0 else FP32)
        shapes.append((dim0, dim1))
    reduce = [BF16] * 350 + [FP32] * 150
    for i in range(499, 0, -1):
        j = next(rng) % (i + 1)
        reduce[i], reduce[j] = reduce[j], reduce[i]
    ts = tuple(Tensor(f"t{i}", shapes[i], grads[i], reduce[i], FP32, grads[i]) for i in range(500))
    return Workload("hetero500", ts, world=128, seed=5, grad_sigma=1e-3, param_sigma=0.02)


WORKLOADS = {"tiny": tiny, "layout500": layout500, "mixed50m": mixed50m,
             "kda_block": kda_block, "hetero500": hetero500}


def get(name: str) -> Workload:
    return WORKLOADS[name]()


def custom(shapes, grad_dtypes, reduce_dtypes, world, seed=0, storage_dtypes=None, param_dtypes=None,
           grad_sigma=1.0, param_sigma=1.0) -> Workload:
    """An ad-hoc layout (used by randomized parity cases)."""
    n = len(shapes)
    storage_dtypes = storage_dtypes or [FP32] * n
    param_dtypes = param_dtypes or list(grad_dtypes)
    ts = tuple(Tensor(f"p{i}", tuple(shapes[i]), grad_dtypes[i], reduce_dtypes[i], storage_dtypes[i],
                      param_dtypes[i]) for i in range(n))
    return Workload("custom", ts, world=world, seed=seed, grad_sigma=grad_sigma, param_sigma=param_sigma)


# --------------------------------------------------------------------------- values

def _draw(rng, count, sigma, dtype):
    x = rng.standard_normal(count, dtype=np.float32)
    x *= np.float32(sigma)
    if dtype == FP32:
        return x
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def make_grads(w: Workload, seed: int | None = None):
    """Flat gradient arrays in each tensor's grad dtype (bf16 as uint16 bits)."""
    rng = np.random.default_rng(w.seed if seed is None else seed)
    return [_draw(rng, t.numel, w.grad_sigma, t.grad_dtype) for t in w.tensors]


def make_params(w: Workload, seed: int | None = None):
    """Flat full parameters in each tensor's storage dtype."""
    rng = np.random.default_rng((w.seed if seed is None else seed) + 1_000_003)
    return [_draw(rng, t.numel, w.param_sigma, t.storage_dtype) for t in w.tensors]


def random_array(count: int, dtype: int, seed: int, sigma: float = 1.0):
    return _draw(np.random.default_rng(seed), count, sigma, dtype)


# fp32 bit patterns that exercise every branch of a float32 -> bfloat16 cast:
# signed zeros, infinities, quiet / signalling NaNs with payloads, subnormals,
# exact ties with even and odd kept parts, values one ulp either side of a
# tie, and the largest finite values (which round to infinity).
F32_SPECIALS = np.array([
    0x00000000, 0x80000000, 0x7F800000, 0xFF800000, 0x7FC00000, 0xFFC00000, 0x7F800001,
    0xFF800001, 0x7FBFFFFF, 0x7FFFFFFF, 0xFFFFFFFF, 0x7FA5A5A5, 0x00000001, 0x80000001,
    0x00007FFF, 0x00008000, 0x00018000, 0x007FFFFF, 0x807FFFFF, 0x00800000, 0x3F808000,
    0x3F818000, 0xBF808000, 0xBF818000, 0x3F807FFF, 0x3F808001, 0x3F817FFF, 0x3F818001,
    0x7F7FFFFF, 0xFF7FFFFF, 0x7F7F8000, 0x7F7F7FFF, 0x7F7E8000, 0x3F800000, 0x47FFFFFF,
], dtype=np.uint32)

# bf16 bit patterns of the same kinds (these pass through unchanged to bf16
# and widen exactly to fp32).
BF16_SPECIALS = np.array([
    0x0000, 0x8000, 0x7F80, 0xFF80, 0x7FC0, 0xFFC0, 0x7F81, 0xFF81, 0x7FFF, 0xFFFF,
    0x0001, 0x8001, 0x007F, 0x0080, 0x7F7F, 0xFF7F, 0x3F80, 0xBF80,
], dtype=np.uint16)


def inject_specials(arrays, dtypes, seed: int):
    """Overwrite a few positions of each array (its first and last elements
    and some random ones) with special bit patterns.  Modifies in place."""
    rng = np.random.default_rng(seed + 77)
    for a, dt in zip(arrays, dtypes):
        n = a.size
        if n == 0:
            continue
        pool = F32_SPECIALS if dt == FP32 else BF16_SPECIALS
        view = a.view(np.uint32) if dt == FP32 else a
        k = min(n, len(pool))
        view[:k] = pool[:k]
        tail = min(n, 3)
        view[n - tail:] = pool[-tail:]
        if n > 8:
            pos = rng.integers(0, n, size=min(n // 4, 16))
            view[pos] = pool[rng.integers(0, len(pool), size=pos.size)]
    return arrays
