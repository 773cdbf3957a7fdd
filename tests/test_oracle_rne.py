"""Brute-force pins of the oracle's dtype conversions against torch's CPU casts.

float32 -> bfloat16: all 2**32 bit patterns.  Non-NaN results must equal
torch's round-to-nearest-even cast bit for bit.  torch maps every NaN to one
pattern, so NaN inputs are checked for the properties the reading fixes: the
result is a quiet NaN of the same sign.  bfloat16 -> float32: all 2**16
patterns, exact.
"""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import oracle

torch = pytest.importorskip("torch")

CHUNK = 1 << 26


def _check_chunk(start):
    u = np.arange(start, start + CHUNK, dtype=np.uint64).astype(np.uint32)
    mine = oracle.convert(u.view(np.float32), oracle.FP32, oracle.BF16)
    ref = torch.from_numpy(u.view(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    exp_bits = (u >> 23) & 0xFF
    nan = (exp_bits == 0xFF) & ((u & 0x7FFFFF) != 0)
    bad = np.flatnonzero((mine != ref) & ~nan)
    if bad.size:
        return f"first mismatch at {int(u[bad[0]]):#010x}: {int(mine[bad[0]]):#06x} vs {int(ref[bad[0]]):#06x}"
    m = mine[nan]
    if not (np.all((m & 0x7F80) == 0x7F80) and np.all((m & 0x7F) != 0) and np.all(m & 0x40)
            and np.array_equal(m >> 15, (u[nan] >> 31).astype(np.uint16))):
        return f"NaN rule broken in chunk {start:#x}"
    return None


def test_f32_to_bf16_all_patterns_vs_torch():
    torch.set_num_threads(2)
    starts = list(range(0, 1 << 32, CHUNK))
    with ThreadPoolExecutor(max_workers=4) as ex:
        errors = [e for e in ex.map(_check_chunk, starts) if e]
    assert not errors, errors[:3]


def test_bf16_to_f32_all_patterns_vs_torch():
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    mine = oracle.convert(h, oracle.BF16, oracle.FP32).view(np.uint32)
    ref = torch.from_numpy(h.view(np.int16)).view(torch.bfloat16).to(torch.float32).numpy().view(np.uint32)
    nan = ((h & 0x7F80) == 0x7F80) & ((h & 0x7F) != 0)
    assert np.array_equal(mine[~nan], ref[~nan])
    # widening is exact for NaNs too: the payload bits are kept
    assert np.array_equal(mine, h.astype(np.uint32) << 16)


def test_same_dtype_conversion_is_a_bit_copy():
    u = np.random.default_rng(0).integers(0, 1 << 32, size=4096, dtype=np.uint64).astype(np.uint32)
    assert np.array_equal(oracle.convert(u.view(np.float32), oracle.FP32, oracle.FP32).view(np.uint32), u)
    h = (u >> 7).astype(np.uint16)
    assert np.array_equal(oracle.convert(h, oracle.BF16, oracle.BF16), h)
