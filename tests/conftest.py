import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU case")


def golden(name):
    """Parse a tests/golden fixture: '#' comments, then 'key v1 v2 ...' lines."""
    rows = {}
    with open(os.path.join(ROOT, "tests", "golden", name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            rows[key] = vals
    return rows


def direct_window_layout():
    """A W=4 layout whose pack windows mostly lie inside one rank chunk (the
    kernel's direct copy): bf16 and fp32 gradients into both reduction
    dtypes, bf16 rank chunks that start at odd elements (2 bytes past a
    dword), and small tensors between large ones (two members in one map
    stretch).  Returns (shapes, grad dtypes, reduce dtypes, W)."""
    BF16, FP32 = 1, 2
    shapes = [(4 * 3001, 1), (8, 5), (4 * 1537, 3), (3,), (4 * 4096, 2), (4 * 2049, 1), (5, 7), (4 * 1025, 8),
              (4 * 777, 11)]
    gdt = [BF16, BF16, FP32, FP32, BF16, FP32, BF16, BF16, BF16]
    rdt = [FP32, FP32, FP32, BF16, BF16, BF16, 0, FP32, BF16]
    return shapes, gdt, rdt, 4


def single_pair_layouts():
    """The shapes of direct_window_layout with every gradient in one dtype and
    every reduction in one dtype, once per (gradient, reduction) dtype pair:
    each is one bucket whose direct windows all have that pair.  Returns a
    list of (shapes, grad dtypes, reduce dtypes, W, pair)."""
    BF16, FP32 = 1, 2
    shapes, _, _, W = direct_window_layout()
    return [(shapes, [g] * len(shapes), [r] * len(shapes), W, g * 4 + r)
            for g, r in ((BF16, FP32), (FP32, FP32), (FP32, BF16), (BF16, BF16))]


def gathered_copy_out_layout():
    """Layouts whose copy-out windows span many small rank chunks (the
    kernel's element-by-element gather): parameters with fewer rows than
    ranks or a handful of rows per rank, in bf16 and fp32, next to ordinary
    ones.  Returns a list of (shapes, param dtypes, W)."""
    BF16, FP32 = 1, 2
    return [
        ([(100, 1), (16 * 188 - 5, 1), (40, 3), (17, 7), (3001, 1), (33, 5), (16 * 64, 64), (7,)],
         [BF16, FP32, BF16, FP32, BF16, FP32, BF16, FP32], 16),
        ([(5000, 1), (129, 1), (4999, 1), (1, 1), (300, 3), (1000, 64)],
         [BF16, FP32, FP32, BF16, BF16, FP32], 128),
        ([(2000, 1), (513, 2), (64, 9)], [FP32, BF16, BF16], 3),
    ]


def small_segment_copy_in_layout():
    """A W=4 layout of 40 small parameters (1-12 rows of 1-9 columns) whose
    all-gather segments are a few vectors long (most of them shorter than a
    window, many with a zero gap), so that nearly every copy-in window is a
    short range at both ends of a segment; storage -> param dtypes cycle
    through all four pairs.  Returns (shapes, storage dtypes, param dtypes,
    W)."""
    BF16, FP32 = 1, 2
    pairs = [(BF16, BF16), (FP32, BF16), (BF16, FP32), (FP32, FP32)]
    shapes = [(1 + (i * 7) % 12, 1 + (i * 5) % 9) for i in range(40)]
    return shapes, [pairs[i % 4][0] for i in range(40)], [pairs[i % 4][1] for i in range(40)], 4
