"""Mutation check of the oracle's pins (opt-in: FSDPPACK_MUTANTS=1; several
minutes, so it is not part of the default CPU run).

Each case plants one plausible mistake in a copy of the oracle -- a wrong
rounding rule, a dropped term, a wrong index or stride, a missing zero fill,
a divide skipped or inverted, a planner step changed -- and runs the pin
tests against it in a subprocess; the case passes when at least one pin
fails.  A mistake no pin catches would be a part of the oracle that is not
pinned to anything outside itself.  The mistakes are planted in the oracle
only, on the CPU; the library is not involved.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PINS = ["tests/test_oracle_pins.py", "tests/test_oracle_props.py", "tests/test_oracle_rne.py",
        "tests/test_oracle_rs_copy_out.py", "tests/test_oracle_flat.py"]

pytestmark = pytest.mark.skipif(os.environ.get("FSDPPACK_MUTANTS") != "1",
                                reason="opt-in mutation check (set FSDPPACK_MUTANTS=1)")

C_MUTANTS = {  # name: (text in oracle.c, the mistake planted in its place)
 'ties_up':       ('    else if (dropped == 0x8000u && (kept & 1u))\n        kept += 1u;', '    else if (dropped == 0x8000u)\n        kept += 1u;'),
 'truncate':      ('    if (dropped > 0x8000u)\n        kept += 1u;', '    if (0)\n        kept += 1u;'),
 'ties_down':     ('    else if (dropped == 0x8000u && (kept & 1u))\n        kept += 1u;', '    else if (0)\n        kept += 1u;'),
 'nan_not_quiet': ('return (uint16_t)(kept | 0x0040u);', 'return (uint16_t)(kept);'),
 'nan_as_number': ('if (exponent == 0xFFu && mantissa != 0u)', 'if (0)'),
 'widen_shift15': ('return ((uint32_t)h) << 16;', 'return ((uint32_t)h) << 15;'),
 'pad_nonzero':   ('                uint32_t bits = 0u;\n                if (s < numel[t])', '                uint32_t bits = 1u;\n                if (s < numel[t])'),
 'interleave':    ('                int64_t s = r * P[t] + j;', '                int64_t s = j * W + r;'),
 'drop_O':        ('store_as(out, dst_dtype, r * S + O[t] + j, bits);', 'store_as(out, dst_dtype, r * S + j, bits);'),
 'valid_short':   ('if (s < numel[t]) bits', 'if (s + 1 < numel[t]) bits'),
 'row_stride_P':  ('store_as(out, dst_dtype, r * S + O[t] + j, bits);', 'store_as(out, dst_dtype, r * P[t] + O[t] * W + j, bits);'),
 'unpack_index':  ('store_as(dst[t], dtype, r * P[t] + j,\n                         load_as(packed, dtype, r * S + O[t] + j, dtype));', 'store_as(dst[t], dtype, r * P[t] + j,\n                         load_as(packed, dtype, r * S + j, dtype));'),
 'copyin_no_zero':('    memset(row, 0, (size_t)B);\n', ''),
 'copyin_storage_stride': ('store_as(seg, param_dtype[t], j, load_as(shards[t], storage_dtype[t], j, param_dtype[t]));', 'store_as(seg, param_dtype[t], j, load_as(shards[t], storage_dtype[t], j, storage_dtype[t]));'),
 'copyout_rank0_only': ('        for (int64_t r = 0; r < W; ++r) {\n            const unsigned char *seg', '        for (int64_t r = 0; r < 1; ++r) {\n            const unsigned char *seg'),
 'same_dtype_convert': ('    return dst_dtype == ORACLE_FP32 ? f : (uint32_t)oracle_f32_to_bf16_bits(f);', '    return dst_dtype == ORACLE_FP32 ? f : (uint32_t)(f >> 16);'),
 # write-back (divide, then cast to storage)
 'wb_no_divide':   ('            if (divide_factor != 1.0f) x = divide_in(x, reduce_dtype, divide_factor);\n            store_as(grads[t], storage_dtype[t], j,', '            store_as(grads[t], storage_dtype[t], j,'),
 'wb_multiply':    ('        x = x / d;', '        x = x * d;'),
 'wb_nan_not_quieted': ('        f |= 0x00400000u;', '        f |= 0u;'),
 'wb_no_requant':  ('    return cast_bits(f, ORACLE_FP32, dtype);\n}', '    return dtype == ORACLE_BF16 ? (f >> 16) : f;\n}'),
 'wb_rank_offset': ('            uint32_t x = load_as(row, reduce_dtype, O[t] + j, reduce_dtype);', '            uint32_t x = load_as(row, reduce_dtype, rank * P[t] + j, reduce_dtype);'),
 'wb_valid_P':     ('        int64_t v = valid_in_chunk(numel[t], P[t], rank);\n        for (int64_t j = 0; j < v; ++j) {\n            uint32_t x = load_as(row, reduce_dtype, O[t] + j', '        int64_t v = P[t] < numel[t] ? P[t] : numel[t];\n        for (int64_t j = 0; j < v; ++j) {\n            uint32_t x = load_as(row, reduce_dtype, O[t] + j'),
 # FSDP1 flat layout
 'flat_pad_one':   ('    for (int64_t k = F; k < (int64_t)W * c; ++k) store_as(out, dst_dtype, k, 0u);', '    for (int64_t k = F; k < (int64_t)W * c; ++k) store_as(out, dst_dtype, k, 1u);'),
 'flat_no_F':      ('            store_as(out, dst_dtype, F + j, load_as(grads[t], grad_dtype[t], j, dst_dtype));', '            store_as(out, dst_dtype, j, load_as(grads[t], grad_dtype[t], j, dst_dtype));'),
 'flat_piece_hi':  ('    *hi = b < s1 ? b : s1;', '    *hi = b;'),
 'flat_wb_row':    ('            uint32_t x = load_as(row, reduce_dtype, f - (int64_t)rank * c, reduce_dtype);', '            uint32_t x = load_as(row, reduce_dtype, f - lo, reduce_dtype);'),
 'flat_ci_nozero': ('    for (int64_t k = 0; k < c; ++k) store_as(row, param_dtype, k, 0u);\n    int64_t F = 0;', '    int64_t F = 0;'),
 'flat_co_skipF':  ('            store_as(params[t], param_dtype, j, load_as(flat, param_dtype, F + j, param_dtype));\n        F += numel[t];', '            store_as(params[t], param_dtype, j, load_as(flat, param_dtype, F + j, param_dtype));\n        F += numel[t] + (t == 0);'),
}

PY_MUTANTS = ["floor_chunk", "no_round16", "bucket_by_grad", "O_not_cumulative", "last_bucket_first"]


def _pins_fail(env, pins):
    env = dict(env, PYTHONPATH=os.pathsep.join([os.path.join(ROOT, "tests"), ROOT, env.get("PYTHONPATH", "")]))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "oracle_mutant_plugin", *pins],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=1800)
    return r.returncode != 0


@pytest.mark.parametrize("name", sorted(C_MUTANTS))
def test_c_mistake_is_caught(name, tmp_path):
    with open(os.path.join(ROOT, "oracle", "oracle.c")) as f:
        src = f.read()
    before, after = C_MUTANTS[name]
    assert src.count(before) == 1, f"{name}: the text to mutate is not unique in oracle.c"
    c = tmp_path / f"{name}.c"
    so = tmp_path / f"{name}.so"
    c.write_text(src.replace(before, after))
    subprocess.check_call(["gcc", "-std=c99", "-O2", "-fPIC", "-shared", str(c), "-o", str(so)])
    assert _pins_fail(dict(os.environ, MUTANT_LIB=str(so)), PINS), f"no pin catches {name}"


@pytest.mark.parametrize("name", PY_MUTANTS)
def test_planner_mistake_is_caught(name):
    assert _pins_fail(dict(os.environ, MUTANT_PY=name), PINS[:2]), f"no pin catches {name}"
