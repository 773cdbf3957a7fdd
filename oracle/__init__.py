"""Plain CPU oracle for FSDP2's mixed-dtype reduce-scatter pack, the write-back
of a reduce-scatter output into sharded gradients, and the all-gather
copy-in / copy-out.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by ``__graft_entry__.smoke()``
and by the CPU-baseline leg of ``bench.py``.  The product package never imports
it, and this module imports nothing from the product package.

The planner below is written in plain Python from the pages' description; the
element loops live in ``oracle.c`` and are reached through ``ctypes``.

Sources (web pages on FSDP2 per-parameter mixed precision):
  * "PyTorch adds per-parameter mixed precision to FSDP2" (ainewsletter.today),
    paragraph 2: one reduction buffer per effective reduction dtype ("a bucket
    and reduce-scatter for each dtype"); paragraph 1: one all-gather per
    fully_shard unit.
  * "The unit you wrapped" (kernels.rudrite.com), padding paragraphs: every
    rank's shard has the padded size; padding sits on the right.
  * "Mixed-Precision Training" (NeMo AutoModel), table "Storage Dtype Compared
    to Compute Dtype": param_dtype / reduce_dtype.

Readings the pages leave open (each is also listed in the design notes):
  * chunking along dim 0 takes ceil(dim0 / W) rows per rank, trailing ranks
    short or empty (torch.chunk's rule);
  * an unset reduce dtype means the gradient's own dtype;
  * buckets are ordered by first appearance, parameters keep unit order;
  * the all-gather row puts each parameter's segment at a 16-byte aligned byte
    offset in unit order, gaps zero (parity unpinned beyond the round trip).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

BF16 = 1
FP32 = 2
ELEM_SIZE = {BF16: 2, FP32: 4}
NP_DTYPE = {BF16: np.uint16, FP32: np.float32}   # bf16 is held as its bit pattern

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with the host C compiler (-O2, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-std=c99", "-O2", "-fPIC", "-shared", "-Wall", "-Wextra",
                               os.path.join(_HERE, "oracle.c"), "-o", tmp])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        lib.oracle_f32_to_bf16_bits.argtypes = [ctypes.c_uint32]
        lib.oracle_f32_to_bf16_bits.restype = ctypes.c_uint16
        lib.oracle_bf16_to_f32_bits.argtypes = [ctypes.c_uint16]
        lib.oracle_bf16_to_f32_bits.restype = ctypes.c_uint32
        lib.oracle_pack.argtypes = [i32, i32, vp, vp, vp, vp, vp, i64, i32, vp]
        lib.oracle_unpack.argtypes = [i32, i32, vp, i32, i64, vp, vp, vp, vp]
        lib.oracle_copy_in.argtypes = [i32, i32, vp, vp, vp, vp, vp, i64, vp]
        lib.oracle_copy_out.argtypes = [i32, i32, vp, i64, vp, vp, vp, vp, vp]
        lib.oracle_convert.argtypes = [vp, i32, vp, i32, i64]
        lib.oracle_rs_copy_out.argtypes = [i32, i32, vp, i32, i64, ctypes.c_float, vp, vp, vp, vp, vp]
        lib.oracle_pack_flat.argtypes = [i32, i32, vp, vp, vp, i64, i32, vp]
        lib.oracle_rs_copy_out_flat.argtypes = [i32, i32, vp, i32, i64, ctypes.c_float, vp, vp, vp]
        lib.oracle_copy_in_flat.argtypes = [i32, i32, vp, vp, i32, vp, i64, vp]
        lib.oracle_copy_out_flat.argtypes = [i32, vp, i32, vp, vp]
        for f in (lib.oracle_pack, lib.oracle_unpack, lib.oracle_copy_in, lib.oracle_copy_out,
                  lib.oracle_rs_copy_out, lib.oracle_pack_flat, lib.oracle_rs_copy_out_flat,
                  lib.oracle_copy_in_flat, lib.oracle_copy_out_flat):
            f.restype = ctypes.c_int
        lib.oracle_convert.restype = None
        _lib = lib
    return _lib


# --------------------------------------------------------------------------- planning

@dataclass(frozen=True)
class ParamDesc:
    """One parameter of a fully_shard unit.

    dim0, inner: the tensor viewed as [dim0, inner] (inner = product of the
    trailing dims; a 0-d tensor is [1, 1]).  grad_dtype: dtype its gradient
    arrives in (the compute dtype).  reduce_dtype: the policy's reduce dtype,
    0 when unset.  storage_dtype: dtype of the resident sharded parameter.
    param_dtype: compute dtype the all-gather delivers.
    """
    dim0: int
    inner: int
    grad_dtype: int
    reduce_dtype: int
    storage_dtype: int
    param_dtype: int

    @property
    def numel(self) -> int:
        return self.dim0 * self.inner


@dataclass
class Bucket:
    dtype: int                 # the effective reduction dtype of every member
    members: list              # parameter indices, unit order
    P: list                    # padded rank-chunk size of each member (elements)
    O: list                    # column offset of each member in a row
    S: int                     # row length: sum of the members' P


@dataclass
class Plan:
    W: int
    params: list
    buckets: list = field(default_factory=list)
    P: list = field(default_factory=list)     # per parameter, unit order
    A: list = field(default_factory=list)     # all-gather byte offset per parameter
    B: int = 0                                # all-gather row bytes


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def _round16(x: int) -> int:
    return (x + 15) // 16 * 16


def plan(params, W: int) -> Plan:
    """Bucket a unit's parameters by effective reduction dtype and lay out the
    reduce-scatter rows and the all-gather row.

    Chunking along dim 0 gives rank r rows [r*c, (r+1)*c) of the parameter,
    c = ceil(dim0 / W); every chunk is padded on the right to P = c * inner
    elements, so each rank's piece has the same size.
    """
    if W < 1:
        raise ValueError("world size must be >= 1")
    params = [p if isinstance(p, ParamDesc) else ParamDesc(*p) for p in params]
    pl = Plan(W=W, params=params)
    for p in params:
        if p.dim0 < 0 or p.inner < 0:
            raise ValueError("negative dimension")
        pl.P.append(_ceil_div(p.dim0, W) * p.inner)
    effective = [p.reduce_dtype if p.reduce_dtype else p.grad_dtype for p in params]
    order = []
    for d in effective:
        if d not in order:
            order.append(d)
    for d in order:
        members = [i for i, e in enumerate(effective) if e == d]
        Ps = [pl.P[i] for i in members]
        Os, acc = [], 0
        for x in Ps:
            Os.append(acc)
            acc += x
        pl.buckets.append(Bucket(dtype=d, members=members, P=Ps, O=Os, S=acc))
    end = 0
    for i, p in enumerate(params):
        start = _round16(end) if i else 0
        pl.A.append(start)
        end = start + pl.P[i] * ELEM_SIZE[p.param_dtype]
    pl.B = _round16(end)
    return pl


def valid_in_chunk(numel: int, P: int, r: int) -> int:
    return max(0, min(P, numel - r * P))


# --------------------------------------------------------------------------- element loops

def _ptrs(arrays):
    return (ctypes.c_void_p * max(1, len(arrays)))(*[a.ctypes.data for a in arrays])


def _i64(xs):
    return np.ascontiguousarray(np.asarray(xs, dtype=np.int64))


def _i32(xs):
    return np.ascontiguousarray(np.asarray(xs, dtype=np.int32))


def _check(arr, dtype, count=None):
    if arr.dtype != NP_DTYPE[dtype] or not arr.flags.c_contiguous:
        raise TypeError(f"expected a contiguous {NP_DTYPE[dtype].__name__} array, got {arr.dtype}")
    if count is not None and arr.size != count:
        raise ValueError(f"expected {count} elements, got {arr.size}")


def pack(pl: Plan, bucket: int, grads) -> np.ndarray:
    """Reduce-scatter input [W, S] of bucket `bucket`; `grads` is the full list
    of the unit's gradients (unit order), each a flat array in its grad dtype."""
    b = pl.buckets[bucket]
    gs = [np.ascontiguousarray(grads[i]).reshape(-1) for i in b.members]
    for i, g in zip(b.members, gs):
        _check(g, pl.params[i].grad_dtype, pl.params[i].numel)
    out = np.empty((pl.W, b.S), dtype=NP_DTYPE[b.dtype])
    gdt = _i32([pl.params[i].grad_dtype for i in b.members])
    numel = _i64([pl.params[i].numel for i in b.members])
    P, O = _i64(b.P), _i64(b.O)
    rc = _load().oracle_pack(pl.W, len(gs), _ptrs(gs), gdt.ctypes.data, numel.ctypes.data,
                             P.ctypes.data, O.ctypes.data, b.S, b.dtype, out.ctypes.data)
    if rc:
        raise RuntimeError("oracle_pack: bad layout")
    return out


def unpack(pl: Plan, bucket: int, packed: np.ndarray):
    """Per-member flat arrays (in the bucket dtype) rebuilt from a packed [W, S]."""
    b = pl.buckets[bucket]
    packed = np.ascontiguousarray(packed)
    _check(packed, b.dtype, pl.W * b.S)
    outs = [np.zeros(pl.params[i].numel, dtype=NP_DTYPE[b.dtype]) for i in b.members]
    numel = _i64([pl.params[i].numel for i in b.members])
    P, O = _i64(b.P), _i64(b.O)
    _load().oracle_unpack(pl.W, len(outs), packed.ctypes.data, b.dtype, b.S, numel.ctypes.data,
                          P.ctypes.data, O.ctypes.data, _ptrs(outs))
    return outs


def copy_in(pl: Plan, rank: int, shards, ag: np.ndarray | None = None) -> np.ndarray:
    """Write row `rank` of the [W, B]-byte all-gather buffer from the rank's
    padded shards (P elements each, storage dtype).  Returns the buffer."""
    if ag is None:
        ag = np.zeros((pl.W, pl.B), dtype=np.uint8)
    shards = [np.ascontiguousarray(s).reshape(-1) for s in shards]
    for p, s, P in zip(pl.params, shards, pl.P):
        _check(s, p.storage_dtype, P)
    if ag.dtype != np.uint8 or ag.size != pl.W * pl.B or not ag.flags.c_contiguous:
        raise ValueError("all-gather buffer must be a contiguous uint8 [W, B] array")
    sdt = _i32([p.storage_dtype for p in pl.params])
    pdt = _i32([p.param_dtype for p in pl.params])
    P, A = _i64(pl.P), _i64(pl.A)
    rc = _load().oracle_copy_in(rank, len(shards), _ptrs(shards), sdt.ctypes.data, pdt.ctypes.data,
                                P.ctypes.data, A.ctypes.data, pl.B, ag.ctypes.data)
    if rc:
        raise RuntimeError("oracle_copy_in: bad layout")
    return ag


def copy_out(pl: Plan, ag: np.ndarray):
    """Full parameters (param dtype, flat) rebuilt from a gathered [W, B] buffer."""
    ag = np.ascontiguousarray(ag)
    if ag.dtype != np.uint8 or ag.size != pl.W * pl.B:
        raise ValueError("all-gather buffer must be a uint8 [W, B] array")
    outs = [np.zeros(p.numel, dtype=NP_DTYPE[p.param_dtype]) for p in pl.params]
    A, P = _i64(pl.A), _i64(pl.P)
    numel = _i64([p.numel for p in pl.params])
    pdt = _i32([p.param_dtype for p in pl.params])
    _load().oracle_copy_out(pl.W, len(outs), ag.ctypes.data, pl.B, A.ctypes.data, P.ctypes.data,
                            numel.ctypes.data, pdt.ctypes.data, _ptrs(outs))
    return outs


def rs_copy_out(pl: Plan, bucket: int, rank: int, row: np.ndarray, divide_factor: float = 1.0):
    """Rank `rank`'s sharded gradients of the members of bucket `bucket` (in
    member order; each the rank chunk's real elements, in the member's storage
    dtype) from the rank's reduced row: S elements of the bucket dtype,
    divided by `divide_factor` (a binary32 value) in that dtype unless it is 1."""
    b = pl.buckets[bucket]
    row = np.ascontiguousarray(row).reshape(-1)
    _check(row, b.dtype, b.S)
    outs = [np.zeros(valid_in_chunk(pl.params[i].numel, P, rank), dtype=NP_DTYPE[pl.params[i].storage_dtype])
            for i, P in zip(b.members, b.P)]
    numel = _i64([pl.params[i].numel for i in b.members])
    sdt = _i32([pl.params[i].storage_dtype for i in b.members])
    P, O = _i64(b.P), _i64(b.O)
    rc = _load().oracle_rs_copy_out(rank, len(outs), row.ctypes.data, b.dtype, b.S, float(np.float32(divide_factor)),
                                    numel.ctypes.data, P.ctypes.data, O.ctypes.data, sdt.ctypes.data, _ptrs(outs))
    if rc:
        raise RuntimeError("oracle_rs_copy_out: bad layout")
    return outs


# --------------------------------------------------------------------------- FSDP1 flat layout

@dataclass
class FlatPlan:
    """A unit laid out as one FSDP1 flat parameter: the parameters flattened and
    concatenated in unit order (N elements, parameter t at flat offset F[t]),
    padded to W*c with c = ceil(N / W); rank r holds flat positions
    [r*c, (r+1)*c).  One reduction dtype and one param dtype for the unit."""
    W: int
    params: list
    dtype: int          # the unit's (effective) reduction dtype
    param_dtype: int
    N: int
    c: int
    F: list


def plan_flat(params, W: int) -> FlatPlan:
    if W < 1:
        raise ValueError("world size must be >= 1")
    params = [p if isinstance(p, ParamDesc) else ParamDesc(*p) for p in params]
    eff = {p.reduce_dtype if p.reduce_dtype else p.grad_dtype for p in params}
    pdt = {p.param_dtype for p in params}
    if len(eff) > 1 or len(pdt) > 1:
        raise ValueError("a flat parameter has one reduction dtype and one param dtype")
    F, acc = [], 0
    for p in params:
        F.append(acc)
        acc += p.numel
    return FlatPlan(W=W, params=params, dtype=eff.pop() if eff else FP32, param_dtype=pdt.pop() if pdt else FP32,
                    N=acc, c=_ceil_div(acc, W), F=F)


def flat_piece(fp: FlatPlan, index: int, rank: int):
    """Parameter `index`'s piece on `rank` as flat positions (lo, hi), lo >= hi when empty."""
    a, b = fp.F[index], fp.F[index] + fp.params[index].numel
    return max(a, rank * fp.c), min(b, (rank + 1) * fp.c)


def piece_len(fp: FlatPlan, index: int, rank: int) -> int:
    lo, hi = flat_piece(fp, index, rank)
    return max(0, hi - lo)


def pack_flat(fp: FlatPlan, grads) -> np.ndarray:
    """Reduce-scatter input [W, c]: the concatenated gradients cast to the reduction dtype, +0 padded."""
    gs = [np.ascontiguousarray(g).reshape(-1) for g in grads]
    for p, g in zip(fp.params, gs):
        _check(g, p.grad_dtype, p.numel)
    out = np.empty((fp.W, fp.c), dtype=NP_DTYPE[fp.dtype])
    gdt = _i32([p.grad_dtype for p in fp.params])
    numel = _i64([p.numel for p in fp.params])
    if _load().oracle_pack_flat(fp.W, len(gs), _ptrs(gs), gdt.ctypes.data, numel.ctypes.data, fp.c, fp.dtype,
                                out.ctypes.data):
        raise RuntimeError("oracle_pack_flat: bad layout")
    return out


def rs_copy_out_flat(fp: FlatPlan, rank: int, row: np.ndarray, divide_factor: float = 1.0):
    """Each parameter's piece of rank `rank`'s sharded gradient (storage dtype) from the
    rank's reduced row (c elements of the reduction dtype), divided as in rs_copy_out."""
    row = np.ascontiguousarray(row).reshape(-1)
    _check(row, fp.dtype, fp.c)
    outs = [np.zeros(piece_len(fp, i, rank), dtype=NP_DTYPE[p.storage_dtype]) for i, p in enumerate(fp.params)]
    numel = _i64([p.numel for p in fp.params])
    sdt = _i32([p.storage_dtype for p in fp.params])
    _load().oracle_rs_copy_out_flat(rank, len(outs), row.ctypes.data, fp.dtype, fp.c,
                                    float(np.float32(divide_factor)), numel.ctypes.data, sdt.ctypes.data, _ptrs(outs))
    return outs


def copy_in_flat(fp: FlatPlan, rank: int, pieces) -> np.ndarray:
    """Rank `rank`'s row of the gathered flat parameter (c elements of the param dtype)
    from its per-parameter pieces (storage dtype)."""
    pieces = [np.ascontiguousarray(x).reshape(-1) for x in pieces]
    for i, (p, x) in enumerate(zip(fp.params, pieces)):
        _check(x, p.storage_dtype, piece_len(fp, i, rank))
    row = np.empty(fp.c, dtype=NP_DTYPE[fp.param_dtype])
    sdt = _i32([p.storage_dtype for p in fp.params])
    numel = _i64([p.numel for p in fp.params])
    _load().oracle_copy_in_flat(rank, len(pieces), _ptrs(pieces), sdt.ctypes.data, fp.param_dtype,
                                numel.ctypes.data, fp.c, row.ctypes.data)
    return row


def copy_out_flat(fp: FlatPlan, flat: np.ndarray):
    """The parameters (param dtype) from the gathered flat parameter (W*c elements)."""
    flat = np.ascontiguousarray(flat).reshape(-1)
    _check(flat, fp.param_dtype, fp.W * fp.c)
    outs = [np.zeros(p.numel, dtype=NP_DTYPE[fp.param_dtype]) for p in fp.params]
    numel = _i64([p.numel for p in fp.params])
    _load().oracle_copy_out_flat(len(outs), flat.ctypes.data, fp.param_dtype, numel.ctypes.data, _ptrs(outs))
    return outs


def shard(pl: Plan, index: int, full: np.ndarray, rank: int) -> np.ndarray:
    """Rank `rank`'s padded shard of parameter `index`: the contiguous row-major
    slice [rank*P, rank*P + P) of the flattened parameter, zero past its end."""
    P = pl.P[index]
    flat = np.ascontiguousarray(full).reshape(-1)
    out = np.zeros(P, dtype=flat.dtype)
    v = valid_in_chunk(flat.size, P, rank)
    out[:v] = flat[rank * P: rank * P + v]
    return out


def convert(arr: np.ndarray, src_dtype: int, dst_dtype: int) -> np.ndarray:
    """Element-wise cast between bf16 (bit patterns) and fp32."""
    arr = np.ascontiguousarray(arr).reshape(-1)
    _check(arr, src_dtype)
    out = np.empty(arr.size, dtype=NP_DTYPE[dst_dtype])
    _load().oracle_convert(arr.ctypes.data, src_dtype, out.ctypes.data, dst_dtype, arr.size)
    return out


def f32_to_bf16_bits(u: int) -> int:
    return int(_load().oracle_f32_to_bf16_bits(u & 0xFFFFFFFF))


def bf16_to_f32_bits(h: int) -> int:
    return int(_load().oracle_bf16_to_f32_bits(h & 0xFFFF))
