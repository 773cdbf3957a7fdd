"""Python binding of libfsdppack: FSDP2's mixed-dtype gradient pack for
reduce-scatter, the write-back of a reduce-scatter output into sharded
gradients, and the all-gather copy-in / copy-out on MI355X (gfx950).

This module only marshals arguments (torch tensors -> device pointers, the
current HIP stream) and calls the C ABI declared in ``include/fsdppack.h``;
every step of the work runs in the library's HIP kernels.  There is no CPU
fallback: if ``libfsdppack.so`` is missing, loading fails loudly.

Functions (same names as the C ABI without the ``fsdppack_`` prefix):
  plan_buckets(params, world)                  -> Plan
  plan_buckets_flat(params, world)             -> Plan   (FSDP1 flat-parameter layout)
  pack_reduce_scatter_input(plan, bucket, grads, out, stream=None)
  pack_reduce_scatter_input_noalloc(plan, bucket, grads, out, stream=None)   (allocates nothing)
  all_gather_copy_in(plan, rank, shards, ag_out, stream=None)
  all_gather_copy_out(plan, ag, params, stream=None)
  reduce_scatter_copy_out(plan, bucket, rank, rs_out, shard_grads, divide_factor=1.0, stream=None)
  reduce_scatter_copy_out_all(plan, rank, rs_outs, shard_grads, divide_factor=1.0, stream=None)
                                               (every bucket's write-back in one launch)

The tensor lists may also be given as a PointerArray from prepare_grads /
prepare_shards / prepare_params / prepare_shard_grads: validated once and
reused across calls, the way a training loop reuses its gradient and shard
buffers every step.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch  # device memory and streams; loaded first so libfsdppack binds to torch's HIP runtime

BF16 = 1
FP32 = 2
DTYPE_NONE = 0
TORCH_DTYPE = {BF16: torch.bfloat16, FP32: torch.float32}
ELEM_SIZE = {BF16: 2, FP32: 4}

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfsdppack.so")

STATUS = {0: "OK", -1: "EINVAL", -2: "EDTYPE", -3: "ENOMEM", -4: "EHIP", -5: "ESTATE"}


class FsdpPackError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"{STATUS.get(code, code)}: {message}")
        self.code = code


class ParamDesc(ctypes.Structure):
    _fields_ = [("dim0", ctypes.c_int64), ("inner", ctypes.c_int64),
                ("grad_dtype", ctypes.c_int32), ("reduce_dtype", ctypes.c_int32),
                ("storage_dtype", ctypes.c_int32), ("param_dtype", ctypes.c_int32)]


_lib = None


def lib():
    """The loaded libfsdppack (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run fsdp2_mixed_dtype_amd.build.build() "
                              "(hipcc --offload-arch=gfx950) first")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        P_i32, P_i64 = ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int64)
        PP_i32, PP_i64 = ctypes.POINTER(P_i32), ctypes.POINTER(P_i64)
        L.fsdppack_plan_buckets.argtypes = [ctypes.POINTER(ParamDesc), i32, i32, ctypes.POINTER(vp)]
        L.fsdppack_plan_buckets_flat.argtypes = [ctypes.POINTER(ParamDesc), i32, i32, ctypes.POINTER(vp)]
        L.fsdppack_plan_info.argtypes = [vp, P_i32, P_i32, P_i32]
        L.fsdppack_plan_bucket.argtypes = [vp, i32, P_i32, P_i64, P_i32, PP_i32, PP_i64, PP_i64]
        L.fsdppack_plan_all_gather_layout.argtypes = [vp, P_i64, PP_i64, PP_i64]
        L.fsdppack_pack_reduce_scatter_input.argtypes = [vp, i32, vp, vp, vp]
        L.fsdppack_pack_reduce_scatter_input_noalloc.argtypes = [vp, i32, vp, vp, vp]
        L.fsdppack_all_gather_copy_in.argtypes = [vp, i32, vp, vp, vp]
        L.fsdppack_all_gather_copy_out.argtypes = [vp, vp, vp, vp]
        L.fsdppack_reduce_scatter_copy_out.argtypes = [vp, i32, i32, vp, ctypes.c_float, vp, vp]
        L.fsdppack_reduce_scatter_copy_out_all.argtypes = [vp, i32, vp, ctypes.c_float, vp, vp]
        L.fsdppack_plan_destroy.argtypes = [vp]
        L.fsdppack_plan_destroy.restype = None
        L.fsdppack_last_error.argtypes = []
        L.fsdppack_last_error.restype = ctypes.c_char_p
        L.fsdppack_counters.argtypes = [P_i64, i32]
        L.fsdppack_time_next_launch.argtypes = [vp, vp]
        L.fsdppack_empty_launch.argtypes = [i32, i32, vp]
        for f in (L.fsdppack_plan_buckets, L.fsdppack_plan_buckets_flat, L.fsdppack_plan_info, L.fsdppack_plan_bucket,
                  L.fsdppack_plan_all_gather_layout, L.fsdppack_pack_reduce_scatter_input,
                  L.fsdppack_pack_reduce_scatter_input_noalloc,
                  L.fsdppack_all_gather_copy_in, L.fsdppack_all_gather_copy_out,
                  L.fsdppack_reduce_scatter_copy_out, L.fsdppack_counters, L.fsdppack_time_next_launch,
                  L.fsdppack_empty_launch):
            f.restype = ctypes.c_int
        _lib = L
    return _lib


def _check(rc: int):
    if rc != 0:
        raise FsdpPackError(rc, lib().fsdppack_last_error().decode())


@dataclass(frozen=True)
class Bucket:
    dtype: int          # effective reduction dtype
    S: int              # row length of the [W, S] reduce-scatter input
    members: tuple      # parameter indices (unit order)
    P: tuple            # padded rank-chunk size of each member
    O: tuple            # column offset of each member


class Plan:
    """A planned fully_shard unit (owns the library handle)."""

    def __init__(self, handle: int, descs, flat: bool = False):
        self._h = ctypes.c_void_p(handle)
        self.descs = tuple(descs)
        self.flat = flat                 # FSDP1 flat-parameter layout (plan_buckets_flat)
        L = lib()
        nb, n, w = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        _check(L.fsdppack_plan_info(self._h, ctypes.byref(nb), ctypes.byref(n), ctypes.byref(w)))
        self.world, self.n = w.value, n.value
        buckets = []
        for b in range(nb.value):
            dt, S, m = ctypes.c_int32(), ctypes.c_int64(), ctypes.c_int32()
            mem = ctypes.POINTER(ctypes.c_int32)()
            P, O = ctypes.POINTER(ctypes.c_int64)(), ctypes.POINTER(ctypes.c_int64)()
            _check(L.fsdppack_plan_bucket(self._h, b, ctypes.byref(dt), ctypes.byref(S), ctypes.byref(m),
                                          ctypes.byref(mem), ctypes.byref(P), ctypes.byref(O)))
            k = m.value
            buckets.append(Bucket(dt.value, S.value, tuple(mem[i] for i in range(k)),
                                  tuple(P[i] for i in range(k)), tuple(O[i] for i in range(k))))
        self.buckets = tuple(buckets)
        B = ctypes.c_int64()
        P, A = ctypes.POINTER(ctypes.c_int64)(), ctypes.POINTER(ctypes.c_int64)()
        _check(L.fsdppack_plan_all_gather_layout(self._h, ctypes.byref(B), ctypes.byref(P), ctypes.byref(A)))
        self.B = B.value
        self.P = tuple(P[i] for i in range(self.n))
        self.A = tuple(A[i] for i in range(self.n))
        self.numel = tuple(d.dim0 * d.inner for d in self.descs)
        self.grad_dtypes = tuple(d.grad_dtype for d in self.descs)
        self.storage_dtypes = tuple(d.storage_dtype for d in self.descs)
        self.param_dtypes = tuple(d.param_dtype for d in self.descs)
        # per bucket: its members, their gradient dtypes and element counts
        self.member_specs = tuple((tuple(b.members), tuple(self.grad_dtypes[i] for i in b.members),
                                   tuple(self.numel[i] for i in b.members)) for b in self.buckets)
        self.shard_grad_specs = {}   # (bucket or None, rank) -> the write-back's members on that rank
        # flat layout: c per rank, parameter t at flat offset O_t of the one bucket
        self.c = self.buckets[0].S if flat and self.buckets else 0

    @property
    def handle(self):
        if not self._h:
            raise FsdpPackError(-5, "plan already destroyed")
        return self._h

    def destroy(self):
        if self._h:
            lib().fsdppack_plan_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass


def plan_buckets(params, world: int) -> Plan:
    """Plan one unit.  params: sequence of (dim0, inner, grad_dtype,
    reduce_dtype, storage_dtype, param_dtype) tuples (or ParamDesc)."""
    descs = [p if isinstance(p, ParamDesc) else ParamDesc(*[int(x) for x in p]) for p in params]
    arr = (ParamDesc * max(1, len(descs)))(*descs)
    h = ctypes.c_void_p()
    _check(lib().fsdppack_plan_buckets(arr, len(descs), int(world), ctypes.byref(h)))
    return Plan(h.value, descs)


def plan_buckets_flat(params, world: int) -> Plan:
    """Plan one unit in the FSDP1 flat-parameter layout: the parameters
    flattened and concatenated into one flat parameter, padded to W*c, rank r
    holding flat positions [r*c, (r+1)*c).  One reduction dtype and one param
    dtype for the unit."""
    descs = [p if isinstance(p, ParamDesc) else ParamDesc(*[int(x) for x in p]) for p in params]
    arr = (ParamDesc * max(1, len(descs)))(*descs)
    h = ctypes.c_void_p()
    _check(lib().fsdppack_plan_buckets_flat(arr, len(descs), int(world), ctypes.byref(h)))
    return Plan(h.value, descs, flat=True)


# torch's raw query of the current stream: the same handle as
# torch.cuda.current_stream().cuda_stream without building a stream object on
# every call (a few microseconds of host time per launch)
_current_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(stream):
    if stream is not None:
        return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    if _current_raw_stream is not None:
        return _current_raw_stream(torch.cuda.current_device())
    return torch.cuda.current_stream().cuda_stream


def _ptr(t, dtype: int | None, numel: int | None, what: str):
    if t is None:
        return 0
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what}: expected a torch.Tensor")
    if not t.is_cuda:             # (cheaper than building t.device; HIP tensors report is_cuda)
        raise ValueError(f"{what}: tensor must live on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{what}: tensor must be contiguous")
    if dtype is not None and t.dtype != TORCH_DTYPE[dtype]:
        raise TypeError(f"{what}: expected {TORCH_DTYPE[dtype]}, got {t.dtype}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{what}: expected {numel} elements, got {t.numel()}")
    return t.data_ptr()


def _ptrs(tensors, dtypes, numels, what: str, index=None):
    """_ptr over a list (dtype codes and element counts by position; `index`:
    the positions' indices for error messages, default 0, 1, ...): a plain
    tensor that passes every check costs one condition; anything else (a
    subclass, a wrong property) goes through _ptr, which accepts it or raises
    the same error it would raise on its own."""
    out = []
    app = out.append
    Tensor = torch.Tensor
    for i, (t, dt, n) in enumerate(zip(tensors, dtypes, numels)):
        if t is None:
            app(0)
        elif (type(t) is Tensor and t.is_cuda and t.dtype is TORCH_DTYPE[dt] and t.is_contiguous()
              and t.numel() == n):
            app(t.data_ptr())
        else:
            app(_ptr(t, dt, n, f"{what}[{i if index is None else index[i]}]"))
    return out


def _member_grads(plan, bucket: int, grads):
    """The pointer array of a gradient list for one bucket's pack: its
    members' pointers, validated, and 0 for every other parameter."""
    if len(grads) != plan.n:
        raise ValueError(f"grads: expected {plan.n} entries, got {len(grads)}")
    mem, dts, ns = plan.member_specs[bucket]
    ptrs = [0] * max(1, plan.n)
    for i, p in zip(mem, _ptrs([grads[i] for i in mem], dts, ns, "grads", mem)):
        ptrs[i] = p
    return (ctypes.c_void_p * len(ptrs))(*ptrs)


def _ptr_array(ptrs):
    return (ctypes.c_void_p * max(1, len(ptrs)))(*ptrs)


class PointerArray:
    """Device pointers of a plan's gradients, shards or parameters, validated
    once (dtype, size, contiguity, device) and reusable across calls.  Keeps
    the tensors alive."""

    def __init__(self, plan: Plan, kind: str, tensors, ptrs):
        self.plan_handle = plan.handle.value
        self.kind = kind
        self.tensors = list(tensors)
        self.array = _ptr_array(ptrs)


def prepare_grads(plan: Plan, grads) -> PointerArray:
    """Gradients by parameter index (grad dtype, numel elements); None allowed
    for parameters that are never packed."""
    if len(grads) != plan.n:
        raise ValueError(f"grads: expected {plan.n} entries, got {len(grads)}")
    ptrs = _ptrs(grads, plan.grad_dtypes, plan.numel, "grads")
    return PointerArray(plan, "grads", grads, ptrs)


def prepare_shards(plan: Plan, shards, rank: int | None = None) -> PointerArray:
    """Local shards by parameter index (storage dtype): the padded rank
    chunks (P elements), or for a flat plan the parameters' pieces on `rank`
    (None allowed for an empty piece)."""
    if len(shards) != plan.n:
        raise ValueError(f"shards: expected {plan.n} entries, got {len(shards)}")
    if plan.flat:
        if rank is None:
            raise ValueError("shards of a flat plan depend on the rank")
        ptrs = [_ptr(s, plan.descs[i].storage_dtype, valid_in_chunk(plan, i, rank), f"shards[{i}]")
                if valid_in_chunk(plan, i, rank) else 0 for i, s in enumerate(shards)]
    else:
        ptrs = _ptrs(shards, plan.storage_dtypes, plan.P, "shards")
    arr = PointerArray(plan, "shards", shards, ptrs)
    arr.rank = rank if plan.flat else None
    return arr


def prepare_params(plan: Plan, params) -> PointerArray:
    """Full parameters by index (param dtype, numel elements)."""
    if len(params) != plan.n:
        raise ValueError(f"params: expected {plan.n} entries, got {len(params)}")
    ptrs = _ptrs(params, plan.param_dtypes, plan.numel, "params")
    return PointerArray(plan, "params", params, ptrs)


def _prepared(plan: Plan, arr, kind: str, make):
    if isinstance(arr, PointerArray):
        if arr.kind != kind or arr.plan_handle != plan.handle.value:
            raise ValueError(f"pointer array was prepared for {arr.kind} of another plan")
        return arr.array
    return make(plan, arr).array


def pack_reduce_scatter_input(plan: Plan, bucket: int, grads, out, stream=None):
    """Fill `out` ([W, S] of the bucket's reduction dtype) with every member's
    gradient chunked along dim 0, cast and zero-padded.  `grads` is indexed by
    parameter (unit order); entries of non-members may be None."""
    b = plan.buckets[bucket]
    if isinstance(grads, PointerArray):
        arr = _prepared(plan, grads, "grads", prepare_grads)
    else:
        arr = _member_grads(plan, bucket, grads)
    optr = _ptr(out, b.dtype, plan.world * b.S, "out")
    _check(lib().fsdppack_pack_reduce_scatter_input(plan.handle, bucket, arr, optr, _stream(stream)))
    return out


def pack_reduce_scatter_input_noalloc(plan: Plan, bucket: int, grads, out, stream=None):
    """pack_reduce_scatter_input for callers that cannot allocate device
    memory: the bucket's tables go through the library's fixed device scratch
    (shared by every such call on the GPU: overlapping calls race)."""
    b = plan.buckets[bucket]
    if isinstance(grads, PointerArray):
        arr = _prepared(plan, grads, "grads", prepare_grads)
    else:
        arr = _member_grads(plan, bucket, grads)
    optr = _ptr(out, b.dtype, plan.world * b.S, "out")
    _check(lib().fsdppack_pack_reduce_scatter_input_noalloc(plan.handle, bucket, arr, optr, _stream(stream)))
    return out


def _bytes_ptr(t, nbytes: int, what: str):
    p = _ptr(t, None, None, what)
    if t.numel() * t.element_size() != nbytes:
        raise ValueError(f"{what}: expected {nbytes} bytes, got {t.numel() * t.element_size()}")
    return p


def all_gather_copy_in(plan: Plan, rank: int, shards, ag_out, stream=None):
    """Write row `rank` of the [W, B]-byte all-gather buffer from the rank's
    padded shards (P elements each, storage dtype)."""
    if plan.flat:
        if isinstance(shards, PointerArray):
            if shards.kind != "shards" or shards.plan_handle != plan.handle.value or shards.rank != rank:
                raise ValueError("pointer array was prepared for another plan or rank")
            arr = shards.array
        else:
            arr = prepare_shards(plan, shards, rank).array
    else:
        arr = _prepared(plan, shards, "shards", prepare_shards)
    aptr = _bytes_ptr(ag_out, plan.world * plan.B, "ag_out")
    _check(lib().fsdppack_all_gather_copy_in(plan.handle, int(rank), arr, aptr, _stream(stream)))
    return ag_out


def all_gather_copy_out(plan: Plan, ag, params, stream=None):
    """Rebuild every full parameter (param dtype) from the gathered buffer."""
    arr = _prepared(plan, params, "params", prepare_params)
    aptr = _bytes_ptr(ag, plan.world * plan.B, "ag")
    _check(lib().fsdppack_all_gather_copy_out(plan.handle, aptr, arr, _stream(stream)))
    return params


def valid_in_chunk(plan: Plan, index: int, rank: int) -> int:
    """Real (non-padding) elements of parameter `index` on rank `rank`: of its
    rank chunk, or for a flat plan of its piece inside the rank's positions."""
    if plan.flat:
        F = plan.buckets[0].O[index]
        return max(0, min(F + plan.numel[index], (rank + 1) * plan.c) - max(F, rank * plan.c))
    P = plan.P[index]
    return max(0, min(P, plan.numel[index] - rank * P))


def prepare_shard_grads(plan: Plan, bucket: int | None, rank: int, grads) -> PointerArray:
    """Sharded gradients by parameter index for the write-back of `bucket`
    (None: of every bucket, for reduce_scatter_copy_out_all) on `rank`: each
    member's entry holds the rank chunk's real elements (storage dtype);
    entries of non-members and of members with nothing on this rank may be
    None."""
    if len(grads) != plan.n:
        raise ValueError(f"shard_grads: expected {plan.n} entries, got {len(grads)}")
    key = (bucket, rank)
    spec = plan.shard_grad_specs.get(key)
    if spec is None:
        # the members with real elements on this rank, their storage dtypes
        # and element counts (the layout is fixed, so once per bucket and rank)
        members = sorted({i for b in plan.buckets for i in b.members} if bucket is None
                         else plan.buckets[bucket].members)
        mem = tuple(i for i in members if valid_in_chunk(plan, i, rank))
        spec = (mem, tuple(plan.storage_dtypes[i] for i in mem), tuple(valid_in_chunk(plan, i, rank) for i in mem))
        plan.shard_grad_specs[key] = spec
    mem, dts, ns = spec
    ptrs = [0] * plan.n
    for i, p in zip(mem, _ptrs([grads[i] for i in mem], dts, ns, "shard_grads", mem)):
        ptrs[i] = p
    arr = PointerArray(plan, "shard_grads", grads, ptrs)
    arr.bucket, arr.rank = bucket, rank
    return arr


def reduce_scatter_copy_out(plan: Plan, bucket: int, rank: int, rs_out, shard_grads, divide_factor: float = 1.0,
                            stream=None):
    """Write rank `rank`'s sharded gradients of the members of `bucket` from
    the rank's reduced row `rs_out` (S elements of the bucket's reduction
    dtype): each element divided by `divide_factor` in the reduction dtype
    (unless it is 1), then cast to the member's storage dtype.  `shard_grads`
    is indexed by parameter (see prepare_shard_grads)."""
    b = plan.buckets[bucket]
    if isinstance(shard_grads, PointerArray):
        if (shard_grads.kind != "shard_grads" or shard_grads.plan_handle != plan.handle.value
                or shard_grads.bucket != bucket or shard_grads.rank != rank):
            raise ValueError("pointer array was prepared for another plan, bucket or rank")
        arr = shard_grads.array
    else:
        arr = prepare_shard_grads(plan, bucket, rank, shard_grads).array
    rptr = _ptr(rs_out, b.dtype, b.S, "rs_out")
    _check(lib().fsdppack_reduce_scatter_copy_out(plan.handle, bucket, int(rank), rptr, float(divide_factor), arr,
                                                  _stream(stream)))
    return shard_grads


def reduce_scatter_copy_out_all(plan: Plan, rank: int, rs_outs, shard_grads, divide_factor: float = 1.0,
                                stream=None):
    """The write-back of every bucket in one launch: for each bucket b, what
    reduce_scatter_copy_out(plan, b, rank, rs_outs[b], ...) writes.  `rs_outs`
    holds one reduced row per bucket (S_b elements of its reduction dtype);
    `shard_grads` is indexed by parameter (prepare_shard_grads(plan, None,
    rank, grads))."""
    if len(rs_outs) != len(plan.buckets):
        raise ValueError(f"rs_outs: expected {len(plan.buckets)} rows, got {len(rs_outs)}")
    if isinstance(shard_grads, PointerArray):
        if (shard_grads.kind != "shard_grads" or shard_grads.plan_handle != plan.handle.value
                or shard_grads.bucket is not None or shard_grads.rank != rank):
            raise ValueError("pointer array was prepared for another plan, bucket or rank")
        arr = shard_grads.array
    else:
        arr = prepare_shard_grads(plan, None, rank, shard_grads).array
    rows = _ptr_array([_ptr(r, b.dtype, b.S, f"rs_outs[{i}]") for i, (r, b) in enumerate(zip(rs_outs, plan.buckets))])
    _check(lib().fsdppack_reduce_scatter_copy_out_all(plan.handle, int(rank), rows, float(divide_factor), arr,
                                                      _stream(stream)))
    return shard_grads


def time_next_launch(start, stop):
    """Have the next compute call on this thread stamp two timing events
    (torch.cuda.Event(enable_timing=True), already recorded once so that they
    exist) at its kernel's start and end."""
    _check(lib().fsdppack_time_next_launch(start.cuda_event, stop.cuda_event))


def counters():
    """(kernel launches, pointer-table uploads, pointer-table reuses, plan
    uploads, pointer tables replaced by a new set, cross-stream waits at such a
    replacement, launches whose pointers travelled in the launch arguments,
    host waits for a replaced table's previous upload, copies of pack tables
    into the allocation-free pack's scratch)."""
    c = (ctypes.c_int64 * 9)()
    _check(lib().fsdppack_counters(c, 9))
    return tuple(c)


def empty_launch(workgroups: int, threads: int = 64, stream=None):
    """Launch a kernel that does nothing with the given grid (the floor of a
    launch of that many workgroups; a measurement aid)."""
    _check(lib().fsdppack_empty_launch(int(workgroups), int(threads), _stream(stream)))
