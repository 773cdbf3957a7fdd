// fsdppack_abi.cpp -- the C ABI of libfsdppack (declared in include/fsdppack.h).
//
// Argument checks are synchronous and on the host; every compute call then
// enqueues one launch of a window kernel on the caller's stream.
// Per-call device pointers (grads, shards, params) travel in the launch's
// arguments when there are at most 64 of them; larger sets reach the kernel
// through a device table cached by content (see PtrCache in
// fsdppack_plan.h), so a training loop that passes the same buffers each step
// pays no upload, and a set of up to 960 that is not cached yet travels in
// the arguments while its table is uploaded behind the launch.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <atomic>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <string>

#include "fsdppack_plan.h"

using namespace fsdppack;

namespace {

thread_local std::string g_error;
thread_local void *g_next_start = nullptr;   // events for the next launch on this thread
thread_local void *g_next_stop = nullptr;
// launches, table uploads, table reuses, plan uploads, table evictions,
// cross-stream waits at an eviction, launches with their pointers inline,
// host waits for a replaced table's upload, allocation-free table copies
constexpr int kCounters = 9;
std::atomic<int64_t> g_counters[kCounters];
std::atomic<uint64_t> g_plan_serial{0};

// What each device's scratch holds: the image the last allocation-free pack
// on that device copied there (plan serial, and region: -1 for the plan-wide
// image, else the bucket) and an event recorded after the copy, on the
// copying stream.  A call whose image is the one held copies nothing.  Once
// a call has been captured into a graph on the device, every replay of that
// graph rewrites the scratch, so from then on the device's calls always copy
// (`captured`).
struct ScratchHolds {
    uint64_t serial = 0;
    int32_t region = 0;
    hipEvent_t copied = nullptr;
    bool captured = false;
};
std::mutex g_scratch_mu;
ScratchHolds g_scratch_holds[kMaxDevices];

int fail(int code, const std::string &msg)
{
    g_error = msg;
    return code;
}

int hip_fail(hipError_t e, const char *what)
{
    return fail(FSDPPACK_EHIP, std::string(what) + ": " + hipGetErrorName(e) + " (" + hipGetErrorString(e) + ")");
}

bool trace_on()
{
    static const bool on = [] {
        const char *v = std::getenv("FSDPPACK_TRACE");
        return v != nullptr && v[0] != '\0' && v[0] != '0';
    }();
    return on;
}

bool plan_ok(const fsdppack_plan *p) { return p != nullptr && p->magic == kPlanMagic; }

bool aligned(const void *p, int64_t bytes) { return (reinterpret_cast<uintptr_t>(p) % bytes) == 0; }

// Timing events armed for this thread's next launch.  Every compute call
// takes them when it starts: its launch stamps them, and a call that launches
// nothing (nothing to write, or rejected) leaves them unstamped.
struct ArmedEvents {
    void *start = nullptr, *stop = nullptr;
};

ArmedEvents take_armed_events()
{
    ArmedEvents ev{g_next_start, g_next_stop};
    g_next_start = g_next_stop = nullptr;
    return ev;
}

// Copy one operation's tables to the device.  A table is kept only once its
// copy has succeeded, so a call retried after a failed upload resumes it
// without leaking or trusting a half-made table.
int upload_table(OpTable &op)
{
    auto put = [](void *&dst, const void *src, size_t bytes, const char *what) -> int {
        if (bytes == 0 || dst != nullptr) return FSDPPACK_OK;
        void *d = nullptr;
        hipError_t e = hipMalloc(&d, bytes);
        if (e != hipSuccess) return hip_fail(e, (std::string("hipMalloc(") + what + ")").c_str());
        if ((e = hipMemcpy(d, src, bytes, hipMemcpyHostToDevice)) != hipSuccess) {
            (void)hipFree(d);
            return hip_fail(e, (std::string("hipMemcpy(") + what + ")").c_str());
        }
        dst = d;
        return FSDPPACK_OK;
    };
    if (int rc = put(op.d_members, op.members.data(), op.members.size(), "member table")) return rc;
    if (int rc = put(op.d_columns, op.columns.data(), op.columns.size() * sizeof(ColumnWindow), "column map"))
        return rc;
    return put(op.d_stretches, op.stretches.data(), op.stretches.size() * sizeof(PackStretch), "stretch records");
}

// Upload the plan's member tables once, on the current device; afterwards
// the plan is bound to that device.  Caller holds plan->mu.
int ensure_device(fsdppack_plan *p)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (p->uploaded) {
        if (dev != p->device)
            return fail(FSDPPACK_ESTATE, "plan was prepared on device " + std::to_string(p->device) +
                                             " but the current device is " + std::to_string(dev));
        return FSDPPACK_OK;
    }
    for (BucketPlan &b : p->buckets) {
        if (int rc = upload_table(b.pack)) return rc;
        if (int rc = upload_table(b.write_back)) return rc;
    }
    if (int rc = upload_table(p->copy_in)) return rc;
    if (int rc = upload_table(p->copy_out)) return rc;
    if (int rc = upload_table(p->write_back_all)) return rc;
    p->caches.resize(2 * p->buckets.size() + 3);
    p->device = dev;
    p->uploaded = true;
    g_counters[3]++;
    return FSDPPACK_OK;
}

// The cached device table holding pointer set `key`, if any (*out = NULL
// when there is none), ordered before work enqueued next on `stream`.
// Caller holds plan->mu.
int find_table(PtrCache &c, const std::vector<uint64_t> &key, hipStream_t stream, PtrSlot **out)
{
    *out = nullptr;
    for (PtrSlot &s : c.slots) {
        if (s.live && s.key == key) {
            bool ordered = false;
            for (void *st : s.streams) ordered |= (st == stream);
            if (!ordered) {
                // first use on this stream: wait once for the upload
                hipError_t e;
                if ((e = hipStreamWaitEvent(stream, static_cast<hipEvent_t>(s.ready), 0)) != hipSuccess)
                    return hip_fail(e, "hipStreamWaitEvent");
                s.streams.push_back(stream);
            }
            s.last_use = ++c.clock;
            g_counters[2]++;
            *out = &s;
            return FSDPPACK_OK;
        }
    }
    return FSDPPACK_OK;
}

// Find or stage the device table for pointer set `key` in cache `c`, ordered
// before work enqueued next on `stream`.  Caller holds plan->mu.
//
// Replacing a cached table needs no device-wide synchronisation:
//  * the slot's previous upload read its pinned staging buffer, so that one
//    copy (issued at least kPtrSlots distinct pointer sets ago) must be done
//    before the buffer is rewritten: a host wait on its event;
//  * kernels that read the old table on `stream` itself precede the new
//    upload in stream order, and those on any other stream that used the slot
//    are waited for on the device (an event recorded on that stream now,
//    waited on by `stream`).
// With may_wait false the table is only staged if that takes no host wait:
// when the slot to replace still has its previous upload in flight, *out is
// NULL and nothing is enqueued.
int acquire_table(PtrCache &c, const std::vector<uint64_t> &key, hipStream_t stream, PtrSlot **out,
                  bool may_wait = true)
{
    hipError_t e;
    if (int rc = find_table(c, key, stream, out)) return rc;
    if (*out != nullptr) return FSDPPACK_OK;
    PtrSlot *victim = nullptr;
    for (PtrSlot &s : c.slots)
        if (!s.live) { victim = &s; break; }
    if (victim == nullptr) {
        victim = &c.slots[0];
        for (PtrSlot &s : c.slots)
            if (s.last_use < victim->last_use) victim = &s;
        if (!may_wait) {
            e = hipEventQuery(static_cast<hipEvent_t>(victim->ready));
            if (e == hipErrorNotReady) return FSDPPACK_OK;      // skip: its staging is still being read
            if (e != hipSuccess) return hip_fail(e, "hipEventQuery(previous upload)");
        } else {
            if ((e = hipEventSynchronize(static_cast<hipEvent_t>(victim->ready))) != hipSuccess)
                return hip_fail(e, "hipEventSynchronize(previous upload)");
            g_counters[7]++;
        }
        size_t used = 0;
        for (void *st : victim->streams) {
            if (st == stream) continue;
            if (used == victim->drain.size()) {
                hipEvent_t ev;
                if ((e = hipEventCreateWithFlags(&ev, hipEventDisableTiming)) != hipSuccess)
                    return hip_fail(e, "hipEventCreate");
                victim->drain.push_back(ev);
            }
            hipEvent_t ev = static_cast<hipEvent_t>(victim->drain[used++]);
            if ((e = hipEventRecord(ev, static_cast<hipStream_t>(st))) != hipSuccess)
                return hip_fail(e, "hipEventRecord(other stream)");
            if ((e = hipStreamWaitEvent(stream, ev, 0)) != hipSuccess) return hip_fail(e, "hipStreamWaitEvent");
            g_counters[5]++;
        }
        victim->live = false;
        g_counters[4]++;
    }
    const size_t bytes = key.size() * sizeof(uint64_t);
    if (victim->d_table == nullptr) {
        // the slot's device table, pinned staging and event, kept only together
        uint64_t *d = nullptr, *h = nullptr;
        hipEvent_t ev = nullptr;
        if ((e = hipMalloc(reinterpret_cast<void **>(&d), bytes)) != hipSuccess)
            return hip_fail(e, "hipMalloc(pointer table)");
        if ((e = hipHostMalloc(reinterpret_cast<void **>(&h), bytes, hipHostMallocDefault)) != hipSuccess) {
            (void)hipFree(d);
            return hip_fail(e, "hipHostMalloc(pointer table)");
        }
        if ((e = hipEventCreateWithFlags(&ev, hipEventDisableTiming)) != hipSuccess) {
            (void)hipFree(d);
            (void)hipHostFree(h);
            return hip_fail(e, "hipEventCreate");
        }
        victim->d_table = d;
        victim->h_stage = h;
        victim->ready = ev;
    }
    std::memcpy(victim->h_stage, key.data(), bytes);
    if ((e = hipMemcpyAsync(victim->d_table, victim->h_stage, bytes, hipMemcpyHostToDevice, stream)) != hipSuccess)
        return hip_fail(e, "hipMemcpyAsync(pointer table)");
    if ((e = hipEventRecord(static_cast<hipEvent_t>(victim->ready), stream)) != hipSuccess) return hip_fail(e, "hipEventRecord");
    victim->key = key;
    victim->streams.assign(1, stream);
    victim->live = true;
    victim->last_use = ++c.clock;
    g_counters[1]++;
    *out = victim;
    return FSDPPACK_OK;
}

// Run one operation: one kernel launch, its pointer table in the launch's
// arguments (up to kInlineLarge entries) or in a cached device table.
int run_op(fsdppack_plan *p, const OpTable &op, size_t cache_index, const std::vector<uint64_t> &key, char *base,
           void *stream, const ArmedEvents &ev, const char *what, int32_t rank = 0, float divisor = 1.0f)
{
    // window boundaries follow the cache lines of memory, not the buffer's start
    const int32_t shift = static_cast<int32_t>(reinterpret_cast<uintptr_t>(base) & (kLineBytes - 1));
    if (op.windows(shift) <= 0) return FSDPPACK_OK;
    std::lock_guard<std::mutex> lock(p->mu);
    if (int rc = ensure_device(p)) return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    WindowArgs args = op.args(true, shift);
    // Up to kInlineSmall pointers travel in the launch's arguments.  A larger
    // set uses its cached device table when there is one (on MI355X a
    // 960-entry argument table made a launch about 0.5 us longer than a device
    // table), else its pointers travel in the arguments (up to kInlineLarge)
    // and the set is uploaded behind this launch, for the next call that
    // passes it, when that needs no host wait; beyond kInlineLarge the device
    // table is staged first.
    const uint64_t *inline_ptrs = nullptr;
    bool upload_after = false;
    if (key.size() <= static_cast<size_t>(kInlineSmall)) {
        inline_ptrs = key.data();
    } else {
        PtrSlot *slot = nullptr;
        if (int rc = find_table(p->caches[cache_index], key, s, &slot)) return rc;
        if (slot == nullptr && key.size() <= static_cast<size_t>(kInlineLarge)) {
            inline_ptrs = key.data();
            upload_after = true;
        } else {
            if (slot == nullptr)
                if (int rc = acquire_table(p->caches[cache_index], key, s, &slot)) return rc;
            args.table = slot->d_table;
        }
    }
    if (inline_ptrs != nullptr) g_counters[6]++;
    args.base = base;
    args.rank = rank;
    args.divisor = divisor;
    const int le = launch_windows(args, inline_ptrs, static_cast<int32_t>(key.size()), stream, ev.start, ev.stop);
    if (le != 0) return hip_fail(static_cast<hipError_t>(le), what);
    g_counters[0]++;
    if (upload_after) {
        // cache the set for the next call that passes it, unless that would
        // make the host wait (the table to replace is still being uploaded)
        PtrSlot *slot = nullptr;
        if (int rc = acquire_table(p->caches[cache_index], key, s, &slot, false)) return rc;
    }
    if (trace_on())
        std::fprintf(stderr, "fsdppack: %s: %d workgroups, %lld bytes read, %lld bytes written\n", what,
                     args.n_windows, static_cast<long long>(op.src_bytes), static_cast<long long>(op.dst_bytes));
    return FSDPPACK_OK;
}

// Argument checks shared by the two pack entry points (`what` names the
// call).  A message is built only for an argument that is rejected.
int check_pack_args(const fsdppack_plan *plan, int32_t bucket, const void *const *grads, const void *out,
                    const char *what)
{
    auto bad = [what](int code, const std::string &msg) { return fail(code, std::string(what) + ": " + msg); };
    if (!plan_ok(plan)) return bad(FSDPPACK_ESTATE, "invalid plan handle");
    if (bucket < 0 || bucket >= static_cast<int32_t>(plan->buckets.size()))
        return bad(FSDPPACK_EINVAL, "bucket index out of range");
    if (grads == nullptr) return bad(FSDPPACK_EINVAL, "grads is NULL");
    const BucketPlan &b = plan->buckets[bucket];
    if (b.S > 0 && (out == nullptr || !aligned(out, dtype_bytes(b.dtype))))
        return bad(FSDPPACK_EINVAL, "out is NULL or not aligned to its element size");
    for (int32_t t : b.members) {
        if (plan->numel[t] == 0) continue;
        const void *g = grads[t];
        if (g == nullptr || !aligned(g, dtype_bytes(plan->params[t].grad_dtype)))
            return bad(FSDPPACK_EINVAL, "grads[" + std::to_string(t) + "] is NULL or not aligned to its element size");
    }
    return FSDPPACK_OK;
}

}  // namespace

extern "C" {

namespace {
int make_plan(const fsdppack_param_desc *params, int32_t n, int32_t world, fsdppack_plan **out_plan, bool flat)
{
    if (out_plan == nullptr) return fail(FSDPPACK_EINVAL, "plan_buckets: out_plan is NULL");
    *out_plan = nullptr;
    fsdppack_plan *p = new (std::nothrow) fsdppack_plan();
    if (p == nullptr) return fail(FSDPPACK_ENOMEM, "plan_buckets: out of host memory");
    std::string err;
    int rc;
    try {
        rc = flat ? build_plan_flat(params, n, world, p, err) : build_plan(params, n, world, p, err);
    } catch (const std::bad_alloc &) {
        rc = FSDPPACK_ENOMEM;
        err = "plan_buckets: out of host memory";
    }
    if (rc != FSDPPACK_OK) {
        delete p;
        return fail(rc, err);
    }
    p->serial = ++g_plan_serial;
    *out_plan = p;
    return FSDPPACK_OK;
}
}  // namespace

int fsdppack_plan_buckets(const fsdppack_param_desc *params, int32_t n, int32_t world,
                          fsdppack_plan **out_plan)
{
    return make_plan(params, n, world, out_plan, false);
}

int fsdppack_plan_buckets_flat(const fsdppack_param_desc *params, int32_t n, int32_t world,
                               fsdppack_plan **out_plan)
{
    return make_plan(params, n, world, out_plan, true);
}

int fsdppack_plan_info(const fsdppack_plan *plan, int32_t *num_buckets, int32_t *num_params, int32_t *world)
{
    if (!plan_ok(plan)) return fail(FSDPPACK_ESTATE, "plan_info: invalid plan handle");
    if (num_buckets) *num_buckets = static_cast<int32_t>(plan->buckets.size());
    if (num_params) *num_params = plan->n;
    if (world) *world = plan->W;
    return FSDPPACK_OK;
}

int fsdppack_plan_bucket(const fsdppack_plan *plan, int32_t bucket, int32_t *reduce_dtype, int64_t *S,
                         int32_t *nmembers, const int32_t **members, const int64_t **P, const int64_t **O)
{
    if (!plan_ok(plan)) return fail(FSDPPACK_ESTATE, "plan_bucket: invalid plan handle");
    if (bucket < 0 || bucket >= static_cast<int32_t>(plan->buckets.size()))
        return fail(FSDPPACK_EINVAL, "plan_bucket: bucket index out of range");
    const BucketPlan &b = plan->buckets[bucket];
    if (reduce_dtype) *reduce_dtype = b.dtype;
    if (S) *S = b.S;
    if (nmembers) *nmembers = static_cast<int32_t>(b.members.size());
    if (members) *members = b.members.data();
    if (P) *P = b.P.data();
    if (O) *O = b.O.data();
    return FSDPPACK_OK;
}

int fsdppack_plan_all_gather_layout(const fsdppack_plan *plan, int64_t *B, const int64_t **P, const int64_t **A)
{
    if (!plan_ok(plan)) return fail(FSDPPACK_ESTATE, "plan_all_gather_layout: invalid plan handle");
    if (B) *B = plan->B;
    if (P) *P = plan->P.data();
    if (A) *A = plan->A.data();
    return FSDPPACK_OK;
}

int fsdppack_pack_reduce_scatter_input(const fsdppack_plan *cplan, int32_t bucket, const void *const *grads,
                                       void *out, void *stream)
{
    const ArmedEvents ev = take_armed_events();
    if (int rc = check_pack_args(cplan, bucket, grads, out, "pack_reduce_scatter_input")) return rc;
    fsdppack_plan *plan = const_cast<fsdppack_plan *>(cplan);
    const BucketPlan &b = plan->buckets[bucket];
    // the pack's pointer table is in member order (entry m = member m)
    std::vector<uint64_t> key(b.pack.table_params.size());
    for (size_t m = 0; m < key.size(); ++m) key[m] = reinterpret_cast<uint64_t>(grads[b.pack.table_params[m]]);
    try {
        return run_op(plan, b.pack, static_cast<size_t>(bucket), key, static_cast<char *>(out), stream, ev,
                      "pack_reduce_scatter_input");
    } catch (const std::bad_alloc &) {
        return fail(FSDPPACK_ENOMEM, "pack_reduce_scatter_input: out of host memory");
    }
}

int fsdppack_pack_reduce_scatter_input_noalloc(const fsdppack_plan *cplan, int32_t bucket, const void *const *grads,
                                               void *out, void *stream)
{
    const ArmedEvents ev = take_armed_events();
    if (int rc = check_pack_args(cplan, bucket, grads, out, "pack_reduce_scatter_input_noalloc")) return rc;
    const fsdppack_plan *plan = cplan;
    const OpTable &op = plan->buckets[bucket].pack;
    if (op.table_params.size() > static_cast<size_t>(kInlineLarge))
        return fail(FSDPPACK_EINVAL, "pack_reduce_scatter_input_noalloc: the bucket has more than " +
                                         std::to_string(kInlineLarge) + " members");
    // the bucket's tables: in the plan-wide image, else in its own
    const bool whole = !plan->scratch_image.empty() && plan->scratch_at[bucket] >= 0;
    if (!whole && op.scratch_image.empty() && op.scratch_need > 0)
        return fail(FSDPPACK_EINVAL, "pack_reduce_scatter_input_noalloc: the bucket's tables need " +
                                         std::to_string(op.scratch_need) + " bytes, more than the " +
                                         std::to_string(kScratchBytes) + "-byte scratch");
    const int32_t shift = static_cast<int32_t>(reinterpret_cast<uintptr_t>(out) & (kLineBytes - 1));
    if (op.windows(shift) <= 0) return FSDPPACK_OK;
    void *sp = nullptr;
    hipError_t e = static_cast<hipError_t>(scratch_address(&sp));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    int dev = -1;
    if ((e = hipGetDevice(&dev)) != hipSuccess) return hip_fail(e, "hipGetDevice");
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if ((e = hipStreamIsCapturing(static_cast<hipStream_t>(stream), &cap)) != hipSuccess)
        return hip_fail(e, "hipStreamIsCapturing");
    const unsigned char *img = whole ? plan->scratch_image.data() : op.scratch_image.data();
    const size_t img_bytes = whole ? plan->scratch_image.size() : op.scratch_image.size();
    const int32_t region = whole ? -1 : bucket;
    char *base = static_cast<char *>(sp) + (whole ? plan->scratch_at[bucket] : 0);
    {
        // Copy the image unless the scratch holds it; when it does and the
        // copy that put it there may still be in flight, the launch waits for
        // that copy on the device (whichever stream made it).  The plan's host
        // images live as long as the plan, and destroying a plan that copied
        // waits for the device, so a copy may complete after this call returns.
        // Under stream capture the copy becomes a node of the graph, ahead of
        // the kernel, and the scratch's contents are unknown from then on.
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        ScratchHolds &h = g_scratch_holds[dev];
        if (cap != hipStreamCaptureStatusNone) {
            h.captured = true;
            h.serial = 0;
        }
        if (!h.captured && h.copied == nullptr) {
            if ((e = hipEventCreateWithFlags(&h.copied, hipEventDisableTiming)) != hipSuccess) {
                h.copied = nullptr;
                return hip_fail(e, "hipEventCreate(scratch copy)");
            }
        }
        if (!h.captured && h.serial == plan->serial && h.region == region) {
            e = hipEventQuery(h.copied);
            if (e == hipErrorNotReady) {
                if ((e = hipStreamWaitEvent(static_cast<hipStream_t>(stream), h.copied, 0)) != hipSuccess)
                    return hip_fail(e, "hipStreamWaitEvent(scratch copy)");
            } else if (e != hipSuccess) {
                return hip_fail(e, "hipEventQuery(scratch copy)");
            }
        } else {
            h.serial = 0;   // unknown until the copy is enqueued
            plan->staged.store(true);
            e = hipMemcpyAsync(static_cast<char *>(sp), img, img_bytes, hipMemcpyHostToDevice,
                               static_cast<hipStream_t>(stream));
            if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync(tables to scratch)");
            if (!h.captured) {
                if ((e = hipEventRecord(h.copied, static_cast<hipStream_t>(stream))) != hipSuccess)
                    return hip_fail(e, "hipEventRecord(scratch copy)");
                h.serial = plan->serial;
                h.region = region;
            }
            g_counters[8]++;
        }
    }
    WindowArgs args = op.args(false, shift);
    args.members = base;
    args.columns = base + op.scratch_c_off;
    args.stretches = op.narrow ? reinterpret_cast<const PackStretch *>(base + op.scratch_s_off) : nullptr;
    args.table = nullptr;
    args.base = static_cast<char *>(out);
    // the pointer table travels in the launch's arguments
    uint64_t key[kInlineLarge];
    const int32_t nk = static_cast<int32_t>(op.table_params.size());
    for (int32_t m = 0; m < nk; ++m) key[m] = reinterpret_cast<uint64_t>(grads[op.table_params[m]]);
    const int le = launch_windows(args, key, nk, stream, ev.start, ev.stop);
    if (le != 0) return hip_fail(static_cast<hipError_t>(le), "pack_reduce_scatter_input_noalloc");
    g_counters[0]++;
    g_counters[6]++;
    return FSDPPACK_OK;
}

int fsdppack_all_gather_copy_in(const fsdppack_plan *cplan, int32_t rank, const void *const *shards, void *ag_out,
                                void *stream)
{
    const ArmedEvents ev = take_armed_events();
    fsdppack_plan *plan = const_cast<fsdppack_plan *>(cplan);
    if (!plan_ok(plan)) return fail(FSDPPACK_ESTATE, "all_gather_copy_in: invalid plan handle");
    if (rank < 0 || rank >= plan->W) return fail(FSDPPACK_EINVAL, "all_gather_copy_in: rank out of range");
    if (shards == nullptr) return fail(FSDPPACK_EINVAL, "all_gather_copy_in: shards is NULL");
    if (plan->flat) {
        // the rank's row of the flat parameter from its per-parameter pieces
        if (plan->B > 0 && (ag_out == nullptr || !aligned(ag_out, dtype_bytes(plan->copy_in.reduce_dt))))
            return fail(FSDPPACK_EINVAL, "all_gather_copy_in: ag_out is NULL or not aligned to its element size");
        const OpTable &op = plan->copy_in;
        std::vector<uint64_t> key(op.table_params.size(), 0);
        for (size_t m = 0; m < key.size(); ++m) {
            const int32_t t = op.table_params[m];
            if (shard_elements(*plan, t, rank) == 0) continue;
            const void *s = shards[t];
            if (s == nullptr || !aligned(s, dtype_bytes(plan->params[t].storage_dtype)))
                return fail(FSDPPACK_EINVAL, "all_gather_copy_in: shards[" + std::to_string(t) +
                                                 "] is NULL or not aligned to its element size");
            key[m] = reinterpret_cast<uint64_t>(s);
        }
        char *row = static_cast<char *>(ag_out) + static_cast<int64_t>(rank) * plan->B;
        try {
            return run_op(plan, op, plan->buckets.size(), key, row, stream, ev, "all_gather_copy_in", rank);
        } catch (const std::bad_alloc &) {
            return fail(FSDPPACK_ENOMEM, "all_gather_copy_in: out of host memory");
        }
    }
    if (plan->B > 0 && (ag_out == nullptr || !aligned(ag_out, 4)))
        return fail(FSDPPACK_EINVAL, "all_gather_copy_in: ag_out is NULL or not 4-byte aligned");
    // the table is in segment-record order (every parameter with P > 0)
    const OpTable &op = plan->copy_in;
    std::vector<uint64_t> key(op.table_params.size(), 0);
    for (size_t m = 0; m < key.size(); ++m) {
        const int32_t t = op.table_params[m];
        const void *s = shards[t];
        if (s == nullptr || !aligned(s, dtype_bytes(plan->params[t].storage_dtype)))
            return fail(FSDPPACK_EINVAL, "all_gather_copy_in: shards[" + std::to_string(t) +
                                             "] is NULL or not aligned to its element size");
        key[m] = reinterpret_cast<uint64_t>(s);
    }
    char *row = static_cast<char *>(ag_out) + static_cast<int64_t>(rank) * plan->B;
    try {
        return run_op(plan, op, plan->buckets.size(), key, row, stream, ev, "all_gather_copy_in");
    } catch (const std::bad_alloc &) {
        return fail(FSDPPACK_ENOMEM, "all_gather_copy_in: out of host memory");
    }
}

int fsdppack_all_gather_copy_out(const fsdppack_plan *cplan, const void *ag, void *const *params, void *stream)
{
    const ArmedEvents ev = take_armed_events();
    fsdppack_plan *plan = const_cast<fsdppack_plan *>(cplan);
    if (!plan_ok(plan)) return fail(FSDPPACK_ESTATE, "all_gather_copy_out: invalid plan handle");
    if (params == nullptr) return fail(FSDPPACK_EINVAL, "all_gather_copy_out: params is NULL");
    const int64_t ag_align = plan->flat && plan->n > 0 ? dtype_bytes(plan->params[0].param_dtype) : 4;
    if (plan->B > 0 && (ag == nullptr || !aligned(ag, ag_align)))
        return fail(FSDPPACK_EINVAL, "all_gather_copy_out: ag is NULL or misaligned");
    std::vector<uint64_t> key(plan->n, 0);
    for (int32_t t = 0; t < plan->n; ++t) {
        if (plan->numel[t] == 0) continue;
        void *d = params[t];
        if (d == nullptr || !aligned(d, dtype_bytes(plan->params[t].param_dtype)))
            return fail(FSDPPACK_EINVAL, "all_gather_copy_out: params[" + std::to_string(t) +
                                             "] is NULL or not aligned to its element size");
        key[t] = reinterpret_cast<uint64_t>(d);
    }
    try {
        return run_op(plan, plan->copy_out, plan->buckets.size() + 1, key,
                      const_cast<char *>(static_cast<const char *>(ag)), stream, ev, "all_gather_copy_out");
    } catch (const std::bad_alloc &) {
        return fail(FSDPPACK_ENOMEM, "all_gather_copy_out: out of host memory");
    }
}

namespace {
// The per-bucket write-back, with the timing events its caller took.
int reduce_scatter_copy_out(const fsdppack_plan *cplan, int32_t bucket, int32_t rank, const void *rs_out,
                            float divide_factor, void *const *shard_grads, void *stream, const ArmedEvents &ev)
{
    fsdppack_plan *plan = const_cast<fsdppack_plan *>(cplan);
    if (!plan_ok(plan)) return fail(FSDPPACK_ESTATE, "reduce_scatter_copy_out: invalid plan handle");
    if (bucket < 0 || bucket >= static_cast<int32_t>(plan->buckets.size()))
        return fail(FSDPPACK_EINVAL, "reduce_scatter_copy_out: bucket index out of range");
    if (rank < 0 || rank >= plan->W) return fail(FSDPPACK_EINVAL, "reduce_scatter_copy_out: rank out of range");
    if (!(divide_factor > 0.0f) || divide_factor > 3.4028235e38f)
        return fail(FSDPPACK_EINVAL, "reduce_scatter_copy_out: divide_factor must be finite and positive");
    if (shard_grads == nullptr) return fail(FSDPPACK_EINVAL, "reduce_scatter_copy_out: shard_grads is NULL");
    BucketPlan &b = plan->buckets[bucket];
    if (b.S > 0 && (rs_out == nullptr || !aligned(rs_out, dtype_bytes(b.dtype))))
        return fail(FSDPPACK_EINVAL, "reduce_scatter_copy_out: rs_out is NULL or not aligned to its element size");
    // the table is indexed by parameter (record order in a flat plan);
    // members with no real element on this rank (and non-members) are not
    // touched and may be NULL
    const bool by_record = plan->flat;
    std::vector<uint64_t> key(by_record ? b.write_back.table_params.size() : plan->n, 0);
    for (size_t k = 0; k < (by_record ? key.size() : b.members.size()); ++k) {
        const int32_t t = by_record ? b.write_back.table_params[k] : b.members[k];
        if (shard_elements(*plan, t, rank) == 0) continue;
        void *g = shard_grads[t];
        if (g == nullptr || !aligned(g, dtype_bytes(plan->params[t].storage_dtype)))
            return fail(FSDPPACK_EINVAL, "reduce_scatter_copy_out: shard_grads[" + std::to_string(t) +
                                             "] is NULL or not aligned to its element size");
        key[by_record ? k : static_cast<size_t>(t)] = reinterpret_cast<uint64_t>(g);
    }
    try {
        return run_op(plan, b.write_back, plan->buckets.size() + 2 + static_cast<size_t>(bucket), key,
                      const_cast<char *>(static_cast<const char *>(rs_out)), stream, ev, "reduce_scatter_copy_out",
                      rank, divide_factor);
    } catch (const std::bad_alloc &) {
        return fail(FSDPPACK_ENOMEM, "reduce_scatter_copy_out: out of host memory");
    }
}
}  // namespace

int fsdppack_reduce_scatter_copy_out(const fsdppack_plan *cplan, int32_t bucket, int32_t rank, const void *rs_out,
                                     float divide_factor, void *const *shard_grads, void *stream)
{
    const ArmedEvents ev = take_armed_events();
    return reduce_scatter_copy_out(cplan, bucket, rank, rs_out, divide_factor, shard_grads, stream, ev);
}

int fsdppack_reduce_scatter_copy_out_all(const fsdppack_plan *cplan, int32_t rank, const void *const *rs_outs,
                                         float divide_factor, void *const *shard_grads, void *stream)
{
    const ArmedEvents ev = take_armed_events();
    fsdppack_plan *plan = const_cast<fsdppack_plan *>(cplan);
    if (!plan_ok(plan)) return fail(FSDPPACK_ESTATE, "reduce_scatter_copy_out_all: invalid plan handle");
    if (rs_outs == nullptr) return fail(FSDPPACK_EINVAL, "reduce_scatter_copy_out_all: rs_outs is NULL");
    const int32_t nb = static_cast<int32_t>(plan->buckets.size());
    if (nb <= 1) {
        // one bucket: the same launch as the per-bucket call
        if (nb == 0) {
            if (rank < 0 || rank >= plan->W) return fail(FSDPPACK_EINVAL, "reduce_scatter_copy_out_all: rank out of range");
            if (!(divide_factor > 0.0f) || divide_factor > 3.4028235e38f)
                return fail(FSDPPACK_EINVAL, "reduce_scatter_copy_out_all: divide_factor must be finite and positive");
            return FSDPPACK_OK;
        }
        return reduce_scatter_copy_out(cplan, 0, rank, rs_outs[0], divide_factor, shard_grads, stream, ev);
    }
    if (rank < 0 || rank >= plan->W) return fail(FSDPPACK_EINVAL, "reduce_scatter_copy_out_all: rank out of range");
    if (!(divide_factor > 0.0f) || divide_factor > 3.4028235e38f)
        return fail(FSDPPACK_EINVAL, "reduce_scatter_copy_out_all: divide_factor must be finite and positive");
    if (shard_grads == nullptr) return fail(FSDPPACK_EINVAL, "reduce_scatter_copy_out_all: shard_grads is NULL");
    // the parameters' entries, then one per bucket: its reduced row
    std::vector<uint64_t> key(static_cast<size_t>(plan->n) + nb, 0);
    for (int32_t bi = 0; bi < nb; ++bi) {
        const BucketPlan &b = plan->buckets[bi];
        if (b.S > 0 && (rs_outs[bi] == nullptr || !aligned(rs_outs[bi], dtype_bytes(b.dtype))))
            return fail(FSDPPACK_EINVAL, "reduce_scatter_copy_out_all: rs_outs[" + std::to_string(bi) +
                                             "] is NULL or not aligned to its element size");
        key[static_cast<size_t>(plan->n) + bi] = reinterpret_cast<uint64_t>(rs_outs[bi]);
        for (int32_t t : b.members) {
            if (shard_elements(*plan, t, rank) == 0) continue;
            void *g = shard_grads[t];
            if (g == nullptr || !aligned(g, dtype_bytes(plan->params[t].storage_dtype)))
                return fail(FSDPPACK_EINVAL, "reduce_scatter_copy_out_all: shard_grads[" + std::to_string(t) +
                                                 "] is NULL or not aligned to its element size");
            key[t] = reinterpret_cast<uint64_t>(g);
        }
    }
    try {
        return run_op(plan, plan->write_back_all, 2 * plan->buckets.size() + 2, key, nullptr, stream, ev,
                      "reduce_scatter_copy_out_all", rank, divide_factor);
    } catch (const std::bad_alloc &) {
        return fail(FSDPPACK_ENOMEM, "reduce_scatter_copy_out_all: out of host memory");
    }
}

void fsdppack_plan_destroy(fsdppack_plan *plan)
{
    if (!plan_ok(plan)) return;
    {
        std::lock_guard<std::mutex> lock(plan->mu);
        // no kernel may still read the tables, and no copy into the scratch
        // still read the plan's host images
        if (plan->uploaded || plan->staged.load()) (void)hipDeviceSynchronize();
        for (PtrCache &c : plan->caches) {
            for (PtrSlot &s : c.slots) {
                if (s.ready) (void)hipEventDestroy(static_cast<hipEvent_t>(s.ready));
                for (void *ev : s.drain) (void)hipEventDestroy(static_cast<hipEvent_t>(ev));
                if (s.d_table) (void)hipFree(s.d_table);
                if (s.h_stage) (void)hipHostFree(s.h_stage);
            }
        }
        auto free_table = [](OpTable &op) {
            if (op.d_members) (void)hipFree(op.d_members);
            if (op.d_columns) (void)hipFree(op.d_columns);
            if (op.d_stretches) (void)hipFree(op.d_stretches);
            op.d_members = nullptr;
            op.d_columns = nullptr;
            op.d_stretches = nullptr;
        };
        for (BucketPlan &b : plan->buckets) {
            free_table(b.pack);
            free_table(b.write_back);
        }
        free_table(plan->copy_in);
        free_table(plan->copy_out);
        free_table(plan->write_back_all);
        plan->magic = 0;
    }
    delete plan;
}

const char *fsdppack_last_error(void) { return g_error.c_str(); }

int fsdppack_time_next_launch(void *start_event, void *stop_event)
{
    g_next_start = start_event;
    g_next_stop = stop_event;
    return FSDPPACK_OK;
}

int fsdppack_empty_launch(int32_t workgroups, int32_t threads, void *stream)
{
    const ArmedEvents ev = take_armed_events();
    if (workgroups < 1 || threads < 64 || threads > 1024 || threads % 64 != 0 ||
        static_cast<int64_t>(workgroups) * threads >= (int64_t{1} << 32))
        return fail(FSDPPACK_EINVAL, "empty_launch: workgroups must be >= 1 and threads a multiple of 64 in [64, 1024], "
                                     "fewer than 2^32 work-items in all");
    const int le = launch_empty(workgroups, threads, stream, ev.start, ev.stop);
    if (le != 0) return hip_fail(static_cast<hipError_t>(le), "empty_launch");
    return FSDPPACK_OK;
}

int fsdppack_counters(int64_t *counters, int32_t n)
{
    if (counters == nullptr || n < 0) return fail(FSDPPACK_EINVAL, "counters: bad arguments");
    for (int32_t i = 0; i < n && i < kCounters; ++i) counters[i] = g_counters[i].load();
    return FSDPPACK_OK;
}

}  // extern "C"
