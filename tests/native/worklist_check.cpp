// worklist_check.cpp -- host-side bounds check of libfsdppack's launches.
//
// Builds a plan with the library's own planner (fsdppack_plan.cpp, compiled
// into this program with the address and undefined-behaviour sanitizers) and
// walks every window of every operation through the very window -> range
// mapping the kernels run (fsdppack_internal.h, compiled for the host here),
// checking the invariants the kernels rely on:
//  * each range lies inside its chunk, reads only the source bytes of its
//    `valid` prefix, and writes inside its destination buffer;
//  * ranges use a valid pointer-table slot and supported dtypes;
//  * over all windows of a launch, every destination byte is written exactly
//    once (checked on the sorted list of written intervals).
//
// Input (stdin): "world n" then n lines
// "dim0 inner grad reduce storage param".  Prints "OK" or the first failure.
#include <algorithm>
#include <cstdio>
#include <cstring>
#include <string>
#include <utility>
#include <vector>

#include "../../fsdp2_mixed_dtype_amd/csrc/fsdppack_plan.h"

using namespace fsdppack;

static std::string g_fail;

#define CHECK(cond, ...)                                                  \
    do {                                                                  \
        if (!(cond)) {                                                    \
            char buf[512];                                                \
            std::snprintf(buf, sizeof buf, __VA_ARGS__);                  \
            g_fail = buf;                                                 \
            return false;                                                 \
        }                                                                 \
    } while (0)

using Intervals = std::vector<std::pair<int64_t, int64_t>>;

// Check one range produced for window w.
template <typename DstSize, typename SrcSize>
static bool check_range(const char *name, int32_t w, const RangeRef &g, const OpTable &op, int32_t nparams,
                        DstSize dst_size, SrcSize src_size, std::vector<Intervals> &written)
{
    CHECK(dtype_ok(g.src_dt) && dtype_ok(g.dst_dt), "%s: window %d bad dtype", name, w);
    const int32_t entries = op.op == kOpPack ? op.n : nparams;     // pointer-table entries
    CHECK(g.slot >= 0 && g.slot < entries, "%s: window %d slot %d out of range", name, w, g.slot);
    CHECK(g.param >= 0 && g.param < nparams, "%s: window %d param %d out of range", name, w, g.param);
    CHECK(op.op != kOpPack || op.table_params[g.slot] == g.param, "%s: window %d table entry mismatch", name, w);
    CHECK(g.lo >= 0 && g.lo < g.hi, "%s: window %d empty or reversed range", name, w);
    CHECK(g.valid >= 0, "%s: window %d negative valid", name, w);
    const int64_t dsz = dtype_bytes(g.dst_dt), ssz = dtype_bytes(g.src_dt);
    const int64_t d0 = g.dst_off + g.lo * dsz, d1 = g.dst_off + g.hi * dsz;
    CHECK(g.dst_off >= 0 && g.dst_off % dsz == 0 && d1 <= dst_size(g), "%s: window %d writes [%lld,%lld) past %lld",
          name, w, (long long)d0, (long long)d1, (long long)dst_size(g));
    if (g.lo < g.valid) {
        const int64_t s1 = g.src_off + std::min(g.hi, g.valid) * ssz;
        CHECK(g.src_off >= 0 && s1 <= src_size(g), "%s: window %d reads up to %lld past %lld", name, w,
              (long long)s1, (long long)src_size(g));
    }
    written[g.table_side == kTableIsDest ? g.param : 0].emplace_back(d0, d1);
    return true;
}

template <typename DstSize, typename SrcSize>
static bool check_op(const char *name, const OpTable &op, int32_t W, int32_t nparams, DstSize dst_size,
                     SrcSize src_size, std::vector<Intervals> &written)
{
    WindowArgs a = op.args(false);
    a.W = W;
    const size_t rec = op.op == kOpPack ? sizeof(PackMember)
                       : op.op == kOpCopyIn ? sizeof(CopyInMember) : sizeof(CopyOutTensor);
    CHECK(op.members.size() == static_cast<size_t>(op.n) * rec, "%s: member table size", name);
    CHECK(op.n_windows == 0 || op.n > 0, "%s: windows without members", name);
    CHECK(op.op != kOpPack || (op.columns.size() == static_cast<size_t>(op.gx) &&
                               op.table_params.size() == static_cast<size_t>(op.n)), "%s: column map size", name);
    for (int32_t w = 0; w < op.n_windows; ++w) {
        int ranges = 0;
        bool ok = true;
        for_each_range(a, w, [&](const RangeRef &g) {
            if (ok) ok = check_range(name, w, g, op, nparams, dst_size, src_size, written);
            ++ranges;
        });
        if (!ok) return false;
        CHECK(ranges > 0, "%s: window %d has no range", name, w);
    }
    return true;
}

// The written intervals of one buffer must tile [0, size) exactly.
static bool tiles(Intervals v, int64_t size, const char *name)
{
    std::sort(v.begin(), v.end());
    int64_t at = 0;
    for (const auto &iv : v) {
        CHECK(iv.first == at, "%s: bytes [%lld,%lld) %s", name, (long long)std::min(at, iv.first),
              (long long)std::max(at, iv.first), iv.first < at ? "written twice" : "never written");
        at = iv.second;
    }
    CHECK(at == size, "%s: bytes [%lld,%lld) never written", name, (long long)at, (long long)size);
    return true;
}

int main()
{
    int32_t world, n;
    if (std::scanf("%d %d", &world, &n) != 2) { std::puts("FAIL bad header"); return 1; }
    std::vector<fsdppack_param_desc> d(n);
    for (int32_t i = 0; i < n; ++i) {
        long long a, b;
        if (std::scanf("%lld %lld %d %d %d %d", &a, &b, &d[i].grad_dtype, &d[i].reduce_dtype, &d[i].storage_dtype,
                       &d[i].param_dtype) != 6) { std::puts("FAIL bad line"); return 1; }
        d[i].dim0 = a;
        d[i].inner = b;
    }
    fsdppack_plan plan;
    std::string err;
    if (build_plan(d.data(), n, world, &plan, err) != FSDPPACK_OK) {
        std::printf("FAIL plan: %s\n", err.c_str());
        return 1;
    }
    const int64_t W = plan.W;
    auto grad_bytes = [&](const RangeRef &g) { return plan.numel[g.param] * dtype_bytes(plan.params[g.param].grad_dtype); };
    for (size_t bi = 0; bi < plan.buckets.size(); ++bi) {
        const BucketPlan &b = plan.buckets[bi];
        const int64_t out_bytes = W * b.S * dtype_bytes(b.dtype);
        std::vector<Intervals> written(1);
        char name[64];
        std::snprintf(name, sizeof name, "pack[%zu]", bi);
        if (!check_op(name, b.pack, plan.W, n, [&](const RangeRef &) { return out_bytes; }, grad_bytes, written) ||
            !tiles(written[0], out_bytes, name)) {
            std::printf("FAIL %s\n", g_fail.c_str());
            return 1;
        }
    }
    {
        std::vector<Intervals> written(1);
        auto shard_bytes = [&](const RangeRef &g) { return plan.P[g.param] * dtype_bytes(plan.params[g.param].storage_dtype); };
        if (!check_op("copy_in", plan.copy_in, plan.W, n, [&](const RangeRef &) { return plan.B; }, shard_bytes,
                      written) ||
            !tiles(written[0], plan.B, "copy_in")) {
            std::printf("FAIL %s\n", g_fail.c_str());
            return 1;
        }
    }
    {
        std::vector<Intervals> written(n);
        auto param_bytes = [&](const RangeRef &g) { return plan.numel[g.param] * dtype_bytes(plan.params[g.param].param_dtype); };
        if (!check_op("copy_out", plan.copy_out, plan.W, n, param_bytes, [&](const RangeRef &) { return W * plan.B; },
                      written)) {
            std::printf("FAIL %s\n", g_fail.c_str());
            return 1;
        }
        for (int32_t t = 0; t < n; ++t) {
            char name[64];
            std::snprintf(name, sizeof name, "copy_out param %d", t);
            if (!tiles(written[t], plan.numel[t] * dtype_bytes(plan.params[t].param_dtype), name)) {
                std::printf("FAIL %s\n", g_fail.c_str());
                return 1;
            }
        }
    }
    std::printf("OK %zu buckets, windows:", plan.buckets.size());
    for (const BucketPlan &b : plan.buckets) std::printf(" %d", b.pack.n_windows);
    std::printf(" copy_in %d copy_out %d\n", plan.copy_in.n_windows, plan.copy_out.n_windows);
    return 0;
}
