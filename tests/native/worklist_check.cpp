// worklist_check.cpp -- host-side bounds check of libfsdppack's work lists.
//
// Builds a plan with the library's own planner (fsdppack_plan.cpp, compiled
// into this program with the address and undefined-behaviour sanitizers) and
// checks, for every work list the kernels would run, the invariants the
// grouped segment kernel relies on:
//  * the item array is a sentinel-terminated, strictly increasing list of
//    (segment, offset) starts inside the segment array;
//  * every segment's destination range lies inside its destination buffer,
//    its source range (the `valid` prefix) inside its source buffer, its
//    pointer-table slot inside the table, and its dtypes are supported;
//  * walking the items exactly as the kernel does writes every destination
//    byte exactly once (checked on the sorted list of written intervals).
//
// Input (stdin): "world item_bytes n" then n lines
// "dim0 inner grad reduce storage param".  Prints "OK" or the first failure.
#include <algorithm>
#include <cstdio>
#include <cstring>
#include <utility>
#include <string>
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

// dst_size(seg): bytes of the buffer the segment writes into;
// src_size(seg): bytes of the buffer it reads from.
template <typename DstSize, typename SrcSize>
static bool check_list(const char *name, const WorkList &wl, int32_t n, DstSize dst_size, SrcSize src_size,
                       std::vector<std::vector<std::pair<int64_t, int64_t>>> &written)
{
    const int64_t nseg = static_cast<int64_t>(wl.segs.size());
    CHECK(!wl.items.empty(), "%s: empty item array", name);
    const Item &sent = wl.items.back();
    CHECK(sent.seg == nseg && sent.off == 0, "%s: bad sentinel (%d,%lld)", name, sent.seg, (long long)sent.off);
    for (size_t k = 0; k + 1 < wl.items.size(); ++k) {
        const Item &a = wl.items[k], &b = wl.items[k + 1];
        CHECK(a.seg >= 0 && a.seg < nseg, "%s: item %zu segment %d out of range", name, k, a.seg);
        CHECK(a.off >= 0 && a.off < wl.segs[a.seg].len, "%s: item %zu offset out of range", name, k);
        CHECK(a.seg < b.seg || (a.seg == b.seg && a.off < b.off), "%s: items %zu,%zu not increasing", name, k, k + 1);
    }
    for (int64_t i = 0; i < nseg; ++i) {
        const Seg &g = wl.segs[i];
        CHECK(dtype_ok(g.src_dt) && dtype_ok(g.dst_dt), "%s: segment %lld bad dtype", name, (long long)i);
        CHECK(g.slot >= 0 && g.slot < n, "%s: segment %lld slot %d out of range", name, (long long)i, g.slot);
        CHECK(g.len >= 0 && g.valid >= 0 && g.valid <= g.len, "%s: segment %lld bad len/valid", name, (long long)i);
        const int64_t dend = g.dst_off + g.len * dtype_bytes(g.dst_dt);
        CHECK(g.dst_off >= 0 && dend <= dst_size(g), "%s: segment %lld writes [%lld,%lld) past %lld", name,
              (long long)i, (long long)g.dst_off, (long long)dend, (long long)dst_size(g));
        CHECK(g.dst_off % dtype_bytes(g.dst_dt) == 0, "%s: segment %lld destination misaligned", name, (long long)i);
        if (g.valid > 0) {
            const int64_t send = g.src_off + g.valid * dtype_bytes(g.src_dt);
            CHECK(g.src_off >= 0 && send <= src_size(g), "%s: segment %lld reads [%lld,%lld) past %lld", name,
                  (long long)i, (long long)g.src_off, (long long)send, (long long)src_size(g));
        }
    }
    // walk items the way the kernel does and mark written bytes
    for (size_t k = 0; k + 1 < wl.items.size(); ++k) {
        const Item first = wl.items[k], last = wl.items[k + 1];
        for (int32_t s = first.seg; s < last.seg || (s == last.seg && last.off > 0); ++s) {
            CHECK(s < nseg, "%s: item walk reads segment %d of %lld", name, s, (long long)nseg);
            const Seg &g = wl.segs[s];
            const int64_t lo = (s == first.seg) ? first.off : 0;
            const int64_t hi = (s == last.seg) ? last.off : g.len;
            if (hi <= lo) continue;
            CHECK(hi <= g.len, "%s: range past segment end", name);
            const int64_t esz = dtype_bytes(g.dst_dt);
            const int buf = g.table_side == kTableIsDest ? g.slot : 0;
            written[buf].emplace_back(g.dst_off + lo * esz, g.dst_off + hi * esz);
        }
    }
    return true;
}

// The written intervals of one buffer must tile [0, size) exactly.
static bool tiles(std::vector<std::pair<int64_t, int64_t>> v, int64_t size, const char *name)
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
    long long item_bytes;
    if (std::scanf("%d %lld %d", &world, &item_bytes, &n) != 3) { std::puts("FAIL bad header"); return 1; }
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
    if (build_plan(d.data(), n, world, item_bytes, &plan, err) != FSDPPACK_OK) {
        std::printf("FAIL plan: %s\n", err.c_str());
        return 1;
    }
    const int64_t W = plan.W;
    auto grad_bytes = [&](const Seg &g) { return plan.numel[g.slot] * dtype_bytes(plan.params[g.slot].grad_dtype); };
    for (size_t bi = 0; bi < plan.buckets.size(); ++bi) {
        const BucketPlan &b = plan.buckets[bi];
        const int64_t out_bytes = W * b.S * dtype_bytes(b.dtype);
        std::vector<std::vector<std::pair<int64_t, int64_t>>> written(1);
        char name[64];
        std::snprintf(name, sizeof name, "pack[%zu]", bi);
        if (!check_list(name, b.pack, n, [&](const Seg &) { return out_bytes; }, grad_bytes, written) ||
            !tiles(written[0], out_bytes, name)) {
            std::printf("FAIL %s\n", g_fail.c_str());
            return 1;
        }
    }
    {
        std::vector<std::vector<std::pair<int64_t, int64_t>>> written(1);
        auto shard_bytes = [&](const Seg &g) { return plan.P[g.slot] * dtype_bytes(plan.params[g.slot].storage_dtype); };
        if (!check_list("copy_in", plan.copy_in, n, [&](const Seg &) { return plan.B; }, shard_bytes, written) ||
            !tiles(written[0], plan.B, "copy_in")) {
            std::printf("FAIL %s\n", g_fail.c_str());
            return 1;
        }
    }
    {
        std::vector<std::vector<std::pair<int64_t, int64_t>>> written(n);
        auto param_bytes = [&](const Seg &g) { return plan.numel[g.slot] * dtype_bytes(plan.params[g.slot].param_dtype); };
        if (!check_list("copy_out", plan.copy_out, n, param_bytes, [&](const Seg &) { return W * plan.B; }, written)) {
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
    std::printf("OK %zu buckets, items:", plan.buckets.size());
    for (const BucketPlan &b : plan.buckets) std::printf(" %d", b.pack.n_items());
    std::printf(" copy_in %d copy_out %d\n", plan.copy_in.n_items(), plan.copy_out.n_items());
    return 0;
}
