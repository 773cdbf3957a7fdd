// worklist_check.cpp -- host-side bounds check of libfsdppack's work lists.
//
// Builds a plan with the library's own planner (fsdppack_plan.cpp, compiled
// into this program with the address and undefined-behaviour sanitizers) and
// checks, for every work list the kernels would run, the invariants the
// grouped segment kernel relies on:
//  * the item records are stored by a bijective slot map, each covers a
//    non-empty range inside the segment array, and consecutive items meet
//    exactly (the last one ends the list);
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
static bool check_list(const char *name, const WorkList &wl, int32_t nparams, DstSize dst_size, SrcSize src_size,
                       std::vector<std::vector<std::pair<int64_t, int64_t>>> &written)
{
    const int64_t nseg = static_cast<int64_t>(wl.segs.size());
    const int32_t n = static_cast<int32_t>(wl.items.size());
    // item_slot must be a bijection on [0, n)
    std::vector<uint8_t> hit(n, 0);
    for (int32_t b = 0; b < n; ++b) {
        const int32_t slot = item_slot(b, n);
        CHECK(slot >= 0 && slot < n && !hit[slot], "%s: item_slot not a bijection at %d", name, b);
        hit[slot] = 1;
    }
    for (int32_t b = 0; b < n; ++b) {
        const Item &it = wl.items[item_slot(b, n)];
        CHECK(it.seg_a >= 0 && it.seg_a < nseg, "%s: item %d start segment %d out of range", name, b, it.seg_a);
        CHECK(it.off_a >= 0 && it.off_a < wl.segs[it.seg_a].len, "%s: item %d start offset out of range", name, b);
        CHECK(it.seg_b >= 0 && it.seg_b <= nseg, "%s: item %d end segment out of range", name, b);
        CHECK(it.seg_b < nseg ? (it.off_b >= 0 && it.off_b < wl.segs[it.seg_b].len) : it.off_b == 0,
              "%s: item %d end offset out of range", name, b);
        CHECK(it.seg_a < it.seg_b || (it.seg_a == it.seg_b && it.off_a < it.off_b), "%s: item %d empty or reversed",
              name, b);
        if (b + 1 < n) {
            const Item &nx = wl.items[item_slot(b + 1, n)];
            CHECK(nx.seg_a == it.seg_b && nx.off_a == it.off_b, "%s: item %d does not end where %d starts", name, b, b + 1);
        } else {
            CHECK(it.seg_b == nseg && it.off_b == 0, "%s: last item does not end the list", name);
        }
    }
    for (int64_t i = 0; i < nseg; ++i) {
        const Seg &g = wl.segs[i];
        CHECK(dtype_ok(g.src_dt) && dtype_ok(g.dst_dt), "%s: segment %lld bad dtype", name, (long long)i);
        CHECK(g.slot >= 0 && g.slot < nparams, "%s: segment %lld slot %d out of range", name, (long long)i, g.slot);
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
    // walk items the way the kernel does and record written byte ranges
    for (int32_t b = 0; b < n; ++b) {
        const Item it = wl.items[item_slot(b, n)];
        for (int32_t s = it.seg_a; s < it.seg_b || (s == it.seg_b && it.off_b > 0); ++s) {
            CHECK(s < nseg, "%s: item walk reads segment %d of %lld", name, s, (long long)nseg);
            const Seg &g = wl.segs[s];
            const int64_t lo = (s == it.seg_a) ? it.off_a : 0;
            const int64_t hi = (s == it.seg_b) ? it.off_b : g.len;
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
