// fsdppack_plan.cpp -- host planner of libfsdppack (no HIP calls).
//
// Buckets: one per effective reduction dtype (the policy's reduce dtype, or
// the gradient's own dtype when unset), in order of first appearance, each
// keeping its members in unit order -- "PyTorch adds per-parameter mixed
// precision to FSDP2" (ainewsletter.today), paragraph 2.
//
// Rank chunks: parameter t viewed as [dim0, inner] gives rank r the rows
// [r*c, (r+1)*c), c = ceil(dim0 / W), padded on the right to P = c * inner
// elements -- "The unit you wrapped" (kernels.rudrite.com), the padding
// paragraphs (every rank holds a shard of the padded size).
//
// All-gather row: each parameter's P elements in its compute dtype at a
// 16-byte aligned byte offset, unit order, so that one all-gather carries
// mixed target dtypes ("PyTorch adds per-parameter mixed precision to
// FSDP2", paragraph 1).
#include "fsdppack_plan.h"

#include <algorithm>
#include <climits>
#include <map>

namespace fsdppack {
namespace {

bool mul_ok(int64_t a, int64_t b, int64_t &out) { return !__builtin_mul_overflow(a, b, &out); }
bool add_ok(int64_t a, int64_t b, int64_t &out) { return !__builtin_add_overflow(a, b, &out); }

int64_t round_up16(int64_t x) { return (x + 15) / 16 * 16; }

// Largest byte count any offset may reach; keeps every derived sum in range.
constexpr int64_t kMaxBytes = INT64_MAX / 4;

}  // namespace

void build_items(const std::vector<Seg> &segs, const std::vector<int64_t> &vpos, int64_t item_bytes,
                 std::vector<Item> &items)
{
    // item starts in list order: a new item wherever the virtual position
    // crosses a multiple of item_bytes
    struct Start { int32_t seg; int64_t off; };
    std::vector<Start> starts;
    int64_t current = -1;   // virtual window of the item being filled
    for (size_t i = 0; i < segs.size(); ++i) {
        const Seg &g = segs[i];
        if (g.len == 0) continue;
        const int64_t esz = dtype_bytes(g.dst_dt);
        const int64_t a = vpos[i], e = vpos[i] + g.len * esz;
        const int64_t k0 = a / item_bytes, k1 = (e - 1) / item_bytes;
        for (int64_t k = k0; k <= k1; ++k) {
            if (k == current) continue;   // the open item runs on into this segment
            const int64_t off = (k == k0) ? 0 : (k * item_bytes - a) / esz;
            starts.push_back(Start{static_cast<int32_t>(i), off});
            current = k;
        }
    }
    const int32_t n = static_cast<int32_t>(starts.size());
    items.assign(n, Item{});
    for (int32_t b = 0; b < n; ++b) {
        Item it{};
        it.seg_a = starts[b].seg;
        it.off_a = starts[b].off;
        if (b + 1 < n) { it.seg_b = starts[b + 1].seg; it.off_b = starts[b + 1].off; }
        else { it.seg_b = static_cast<int32_t>(segs.size()); it.off_b = 0; }
        items[item_slot(b, n)] = it;
    }
}

int build_plan(const fsdppack_param_desc *params, int32_t n, int32_t world, int64_t item_bytes,
               fsdppack_plan *plan, std::string &err)
{
    if (n < 0 || (n > 0 && params == nullptr)) { err = "plan_buckets: params is NULL or n < 0"; return FSDPPACK_EINVAL; }
    if (world < 1) { err = "plan_buckets: world size must be >= 1"; return FSDPPACK_EINVAL; }
    if (item_bytes < 256 || item_bytes % 16) { err = "plan_buckets: bad work-item size"; return FSDPPACK_EINVAL; }
    const int64_t W = world;
    plan->W = world;
    plan->n = n;
    plan->item_bytes = item_bytes;
    plan->params.assign(params, params + n);
    plan->numel.resize(n);
    plan->P.resize(n);
    plan->A.resize(n);

    for (int32_t t = 0; t < n; ++t) {
        const fsdppack_param_desc &p = params[t];
        if (!dtype_ok(p.grad_dtype) || !dtype_ok(p.storage_dtype) || !dtype_ok(p.param_dtype) ||
            !(p.reduce_dtype == kNone || dtype_ok(p.reduce_dtype))) {
            err = "plan_buckets: parameter " + std::to_string(t) + " has an unsupported dtype code";
            return FSDPPACK_EDTYPE;
        }
        if (p.dim0 < 0 || p.inner < 0) {
            err = "plan_buckets: parameter " + std::to_string(t) + " has a negative dimension";
            return FSDPPACK_EINVAL;
        }
        const int64_t rows = p.dim0 == 0 ? 0 : (p.dim0 - 1) / W + 1;   // ceil(dim0 / W)
        int64_t numel, chunk, all_ranks, bytes;
        if (!mul_ok(p.dim0, p.inner, numel) || !mul_ok(rows, p.inner, chunk) ||
            !mul_ok(chunk, W, all_ranks) || !mul_ok(all_ranks, 4, bytes) || bytes > kMaxBytes) {
            err = "plan_buckets: parameter " + std::to_string(t) + " is too large";
            return FSDPPACK_EINVAL;
        }
        plan->numel[t] = numel;
        plan->P[t] = chunk;
    }

    // buckets by effective reduction dtype, first appearance order
    std::map<int32_t, size_t> index_of;
    for (int32_t t = 0; t < n; ++t) {
        const fsdppack_param_desc &p = params[t];
        const int32_t eff = p.reduce_dtype != kNone ? p.reduce_dtype : p.grad_dtype;
        auto it = index_of.find(eff);
        if (it == index_of.end()) {
            it = index_of.emplace(eff, plan->buckets.size()).first;
            plan->buckets.emplace_back();
            plan->buckets.back().dtype = eff;
        }
        BucketPlan &b = plan->buckets[it->second];
        b.members.push_back(t);
        b.P.push_back(plan->P[t]);
        b.O.push_back(b.S);
        int64_t s2, row_bytes;
        if (!add_ok(b.S, plan->P[t], s2) || !mul_ok(s2, W * 4, row_bytes) || row_bytes > kMaxBytes) {
            err = "plan_buckets: reduce-scatter buffer too large";
            return FSDPPACK_EINVAL;
        }
        b.S = s2;
    }

    // all-gather row layout
    int64_t cursor = 0;
    for (int32_t t = 0; t < n; ++t) {
        plan->A[t] = round_up16(cursor);
        cursor = plan->A[t] + plan->P[t] * dtype_bytes(plan->params[t].param_dtype);
        if (cursor > kMaxBytes / W) { err = "plan_buckets: all-gather buffer too large"; return FSDPPACK_EINVAL; }
    }
    plan->B = round_up16(cursor);

    // ---- work lists
    std::vector<int64_t> vpos;
    for (BucketPlan &b : plan->buckets) {
        // reduce-scatter pack: rank-major, members in unit order, i.e. the
        // order of the [W, S] destination in memory
        WorkList &wl = b.pack;
        const int64_t dsz = dtype_bytes(b.dtype);
        vpos.clear();
        for (int64_t r = 0; r < W; ++r) {
            for (size_t k = 0; k < b.members.size(); ++k) {
                const int32_t t = b.members[k];
                const int64_t Pt = b.P[k];
                if (Pt == 0) continue;
                const int64_t valid = std::max<int64_t>(0, std::min<int64_t>(Pt, plan->numel[t] - r * Pt));
                Seg g{};
                g.dst_off = (r * b.S + b.O[k]) * dsz;
                g.src_off = r * Pt * dtype_bytes(plan->params[t].grad_dtype);
                g.len = Pt;
                g.valid = valid;
                g.slot = t;
                g.src_dt = static_cast<uint8_t>(plan->params[t].grad_dtype);
                g.dst_dt = static_cast<uint8_t>(b.dtype);
                g.table_side = kTableIsSource;
                wl.segs.push_back(g);
                vpos.push_back(g.dst_off);
                wl.src_bytes += valid * dtype_bytes(g.src_dt);
            }
        }
        wl.dst_bytes = W * b.S * dsz;
        if (wl.segs.size() > static_cast<size_t>(INT32_MAX) - 1) { err = "plan_buckets: too many rank chunks"; return FSDPPACK_EINVAL; }
        build_items(wl.segs, vpos, item_bytes, wl.items);
    }

    {   // all-gather copy-in: one segment per parameter, each covering its
        // 16-byte aligned slot (cast shard, then zero gap up to the next
        // slot); grouped by (storage, param) dtype pair, unit order inside
        WorkList &wl = plan->copy_in;
        std::map<int32_t, int32_t> pair_group;   // dtype pair -> first-appearance index
        std::vector<int32_t> group(n), order(n);
        for (int32_t t = 0; t < n; ++t) {
            const int32_t key = plan->params[t].storage_dtype * 4 + plan->params[t].param_dtype;
            group[t] = pair_group.emplace(key, static_cast<int32_t>(pair_group.size())).first->second;
            order[t] = t;
        }
        std::stable_sort(order.begin(), order.end(),
                         [&](int32_t x, int32_t y) { return group[x] < group[y]; });
        vpos.clear();
        int64_t v = 0;
        for (int32_t t : order) {
            const int64_t next = (t + 1 < n) ? plan->A[t + 1] : plan->B;
            const int64_t span = next - plan->A[t];
            if (span == 0) continue;
            const int64_t psz = dtype_bytes(plan->params[t].param_dtype);
            Seg g{};
            g.dst_off = plan->A[t];
            g.src_off = 0;
            g.len = span / psz;
            g.valid = plan->P[t];
            g.slot = t;
            g.src_dt = static_cast<uint8_t>(plan->params[t].storage_dtype);
            g.dst_dt = static_cast<uint8_t>(plan->params[t].param_dtype);
            g.table_side = kTableIsSource;
            wl.segs.push_back(g);
            vpos.push_back(v);
            v += span;
            wl.src_bytes += plan->P[t] * dtype_bytes(g.src_dt);
        }
        wl.dst_bytes = plan->B;
        build_items(wl.segs, vpos, item_bytes, wl.items);
    }

    {   // all-gather copy-out: per parameter, per rank, the non-padding part
        // of the gathered segment back into the full tensor
        WorkList &wl = plan->copy_out;
        vpos.clear();
        int64_t v = 0;
        for (int32_t t = 0; t < n; ++t) {
            const int64_t psz = dtype_bytes(plan->params[t].param_dtype);
            const int64_t Pt = plan->P[t];
            v = round_up16(v);
            for (int64_t r = 0; r < W && Pt > 0; ++r) {
                const int64_t valid = std::max<int64_t>(0, std::min<int64_t>(Pt, plan->numel[t] - r * Pt));
                if (valid == 0) break;
                Seg g{};
                g.dst_off = r * Pt * psz;
                g.src_off = r * plan->B + plan->A[t];
                g.len = valid;
                g.valid = valid;
                g.slot = t;
                g.src_dt = static_cast<uint8_t>(plan->params[t].param_dtype);
                g.dst_dt = g.src_dt;
                g.table_side = kTableIsDest;
                wl.segs.push_back(g);
                vpos.push_back(v + g.dst_off);
            }
            v += plan->numel[t] * psz;
            wl.src_bytes += plan->numel[t] * psz;
        }
        wl.dst_bytes = wl.src_bytes;
        if (wl.segs.size() > static_cast<size_t>(INT32_MAX) - 1) { err = "plan_buckets: too many rank chunks"; return FSDPPACK_EINVAL; }
        build_items(wl.segs, vpos, item_bytes, wl.items);
    }
    return FSDPPACK_OK;
}

}  // namespace fsdppack
