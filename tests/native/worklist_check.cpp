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
//    once (checked on the sorted list of written intervals);
//  * for the pack and the copy-in, whose windows follow memory, each window
//    starts and ends on a cache-line boundary of memory unless it starts or
//    ends with its row, for several offsets of the destination past a line
//    boundary; only the pack's spare window at the end of a row may have no
//    range;
//  * a pack or copy-in window that takes the kernel's direct copy (for the
//    pack also through the stretch records of a made-up pointer set) is
//    exactly the one range the general walk gives for it, the pack's 2-D
//    grid maps every workgroup to the window the linear index names, and a copy-out window the
//    kernel gathers element by element reads, for every element, the byte
//    the chunk walk reads for it, and a copy-in window it gathers vector by
//    vector takes each vector from the record the walk takes it from;
//  * the record maps have one entry per 2^map_lg bytes of a row (pack,
//    copy-in, flat ops; at least a window) or per group of windows
//    (copy-out, write-back);
//  * the reduce-scatter write-back of every rank (a sample of ranks for large
//    W) writes each member's real rank-chunk elements exactly once and reads
//    only the rank's reduced row.
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
static int64_t g_direct = 0;      // pack windows taking the direct copy (column map)
static int64_t g_direct_st = 0;   // pack windows taking it through the stretch records
static int64_t g_direct_flat = 0;   // flat copy-in windows taking the direct copy
static int64_t g_direct_in = 0;   // copy-in windows taking it
static int64_t g_gather = 0;      // copy-out windows gathered element by element
static int64_t g_scratch_images = 0;   // buckets whose tables fit the allocation-free pack's scratch

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
static bool check_range(const char *name, int32_t w, int32_t shift, const RangeRef &g, const OpTable &op,
                        int32_t nparams, DstSize dst_size, SrcSize src_size, std::vector<Intervals> &written)
{
    CHECK(dtype_ok(g.src_dt) && dtype_ok(g.dst_dt), "%s: window %d bad dtype", name, w);
    CHECK(g.lo >= 0 && g.lo < g.hi, "%s: window %d empty or reversed range", name, w);
    const bool by_record = op.op == kOpPack || op.op == kOpCopyIn || op.op == kOpWriteBackFlat || op.op == kOpCopyInFlat;
    if (g.param < 0) {
        // a flat copy-in's padding: +0 only, no source and no table entry
        CHECK(op.op == kOpCopyInFlat && g.valid == 0 && g.table_side == kTableIsSource,
              "%s: window %d has a range without a parameter", name, w);
        const int64_t d1 = g.dst_off + g.hi * dtype_bytes(g.dst_dt);
        CHECK(g.dst_off >= 0 && d1 <= dst_size(g), "%s: window %d zero range [%lld,%lld) past %lld", name, w,
              (long long)(g.dst_off + g.lo * dtype_bytes(g.dst_dt)), (long long)d1, (long long)dst_size(g));
        written[0].emplace_back(g.dst_off + g.lo * dtype_bytes(g.dst_dt), d1);
        return true;
    }
    const int32_t entries = by_record ? op.n : nparams;             // pointer-table entries
    CHECK(g.slot >= 0 && g.slot < entries, "%s: window %d slot %d out of range", name, w, g.slot);
    CHECK(g.param >= 0 && g.param < nparams, "%s: window %d param %d out of range", name, w, g.param);
    CHECK(!by_record || op.table_params[g.slot] == g.param, "%s: window %d table entry mismatch", name, w);
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
static bool check_op(const char *name, const OpTable &op, int32_t W, int32_t shift, int32_t nparams,
                     DstSize dst_size, SrcSize src_size, std::vector<Intervals> &written, int32_t rank = 0)
{
    WindowArgs a = op.args(false, shift);
    (void)W;   // rows come from the op table
    a.rank = rank;
    a.divisor = 1.0f;
    CHECK(a.n_windows == op.windows(shift) && (shift != 0 || a.n_windows == op.n_windows), "%s: window count", name);
    const size_t rec = op.op == kOpPack ? sizeof(PackMember)
                       : op.op == kOpCopyIn ? sizeof(CopyInSeg)
                       : (op.op == kOpCopyInFlat || op.op == kOpWriteBackFlat) ? sizeof(FlatMember)
                                                                                  : sizeof(CopyOutTensor);
    CHECK(op.members.size() == static_cast<size_t>(op.n) * rec, "%s: member table size", name);
    CHECK(op.n_windows == 0 || op.n > 0, "%s: windows without members", name);
    // maps over a row: one entry per 2^map_lg bytes, at least a window's worth
    const int64_t stretch = int64_t{1} << op.map_lg;
    CHECK(op.map_lg >= kWindowLog2 && op.map_lg < 48, "%s: map stretch 2^%d bytes", name, op.map_lg);
    CHECK(op.op != kOpPack ||
              (op.columns.size() == static_cast<size_t>((op.S * dtype_bytes(op.reduce_dt) + stretch - 1) / stretch) &&
               op.table_params.size() == static_cast<size_t>(op.n)), "%s: column map size", name);
    CHECK(op.op != kOpCopyIn ||
              (op.columns.size() == static_cast<size_t>((op.n_windows + (1 << kGroupLog2) - 1) >> kGroupLog2) &&
               op.table_params.size() == static_cast<size_t>(op.n)),
          "%s: copy-in group map size", name);
    CHECK((op.op != kOpCopyInFlat && op.op != kOpWriteBackFlat) ||
              op.columns.size() == static_cast<size_t>((op.flat_n * dtype_bytes(op.reduce_dt) + stretch - 1) / stretch),
          "%s: flat map size", name);
    CHECK((op.op != kOpCopyOut && op.op != kOpWriteBack) ||
              op.columns.size() == static_cast<size_t>((op.n_windows + (1 << kGroupLog2) - 1) >> kGroupLog2),
          "%s: group map size", name);
    // a made-up pointer set for the pack's stretch-record test: member m's
    // gradient at 2^32 * (m + 1), plus one element for odd m (bf16 sources
    // then start 2 bytes past a dword)
    std::vector<uint64_t> ptrs(static_cast<size_t>(op.n));
    if (op.op == kOpCopyInFlat) {
        const FlatMember *M = reinterpret_cast<const FlatMember *>(op.members.data());
        for (int32_t m = 0; m < op.n; ++m)
            ptrs[m] = (static_cast<uint64_t>(m + 1) << 32) + ((m & 1) ? dtype_bytes(M[m].dt) : 0);
    }
    if (op.op == kOpPack) {
        const PackMember *M = reinterpret_cast<const PackMember *>(op.members.data());
        for (int32_t m = 0; m < op.n; ++m)
            ptrs[m] = (static_cast<uint64_t>(m + 1) << 32) + ((m & 1) ? dtype_bytes(M[m].src_dt) : 0);
        // every window of the grid (k = 0 .. gx) finds its record
        const size_t n_rec = op.narrow ? static_cast<size_t>(((op.gx + 1) * kWindowBytes - 1) >> op.map_lg) + 1 : 0;
        CHECK(op.stretches.size() >= n_rec && op.stretches.size() >= (op.narrow ? op.columns.size() : 0) &&
                  (!op.narrow || op.stretches.size() <= std::max(n_rec, op.columns.size())) &&
                  (a.stretches != nullptr) == op.narrow,
              "%s: stretch records", name);
        const int64_t rb = op.S * dtype_bytes(op.reduce_dt);
        for (const PackStretch &e : op.stretches)
            for (int i = 0; i < 2; ++i) {
                const PackCand &c = e.c[i];
                const bool none = c.full == 0 && c.end == 0;
                CHECK(none || (c.moff % 8 == 0 && c.moff / 8 < static_cast<uint32_t>(op.n) &&
                               int64_t{c.lo} + c.span + kWindowBytes <= rb && c.sh <= 2 && (c.code & 3u) == static_cast<uint32_t>(op.reduce_dt)),
                      "%s: stretch record", name);
            }
    }
    for (int32_t w = 0; w < a.n_windows; ++w) {
        int ranges = 0;
        bool ok = true;
        int64_t lo = INT64_MAX, hi = INT64_MIN;       // bytes the window writes, from the aligned origin
        for_each_range(a, w, [&](const RangeRef &g) {
            if (ok) ok = check_range(name, w, a.shift, g, op, nparams, dst_size, src_size, written);
            const int64_t dsz = dtype_bytes(g.dst_dt);
            lo = std::min(lo, a.shift + g.dst_off + g.lo * dsz);
            hi = std::max(hi, a.shift + g.dst_off + g.hi * dsz);
            ++ranges;
        });
        if (!ok) return false;
        if (op.op == kOpPack) {
            // the kernel's direct copy of a whole single-member window must
            // be exactly the one range the general walk gives for it
            DirectWindow d{};
            if (pack_direct(a, w, d)) {
                int n_rng = 0;
                bool same = false;
                for_each_range(a, w, [&](const RangeRef &g) {
                    ++n_rng;
                    const int64_t ssz = dtype_bytes(g.src_dt), dsz = dtype_bytes(g.dst_dt);
                    same = g.hi - g.lo == kWindowBytes / dsz && g.valid >= g.hi && g.src_dt == d.src_dt &&
                           g.dst_dt == d.dst_dt && static_cast<int64_t>(d.src) == g.src_off + g.lo * ssz &&
                           d.dst_off == g.dst_off + g.lo * dsz && (a.shift + d.dst_off) % 16 == 0;
                });
                CHECK(n_rng == 1 && same, "%s: window %d (shift %d): direct copy differs from its range", name, w, shift);
                ++g_direct;
            }
            // the launch's 2-D grid gives the same row and window
            int32_t r, k, r2, k2;
            pack_row_window(a, w, r, k);
            const int32_t span = (a.gx + 1) << a.group_lg;
            pack_row_window_2d(a, static_cast<uint32_t>(w % span), static_cast<uint32_t>(w / span), r2, k2);
            CHECK(r == r2 && k == k2, "%s: window %d: 2-D grid maps to row %d window %d, not %d / %d", name, w, r2, k2,
                  r, k);
            // the direct copy through the stretch records is likewise the one
            // range of the walk, read from the member's own pointer
            if (op.narrow) {
                WindowArgs as = a;
                as.table = ptrs.data();
                DirectWindow ds{};
                if (pack_direct_stretch(as, r, k, ds)) {
                    int n_rng = 0;
                    bool same = false;
                    for_each_range(a, w, [&](const RangeRef &g) {
                        ++n_rng;
                        const int64_t ssz = dtype_bytes(g.src_dt), dsz = dtype_bytes(g.dst_dt);
                        same = g.hi - g.lo == kWindowBytes / dsz && g.valid >= g.hi && g.src_dt == ds.src_dt &&
                               g.dst_dt == ds.dst_dt && ds.src == ptrs[g.slot] + static_cast<uint64_t>(g.src_off + g.lo * ssz) &&
                               ds.dst_off == g.dst_off + g.lo * dsz && (a.shift + ds.dst_off) % 16 == 0;
                    });
                    CHECK(n_rng == 1 && same, "%s: window %d (shift %d): stretch-direct copy differs from its range",
                          name, w, shift);
                    ++g_direct_st;
                }
            }
        }
        if (op.op == kOpCopyIn) {
            // a copy-in window is one range of one segment (or empty: the
            // segment's spare window), bounded by line boundaries of memory
            // or by the segment's own ends; its direct copy, when it takes
            // one, is exactly that range
            const CopyInWindow c = copy_in_span(a.columns, a.members, nullptr, a.shift, w);
            CHECK(ranges <= 1 && (ranges == 1) == (c.y1 > c.y0), "%s: window %d has %d ranges", name, w, ranges);
            if (ranges == 1) {
                CHECK((c.y0 == c.s.A || (shift + c.y0) % kLineBytes == 0) &&
                          (c.y1 == c.A_next || (shift + c.y1) % kLineBytes == 0) && c.y1 - c.y0 <= kWindowBytes,
                      "%s: window %d (shift %d) writes [%lld,%lld) of a segment [%lld,%lld), off the line boundaries",
                      name, w, shift, (long long)c.y0, (long long)c.y1, (long long)c.s.A, (long long)c.A_next);
                CHECK(w == c.s.win0 || c.y0 > c.s.A, "%s: window %d: a segment's later window starts at its first byte",
                      name, w);
            } else {
                CHECK(w > c.s.win0 && c.y0 >= c.A_next, "%s: window %d: an empty window before its segment's end", name,
                      w);
            }
            DirectWindow d{};
            if (ranges == 1 && copy_in_direct(c, shift, d)) {
                const RangeRef g = copy_in_range(c);
                const int64_t ssz = dtype_bytes(g.src_dt), dsz = dtype_bytes(g.dst_dt);
                CHECK(g.hi - g.lo == kWindowBytes / dsz && g.valid >= g.hi && g.src_dt == d.src_dt && g.dst_dt == d.dst_dt &&
                          static_cast<int64_t>(d.src) == g.src_off + g.lo * ssz && d.dst_off == g.dst_off + g.lo * dsz &&
                          (a.shift + d.dst_off) % 16 == 0,
                      "%s: window %d (shift %d): direct copy-in differs from its range", name, w, shift);
                ++g_direct_in;
            }
        }
        if (op.op == kOpCopyInFlat) {
            // the flat copy-in's direct copy of a whole window of one piece
            // is exactly the one range the walk gives for it
            DirectWindow d{};
            WindowArgs at = a;
            at.table = ptrs.data();
            if (flat_copy_in_direct(at, w, d)) {
                int n_rng = 0;
                bool same = false;
                for_each_range(a, w, [&](const RangeRef &g) {
                    ++n_rng;
                    const int64_t ssz = dtype_bytes(g.src_dt), dsz = dtype_bytes(g.dst_dt);
                    same = g.hi - g.lo == kWindowBytes / dsz && g.valid >= g.hi && g.src_dt == d.src_dt &&
                           g.dst_dt == d.dst_dt && g.table_side == kTableIsSource &&
                           d.src == ptrs[g.slot] + static_cast<uint64_t>(g.src_off + g.lo * ssz) &&
                           d.dst_off == g.dst_off + g.lo * dsz && (a.shift + d.dst_off) % 16 == 0;
                });
                CHECK(n_rng == 1 && same, "%s: window %d (shift %d): direct flat copy-in differs from its range", name,
                      w, shift);
                ++g_direct_flat;
            }
        }
        if (op.op == kOpCopyOut) {
            // a gathered copy-out window reads, for each of its elements, the
            // very byte the chunk walk reads for it, and covers the same elements
            const CopyOutTensor t = find_tensor(a, w);
            int64_t e0, e1;
            copy_out_span(t, w, e0, e1);
            if (copy_out_gathered(t, e0, e1)) {
                int64_t covered = 0;
                bool same = true;
                for_each_range(a, w, [&](const RangeRef &g) {
                    const int64_t esz = dtype_bytes(g.dst_dt);
                    for (int64_t j = g.lo; j < g.hi && same; ++j) {
                        const int64_t i = g.dst_off / esz + j;
                        same = i >= e0 && i < e1 && g.src_dt == t.dt && g.dst_dt == t.dt &&
                               copy_out_source(a, t, static_cast<uint32_t>(i)) == g.src_off + j * esz;
                    }
                    covered += g.hi - g.lo;
                });
                CHECK(same && covered == e1 - e0 && (t.numel >> 32) == 0,
                      "%s: window %d: gathered copy differs from its chunk ranges", name, w);
                ++g_gather;
            }
        }
        int64_t row0 = shift, row1 = shift + op.B;        // the window's row, from the aligned origin
        if (op.op == kOpPack) {
            // window k of row r is empty exactly when the row ends before it
            int32_t r, k;
            pack_row_window(a, w, r, k);
            const int64_t rb = op.S * dtype_bytes(op.reduce_dt);
            const int64_t s_r = (shift + r * rb) % kLineBytes;
            const bool spare = static_cast<int64_t>(k) * kWindowBytes - s_r >= rb;
            CHECK((ranges == 0) == spare, "%s: window %d (row %d, shift %d) has %d ranges", name, w, r, shift, ranges);
            row0 = shift + r * rb;
            row1 = row0 + rb;
        } else if (op.op != kOpWriteBack && op.op != kOpWriteBackFlat && op.op != kOpCopyIn) {
            // (write-back windows past a rank's real elements, and a copy-in
            // segment's spare window, are empty)
            CHECK(ranges > 0, "%s: window %d has no range", name, w);
        }
        if ((op.op == kOpPack || op.op == kOpCopyInFlat) && ranges > 0)
            CHECK((lo == row0 || lo % kLineBytes == 0) && (hi == row1 || hi % kLineBytes == 0) &&
                      hi - lo <= kWindowBytes,
                  "%s: window %d (shift %d) writes [%lld,%lld) from the aligned origin, off the line boundaries",
                  name, w, shift, (long long)lo, (long long)hi);
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

int main(int argc, char **argv)
{
    const bool flat = argc > 1 && std::strcmp(argv[1], "flat") == 0;
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
    const int rc = flat ? build_plan_flat(d.data(), n, world, &plan, err) : build_plan(d.data(), n, world, &plan, err);
    if (rc != FSDPPACK_OK) {
        std::printf("FAIL plan: %s\n", err.c_str());
        return 1;
    }
    const int64_t W = plan.W;
    auto fail = [] { std::printf("FAIL %s\n", g_fail.c_str()); return 1; };
    auto grad_bytes = [&](const RangeRef &g) { return plan.numel[g.param] * dtype_bytes(plan.params[g.param].grad_dtype); };
    auto piece_bytes = [&](int32_t t, int32_t r) {
        return shard_elements(plan, t, r) * dtype_bytes(plan.params[t].storage_dtype);
    };
    // ranks walked by the rank-dependent operations (a sample for large W)
    std::vector<int32_t> ranks;
    for (int32_t r = 0; r < plan.W; ++r)
        if (plan.W <= 16 || r < 2 || r == plan.W / 2 || r >= plan.W - 2) ranks.push_back(r);
    // destination offsets past a line boundary: the pack's output is only
    // element aligned, the copy-in row 4-byte aligned (element aligned, flat)
    const int32_t kShiftUnits[] = {0, 1, 4, 27, 31};
    for (size_t bi = 0; bi < plan.buckets.size(); ++bi) {
        const BucketPlan &b = plan.buckets[bi];
        const int64_t out_bytes = W * b.S * dtype_bytes(b.dtype);
        // the planner's row grouping, and every other one the rows allow
        for (int32_t glg = -1; glg <= 3; ++glg) {
            if (glg >= 0 && (glg == b.pack.group_lg || b.pack.rows % (1 << glg) != 0)) continue;
            OpTable op = b.pack;
            if (glg >= 0) op.group_lg = glg;
            for (int32_t u : kShiftUnits) {
                const int32_t shift = static_cast<int32_t>((u * dtype_bytes(b.dtype)) % kLineBytes);
                std::vector<Intervals> written(1);
                char name[80];
                std::snprintf(name, sizeof name, "pack[%zu] rows/group %d shift %d", bi, 1 << op.group_lg, shift);
                if (!check_op(name, op, plan.W, shift, n, [&](const RangeRef &) { return out_bytes; }, grad_bytes,
                              written) ||
                    !tiles(written[0], out_bytes, name))
                    return fail();
            }
        }
    }
    // the allocation-free pack's scratch images: each eligible bucket's three
    // tables, each at a 256-byte boundary, byte for byte -- all of them in
    // one plan-wide image, one after another, when they fit it together,
    // else each bucket that fits alone in its own
    {
        int64_t total = 0;
        auto eligible = [](const OpTable &op) {
            return op.scratch_need > 0 && op.table_params.size() <= static_cast<size_t>(kInlineLarge);
        };
        for (const BucketPlan &b : plan.buckets)
            if (eligible(b.pack)) total += (b.pack.scratch_need + 255) / 256 * 256;
        const bool whole = total > 0 && total <= kScratchBytes;
        if (whole != !plan.scratch_image.empty() || plan.scratch_at.size() != plan.buckets.size()) {
            g_fail = "plan-wide scratch image present when it should not be, or missing";
            return fail();
        }
        int64_t next = 0;
        for (size_t bi = 0; bi < plan.buckets.size(); ++bi) {
            const OpTable &op = plan.buckets[bi].pack;
            const size_t mb = op.members.size(), cb = op.columns.size() * sizeof(ColumnWindow),
                         sb = op.stretches.size() * sizeof(PackStretch);
            bool ok = op.scratch_c_off % 256 == 0 && op.scratch_s_off % 256 == 0 &&
                      op.scratch_c_off >= static_cast<int64_t>(mb) &&
                      op.scratch_s_off >= op.scratch_c_off + static_cast<int64_t>(cb) &&
                      op.scratch_need == op.scratch_s_off + static_cast<int64_t>(sb);
            const unsigned char *img = nullptr;
            if (whole) {
                ok = ok && op.scratch_image.empty() && plan.scratch_at[bi] == (eligible(op) ? next : -1);
                if (eligible(op)) {
                    img = plan.scratch_image.data() + next;
                    next += (op.scratch_need + 255) / 256 * 256;
                    ok = ok && next <= static_cast<int64_t>(plan.scratch_image.size());
                }
            } else {
                const bool own = eligible(op) && op.scratch_need <= kScratchBytes;
                ok = ok && plan.scratch_at[bi] == -1 && own == !op.scratch_image.empty() &&
                     (!own || op.scratch_image.size() == static_cast<size_t>(op.scratch_need));
                if (own) img = op.scratch_image.data();
            }
            if (ok && img)
                ok = (mb == 0 || std::memcmp(img, op.members.data(), mb) == 0) &&
                     (cb == 0 || std::memcmp(img + op.scratch_c_off, op.columns.data(), cb) == 0) &&
                     (sb == 0 || std::memcmp(img + op.scratch_s_off, op.stretches.data(), sb) == 0);
            if (!ok) {
                g_fail = "pack[" + std::to_string(bi) + "] scratch image does not hold the pack's tables";
                return fail();
            }
            if (img) ++g_scratch_images;
        }
    }
    const int64_t row_esz = flat ? dtype_bytes(plan.copy_in.reduce_dt) : 4;
    for (int32_t r : flat ? ranks : std::vector<int32_t>{0}) {
        for (int32_t u : kShiftUnits) {
            const int32_t shift = static_cast<int32_t>((u * row_esz) % kLineBytes);
            std::vector<Intervals> written(1);
            char name[64];
            std::snprintf(name, sizeof name, "copy_in rank %d shift %d", r, shift);
            auto shard_bytes = [&](const RangeRef &g) {
                return flat ? piece_bytes(g.param, r) : plan.P[g.param] * dtype_bytes(plan.params[g.param].storage_dtype);
            };
            if (!check_op(name, plan.copy_in, plan.W, shift, n, [&](const RangeRef &) { return plan.B; }, shard_bytes,
                          written, r) ||
                !tiles(written[0], plan.B, name))
                return fail();
        }
    }
    {
        std::vector<Intervals> written(n);
        auto param_bytes = [&](const RangeRef &g) { return plan.numel[g.param] * dtype_bytes(plan.params[g.param].param_dtype); };
        if (!check_op("copy_out", plan.copy_out, plan.W, 0, n, param_bytes, [&](const RangeRef &) { return W * plan.B; },
                      written))
            return fail();
        for (int32_t t = 0; t < n; ++t) {
            char name[64];
            std::snprintf(name, sizeof name, "copy_out param %d", t);
            if (!tiles(written[t], plan.numel[t] * dtype_bytes(plan.params[t].param_dtype), name)) return fail();
        }
    }
    for (size_t bi = 0; bi < plan.buckets.size(); ++bi) {
        const BucketPlan &b = plan.buckets[bi];
        const int64_t row_bytes = b.S * dtype_bytes(b.dtype);
        for (int32_t r : ranks) {
            std::vector<Intervals> written(n);
            char name[64];
            std::snprintf(name, sizeof name, "write-back[%zu] rank %d", bi, r);
            std::vector<int64_t> dst_limit(n, 0);
            for (int32_t t : b.members) dst_limit[t] = piece_bytes(t, r);
            if (!check_op(name, b.write_back, plan.W, 0, n, [&](const RangeRef &g) { return dst_limit[g.param]; },
                          [&](const RangeRef &) { return row_bytes; }, written, r))
                return fail();
            for (int32_t t = 0; t < n; ++t) {
                char tn[96];
                std::snprintf(tn, sizeof tn, "%s param %d", name, t);
                if (!tiles(written[t], dst_limit[t], tn)) return fail();
            }
        }
    }
    if (plan.buckets.size() > 1) {
        // the write-back of every bucket in one launch: each member written
        // exactly once from its own bucket's row (pointer-table entry
        // n + bucket), in that bucket's reduction dtype
        std::vector<int32_t> bucket_of(n, -1);
        for (size_t bi = 0; bi < plan.buckets.size(); ++bi)
            for (int32_t t : plan.buckets[bi].members) bucket_of[t] = static_cast<int32_t>(bi);
        for (int32_t r : ranks) {
            std::vector<Intervals> written(n);
            char name[64];
            std::snprintf(name, sizeof name, "write-back of all buckets, rank %d", r);
            std::vector<int64_t> dst_limit(n, 0);
            for (int32_t t = 0; t < n; ++t) dst_limit[t] = bucket_of[t] >= 0 ? piece_bytes(t, r) : 0;
            bool sources_ok = true;
            auto row_bytes = [&](const RangeRef &g) -> int64_t {
                const int32_t bi = g.src_slot - n;
                if (g.param < 0 || bi != bucket_of[g.param] || g.src_dt != plan.buckets[bi].dtype) {
                    sources_ok = false;
                    return -1;
                }
                return plan.buckets[bi].S * dtype_bytes(plan.buckets[bi].dtype);
            };
            if (!check_op(name, plan.write_back_all, plan.W, 0, n, [&](const RangeRef &g) { return dst_limit[g.param]; },
                          row_bytes, written, r))
                return fail();
            if (!sources_ok) {
                std::printf("FAIL %s: a range reads another bucket's row or dtype\n", name);
                return 1;
            }
            for (int32_t t = 0; t < n; ++t) {
                char tn[96];
                std::snprintf(tn, sizeof tn, "%s param %d", name, t);
                if (!tiles(written[t], dst_limit[t], tn)) return fail();
            }
        }
    } else if (plan.write_back_all.n_windows != 0 || plan.write_back_all.n != 0) {
        std::puts("FAIL a one-bucket plan has an all-bucket write-back table");
        return 1;
    }
    std::printf("OK %s%zu buckets, windows:", flat ? "flat, " : "", plan.buckets.size());
    for (const BucketPlan &b : plan.buckets) std::printf(" %d (rows/group %d)", b.pack.n_windows, 1 << b.pack.group_lg);
    std::printf(" copy_in %d copy_out %d; direct pack windows %lld, stretch-direct pack windows %lld, "
                "direct copy-in windows %lld, gathered copy-out windows %lld, direct flat copy-in windows %lld, "
                "scratch images %lld\n",
                plan.copy_in.n_windows, plan.copy_out.n_windows, static_cast<long long>(g_direct),
                static_cast<long long>(g_direct_st),
                static_cast<long long>(g_direct_in), static_cast<long long>(g_gather), static_cast<long long>(g_direct_flat),
                static_cast<long long>(g_scratch_images));
    return 0;
}
