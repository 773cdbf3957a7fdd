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
//
// FSDP1 flat layout (build_plan_flat): the unit's parameters flattened and
// concatenated in unit order into one flat parameter, padded to W*ceil(N/W),
// one contiguous piece per rank -- "The unit you wrapped", the
// auto_wrap_policy and padding paragraphs.
//
// Each operation also gets its launch tables here: records, the map from a
// window to the records it touches, and the launch geometry.
#include "fsdppack_plan.h"

#include <algorithm>
#include <climits>
#include <cstring>
#include <map>
#include <utility>

namespace fsdppack {
namespace {

bool mul_ok(int64_t a, int64_t b, int64_t &out) { return !__builtin_mul_overflow(a, b, &out); }
bool add_ok(int64_t a, int64_t b, int64_t &out) { return !__builtin_add_overflow(a, b, &out); }

int64_t round_up16(int64_t x) { return (x + 15) / 16 * 16; }

// Largest byte count any offset may reach; keeps every derived sum in range.
constexpr int64_t kMaxBytes = INT64_MAX / 4;

// Largest number of workgroups along one dimension of a launch.  A dispatch
// counts its grid in work-items in 32 bits, so a dimension of 64-thread
// workgroups holds fewer than 2^26 of them (each writing a 2 KiB window:
// about 128 GiB per launch); the pack's rows are its second dimension.
constexpr int64_t kMaxGridX = (int64_t{1} << 26) - 1;
// Total workgroups of a launch (the kernels index windows in 32 bits).
constexpr int64_t kMaxWindows = INT32_MAX;

}  // namespace

// Record map over positions [0, total) for records whose spans [b, e) tile
// it in order (span(i) gives record i's span): for each stretch of
// 2^(map_lg - esz_lg) positions (2^map_lg bytes of elements of 2^esz_lg
// bytes), the records overlapping it.  Each workgroup reads the entries of
// the one or two stretches its window touches before any of its data, so the
// map is kept small enough to stay resident in the scalar cache and L2: the
// stretch is the coarsest power of two bytes, from one window up, that gives
// at most kMapEntries entries, made finer (down to one window) while its
// stretches list too many records on average (a window walks every record
// of its stretches, skipping those it does not overlap).  On MI355X a plain
// cast kernel that reads one entry of a ~100 KB table per workgroup (the
// size of a one-entry-per-window map for a 25 MB row) ran up to 8 % slower
// than with a table of a few KB when its waves move one vector per lane;
// with the pack's two vectors per lane the difference was within noise.
constexpr int64_t kMapEntries = 1024;
constexpr double kMapMeanRecords = 2.0;
constexpr int64_t kMapMaxRecords = 32;

template <typename Span>
static int32_t build_record_map(std::vector<ColumnWindow> &map, int64_t total, int esz_lg, size_t nrec, Span span)
{
    const int64_t total_bytes = total << esz_lg;
    int32_t lg = kWindowLog2;
    while (lg < 40 && ((total_bytes + (int64_t{1} << lg) - 1) >> lg) > kMapEntries) ++lg;
    for (;; --lg) {
        const int64_t E = int64_t{1} << (lg - esz_lg);
        const int64_t nx = (total + E - 1) / E;
        map.resize(static_cast<size_t>(nx));
        size_t first = 0;
        int64_t sum = 0, most = 0;
        for (int64_t x = 0; x < nx; ++x) {
            const int64_t p0 = x * E, p1 = std::min(total, p0 + E);
            while (first < nrec && span(first).second <= p0) ++first;
            size_t last = first;
            while (last < nrec && span(last).first < p1) ++last;
            map[x] = ColumnWindow{static_cast<int32_t>(first), static_cast<int32_t>(last - first)};
            sum += static_cast<int64_t>(last - first);
            most = std::max(most, static_cast<int64_t>(last - first));
        }
        if (lg == kWindowLog2 || (most <= kMapMaxRecords && sum <= kMapMeanRecords * static_cast<double>(nx)))
            return lg;
    }
}

// Whether a pack table gets stretch records: the kernel's direct test works
// in 32-bit column and row-byte arithmetic (rows of fewer than 2^31 bytes)
// and steps between a member's rank chunks by a 32-bit byte count.
static bool pack_narrow(const OpTable &op, const std::vector<PackMember> &mem)
{
    if (mem.empty() || (op.S * dtype_bytes(op.reduce_dt)) >= (int64_t{1} << 31)) return false;
    for (const PackMember &m : mem)
        if (m.P * dtype_bytes(m.src_dt) >= (int64_t{1} << 32) || m.numel >= (int64_t{1} << 32)) return false;
    return true;
}

// Group map of a table of records (CopyOutTensor, CopyInSeg) whose windows
// are consecutive (record t owns windows [win0_t, win0_{t+1})): for each group
// of 2^kGroupLog2 windows, the records owning its first and last windows.
template <typename T = CopyOutTensor>
static void build_group_map(OpTable &op)
{
    const T *R = reinterpret_cast<const T *>(op.members.data());
    const int64_t win = op.n_windows;
    const int64_t ng = (win + (int64_t{1} << kGroupLog2) - 1) >> kGroupLog2;
    op.columns.resize(static_cast<size_t>(ng));
    int32_t t0 = 0;
    for (int64_t j = 0; j < ng; ++j) {
        const int64_t w0 = j << kGroupLog2, w1 = std::min(win, (j + 1) << kGroupLog2) - 1;
        while (t0 + 1 < op.n && R[t0 + 1].win0 <= w0) ++t0;     // owner of the group's first window
        int32_t t1 = t0;
        while (t1 + 1 < op.n && R[t1 + 1].win0 <= w1) ++t1;     // owner of its last window
        op.columns[j] = ColumnWindow{t0, t1 - t0 + 1};
    }
}

// Checks shared by both layouts; fills W, n, params, numel and the
// per-parameter rank-chunk sizes P.
static int validate(const fsdppack_param_desc *params, int32_t n, int32_t world, fsdppack_plan *plan,
                    std::string &err)
{
    if (n < 0 || (n > 0 && params == nullptr)) { err = "plan_buckets: params is NULL or n < 0"; return FSDPPACK_EINVAL; }
    if (world < 1) { err = "plan_buckets: world size must be >= 1"; return FSDPPACK_EINVAL; }
    const int64_t W = world;
    plan->W = world;
    plan->n = n;
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
    return FSDPPACK_OK;
}

int build_plan(const fsdppack_param_desc *params, int32_t n, int32_t world, fsdppack_plan *plan,
               std::string &err)
{
    if (int rc = validate(params, n, world, plan, err)) return rc;
    const int64_t W = world;

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

    // ---- operation tables (members with nothing to move are left out, so
    // every lookup lands on a non-empty member)
    for (BucketPlan &b : plan->buckets) {
        // reduce-scatter pack: members in unit order along the columns of
        // every row
        OpTable &op = b.pack;
        op.op = kOpPack;
        op.rows = static_cast<int32_t>(W);
        op.reduce_dt = b.dtype;
        op.S = b.S;
        const int64_t dsz = dtype_bytes(b.dtype);
        std::vector<PackMember> mem;
        for (size_t k = 0; k < b.members.size(); ++k) {
            const int32_t t = b.members[k];
            if (b.P[k] == 0) continue;
            PackMember m{};
            m.O = b.O[k];
            m.P = b.P[k];
            m.numel = plan->numel[t];
            m.param = t;
            m.src_dt = plan->params[t].grad_dtype;
            op.add(m);
            mem.push_back(m);
            op.table_params.push_back(t);
            op.src_bytes += plan->numel[t] * dtype_bytes(m.src_dt);
        }
        const int64_t gx = (b.S * dsz + kWindowBytes - 1) / kWindowBytes;
        if ((gx + 1) * W > kMaxWindows || (gx + 1) * 2 > kMaxGridX) {
            err = "plan_buckets: reduce-scatter buffer needs too many workgroups";
            return FSDPPACK_EINVAL;
        }
        op.gx = static_cast<int32_t>(gx);
        op.dst_bytes = W * b.S * dsz;
        op.n_windows = static_cast<int32_t>(op.windows(0));
        // Row order: rows in pairs (window k of rows 2i and 2i+1, then window
        // k + 1) when W is even, one row at a time otherwise.  Measured on
        // MI355X over groups of 1, 2 and 4 rows: pairs gained 2-4 % on
        // layouts of ~100-400 KB chunks (445 tensors, or 32 tensors at W=8)
        // and 2.5 % on multi-MB chunks (12 tensors of a 218M-element block),
        // and lost nothing at W=128; groups of 4 were no better than pairs
        // and slower at W=128.
        if (!mem.empty() && W % 2 == 0) op.group_lg = 1;

        // reduce-scatter write-back: each member's rank chunk (P elements in
        // its storage dtype) cut into windows from its first byte; a launch
        // clips them to the chunk's real elements for its rank
        OpTable &wb = b.write_back;
        wb.op = kOpWriteBack;
        wb.reduce_dt = b.dtype;
        wb.S = b.S;
        int64_t win = 0;
        for (size_t k = 0; k < b.members.size(); ++k) {
            if (b.P[k] == 0) continue;
            const int32_t t = b.members[k];
            const int64_t bytes = b.P[k] * dtype_bytes(plan->params[t].storage_dtype);
            CopyOutTensor m{};
            m.win0 = win;
            m.numel = plan->numel[t];
            m.P = b.P[k];
            m.A = b.O[k] * dsz;
            m.slot = t;
            m.dt = plan->params[t].storage_dtype;
            m.src_dt = b.dtype;
            m.src_slot = -1;
            wb.add(m);
            win += (bytes + kWindowBytes - 1) / kWindowBytes;
            if (win > kMaxGridX) { err = "plan_buckets: sharded gradients need too many write-back workgroups"; return FSDPPACK_EINVAL; }
            wb.dst_bytes += bytes;
            wb.src_bytes += b.P[k] * dsz;
        }
        wb.n_windows = static_cast<int32_t>(win);
        build_group_map(wb);
        // column map: the members each stretch of a row's columns overlaps
        // (members tile [0, S) in column order, so one sweep finds them all)
        op.map_lg = build_record_map(op.columns, b.S, dsz == 2 ? 1 : 2, mem.size(), [&](size_t i) {
            return std::make_pair(mem[i].O, mem[i].O + mem[i].P);
        });
        op.narrow = pack_narrow(op, mem);
        if (op.narrow) {
            build_pack_stretches(op);
        }
    }

    if (plan->buckets.size() > 1) {
        // the write-back of every bucket in one launch: the buckets' records
        // one after another, each reading its bucket's reduced row from
        // pointer-table entry n + bucket (after the parameters' entries)
        OpTable &op = plan->write_back_all;
        op.op = kOpWriteBack;
        op.reduce_dt = plan->buckets[0].dtype;
        int64_t win = 0;
        for (size_t bi = 0; bi < plan->buckets.size(); ++bi) {
            const OpTable &wb = plan->buckets[bi].write_back;
            const CopyOutTensor *T = reinterpret_cast<const CopyOutTensor *>(wb.members.data());
            for (int32_t k = 0; k < wb.n; ++k) {
                CopyOutTensor m = T[k];
                m.win0 += win;
                m.src_slot = n + static_cast<int32_t>(bi);
                op.add(m);
            }
            win += wb.n_windows;
            op.dst_bytes += wb.dst_bytes;
            op.src_bytes += wb.src_bytes;
        }
        if (win > kMaxGridX) { err = "plan_buckets: sharded gradients need too many write-back workgroups"; return FSDPPACK_EINVAL; }
        op.n_windows = static_cast<int32_t>(win);
        build_group_map(op);
    }

    {   // all-gather copy-in: each parameter owns bytes [A_t, A_{t+1}) of the
        // row, its cast shard then zero gap bytes up to the next slot, cut
        // into windows of its own
        OpTable &op = plan->copy_in;
        op.op = kOpCopyIn;
        op.B = plan->B;
        int64_t win = 0;
        for (int32_t t = 0; t < n; ++t) {
            const int64_t next = (t + 1 < n) ? plan->A[t + 1] : plan->B;
            if (next == plan->A[t]) continue;
            CopyInSeg m{};
            m.A = plan->A[t];
            m.P = plan->P[t];
            m.win0 = static_cast<int32_t>(win);
            m.param = t;
            m.src_dt = static_cast<int16_t>(plan->params[t].storage_dtype);
            m.dst_dt = static_cast<int16_t>(plan->params[t].param_dtype);
            op.add(m);
            op.table_params.push_back(t);
            win += copy_in_windows(next - m.A);
            if (win > kMaxGridX) { err = "plan_buckets: all-gather row needs too many workgroups"; return FSDPPACK_EINVAL; }
            op.src_bytes += plan->P[t] * dtype_bytes(m.src_dt);
        }
        op.dst_bytes = plan->B;
        op.n_windows = static_cast<int32_t>(win);
        // group map with split windows (WindowGroup)
        build_group_map<CopyInSeg>(op);
        const CopyInSeg *R = reinterpret_cast<const CopyInSeg *>(op.members.data());
        for (ColumnWindow &g : op.columns) {
            const int32_t count = g.count;
            g.count = count == 1 ? INT32_MAX : count == 2 ? R[g.first + 1].win0 : -count;
        }
        static_assert(sizeof(ColumnWindow) == sizeof(WindowGroup), "the same map entries");
    }

    {   // all-gather copy-out: each parameter's bytes cut into windows; a
        // window is split at rank-chunk boundaries by the kernel
        OpTable &op = plan->copy_out;
        op.op = kOpCopyOut;
        op.B = plan->B;
        int64_t win = 0;
        for (int32_t t = 0; t < n; ++t) {
            if (plan->numel[t] == 0) continue;
            const int64_t bytes = plan->numel[t] * dtype_bytes(plan->params[t].param_dtype);
            CopyOutTensor m{};
            m.win0 = win;
            m.numel = plan->numel[t];
            m.P = plan->P[t];
            m.A = plan->A[t];
            m.slot = t;
            m.dt = plan->params[t].param_dtype;
            m.src_dt = m.dt;
            m.src_slot = -1;
            op.add(m);
            win += (bytes + kWindowBytes - 1) / kWindowBytes;
            if (win > kMaxGridX) { err = "plan_buckets: parameters need too many copy-out workgroups"; return FSDPPACK_EINVAL; }
            op.src_bytes += bytes;
        }
        op.n_windows = static_cast<int32_t>(win);
        op.dst_bytes = op.src_bytes;
        build_group_map(op);
    }
    build_scratch_images(plan);
    return FSDPPACK_OK;
}

void build_scratch_images(fsdppack_plan *plan)
{
    auto up = [](int64_t x) { return (x + 255) / 256 * 256; };
    const size_t nb = plan->buckets.size();
    plan->scratch_image.clear();
    plan->scratch_at.assign(nb, -1);
    auto eligible = [](const OpTable &op) {
        return op.scratch_need > 0 && op.table_params.size() <= static_cast<size_t>(kInlineLarge);
    };
    auto lay = [](const OpTable &op, unsigned char *img) {
        if (!op.members.empty()) std::memcpy(img, op.members.data(), op.members.size());
        if (!op.columns.empty())
            std::memcpy(img + op.scratch_c_off, op.columns.data(), op.columns.size() * sizeof(ColumnWindow));
        if (!op.stretches.empty())
            std::memcpy(img + op.scratch_s_off, op.stretches.data(), op.stretches.size() * sizeof(PackStretch));
    };
    int64_t total = 0;
    for (BucketPlan &b : plan->buckets) {
        OpTable &op = b.pack;
        op.scratch_c_off = up(static_cast<int64_t>(op.members.size()));
        op.scratch_s_off = op.scratch_c_off + up(static_cast<int64_t>(op.columns.size() * sizeof(ColumnWindow)));
        op.scratch_need = op.scratch_s_off + static_cast<int64_t>(op.stretches.size() * sizeof(PackStretch));
        op.scratch_image.clear();
        if (eligible(op)) total += up(op.scratch_need);
    }
    if (total > 0 && total <= kScratchBytes) {
        plan->scratch_image.assign(static_cast<size_t>(total), 0);
        int64_t at = 0;
        for (size_t bi = 0; bi < nb; ++bi) {
            const OpTable &op = plan->buckets[bi].pack;
            if (!eligible(op)) continue;
            plan->scratch_at[bi] = at;
            lay(op, plan->scratch_image.data() + at);
            at += up(op.scratch_need);
        }
        return;
    }
    for (BucketPlan &b : plan->buckets) {
        OpTable &op = b.pack;
        if (!eligible(op) || op.scratch_need > kScratchBytes) continue;
        op.scratch_image.assign(static_cast<size_t>(op.scratch_need), 0);
        lay(op, op.scratch_image.data());
    }
}

void build_pack_stretches(OpTable &op)
{
    const PackMember *M = reinterpret_cast<const PackMember *>(op.members.data());
    const int lg = op.reduce_dt == kBF16 ? 1 : 2;
    const int64_t rb = op.S << lg, E = int64_t{1} << op.map_lg;
    const int64_t nx = static_cast<int64_t>(op.columns.size());
    // the grid's windows k = 0 .. gx of a row start at most at byte k*2048:
    // records up to the stretch of the last byte of window gx
    const int64_t n_rec = ((op.gx * kWindowBytes + kWindowBytes - 1) >> op.map_lg) + 1;
    PackStretch none{};                                    // full = end = 0: no window passes
    none.c[1].lo = ~0u;
    op.stretches.assign(static_cast<size_t>(std::max(n_rec, nx)), none);
    // Members whose rank chunk is shorter than a window can hold no direct
    // window, so they take no candidate place: a stretch of large chunks with
    // a few norms or biases between them still lists its large members
    // (a window that touches a small member lies in no large one's columns
    // and fails the range test).
    std::vector<int32_t> big;
    for (int32_t i = 0; i < op.n; ++i)
        if ((M[i].P << lg) >= kWindowBytes) big.push_back(i);
    const int32_t nbig = static_cast<int32_t>(big.size());
    int32_t first = 0;
    for (int64_t x = 0; x < nx; ++x) {
        // the columns of row bytes [x*E - window, (x+1)*E), clipped to the row:
        // every window whose last byte lies in stretch x starts in there
        const int64_t b0 = std::max<int64_t>(0, x * E - kWindowBytes), b1 = std::min(rb, (x + 1) * E);
        const int64_t c0 = b0 >> lg, c1 = (b1 + (int64_t{1} << lg) - 1) >> lg;
        while (first < nbig && M[big[first]].O + M[big[first]].P <= c0) ++first;
        int32_t last = first;
        while (last < nbig && M[big[last]].O < c1) ++last;
        if (last - first < 1 || last - first > 2) continue;
        PackStretch &s = op.stretches[static_cast<size_t>(x)];
        for (int32_t j = first; j < last; ++j) {
            const int32_t i = big[j];
            const PackMember &m = M[i];
            const int64_t ssz = dtype_bytes(m.src_dt), full = m.numel / m.P, Pb = m.P << lg;
            PackCand &c = s.c[j - first];
            c.lo = static_cast<uint32_t>(m.O << lg);
            c.span = static_cast<uint32_t>(Pb - kWindowBytes);
            c.full = static_cast<uint32_t>(full);
            c.end = static_cast<uint32_t>((m.O + m.numel - full * m.P) << lg);
            c.Pss = static_cast<uint32_t>(m.P * ssz);
            c.moff = static_cast<uint32_t>(i) * 8u;
            c.sh = static_cast<uint32_t>(1 + lg - (ssz == 2 ? 1 : 2));
            c.code = static_cast<uint32_t>(m.src_dt * 4 + op.reduce_dt);
        }
    }
}

int64_t shard_elements(const fsdppack_plan &plan, int32_t t, int32_t r)
{
    if (plan.flat) {
        const int64_t lo = std::max(plan.fl.F[t], int64_t{r} * plan.fl.c);
        const int64_t hi = std::min(plan.fl.F[t] + plan.numel[t], (int64_t{r} + 1) * plan.fl.c);
        return std::max<int64_t>(0, hi - lo);
    }
    return std::max<int64_t>(0, std::min(plan.P[t], plan.numel[t] - int64_t{r} * plan.P[t]));
}

// Flat-position map of FlatMember records (consecutive, tiling [0, N) in
// order, empty parameters left out), for a row of elements of 2^esz_lg bytes.
static void build_flat_map(OpTable &op, const std::vector<FlatMember> &mem, int64_t N, int esz_lg)
{
    op.map_lg = build_record_map(op.columns, N, esz_lg, mem.size(), [&](size_t i) {
        return std::make_pair(mem[i].F, mem[i].F + mem[i].numel);
    });
}

int build_plan_flat(const fsdppack_param_desc *params, int32_t n, int32_t world, fsdppack_plan *plan,
                    std::string &err)
{
    if (int rc = validate(params, n, world, plan, err)) return rc;
    const int64_t W = world;
    plan->flat = true;
    if (n == 0) return FSDPPACK_OK;
    // one flat parameter: one reduction dtype, one param dtype
    const int32_t rdt = params[0].reduce_dtype != kNone ? params[0].reduce_dtype : params[0].grad_dtype;
    const int32_t pdt = params[0].param_dtype;
    for (int32_t t = 1; t < n; ++t) {
        const int32_t eff = params[t].reduce_dtype != kNone ? params[t].reduce_dtype : params[t].grad_dtype;
        if (eff != rdt || params[t].param_dtype != pdt) {
            err = "plan_buckets_flat: a flat parameter needs one reduction dtype and one param dtype (parameter " +
                  std::to_string(t) + " differs)";
            return FSDPPACK_EDTYPE;
        }
    }
    FlatLayout &fl = plan->fl;
    fl.F.resize(n);
    for (int32_t t = 0; t < n; ++t) {
        fl.F[t] = fl.N;
        fl.N += plan->numel[t];
        if (fl.N > kMaxBytes / 4) { err = "plan_buckets_flat: flat parameter too large"; return FSDPPACK_EINVAL; }
    }
    fl.c = (fl.N + W - 1) / W;
    const int64_t bsz = dtype_bytes(rdt), psz = dtype_bytes(pdt);

    // introspection: one bucket whose members sit at flat offsets
    plan->buckets.emplace_back();
    BucketPlan &b = plan->buckets.back();
    b.dtype = rdt;
    b.S = fl.c;
    for (int32_t t = 0; t < n; ++t) {
        b.members.push_back(t);
        b.P.push_back(plan->numel[t]);
        b.O.push_back(fl.F[t]);
        plan->P[t] = plan->numel[t];
        plan->A[t] = fl.F[t] * psz;
    }
    plan->B = fl.c * psz;

    // pack: one row of W*c elements, members at their flat offsets; the last
    // member's chunk also covers the padding up to W*c (+0, never read)
    {
        OpTable &op = b.pack;
        op.op = kOpPack;
        op.rows = 1;
        op.reduce_dt = rdt;
        op.S = W * fl.c;
        std::vector<PackMember> mem;
        for (int32_t t = 0; t < n; ++t) {
            if (plan->numel[t] == 0) continue;
            PackMember m{};
            m.O = fl.F[t];
            m.P = plan->numel[t];
            m.numel = plan->numel[t];
            m.param = t;
            m.src_dt = params[t].grad_dtype;
            mem.push_back(m);
            op.table_params.push_back(t);
            op.src_bytes += plan->numel[t] * dtype_bytes(m.src_dt);
        }
        if (!mem.empty()) mem.back().P += op.S - fl.N;
        for (const PackMember &m : mem) op.add(m);
        const int64_t gx = (op.S * bsz + kWindowBytes - 1) / kWindowBytes;
        if (gx + 1 > kMaxGridX) { err = "plan_buckets_flat: reduce-scatter buffer needs too many workgroups"; return FSDPPACK_EINVAL; }
        op.gx = static_cast<int32_t>(gx);
        op.dst_bytes = op.S * bsz;
        op.n_windows = static_cast<int32_t>(op.windows(0));
        op.map_lg = build_record_map(op.columns, op.S, bsz == 2 ? 1 : 2, mem.size(), [&](size_t i) {
            return std::make_pair(mem[i].O, mem[i].O + mem[i].P);
        });
        op.narrow = pack_narrow(op, mem);
        if (op.narrow) {
            build_pack_stretches(op);
        }
    }

    // write-back and copy-in: windows over a rank's row, records by flat offset
    std::vector<FlatMember> fm;
    std::vector<int32_t> fm_params;
    for (int32_t t = 0; t < n; ++t) {
        if (plan->numel[t] == 0) continue;
        FlatMember m{};
        m.F = fl.F[t];
        m.numel = plan->numel[t];
        m.slot = t;
        m.dt = params[t].storage_dtype;
        fm.push_back(m);
        fm_params.push_back(t);
    }
    for (int which = 0; which < 2; ++which) {
        const bool copy_in = which == 1;
        OpTable &op = copy_in ? plan->copy_in : b.write_back;
        op.op = copy_in ? kOpCopyInFlat : kOpWriteBackFlat;
        op.reduce_dt = copy_in ? pdt : rdt;        // the row's dtype
        op.S = fl.c;
        op.flat_n = fl.N;
        for (const FlatMember &m : fm) op.add(m);
        op.table_params = fm_params;               // pointer table in record order
        const int64_t rsz = copy_in ? psz : bsz;
        const int64_t row_bytes = fl.c * rsz;
        op.B = row_bytes;
        // the copy-in's windows follow the lines of its destination row; the
        // write-back's row is its source, so its windows start at the row
        op.dst_bytes = copy_in ? row_bytes : 0;
        if ((row_bytes + kLineBytes - 1 + kWindowBytes - 1) / kWindowBytes > kMaxGridX) {
            err = "plan_buckets_flat: a rank's row needs too many workgroups";
            return FSDPPACK_EINVAL;
        }
        op.n_windows = static_cast<int32_t>(copy_in ? op.windows(0) : (row_bytes + kWindowBytes - 1) / kWindowBytes);
        build_flat_map(op, fm, fl.N, rsz == 2 ? 1 : 2);
    }

    // copy-out: each parameter is one contiguous stretch of the gathered flat parameter
    {
        OpTable &op = plan->copy_out;
        op.op = kOpCopyOut;
        op.B = plan->B;
        int64_t win = 0;
        for (int32_t t = 0; t < n; ++t) {
            if (plan->numel[t] == 0) continue;
            const int64_t bytes = plan->numel[t] * psz;
            CopyOutTensor m{};
            m.win0 = win;
            m.numel = plan->numel[t];
            m.P = plan->numel[t];
            m.A = fl.F[t] * psz;
            m.slot = t;
            m.dt = pdt;
            m.src_dt = pdt;
            m.src_slot = -1;
            op.add(m);
            win += (bytes + kWindowBytes - 1) / kWindowBytes;
            if (win > kMaxGridX) { err = "plan_buckets_flat: parameters need too many copy-out workgroups"; return FSDPPACK_EINVAL; }
            op.src_bytes += bytes;
        }
        op.n_windows = static_cast<int32_t>(win);
        op.dst_bytes = op.src_bytes;
        build_group_map(op);
    }
    build_scratch_images(plan);
    return FSDPPACK_OK;
}

}  // namespace fsdppack
