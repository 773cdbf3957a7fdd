// fsdppack_internal.h -- plan tables and the window -> range mapping shared
// by the host planner, the ABI layer and the HIP kernels of libfsdppack.
//
// Every operation of the library (reduce-scatter pack, all-gather copy-in,
// all-gather copy-out) is the same primitive over *ranges*: a contiguous
// destination run whose first `valid` elements are the cast of a contiguous
// source run and whose remaining elements are +0 (the right-hand padding of
// a rank chunk, or the zero gap after an all-gather segment).  One side of
// every range lives in a caller tensor reached through a per-call pointer
// table; the other side is an offset into the call's single packed buffer.
//
// Work is cut into fixed *windows* of kWindowBytes of destination, one per
// workgroup.  A workgroup finds its ranges arithmetically from its window
// index plus small per-plan tables (a column map and member records for the
// pack, a binary search over member offsets for the all-gather copies).  The
// tables are a few KB to a few hundred KB and read by many workgroups, so
// they stay resident in the scalar cache and L2: no workgroup waits on a
// cold record of its own before touching data (a per-workgroup record, read
// cold, measured ~20 % slower on MI355X), and the dependent table reads in
// front of a wave's data are kept to two for the pack.  The mapping functions below are compiled both for the device
// (the kernels) and for the host (the planner's bounds checker), so the
// checker runs exactly the code the kernels run.
#pragma once

#include <cstdint>

#if defined(__HIP__)
#define FSDPPACK_HD __attribute__((host, device))
#else
#define FSDPPACK_HD
#endif

// Plan tables are read-only for a kernel's whole life.  In device code they
// are read through the constant address space, which lets the compiler use
// scalar loads for them even after the kernel has issued stores: a vector
// load there would make the wave wait for its own outstanding stores.
#if defined(__HIP_DEVICE_COMPILE__)
#define FSDPPACK_TABLE __attribute__((address_space(4)))
#else
#define FSDPPACK_TABLE
#endif

namespace fsdppack {

enum : int32_t { kNone = 0, kBF16 = 1, kFP32 = 2 };

FSDPPACK_HD inline int64_t dtype_bytes(int32_t dt) { return dt == kBF16 ? 2 : 4; }
inline bool dtype_ok(int32_t dt) { return dt == kBF16 || dt == kFP32; }

// Destination bytes per workgroup (one wave64 moving two 16-byte vectors
// per lane).
constexpr int64_t kWindowBytes = 2048;

// Which side of a range is the caller's tensor (reached through the pointer
// table); the other side is the call's packed buffer.
enum : int32_t { kTableIsSource = 0, kTableIsDest = 1 };

enum : int32_t { kOpPack = 0, kOpCopyIn = 1, kOpCopyOut = 2 };

// One bucket member of a reduce-scatter pack: columns [O, O + P) of every
// row; `numel` elements of dtype src_dt.  The pack's pointer table is in
// member order (entry m is member m's gradient); `param` is the parameter
// index, for the host.
struct PackMember {
    int64_t O;
    int64_t P;
    int64_t numel;
    int32_t param;
    int32_t src_dt;
};
static_assert(sizeof(PackMember) == 32, "shared with the device");

// The members a pack column window overlaps: first, first + 1, ...,
// first + count - 1.  One entry per window of a row, shared by all W rows.
struct ColumnWindow {
    int32_t first;
    int32_t count;
};
static_assert(sizeof(ColumnWindow) == 8, "shared with the device");

// One parameter of the all-gather copy-in: bytes [A, A_next) of the row,
// the first P elements (param dtype) cast from the shard, the rest zero.
struct CopyInMember {
    int64_t A;
    int64_t A_next;
    int64_t P;
    int32_t slot;
    int16_t src_dt;
    int16_t dst_dt;
};
static_assert(sizeof(CopyInMember) == 32, "shared with the device");

// One parameter of the all-gather copy-out: its windows start at window
// index win0; numel elements of dtype dt, rank chunks of P elements found
// at byte A of each all-gather row.
struct CopyOutTensor {
    int64_t win0;
    int64_t numel;
    int64_t P;
    int64_t A;
    int32_t slot;
    int32_t dt;
};
static_assert(sizeof(CopyOutTensor) == 40, "shared with the device");

// Arguments of one launch (all three operations).
struct WindowArgs {
    int32_t op;              // kOpPack / kOpCopyIn / kOpCopyOut
    int32_t n;               // entries of `members`
    int32_t n_windows;       // workgroups
    int32_t gx;              // pack: windows per row
    int32_t W;               // world size
    int32_t dst_dt;          // pack: reduction dtype
    int64_t S;               // pack: row length in elements
    int64_t B;               // copy-in row bytes / copy-out row stride
    const void *members;     // PackMember / CopyInMember / CopyOutTensor array
    const void *columns;     // pack: ColumnWindow per window of a row
    const uint64_t *table;   // device pointer table, indexed by slot
    char *base;              // the call's packed buffer (destination or source)
};

// One contiguous range for the copy primitive: elements [lo, hi) of a chunk
// whose element 0 sits at byte src_off of its source and dst_off of its
// destination; elements >= valid are +0.
struct RangeRef {
    uint64_t ptr;            // the caller tensor's address (pointer-table entry `slot`)
    int64_t src_off;
    int64_t dst_off;
    int64_t lo;
    int64_t hi;
    int64_t valid;
    int32_t slot;            // pointer-table entry
    int32_t param;           // parameter index (host-side checks)
    int32_t src_dt;
    int32_t dst_dt;
    int32_t table_side;
};

// Pointer-table entry; the host-side checker walks windows without a table.
FSDPPACK_HD inline uint64_t table_entry(const WindowArgs &a, int32_t slot)
{
    return a.table ? ((const FSDPPACK_TABLE uint64_t *)a.table)[slot] : 0;
}

FSDPPACK_HD inline int64_t imin(int64_t a, int64_t b) { return a < b ? a : b; }
FSDPPACK_HD inline int64_t imax(int64_t a, int64_t b) { return a > b ? a : b; }

// Non-negative division that takes the 32-bit path when both operands fit.
FSDPPACK_HD inline int64_t udiv(int64_t a, int64_t b)
{
    if (((a | b) >> 32) == 0) return static_cast<int64_t>(static_cast<uint32_t>(a) / static_cast<uint32_t>(b));
    return static_cast<int64_t>(static_cast<uint64_t>(a) / static_cast<uint64_t>(b));
}

// Pack window w: row r = w / gx, columns [x*E, min(S, (x+1)*E)) with x = w %
// gx and E the window in elements.  The column map names the members the
// window overlaps, so a wave needs two dependent table reads (the column
// entry, then the member record and its pointer together) before its data.
template <typename F>
FSDPPACK_HD inline void pack_window(const WindowArgs &a, int32_t w, F &&f)
{
    const FSDPPACK_TABLE PackMember *M = (const FSDPPACK_TABLE PackMember *)a.members;
    const FSDPPACK_TABLE ColumnWindow *C = (const FSDPPACK_TABLE ColumnWindow *)a.columns;
    const int64_t dsz = dtype_bytes(a.dst_dt);
    const int64_t E = kWindowBytes / dsz;
    const int32_t r = w / a.gx, x = w % a.gx;
    const int64_t c0 = static_cast<int64_t>(x) * E, c1 = imin(a.S, c0 + E);
    const ColumnWindow cw = C[x];
    for (int32_t i = 0; i < cw.count; ++i) {
        const int32_t m = cw.first + i;
        const uint64_t ptr = table_entry(a, m);          // issued with the member read
        const PackMember pm = M[m];
        const int64_t b0 = imax(c0, pm.O), b1 = imin(c1, pm.O + pm.P);
        RangeRef g;
        g.ptr = ptr;
        g.src_off = static_cast<int64_t>(r) * pm.P * dtype_bytes(pm.src_dt);
        g.dst_off = (static_cast<int64_t>(r) * a.S + pm.O) * dsz;
        g.lo = b0 - pm.O;
        g.hi = b1 - pm.O;
        g.valid = imax(0, imin(pm.P, pm.numel - static_cast<int64_t>(r) * pm.P));
        g.slot = m;
        g.param = pm.param;
        g.src_dt = pm.src_dt;
        g.dst_dt = a.dst_dt;
        g.table_side = kTableIsSource;
        f(g);
    }
}

// Copy-in window w: bytes [w*kWindowBytes, ...) of the row; members by
// binary search on A.  Every member's span is a multiple of 16 bytes.
template <typename F>
FSDPPACK_HD inline void copy_in_window(const WindowArgs &a, int32_t w, F &&f)
{
    const FSDPPACK_TABLE CopyInMember *M = (const FSDPPACK_TABLE CopyInMember *)a.members;
    const int64_t y0 = static_cast<int64_t>(w) * kWindowBytes, y1 = imin(a.B, y0 + kWindowBytes);
    int32_t lo = 0, hi = a.n - 1;                        // last member with A <= y0
    while (lo < hi) {
        const int32_t mid = (lo + hi + 1) >> 1;
        if (M[mid].A <= y0) lo = mid; else hi = mid - 1;
    }
    for (int32_t m = lo; m < a.n && M[m].A < y1; ++m) {
        const CopyInMember cm = M[m];
        const int64_t b0 = imax(y0, cm.A), b1 = imin(y1, cm.A_next);
        if (b1 <= b0) continue;
        const int64_t esz = dtype_bytes(cm.dst_dt);
        RangeRef g;
        g.ptr = table_entry(a, cm.slot);
        g.src_off = 0;
        g.dst_off = cm.A;
        g.lo = (b0 - cm.A) / esz;
        g.hi = (b1 - cm.A) / esz;
        g.valid = cm.P;
        g.slot = cm.slot;
        g.param = cm.slot;
        g.src_dt = cm.src_dt;
        g.dst_dt = cm.dst_dt;
        g.table_side = kTableIsSource;
        f(g);
    }
}

// Copy-out window w: the tensor whose windows contain w (binary search on
// win0), bytes [x*kWindowBytes, ...) of that tensor, split at rank-chunk
// boundaries; chunk r comes from byte r*B + A of the gathered buffer.
template <typename F>
FSDPPACK_HD inline void copy_out_window(const WindowArgs &a, int32_t w, F &&f)
{
    const FSDPPACK_TABLE CopyOutTensor *T = (const FSDPPACK_TABLE CopyOutTensor *)a.members;
    int32_t lo = 0, hi = a.n - 1;                        // last tensor with win0 <= w
    while (lo < hi) {
        const int32_t mid = (lo + hi + 1) >> 1;
        if (T[mid].win0 <= w) lo = mid; else hi = mid - 1;
    }
    const CopyOutTensor t = T[lo];
    const uint64_t ptr = table_entry(a, t.slot);
    const int64_t esz = dtype_bytes(t.dt);
    const int64_t e0 = (w - t.win0) * (kWindowBytes / esz);
    const int64_t e1 = imin(t.numel, e0 + kWindowBytes / esz);
    for (int64_t r = udiv(e0, t.P); r * t.P < e1; ++r) {
        const int64_t b0 = imax(e0, r * t.P), b1 = imin(e1, (r + 1) * t.P);
        RangeRef g;
        g.ptr = ptr;
        g.src_off = r * a.B + t.A;
        g.dst_off = r * t.P * esz;
        g.lo = b0 - r * t.P;
        g.hi = b1 - r * t.P;
        g.valid = g.hi;
        g.slot = t.slot;
        g.param = t.slot;
        g.src_dt = t.dt;
        g.dst_dt = t.dt;
        g.table_side = kTableIsDest;
        f(g);
    }
}

template <typename F>
FSDPPACK_HD inline void for_each_range(const WindowArgs &a, int32_t w, F &&f)
{
    if (a.op == kOpPack) pack_window(a, w, f);
    else if (a.op == kOpCopyIn) copy_in_window(a, w, f);
    else copy_out_window(a, w, f);
}

// Launch the window kernel on `stream`: one workgroup per window.
// start_event / stop_event (hipEvent_t, may be NULL) are stamped at the
// kernel's start and end.  Returns the hipError_t of the launch as an int.
int launch_windows(const WindowArgs &args, void *stream, void *start_event, void *stop_event);

}  // namespace fsdppack
