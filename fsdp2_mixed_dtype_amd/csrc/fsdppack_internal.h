// fsdppack_internal.h -- plan tables and the window -> range mapping shared
// by the host planner, the ABI layer and the HIP kernels of libfsdppack.
//
// Every operation of the library (reduce-scatter pack, reduce-scatter
// write-back, all-gather copy-in and copy-out, in the per-parameter and the
// FSDP1 flat layouts) is the same primitive over *ranges*: a contiguous
// destination run whose first `valid` elements are the cast of a contiguous
// source run and whose remaining elements are +0 (the right-hand padding of
// a rank chunk, or the zero gap after an all-gather segment).  One side of
// every range lives in a caller tensor reached through a per-call pointer
// table; the other side is an offset into the call's single packed buffer
// (a range that is all +0 has no source).
//
// Work is cut into fixed *windows* of kWindowBytes of destination, one per
// workgroup.  For the pack (per row) and the copy-in, window boundaries sit
// on cache-line boundaries of memory (the launch passes how far the buffer
// starts past one), so a line is written by one workgroup only: a line split
// between two workgroups, possibly on different XCDs with separate L2s,
// reaches HBM as two partial writes.  A workgroup finds its ranges
// arithmetically from its window index plus small per-plan tables: a map
// with one entry per stretch of 2^map_lg bytes of a row (pack, copy-in, flat
// layout; the planner sizes the stretch so the map has at most about a
// thousand entries) or per group of windows (copy-out, write-back) that
// names the records to visit, and the records.  The tables are a few KB and
// every entry is read by many workgroups, so they stay resident in the
// scalar cache and L2: no workgroup waits on a cold record of its own before
// touching data (a per-workgroup record, read cold, measured ~20 % slower on
// MI355X), and a wave makes two rounds of table reads before its data (a
// binary search over hundreds of records would make nine).  The mapping
// functions below are compiled both for the device (the kernels) and for
// the host (the planner's bounds checker), so the checker runs exactly the
// code the kernels run.
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
constexpr int kWindowLog2 = 11;
constexpr int64_t kWindowBytes = int64_t{1} << kWindowLog2;
// Cache line of the L2 (window boundaries are aligned to it in memory).
constexpr int64_t kLineBytes = 128;
// Copy-out windows per entry of its group map.
constexpr int kGroupLog2 = 6;

// Which side of a range is the caller's tensor (reached through the pointer
// table); the other side is the call's packed buffer.
enum : int32_t { kTableIsSource = 0, kTableIsDest = 1 };

enum : int32_t { kOpPack = 0, kOpCopyIn = 1, kOpCopyOut = 2, kOpWriteBack = 3, kOpWriteBackFlat = 4, kOpCopyInFlat = 5 };

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

// The records a stretch of work touches: first, first + 1, ...,
// first + count - 1.  Pack: the members overlapping columns [x*E, (x+1)*E)
// of a row (E = 2^map_lg bytes of elements), shared by all W rows.  Copy-in:
// the members overlapping bytes [x*2^map_lg, (x+1)*2^map_lg) of the row.
// Copy-out, write-back: the records owning windows [j*64, (j+1)*64).  Flat
// layout: the parameters overlapping flat positions [x*E, (x+1)*E).
struct ColumnWindow {
    int32_t first;
    int32_t count;
};
static_assert(sizeof(ColumnWindow) == 8, "shared with the device");

// One parameter's segment of the all-gather copy-in row: bytes [A, A_next)
// with A_next = A + P*size(dst_dt) rounded up to 16 bytes; its first P
// elements (param dtype dst_dt) are the shard (storage dtype src_dt) cast,
// the rest (fewer than 16 bytes) zero.  Its windows are win0, win0 + 1, ...
// (copy_in_windows of them).  The copy-in's pointer table is in record
// order: entry m is record m's shard.
struct CopyInSeg {
    int64_t A;
    int64_t P;
    int32_t win0;
    int32_t param;           // parameter index (host-side checks)
    int16_t src_dt;
    int16_t dst_dt;
    int32_t reserved;
};
static_assert(sizeof(CopyInSeg) == 32, "shared with the device");

// Windows of a copy-in segment of `bytes` bytes: its bytes cut at the
// 2 KiB-spaced line boundaries of memory, counted from the line holding its
// first byte, for the worst start in a line (the row is 4-byte aligned and
// segments start on 16-byte boundaries of it, so a segment starts at most
// 124 bytes past a line); a window past the segment's end for its start is
// empty.
FSDPPACK_HD inline int64_t copy_in_windows(int64_t bytes) { return (bytes + 124 + 2047) >> 11; }

// One parameter of the all-gather copy-out: its windows start at window
// index win0; numel elements of dtype dt, rank chunks of P elements found
// at byte A of each all-gather row.  The reduce-scatter write-back uses the
// same record for a bucket member: its windows cover the P-element rank
// chunk in the storage dtype dt, read from byte A = O * size(src_dt) of the
// rank's reduced row, whose elements have the bucket's reduction dtype src_dt.
// That row is the call's buffer (src_slot -1) or, in the write-back of all
// buckets in one launch, pointer-table entry src_slot.
struct CopyOutTensor {
    int64_t win0;
    int64_t numel;
    int64_t P;
    int64_t A;
    int32_t slot;
    int32_t dt;
    int32_t src_dt;          // write-back: the reduced row's dtype (copy-out: dt)
    int32_t src_slot;        // write-back: pointer-table entry of the reduced row, -1: the call's buffer
};
static_assert(sizeof(CopyOutTensor) == 48, "shared with the device");

// One parameter of an FSDP1 flat layout, for the flat write-back and copy-in:
// flat positions [F, F + numel); its pieces (the part inside a rank's
// positions) live in caller tensors of dtype dt.  `slot` is the parameter
// index; the pointer table of these operations is in record order.
struct FlatMember {
    int64_t F;
    int64_t numel;
    int32_t slot;
    int32_t dt;
    int64_t reserved;
};
static_assert(sizeof(FlatMember) == 32, "shared with the device");

// One candidate member of a pack stretch, in bytes of the destination row
// (column c of the row is bytes [c*dsz, (c+1)*dsz), dsz the reduction
// dtype's size), laid out so that the kernel's direct test is a handful of
// scalar instructions: a whole window starting at row byte y0 lies in the
// member's columns iff y0 - lo <= span (unsigned), and has no padding in row
// r iff (r, y0 + window) <= (full, end) in lexicographic order.  Stretch
// records are only built for buckets whose rows hold fewer than 2^31 bytes
// and whose members' rank chunks hold fewer than 2^32 source bytes
// (pack_narrow).
//   source of row r, row byte y (lo <= y < lo + P*dsz):
//       table[m] + r*Pss + (((y - lo) << 1) >> sh)
struct PackCand {
    uint32_t lo;             // O*dsz, the member's first row byte
    uint32_t span;           // P*dsz - window bytes (listed members hold at least one window)
    uint32_t end;            // row `full`'s first byte past its real columns: (O + numel - full*P)*dsz
    uint32_t full;           // ranks whose chunk is all real: numel / P
    uint32_t Pss;            // P*size(src): source bytes between consecutive rank chunks
    uint32_t moff;           // 8*m: the byte offset of the member's pointer-table entry
    uint32_t sh;             // 1 + log2(dsz) - log2(size(src))
    uint32_t code;           // src_dt*4 + dst_dt
};
static_assert(sizeof(PackCand) == 32, "shared with the device");

// The members a pack window may lie in, for the windows whose last byte falls
// in one stretch of 2^map_lg bytes of a row: the members of at least one
// window's length overlapping the stretch extended one window to the left
// (so the window's first byte is covered too), in column order, when there
// are at most two of them.  A window starting at or past c[1].lo lies in
// c[1] if anywhere.  A missing candidate has full = end = 0 (no window
// passes) and, as c[1], lo = ~0u.  The records run past the row's end, to
// the stretch of the last byte of the grid's last window, so that the record
// of any window of the grid exists.
struct PackStretch {
    PackCand c[2];
};
static_assert(sizeof(PackStretch) == 64, "one scalar load");

// Arguments of one launch (every operation).
struct WindowArgs {
    int32_t op;              // kOpPack, kOpCopyIn, kOpCopyOut, kOpWriteBack, kOpWriteBackFlat, kOpCopyInFlat
    int32_t n;               // entries of `members`
    int32_t n_windows;       // workgroups
    int32_t gx;              // pack: windows per row, less the row's spare window
    int32_t W;               // pack: rows (the world size; 1 for a flat layout)
    int32_t reduce_dt;       // pack: destination dtype, write-back: source dtype (the bucket's
                             // reduction dtype); flat ops: the rank row's dtype
    int32_t shift;           // pack / copy-in: bytes the destination starts past a cache-line boundary
    int32_t group_lg;        // pack: rows interleaved per row group, log2 (W is a multiple of 2^group_lg)
    int32_t rank;            // write-back, flat copy-in: the rank
    float divisor;           // write-back: divide factor (1: no division)
    int32_t map_lg;          // pack, copy-in, flat ops: log2 of the row bytes per entry of `columns`
    int64_t flat_n;          // flat layout: the flat parameter's real length N (its rows hold S = c each)
    int64_t S;               // pack: row length in elements; flat ops: c, a rank's row length
    int64_t B;               // copy-in row bytes / copy-out row stride
    const void *members;     // PackMember / CopyInSeg / CopyOutTensor / FlatMember records
    const void *columns;     // ColumnWindow map: per 2^map_lg bytes of a row (pack, copy-in) or of
                             // flat positions (flat ops), or per group of windows (copy-out, write-back)
    const uint64_t *table;   // device pointer table (by record for the pack and flat ops, else by parameter)
    char *base;              // the call's packed buffer or row (destination or source)
    const PackStretch *stretches;   // pack: one record per map stretch (null: no direct windows)
};

// Pointer tables of up to this many entries travel in the launch's own
// arguments (the kernel argument segment: no upload, no device memory, nothing
// cached), in two sizes so that small units copy few argument bytes; larger
// tables go through a device table.
constexpr int kInlineSmall = 64;
constexpr int kInlineLarge = 960;

// One contiguous range for the copy primitive: elements [lo, hi) of a chunk
// whose element 0 sits at byte src_off of its source and dst_off of its
// destination; elements >= valid are +0.
struct RangeRef {
    uint64_t ptr;            // the caller tensor's address (pointer-table entry `slot`)
    uint64_t src_ptr = 0;    // a source other than the call's buffer (pointer-table entry src_slot),
    int32_t src_slot = -1;   // for a range whose table side is its destination; 0 / -1: none
    int64_t src_off;
    int64_t dst_off;
    int64_t lo;
    int64_t hi;
    int64_t valid;
    int32_t slot;            // pointer-table entry
    int32_t param;           // parameter index (host-side checks; -1 for a range that is all +0)
    int32_t src_dt;
    int32_t dst_dt;
    int32_t table_side;
};

// Pointer-table entry; the host-side checker walks windows without a table.
FSDPPACK_HD inline uint64_t table_entry(const WindowArgs &a, int32_t slot)
{
    return a.table ? ((const FSDPPACK_TABLE uint64_t *)a.table)[slot] : 0;
}

// Record m of a table of 32-byte records, in one scalar load.  Read field by
// field, the compiler may defer the fields a later branch does not test (a
// second wait on the scalar cache before the wave's first data load), and it
// reads a 16-bit field with a vector load, whose wait also waits for every
// store the wave has issued.
template <typename T>
FSDPPACK_HD inline T read_record(const void *table, int32_t m)
{
    static_assert(sizeof(T) == 32, "32-byte records");
#if defined(__HIP_DEVICE_COMPILE__)
    typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));
    const u32x8 v = ((const FSDPPACK_TABLE u32x8 *)table)[m];
    T rec;
    __builtin_memcpy(&rec, &v, sizeof rec);
    return rec;
#else
    return static_cast<const T *>(table)[m];
#endif
}

FSDPPACK_HD inline int64_t imin(int64_t a, int64_t b) { return a < b ? a : b; }
FSDPPACK_HD inline int64_t imax(int64_t a, int64_t b) { return a > b ? a : b; }

// Non-negative division that takes the 32-bit path when both operands fit.
FSDPPACK_HD inline int64_t udiv(int64_t a, int64_t b)
{
    if (((a | b) >> 32) == 0) return static_cast<int64_t>(static_cast<uint32_t>(a) / static_cast<uint32_t>(b));
    return static_cast<int64_t>(static_cast<uint64_t>(a) / static_cast<uint64_t>(b));
}

// Bytes [y0, y1) of a destination of `total` bytes that window w covers when
// the destination starts `shift` bytes past a cache-line boundary: window
// boundaries fall on line boundaries of memory.
FSDPPACK_HD inline void window_span(int32_t w, int32_t shift, int64_t total, int64_t &y0, int64_t &y1)
{
    const int64_t start = (static_cast<int64_t>(w) << kWindowLog2) - shift;
    y0 = imax(0, start);
    y1 = imin(total, start + kWindowBytes);
}

// Row r and window k of that row for pack window w.  Every row has gx + 1
// windows; rows go in groups of G = 2^group_lg, and inside a group the
// windows interleave row by row (window k of rows g*G ... g*G + G - 1, then
// window k + 1): with small rank chunks, the windows in flight then read a
// few contiguous stretches of each gradient instead of many scattered ones.
FSDPPACK_HD inline void pack_row_window(const WindowArgs &a, int32_t w, int32_t &r, int32_t &k)
{
    const int32_t span = (a.gx + 1) << a.group_lg;       // windows per row group
    const int32_t g = w / span, within = w - g * span;
    k = within >> a.group_lg;
    r = (g << a.group_lg) + (within & ((1 << a.group_lg) - 1));
}

// Row r and window k of the pack window at (x, g) of the launch's 2-D grid:
// g is the row group, x runs over its windows (window k of each of the
// group's 2^group_lg rows in turn) -- the same (r, k) as pack_row_window for
// w = g * (gx + 1) * 2^group_lg + x, without a division.
FSDPPACK_HD inline void pack_row_window_2d(const WindowArgs &a, uint32_t x, uint32_t g, int32_t &r, int32_t &k)
{
    k = static_cast<int32_t>(x >> a.group_lg);
    r = static_cast<int32_t>((g << a.group_lg) + (x & ((1u << a.group_lg) - 1)));
}

// Pack window k of row r.  The row's window boundaries sit on line boundaries
// of memory: window k covers bytes [k*kWindowBytes - s_r, (k+1)*kWindowBytes
// - s_r) of the row, clipped to it, with s_r how far the row starts past a
// line boundary (a row's last window is empty when its bytes fit in gx
// windows).  Its columns [c0, c1) lie in one or two stretches of the column
// map, whose entries name the members to visit: a wave makes two rounds of
// table reads (the column entries, then each member record with its pointer)
// before its data.
template <typename F>
FSDPPACK_HD inline void pack_window_rk(const WindowArgs &a, int32_t r, int32_t k, F &&f)
{
    const FSDPPACK_TABLE ColumnWindow *C = (const FSDPPACK_TABLE ColumnWindow *)a.columns;
    const int lg = a.reduce_dt == kBF16 ? 1 : 2;            // log2 of the element size
    const int64_t rb = a.S << lg;                         // bytes per row
    const int32_t s_r = static_cast<int32_t>((a.shift + r * rb) & (kLineBytes - 1));
    int64_t y0, y1;
    window_span(k, s_r, rb, y0, y1);
    if (y1 <= y0) return;                                 // the row's spare window
    const int64_t c0 = y0 >> lg, c1 = y1 >> lg;
    const int32_t x0 = static_cast<int32_t>(c0 >> (a.map_lg - lg));
    const int32_t x1 = static_cast<int32_t>((c1 - 1) >> (a.map_lg - lg));
    const int32_t m0 = C[x0].first;
    const ColumnWindow last = C[x1];
    for (int32_t m = m0; m < last.first + last.count; ++m) {
        const uint64_t ptr = table_entry(a, m);          // issued with the member read
        const PackMember pm = read_record<PackMember>(a.members, m);
        const int64_t b0 = imax(c0, pm.O), b1 = imin(c1, pm.O + pm.P);
        if (b1 <= b0) continue;                          // in the column window, not in this window
        RangeRef g;
        g.ptr = ptr;
        g.src_off = r * pm.P * dtype_bytes(pm.src_dt);
        g.dst_off = (r * a.S + pm.O) << lg;
        g.lo = b0 - pm.O;
        g.hi = b1 - pm.O;
        g.valid = imax(0, imin(pm.P, pm.numel - r * pm.P));
        g.slot = m;
        g.param = pm.param;
        g.src_dt = pm.src_dt;
        g.dst_dt = a.reduce_dt;
        g.table_side = kTableIsSource;
        f(g);
    }
}

// Pack window w (linear index, pack_row_window).
template <typename F>
FSDPPACK_HD inline void pack_window(const WindowArgs &a, int32_t w, F &&f)
{
    int32_t r, k;
    pack_row_window(a, w, r, k);
    pack_window_rk(a, r, k, f);
}

// A pack window that is one whole window of a single member's rank chunk,
// every element real: the common case, which the kernel moves with a short
// direct copy instead of the general range walk.  `src` is the address of
// the window's first source element (dword aligned, or 2 bytes past a dword
// for a bf16 source), `dst_off` the byte offset of its first destination
// element in the packed buffer (16-byte aligned in memory).
struct DirectWindow {
    uint64_t src;
    int64_t dst_off;
    int32_t src_dt;
    int32_t dst_dt;
};

// Whether window k of row r is such a window (its stretches of the column map
// name one or two members, one of whose chunks holds the whole window with
// no padding, and both ends are aligned for whole 16-byte destination
// vectors and dword source loads); fills `d` when it is.  Both candidate
// records and pointers are read in the same round trip.  The window then
// equals the single range pack_window produces for it, with lo = c0 - O,
// hi = c1 - O and every element below `valid`.
FSDPPACK_HD inline bool pack_direct_rk(const WindowArgs &a, int32_t r, int32_t k, DirectWindow &d)
{
    const FSDPPACK_TABLE ColumnWindow *C = (const FSDPPACK_TABLE ColumnWindow *)a.columns;
    const int lg = a.reduce_dt == kBF16 ? 1 : 2;
    const int64_t rb = a.S << lg;
    const int32_t s_r = static_cast<int32_t>((a.shift + r * rb) & (kLineBytes - 1));
    int64_t y0, y1;
    window_span(k, s_r, rb, y0, y1);
    if (y1 - y0 != kWindowBytes) return false;
    const int64_t c0 = y0 >> lg, c1 = y1 >> lg;
    const ColumnWindow e0 = C[static_cast<int32_t>(c0 >> (a.map_lg - lg))];
    const ColumnWindow e1 = C[static_cast<int32_t>((c1 - 1) >> (a.map_lg - lg))];
    const int32_t m0 = e0.first, n = e1.first + e1.count - m0;   // candidates m0, m0 + 1
    if (n < 1 || n > 2) return false;
    const int32_t m1 = m0 + n - 1;
    const uint64_t ptr0 = table_entry(a, m0), ptr1 = table_entry(a, m1);
    const PackMember pm0 = read_record<PackMember>(a.members, m0);
    const PackMember pm1 = read_record<PackMember>(a.members, m1);
    const bool second = c0 >= pm1.O;                     // members tile the columns in order
    const PackMember pm = second ? pm1 : pm0;
    const uint64_t ptr = second ? ptr1 : ptr0;
    if (c0 < pm.O || c1 > pm.O + pm.P || r * pm.P + (c1 - pm.O) > pm.numel) return false;
    d.src = ptr + static_cast<uint64_t>((r * pm.P + (c0 - pm.O)) * dtype_bytes(pm.src_dt));
    d.dst_off = (r * a.S + c0) << lg;
    d.src_dt = pm.src_dt;
    d.dst_dt = a.reduce_dt;
    // a bf16 source may start 2 bytes past a dword (the kernel then shifts)
    return (d.src & (pm.src_dt == kBF16 ? 1u : 3u)) == 0 && ((a.shift + d.dst_off) & 15) == 0;
}

// pack_direct_rk for pack window w (linear index, pack_row_window).
FSDPPACK_HD inline bool pack_direct(const WindowArgs &a, int32_t w, DirectWindow &d)
{
    int32_t r, k;
    pack_row_window(a, w, r, k);
    return pack_direct_rk(a, r, k, d);
}

// Whether window k of row r is a direct window according to the stretch
// records (a.stretches, built with the plan by build_pack_stretches): one
// whole window inside one member's rank chunk, every element real.  Three
// short scalar loads (the second candidate's first byte in the stretch
// record of the window's last byte, then the one candidate the window can
// lie in, then the member's pointer) stand between the launch arguments and
// the data, with few scalar instructions around them: the record holds each
// candidate's bounds in row bytes, so the test is two unsigned compares.
// The index arithmetic is 32-bit (rows of fewer than 2^31 bytes).  Fills `d`
// as pack_direct does; the window then equals the single range pack_window_rk
// produces for it.  Both ends are always aligned for whole 16-byte
// destination vectors (a window starts k*2048 bytes past the line boundary
// at or before the row's start) and for element loads of the source (the
// caller's pointers are aligned to their element size).
// (The launch's fields the test reads are passed one by one: the kernel takes
// them as leading scalar arguments, which the hardware can place in scalar
// registers before the wave starts.)  table: the pointer table; rb: row
// bytes.
FSDPPACK_HD inline bool pack_direct_stretch_s(const PackStretch *stretches, const uint64_t *table, uint32_t rb,
                                              uint32_t shift, uint32_t map_lg, int32_t r, int32_t k, DirectWindow &d)
{
    constexpr uint32_t kWin = static_cast<uint32_t>(kWindowBytes);
    const uint32_t ur = static_cast<uint32_t>(r);
    const uint32_t s_r = (shift + ur * rb) & static_cast<uint32_t>(kLineBytes - 1);
    // the row's first window wraps y0 below 0 (mod 2^32) when the row starts
    // off a line; y0 + kWin - 1 wraps back, so its record is still in range,
    // and it fails the range test
    const uint32_t y0 = (static_cast<uint32_t>(k) << kWindowLog2) - s_r, y1 = y0 + kWin;
    const uint32_t rec = ((y0 + (kWin - 1u)) >> map_lg) * static_cast<uint32_t>(sizeof(PackStretch));
#if defined(__HIP_DEVICE_COMPILE__)
    // the second candidate's first byte decides which of the two 32-byte
    // candidates to load, so that no field needs a select
    const FSDPPACK_TABLE char *R = (const FSDPPACK_TABLE char *)stretches;
    const uint32_t split = *(const FSDPPACK_TABLE uint32_t *)(R + rec + sizeof(PackCand));
    typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));
    const u32x8 v = *(const FSDPPACK_TABLE u32x8 *)(R + (rec | (y0 >= split ? static_cast<uint32_t>(sizeof(PackCand)) : 0u)));
    const uint32_t lo = v[0], span = v[1], end = v[2], full = v[3], Pss = v[4], moff = v[5], sh = v[6], code = v[7];
    const uint64_t ptr = *(const FSDPPACK_TABLE uint64_t *)((const FSDPPACK_TABLE char *)table + moff);
#else
    const PackStretch &e = *reinterpret_cast<const PackStretch *>(reinterpret_cast<const char *>(stretches) + rec);
    const PackCand &c = y0 >= e.c[1].lo ? e.c[1] : e.c[0];
    const uint32_t lo = c.lo, span = c.span, end = c.end, full = c.full, Pss = c.Pss, sh = c.sh, code = c.code;
    const uint64_t ptr = table ? table[c.moff / 8] : 0;
#endif
    // inside the member's columns, and no padding: r < full, or r == full
    // and y1 <= end, which is r < full + (y1 <= end) (full < 2^31)
    const uint32_t t = y0 - lo;
    if (!((t <= span) & (ur < full + (y1 <= end ? 1u : 0u)))) return false;
    d.src = ptr + static_cast<uint64_t>(ur) * Pss + ((t << 1) >> sh);
    d.dst_off = static_cast<int64_t>(static_cast<uint64_t>(ur) * rb + y0);
    d.src_dt = static_cast<int32_t>(code >> 2);
    d.dst_dt = static_cast<int32_t>(code & 3u);
    return true;
}

FSDPPACK_HD inline bool pack_direct_stretch(const WindowArgs &a, int32_t r, int32_t k, DirectWindow &d)
{
    const uint32_t lg = a.reduce_dt == kBF16 ? 1u : 2u;
    return pack_direct_stretch_s(a.stretches, a.table, static_cast<uint32_t>(a.S) << lg, static_cast<uint32_t>(a.shift),
                                 static_cast<uint32_t>(a.map_lg), r, k, d);
}

// The record of the window-indexed table `T` (records sorted by win0)
// whose windows contain window w: a binary search among the few records the
// group map names for w's group (usually one).
template <typename T>
FSDPPACK_HD inline int32_t find_record(const void *groups, const void *records, int32_t w)
{
    const FSDPPACK_TABLE T *R = (const FSDPPACK_TABLE T *)records;
    const ColumnWindow grp = ((const FSDPPACK_TABLE ColumnWindow *)groups)[w >> kGroupLog2];
    int32_t lo = grp.first, hi = grp.first + grp.count - 1;   // last record with win0 <= w
    while (lo < hi) {
        const int32_t mid = (lo + hi + 1) >> 1;
        if (R[mid].win0 <= w) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// Group map of the copy-in, per 2^kGroupLog2 windows: the record owning the
// group's first window and, when one more record starts inside the group,
// the window where it starts (split; INT32_MAX when the group has one record),
// so that a window names its record without reading any; a group over three
// or more records holds -(their number) in split, and its windows search.
struct WindowGroup {
    int32_t first;
    int32_t split;
};
static_assert(sizeof(WindowGroup) == 8, "shared with the device");

FSDPPACK_HD inline int32_t find_copy_in_record(const void *groups, const void *segs, int32_t w)
{
    const WindowGroup g = ((const FSDPPACK_TABLE WindowGroup *)groups)[w >> kGroupLog2];
    if (g.split >= 0) return g.first + (w >= g.split ? 1 : 0);
    const FSDPPACK_TABLE CopyInSeg *R = (const FSDPPACK_TABLE CopyInSeg *)segs;
    int32_t lo = g.first, hi = g.first - g.split - 1;   // last record with win0 <= w
    while (lo < hi) {
        const int32_t mid = (lo + hi + 1) >> 1;
        if (R[mid].win0 <= w) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// Copy-in window w of a row that starts `shift` bytes past a cache line:
// segment m (from the group map; its record `s` read in one scalar load
// together with its shard's pointer, table entry m) and its bytes [y0, y1) of the row, which
// end on line boundaries of memory except at the segment's own ends.  Every
// window is thus one range of one segment; y1 <= y0 for a spare window.
struct CopyInWindow {
    CopyInSeg s;
    uint64_t ptr;
    int32_t m;
    int64_t y0, y1, A_next;
};
FSDPPACK_HD inline CopyInWindow copy_in_span(const void *groups, const void *segs, const uint64_t *table,
                                             int32_t shift, int32_t w)
{
    CopyInWindow c;
    c.m = find_copy_in_record(groups, segs, w);
    c.s = read_record<CopyInSeg>(segs, c.m);
    c.ptr = table ? ((const FSDPPACK_TABLE uint64_t *)table)[c.m] : 0;
    const int lg = c.s.dst_dt == kBF16 ? 1 : 2;
    c.A_next = c.s.A + ((((c.s.P << lg) + 15) >> 4) << 4);
    const int64_t line0 = ((shift + c.s.A) & ~static_cast<int64_t>(kLineBytes - 1)) - shift;
    const int64_t start = line0 + (static_cast<int64_t>(w - c.s.win0) << kWindowLog2);
    c.y0 = imax(c.s.A, start);
    c.y1 = imin(c.A_next, start + kWindowBytes);
    return c;
}

// The window's one range (elements [lo, hi) of the segment; those past P
// are the zero gap).
FSDPPACK_HD inline RangeRef copy_in_range(const CopyInWindow &c)
{
    const int lg = c.s.dst_dt == kBF16 ? 1 : 2;
    RangeRef g;
    g.ptr = c.ptr;
    g.src_off = 0;
    g.dst_off = c.s.A;
    g.lo = (c.y0 - c.s.A) >> lg;
    g.hi = (c.y1 - c.s.A) >> lg;
    g.valid = c.s.P;
    g.slot = c.m;
    g.param = c.s.param;
    g.src_dt = c.s.src_dt;
    g.dst_dt = c.s.dst_dt;
    g.table_side = kTableIsSource;
    return g;
}

// Whether the window is copied whole by the direct copy: 2 KiB of real
// elements on 16-byte destination vectors (every window but a segment's
// first and last, on a row 16-byte aligned in memory); fills `d`.  The copy
// is then exactly the window's range.
FSDPPACK_HD inline bool copy_in_direct(const CopyInWindow &c, int32_t shift, DirectWindow &d)
{
    const int lg = c.s.dst_dt == kBF16 ? 1 : 2;
    if (c.y1 - c.y0 != kWindowBytes || ((c.y1 - c.s.A) >> lg) > c.s.P || ((shift + c.y0) & 15) != 0) return false;
    d.src = c.ptr + static_cast<uint64_t>(((c.y0 - c.s.A) >> lg) * dtype_bytes(c.s.src_dt));
    d.dst_off = c.y0;
    d.src_dt = c.s.src_dt;
    d.dst_dt = c.s.dst_dt;
    return true;
}

// Copy-in window w of the launch `a` as a range (none for a spare window).
template <typename F>
FSDPPACK_HD inline void copy_in_window(const WindowArgs &a, int32_t w, F &&f)
{
    const CopyInWindow c = copy_in_span(a.columns, a.members, a.table, a.shift, w);
    if (c.y1 > c.y0) f(copy_in_range(c));
}

// The tensor record whose windows contain window w: a binary search on win0
// among the few records the group map names for w's group (usually one).
FSDPPACK_HD inline CopyOutTensor find_tensor(const WindowArgs &a, int32_t w)
{
    return ((const FSDPPACK_TABLE CopyOutTensor *)a.members)[find_record<CopyOutTensor>(a.columns, a.members, w)];
}

// Elements [e0, e1) of tensor t that copy-out window w covers: bytes
// [x*kWindowBytes, ...) of the tensor (windows start at each tensor's own
// first byte; `shift` is unused).
FSDPPACK_HD inline void copy_out_span(const CopyOutTensor &t, int32_t w, int64_t &e0, int64_t &e1)
{
    const int64_t per = kWindowBytes / dtype_bytes(t.dt);
    e0 = (w - t.win0) * per;
    e1 = imin(t.numel, e0 + per);
}

// Byte offset in the gathered buffer of element i of tensor t: element
// i - r*P of rank r's chunk, r = i / P, which sits at byte r*B + A.  For
// tensors of fewer than 2^32 elements (P <= numel), in 32-bit division.
FSDPPACK_HD inline int64_t copy_out_source(const WindowArgs &a, const CopyOutTensor &t, uint32_t i)
{
    const uint32_t P = static_cast<uint32_t>(t.P), r = i / P;
    return static_cast<int64_t>(r) * a.B + t.A + static_cast<int64_t>(i - r * P) * dtype_bytes(t.dt);
}

// Rank chunks above which a copy-out window is gathered element by element
// in one pass (copy_out_source per element) instead of walked chunk by
// chunk.  A parameter with fewer rows than ranks has chunks of a few
// elements, and a window over them meets dozens; walking them costs a full
// round trip of loads and stores per chunk, since a wave's wait for its
// loads also waits for its earlier stores.
constexpr int64_t kGatherChunks = 2;

FSDPPACK_HD inline bool copy_out_gathered(const CopyOutTensor &t, int64_t e0, int64_t e1)
{
    return (t.numel >> 32) == 0 && udiv(e1 - 1, t.P) - udiv(e0, t.P) >= kGatherChunks;
}

// Copy-out window w of tensor t, split at rank-chunk boundaries; chunk r
// comes from byte r*B + A of the gathered buffer.
template <typename F>
FSDPPACK_HD inline void copy_out_chunks(const WindowArgs &a, const CopyOutTensor &t, int32_t w, F &&f)
{
    const uint64_t ptr = table_entry(a, t.slot);
    const int64_t esz = dtype_bytes(t.dt);
    int64_t e0, e1;
    copy_out_span(t, w, e0, e1);
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

// Copy-out window w: the chunks of the tensor owning it.
template <typename F>
FSDPPACK_HD inline void copy_out_window(const WindowArgs &a, int32_t w, F &&f)
{
    copy_out_chunks(a, find_tensor(a, w), w, f);
}

// Reduce-scatter write-back window w: bytes [x*kWindowBytes, ...) of the
// rank chunk of the member owning w, in its storage dtype, clipped to the
// chunk's real elements for rank a.rank (a window past them does nothing);
// the source is the member's columns of the rank's reduced row.
template <typename F>
FSDPPACK_HD inline void write_back_window(const WindowArgs &a, int32_t w, F &&f)
{
    const CopyOutTensor t = find_tensor(a, w);
    const int64_t esz = dtype_bytes(t.dt);
    const int64_t e0 = (w - t.win0) * (kWindowBytes / esz);
    const int64_t valid = imax(0, imin(t.P, t.numel - static_cast<int64_t>(a.rank) * t.P));
    const int64_t e1 = imin(valid, e0 + kWindowBytes / esz);
    if (e1 <= e0) return;
    RangeRef g;
    g.ptr = table_entry(a, t.slot);
    g.src_slot = t.src_slot;
    if (t.src_slot >= 0) g.src_ptr = table_entry(a, t.src_slot);
    g.src_off = t.A;
    g.dst_off = 0;
    g.lo = e0;
    g.hi = e1;
    g.valid = e1;
    g.slot = t.slot;
    g.param = t.slot;
    g.src_dt = t.src_dt;
    g.dst_dt = t.dt;
    g.table_side = kTableIsDest;
    f(g);
}

// FSDP1 flat layout, write-back (COPY_IN false) or copy-in (COPY_IN true)
// window w of rank a.rank's row: S = c elements of dtype reduce_dt (the
// reduction dtype for the write-back, the param dtype for the copy-in), flat
// positions [rank*c, rank*c + c).  The window's row elements [e0, e1) lie in
// one or two stretches of the flat-position map, which names the
// parameters there; each overlap is a range between the row and that
// parameter's piece (its part inside the rank's positions, starting at flat
// position max(F, rank*c)).  The copy-in also writes the row's padding
// (positions past N) as +0, a range with no source.
template <bool COPY_IN, typename F>
FSDPPACK_HD inline void flat_window(const WindowArgs &a, int32_t w, F &&f)
{
    const FSDPPACK_TABLE ColumnWindow *C = (const FSDPPACK_TABLE ColumnWindow *)a.columns;
    const int lg = a.reduce_dt == kBF16 ? 1 : 2;          // log2 of the row's element size
    int64_t y0, y1;
    window_span(w, a.shift, a.S << lg, y0, y1);
    const int64_t e0 = y0 >> lg, e1 = y1 >> lg;
    const int64_t base = static_cast<int64_t>(a.rank) * a.S;   // flat position of row element 0
    const int64_t f0 = base + e0, f1 = imin(base + e1, a.flat_n);
    if (f0 < f1) {
        const int32_t m0 = C[f0 >> (a.map_lg - lg)].first;
        const ColumnWindow last = C[(f1 - 1) >> (a.map_lg - lg)];
        for (int32_t m = m0; m < last.first + last.count; ++m) {
            const uint64_t ptr = table_entry(a, m);      // pointer table in record order
            const FlatMember fm = read_record<FlatMember>(a.members, m);
            const int64_t b0 = imax(f0, fm.F), b1 = imin(f1, fm.F + fm.numel);
            if (b1 <= b0) continue;                      // in the map's stretch, not in this window
            const int64_t piece0 = imax(fm.F, base);
            const int64_t in_piece = (b0 - piece0) * dtype_bytes(fm.dt), in_row = (b0 - base) << lg;
            RangeRef g;
            g.ptr = ptr;
            g.src_off = COPY_IN ? in_piece : in_row;
            g.dst_off = COPY_IN ? in_row : in_piece;
            g.lo = 0;
            g.hi = b1 - b0;
            g.valid = g.hi;
            g.slot = m;
            g.param = fm.slot;
            g.src_dt = COPY_IN ? fm.dt : a.reduce_dt;
            g.dst_dt = COPY_IN ? a.reduce_dt : fm.dt;
            g.table_side = COPY_IN ? kTableIsSource : kTableIsDest;
            f(g);
        }
    }
    if (COPY_IN && base + e1 > a.flat_n) {
        const int64_t z0 = imax(e0, a.flat_n - base);    // first padding element of the window
        RangeRef g;
        g.ptr = 0;
        g.src_off = 0;
        g.dst_off = z0 << lg;
        g.lo = 0;
        g.hi = e1 - z0;
        g.valid = 0;                                      // all +0: no source element is read
        g.slot = 0;
        g.param = -1;
        g.src_dt = a.reduce_dt;
        g.dst_dt = a.reduce_dt;
        g.table_side = kTableIsSource;
        f(g);
    }
}

// Whether FSDP1 flat copy-in window w is one whole window inside a single
// parameter's piece of the rank's row, with every element real and its
// destination on 16-byte vectors; fills `d` (source: the piece's pointer
// plus the window's offset in it; destination: the window's row offset).
// With one or two records in the window's map stretches, both records and
// pointers (table in record order) are read in one round trip.  The window
// then equals the single range flat_window<true> produces for it.
FSDPPACK_HD inline bool flat_copy_in_direct(const WindowArgs &a, int32_t w, DirectWindow &d)
{
    const FSDPPACK_TABLE ColumnWindow *C = (const FSDPPACK_TABLE ColumnWindow *)a.columns;
    const int lg = a.reduce_dt == kBF16 ? 1 : 2;          // log2 of the row's element size
    int64_t y0, y1;
    window_span(w, a.shift, a.S << lg, y0, y1);
    if (y1 - y0 != kWindowBytes || ((a.shift + y0) & 15) != 0) return false;
    const int64_t base = static_cast<int64_t>(a.rank) * a.S;   // flat position of row element 0
    const int64_t f0 = base + (y0 >> lg), f1 = base + (y1 >> lg);
    if (f1 > a.flat_n) return false;                      // padding in the window
    const ColumnWindow e0 = C[f0 >> (a.map_lg - lg)], e1 = C[(f1 - 1) >> (a.map_lg - lg)];
    const int32_t m0 = e0.first, n = e1.first + e1.count - m0;
    if (n < 1 || n > 2) return false;
    const FlatMember r0 = read_record<FlatMember>(a.members, m0);
    const FlatMember r1 = read_record<FlatMember>(a.members, m0 + n - 1);
    const uint64_t p0 = table_entry(a, m0), p1 = table_entry(a, m0 + n - 1);
    const bool second = f0 >= r1.F;                       // records tile the flat positions in order
    const FlatMember &fm = second ? r1 : r0;
    if (f0 < fm.F || f1 > fm.F + fm.numel) return false;
    d.src = (second ? p1 : p0) + static_cast<uint64_t>((f0 - imax(fm.F, base)) * dtype_bytes(fm.dt));
    d.dst_off = y0;
    d.src_dt = fm.dt;
    d.dst_dt = a.reduce_dt;
    return true;
}

template <typename F>
FSDPPACK_HD inline void for_each_range(const WindowArgs &a, int32_t w, F &&f)
{
    if (a.op == kOpPack) pack_window(a, w, f);
    else if (a.op == kOpCopyIn) copy_in_window(a, w, f);
    else if (a.op == kOpCopyOut) copy_out_window(a, w, f);
    else if (a.op == kOpWriteBack) write_back_window(a, w, f);
    else if (a.op == kOpWriteBackFlat) flat_window<false>(a, w, f);
    else flat_window<true>(a, w, f);
}

// Launch the window kernel on `stream`: one workgroup per window.  With
// `inline_ptrs` (n <= kInlineLarge entries) the pointer table travels in the
// launch's arguments; otherwise args.table is a device table.
// start_event / stop_event (hipEvent_t, may be NULL) are stamped at the
// kernel's start and end.  Returns the hipError_t of the launch as an int.
int launch_windows(const WindowArgs &args, const uint64_t *inline_ptrs, int32_t n, void *stream, void *start_event,
                   void *stop_event);

// Bytes of the device scratch the allocation-free pack copies a bucket's
// pack tables into, and the devices it serves.
constexpr int64_t kScratchBytes = int64_t{1} << 20;
constexpr int kMaxDevices = 64;

// The address of the scratch on the current device (looked up once per
// device).  Returns the hipError_t as an int.
int scratch_address(void **out);

// Launch a kernel that does nothing: `workgroups` workgroups of `threads`
// threads (checked by the caller).
int launch_empty(int32_t workgroups, int32_t threads, void *stream, void *start_event, void *stop_event);

}  // namespace fsdppack
