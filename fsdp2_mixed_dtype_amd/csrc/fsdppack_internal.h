// fsdppack_internal.h -- plan, work-list and device-table types shared by the
// host planner, the ABI layer and the HIP kernels of libfsdppack.
//
// Every operation of the library (reduce-scatter pack, all-gather copy-in,
// all-gather copy-out) is the same primitive over a list of *segments*: a
// contiguous destination run of `len` elements whose first `valid` elements
// are the cast of a contiguous source run and whose remaining elements are
// +0 (the right-hand padding of a rank chunk, or the zero gap after an
// all-gather segment).  One side of every segment lives in a caller tensor
// reached through a per-call pointer table; the other side is an offset into
// the call's single packed buffer.
//
// Work is split into *items*, one per workgroup: item k covers everything
// from one (segment, element offset) to the next, so a workgroup may cover
// part of one large segment or many small ones.  This array is the prefix
// map from workgroup to (tensor, rank chunk).
#pragma once

#include <cstdint>

namespace fsdppack {

enum : int32_t { kNone = 0, kBF16 = 1, kFP32 = 2 };

// Destination bytes per work item (one workgroup): the kernel's block size x
// unroll x 16-byte vectors.  Plans may be cut finer or coarser (the kernel is
// correct for any item size); this is the size it is tuned for.
constexpr int64_t kItemBytes = 4096;

inline int64_t dtype_bytes(int32_t dt) { return dt == kBF16 ? 2 : 4; }
inline bool dtype_ok(int32_t dt) { return dt == kBF16 || dt == kFP32; }

// Which side of a segment is the caller's tensor (reached through the
// pointer table); the other side is the call's packed buffer.
enum : uint8_t { kTableIsSource = 0, kTableIsDest = 1 };

struct Seg {
    int64_t dst_off;   // byte offset of element 0 from the destination base
    int64_t src_off;   // byte offset of element 0 from the source base
    int64_t len;       // destination elements
    int64_t valid;     // leading elements taken from the source, 0 <= valid <= len
    int32_t slot;      // pointer-table entry (parameter index)
    uint8_t src_dt;    // kBF16 / kFP32
    uint8_t dst_dt;
    uint8_t table_side;
    uint8_t pad_;
};
static_assert(sizeof(Seg) == 40, "Seg layout is shared with the device");

// One work item: the elements from (seg_a, off_a) up to, not including,
// (seg_b, off_b) of the segment list, where (seg_b, off_b) may be
// (n_segs, 0), the end of the list.
struct Item {
    int32_t seg_a;
    int32_t seg_b;
    int64_t off_a;
    int64_t off_b;
    int64_t pad_;
};
static_assert(sizeof(Item) == 32, "Item layout is shared with the device");

// Workgroups are dealt to the GPU's XCDs round-robin (workgroup b runs on XCD
// b % kXcds), and each XCD has its own L2.  Item b is therefore stored at
// item_slot(b): the workgroups of one XCD read consecutive records, so one
// 128-byte line serves four workgroups of the same XCD instead of being
// fetched by several XCDs.  A bijection on [0, n); only locality depends on
// the XCD count being right.
constexpr int32_t kXcds = 8;
#if defined(__HIP__)
__attribute__((host, device))   // shared by the host planner and the kernel
#endif
inline int32_t item_slot(int32_t b, int32_t n)
{
    const int32_t per = n / kXcds;
    return b < per * kXcds ? (b % kXcds) * per + b / kXcds : b;
}

// Arguments of one launch of the grouped segment kernel.
struct LaunchArgs {
    const Seg *segs;
    const Item *items;       // n_items records, item b at item_slot(b, n_items)
    const uint64_t *table;   // device pointer table, indexed by Seg::slot
    char *base;              // the call's packed buffer (destination or source)
    int32_t n_items;
    int32_t pad_;
};

// Launch the grouped segment kernel on `stream`: one workgroup per item.
// start_event / stop_event (hipEvent_t, may be NULL) are stamped at the
// kernel's start and end.  Returns the hipError_t of the launch as an int.
int launch_segments(const LaunchArgs &args, void *stream, void *start_event, void *stop_event);

}  // namespace fsdppack
