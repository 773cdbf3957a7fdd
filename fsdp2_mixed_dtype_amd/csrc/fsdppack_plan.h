// fsdppack_plan.h -- host-side plan of one fully_shard unit (internal).
//
// The planner follows "PyTorch adds per-parameter mixed precision to FSDP2"
// (ainewsletter.today), paragraph 2, for bucketing (one reduction buffer per
// effective reduction dtype), and "The unit you wrapped" (kernels.rudrite.com),
// padding paragraphs, for the equal right-padded rank pieces (or, for the
// FSDP1 flat layout, one flat parameter split into equal pieces).  It also
// builds the record tables and maps the kernels read (one per operation).
#pragma once

#include <atomic>
#include <cstdint>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/fsdppack.h"
#include "fsdppack_internal.h"

namespace fsdppack {

// One launchable operation: its member table (uploaded once) and launch
// geometry.
struct OpTable {
    int32_t op = kOpPack;
    std::vector<unsigned char> members;   // PackMember / CopyInSeg / CopyOutTensor / FlatMember records
    std::vector<ColumnWindow> columns;    // record map (pack, flat ops: per 2^map_lg bytes of a row;
                                          // copy-in, copy-out, write-back: per window group)
    std::vector<int32_t> table_params;    // pointer-table entry -> parameter index
    int32_t n = 0;                        // records
    int32_t n_windows = 0;                // workgroups per launch (pack, flat copy-in: destination window-aligned)
    int32_t gx = 0;                       // pack: windows per row, less the spare one
    int32_t map_lg = kWindowLog2;         // pack, flat ops: log2 of the bytes per map entry
    int32_t group_lg = 0;                 // pack: log2 of the rows interleaved per row group
    int32_t rows = 1;                     // pack: rows of the launch (W; 1 for a flat layout)
    int64_t flat_n = 0;                   // flat ops: the flat parameter's real length N
    int32_t reduce_dt = 0;                // pack, write-back: the bucket's reduction dtype
    int64_t S = 0;                        // pack: row length (elements)
    int64_t B = 0;                        // all-gather row bytes
    int64_t dst_bytes = 0;                // bytes the operation writes
    int64_t src_bytes = 0;                // bytes it reads
    bool narrow = false;                  // pack: rows of fewer than 2^31 bytes and rank chunks of fewer
                                          // than 2^32 source bytes, so the plan holds stretch records
                                          // (one per column-map entry) for the direct windows
    std::vector<PackStretch> stretches;   // pack: the stretch records (narrow tables only)
    // pack: where the allocation-free pack finds the member table, column map
    // and stretch records in the device scratch (byte offsets from the
    // bucket's place there: members at 0, the others each at a 256-byte
    // boundary; scratch_need bytes in all), and the bucket's own image of them
    // when the plan has no plan-wide image (empty when they need more than
    // kScratchBytes or the pointer table has more than kInlineLarge entries)
    std::vector<unsigned char> scratch_image;
    int64_t scratch_c_off = 0, scratch_s_off = 0, scratch_need = 0;
    void *d_members = nullptr;            // device copies (owned by the plan)
    void *d_columns = nullptr;
    void *d_stretches = nullptr;

    template <typename T> void add(const T &rec)
    {
        const unsigned char *p = reinterpret_cast<const unsigned char *>(&rec);
        members.insert(members.end(), p, p + sizeof(T));
        ++n;
    }
    // Workgroups of a launch whose destination starts `shift` bytes past a
    // cache-line boundary: the pack gives every row gx + 1 windows (enough
    // for any alignment of the row), the flat copy-in cuts its row at line
    // boundaries of memory, the copy-in gives each parameter's segment the
    // windows its worst alignment needs, and the copy-out's and write-back's
    // windows start at each parameter's first byte.
    int64_t windows(int32_t shift) const
    {
        if (op == kOpCopyIn || op == kOpCopyOut || op == kOpWriteBack || op == kOpWriteBackFlat) return n_windows;
        if (dst_bytes == 0) return 0;
        if (op == kOpPack) return (static_cast<int64_t>(gx) + 1) * (dst_bytes / (S * dtype_bytes(reduce_dt)));
        return (shift + dst_bytes + kWindowBytes - 1) >> kWindowLog2;
    }
    // launch arguments against host (`device == false`) or device members
    WindowArgs args(bool device, int32_t shift) const
    {
        WindowArgs a{};
        a.op = op;
        a.n = n;
        a.shift = (op == kOpCopyOut || op == kOpWriteBack || op == kOpWriteBackFlat) ? 0 : shift;
        a.W = rows;
        a.flat_n = flat_n;
        a.n_windows = static_cast<int32_t>(windows(a.shift));
        a.gx = gx;
        a.group_lg = group_lg;
        a.map_lg = map_lg;
        a.reduce_dt = reduce_dt;
        a.S = S;
        a.B = B;
        a.members = device ? d_members : static_cast<const void *>(members.data());
        a.columns = device ? d_columns : static_cast<const void *>(columns.data());
        a.stretches = narrow ? (device ? static_cast<const PackStretch *>(d_stretches) : stretches.data()) : nullptr;
        return a;
    }
};

struct BucketPlan {
    int32_t dtype = 0;
    int64_t S = 0;
    std::vector<int32_t> members;
    std::vector<int64_t> P, O;
    OpTable pack;
    OpTable write_back;   // reduce-scatter output -> the members' sharded gradients
};

// FSDP1 flat layout of a unit: one flat parameter of N elements, c per rank;
// parameter t at flat offset F[t].
struct FlatLayout {
    int64_t N = 0;
    int64_t c = 0;
    std::vector<int64_t> F;
};

// Per-call pointer tables of more than kInlineLarge entries (smaller ones
// travel in the launch's arguments), cached on the device by content: the
// same grads / shards / params pointers (the usual case from step to step)
// reuse an uploaded table; a new set is staged through pinned host memory and
// copied on the caller's stream.  A steady-state call records no event; a stream
// that first uses a slot uploaded on another stream waits once for the
// upload.  Rewriting a slot for a new set waits on the host for the slot's
// previous upload only, and on the device for the other streams that used it
// (acquire_table), never for the whole device.
struct PtrSlot {
    std::vector<uint64_t> key;
    uint64_t *d_table = nullptr;
    uint64_t *h_stage = nullptr;      // pinned host staging of this slot
    void *ready = nullptr;            // hipEvent_t: upload finished
    std::vector<void *> streams;      // streams ordered after the upload
    std::vector<void *> drain;        // hipEvent_t pool: other streams' work, at an eviction
    uint64_t last_use = 0;
    bool live = false;
};

constexpr int kPtrSlots = 16;

struct PtrCache {
    PtrSlot slots[kPtrSlots];
    uint64_t clock = 0;
};

constexpr uint64_t kPlanMagic = 0x6673647070616b31ull;   // "fsdppak1"

}  // namespace fsdppack

struct fsdppack_plan {
    uint64_t magic = fsdppack::kPlanMagic;
    int32_t W = 1;
    int32_t n = 0;
    bool flat = false;                        // FSDP1 flat-parameter layout (build_plan_flat)
    fsdppack::FlatLayout fl;
    std::vector<fsdppack_param_desc> params;
    std::vector<int64_t> numel, P, A;
    int64_t B = 0;
    std::vector<fsdppack::BucketPlan> buckets;
    fsdppack::OpTable copy_in, copy_out;
    fsdppack::OpTable write_back_all;         // every bucket's write-back in one launch (two or more buckets)
    uint64_t serial = 0;                      // unique among the process's plans, never reused
    // allocation-free pack: every eligible bucket's pack tables one after
    // another, as they sit in the device scratch (bucket bi at scratch_at[bi];
    // -1 for a bucket with nothing to pack or more than kInlineLarge
    // pointers), when they fit it together, so one copy serves every bucket;
    // empty otherwise
    std::vector<unsigned char> scratch_image;
    std::vector<int64_t> scratch_at;
    mutable std::atomic<bool> staged{false};  // an allocation-free pack has copied from this plan's images

    // device state (guarded by mu)
    std::mutex mu;
    int device = -1;
    bool uploaded = false;
    std::vector<fsdppack::PtrCache> caches;   // pack per bucket, copy-in, copy-out, write-back per bucket,
                                              // write-back of all buckets
};

namespace fsdppack {

// Build the plan (host work only).  Returns a status code and fills `err`.
int build_plan(const fsdppack_param_desc *params, int32_t n, int32_t world, fsdppack_plan *plan,
               std::string &err);

// Build an FSDP1 flat-parameter plan (one reduction dtype and one param
// dtype for the unit).
int build_plan_flat(const fsdppack_param_desc *params, int32_t n, int32_t world, fsdppack_plan *plan,
                    std::string &err);

// Real elements of parameter t on rank r: the rank chunk's (per-parameter
// layout) or the piece inside the rank's flat positions (flat layout).
int64_t shard_elements(const fsdppack_plan &plan, int32_t t, int32_t r);

// Lay every bucket's pack tables out as the allocation-free pack copies them
// into the device scratch: one plan-wide image when they fit it together,
// else one image per bucket that fits alone.
void build_scratch_images(fsdppack_plan *plan);

// The stretch records of a narrow pack table (op.stretches): for each
// column-map stretch, the members of at least one window's length
// overlapping its bytes extended one window to the left, when there are one
// or two of them (else none); then records
// with no candidate up to the stretch of the last byte of the grid's last
// window of a row.
void build_pack_stretches(OpTable &op);

}  // namespace fsdppack
