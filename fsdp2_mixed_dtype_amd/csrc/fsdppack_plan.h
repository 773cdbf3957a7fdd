// fsdppack_plan.h -- host-side plan of one fully_shard unit (internal).
//
// The planner follows "PyTorch adds per-parameter mixed precision to FSDP2"
// (ainewsletter.today), paragraph 2, for bucketing (one reduction buffer per
// effective reduction dtype), and "The unit you wrapped" (kernels.rudrite.com),
// padding paragraphs, for the equal right-padded rank pieces.  It also builds
// the three work lists the kernels consume (segments + prefix map).
#pragma once

#include <cstdint>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/fsdppack.h"
#include "fsdppack_internal.h"

namespace fsdppack {

// A work list and, once uploaded, its device copy.
struct WorkList {
    std::vector<Seg> segs;
    std::vector<Item> items;          // n_items records, stored by item_slot()
    int64_t dst_bytes = 0;            // bytes the list writes
    int64_t src_bytes = 0;            // bytes the list reads
    // device side (owned by the plan)
    Seg *d_segs = nullptr;
    Item *d_items = nullptr;
    int32_t n_items() const { return static_cast<int32_t>(items.size()); }
};

struct BucketPlan {
    int32_t dtype = 0;
    int64_t S = 0;
    std::vector<int32_t> members;
    std::vector<int64_t> P, O;
    WorkList pack;
};

// Per-call pointer tables, cached on the device by content: the same grads /
// shards / params pointers (the usual case from step to step) reuse an
// uploaded table; a new set is staged through pinned host memory and copied
// on the caller's stream.  A steady-state call records no event: a slot is
// only rewritten after a device-wide synchronisation (eviction is rare), and
// a stream that first uses a slot uploaded on another stream waits once for
// the upload.
struct PtrSlot {
    std::vector<uint64_t> key;
    uint64_t *d_table = nullptr;
    uint64_t *h_stage = nullptr;      // pinned host staging of this slot
    void *ready = nullptr;            // hipEvent_t: upload finished
    std::vector<void *> streams;      // streams ordered after the upload
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
    std::vector<fsdppack_param_desc> params;
    std::vector<int64_t> numel, P, A;
    int64_t B = 0;
    std::vector<fsdppack::BucketPlan> buckets;
    fsdppack::WorkList copy_in, copy_out;
    int64_t item_bytes = 0;

    // device state (guarded by mu)
    std::mutex mu;
    int device = -1;
    bool uploaded = false;
    std::vector<fsdppack::PtrCache> caches;   // one per bucket, then copy-in, copy-out
};

namespace fsdppack {

// Build the plan (host work only).  Returns a status code and fills `err`.
int build_plan(const fsdppack_param_desc *params, int32_t n, int32_t world, int64_t item_bytes,
               fsdppack_plan *plan, std::string &err);

// Cut a segment list into items of about `item_bytes` destination bytes;
// vpos[i] is segment i's position in a virtual destination space
// (monotonic; gaps allowed) so that cuts land on aligned offsets.
void build_items(const std::vector<Seg> &segs, const std::vector<int64_t> &vpos, int64_t item_bytes,
                 std::vector<Item> &items);

}  // namespace fsdppack
